// Float32 grouped GEMM over group-sorted rows, shared by GroupedMatMul
// (ONNX operator page "GroupedMatMul - 29", Summary) and the float MoE
// operator's FC1, FC3 and FC2 (com.microsoft.MoE README, Inputs):
//
//   out[orow(p), n] = sum_k a[arow(p), k] * W[g](k, n)  (+ bias[g, n])
//
// for every sorted position p of a tile whose rows all belong to group g.
// The rows come from the routing front end (route.hip): its stable
// permutation perm maps sorted position -> slot id, and its tile table cuts
// each group's positions into tiles.  Operand row arow(p) is
// a_perm[p] / a_div (rows gathered from tokens) or p (rows already in sorted
// order); output row orow(p) is perm[p] (by slot id) or p (sorted order).
// W[g](k, n) is w[g][k][n] (KN layout, GroupedMatMul's weights [G, K, N]) or
// w[g][n][k] (NK layout, the MoE weights whose rows are output features).
// Tiles of group g >= G write zero rows (GroupedMatMul's invalid indices).
//
// All products and sums are float32 on v_mfma_f32_16x16x4_f32 (fp32 operands,
// fp32 accumulation); the bias is added last.
//
// Two kernels:
//  * qmoe_gmm_f32: LDS-tiled, 64-row x 128-column tiles, 4 wavefronts of
//    32 x 64, both operands of each 16-deep K step staged in LDS (double
//    buffered, the next step's loads in flight during the matrix
//    instructions).  Any K, N, alignment (scalar loads off the vector path).
//  * qmoe_gmm_f32_rows16: weight streaming for tiles of at most 16 rows: each
//    wavefront owns 64 columns of one tile and streams that strip of W[g]
//    from HBM straight into matrix-core operands (no LDS, no barriers).
#include <type_traits>

#include "common.hpp"
#include "launch.h"

namespace qmoe {

namespace {

constexpr int kGM = 64;            // tile rows
constexpr int kGN = 128;           // tile columns
constexpr int kGK = 16;            // K per step
constexpr int kGThreads = 256;
constexpr int kAStride = kGK + 1;  // LDS floats per A row, and per B column in NK layout (bank spread)
constexpr int kBStride = kGN + 16; // LDS floats per B row in KN layout (bank spread)
constexpr int kBBuf = kGK * kBStride > kGN * kAStride ? kGK * kBStride : kGN * kAStride;

}  // namespace

// Index conversion: out[j] = idx[j] if 0 <= idx[j] < G, else G.
template <typename IT>
__global__ void __launch_bounds__(256) qmoe_gmm_index(const IT* __restrict__ idx, long n, int G,
                                                      int* __restrict__ out) {
  const long j = (long)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  const IT v = idx[j];
  out[j] = (v >= 0 && v < (IT)G) ? (int)v : G;
}

__device__ __forceinline__ int gmm_arow(const F32Gemm& g, int p) { return g.a_perm ? g.a_perm[p] / g.a_div : p; }
__device__ __forceinline__ int gmm_orow(const F32Gemm& g, int p) { return g.out_by_slot ? g.perm[p] : p; }

// VEC: 16-byte loads (K % 4 == 0, a and w 16-byte aligned; KN also N % 4 == 0).
template <bool NK, bool VEC>
__global__ void __launch_bounds__(kGThreads) qmoe_gmm_f32(const F32Gemm g, int nblk) {
  __shared__ __attribute__((aligned(16))) float sa[2][kGM * kAStride];
  __shared__ __attribute__((aligned(16))) float sb[2][kBBuf];
  __shared__ int s_arow[kGM];
  __shared__ int s_orow[kGM];
  // one workgroup per (tile, 128-column block); column blocks of a tile are
  // adjacent, so they run together and share its operand rows in L2
  const int tile = blockIdx.x / nblk;
  if (tile >= g.ntiles[0]) return;
  const int grp = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int n0 = (blockIdx.x % nblk) * kGN;
  const int K = g.K, N = g.N;
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col = lane & 15, kq = lane >> 4;

  if (tid < kGM) {
    const int p = p0 + min(tid, rows - 1);
    s_arow[tid] = gmm_arow(g, p);
    s_orow[tid] = gmm_orow(g, p);
  }
  __syncthreads();

  if (grp >= g.G) {
    for (int idx = tid; idx < rows * kGN; idx += kGThreads) {
      const int rr = idx / kGN, c = idx % kGN;
      if (n0 + c < N) g.out[(long)s_orow[rr] * N + n0 + c] = 0.f;
    }
    return;
  }

  // Global -> register staging of one K step.  A: row tid / 4, four k from
  // 4 * (tid % 4).  B, KN: k row tid / 16, eight columns from 8 * (tid % 16);
  // NK: column tid / 2, eight k from 8 * (tid % 2).  Elements past K or N
  // are zero; rows past the tile re-read a valid row.
  const float* arow = g.a + (long)s_arow[tid >> 2] * K;
  const float* wg = g.w + (long)grp * K * N;
  const int ak = (tid & 3) * 4;
  const int bk = NK ? (tid & 1) * 8 : tid >> 4;
  const int bn = NK ? tid >> 1 : (tid & 15) * 8;
  f32x4 ra;
  f32x4 rb[2];
  // VEC: unconditional 16-byte loads (addresses clamped into the row and the
  // matrix), the pieces past K or N zeroed at the LDS store, so that no load
  // waits on a branch (per-lane conditional loads with a scalar fallback
  // made each load wait on the one before)
  auto load = [&](int kt) {
    const int k0 = kt * kGK;
    if constexpr (VEC) {
      ra = *(const f32x4*)(arow + min(k0 + ak, K - 4));
      if (NK) {
        const float* brow = wg + (long)min(n0 + bn, N - 1) * K;
#pragma unroll
        for (int h = 0; h < 2; ++h) rb[h] = *(const f32x4*)(brow + min(k0 + bk + 4 * h, K - 4));
      } else {
        const float* brow = wg + (long)min(k0 + bk, K - 1) * N;
#pragma unroll
        for (int h = 0; h < 2; ++h) rb[h] = *(const f32x4*)(brow + min(n0 + bn + 4 * h, N - 4));
      }
      return;
    }
    if (VEC && k0 + ak + 4 <= K) {
      ra = *(const f32x4*)(arow + k0 + ak);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = k0 + ak + i < K ? arow[k0 + ak + i] : 0.f;
    }
    if (NK) {
      const int n = n0 + bn;
      const float* brow = wg + (long)min(n, N - 1) * K;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = k0 + bk + 4 * h;
        if (VEC && n < N && kk + 4 <= K) {
          rb[h] = *(const f32x4*)(brow + kk);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) rb[h][i] = (n < N && kk + i < K) ? brow[kk + i] : 0.f;
        }
      }
    } else {
      const int kk = k0 + bk;
      const float* brow = wg + (long)min(kk, K - 1) * N;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = n0 + bn + 4 * h;
        if (VEC && kk < K && n + 4 <= N) {
          rb[h] = *(const f32x4*)(brow + n);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) rb[h][i] = (kk < K && n + i < N) ? brow[n + i] : 0.f;
        }
      }
    }
  };
  auto store = [&](int buf, int kt) {
    if constexpr (VEC) {
      const int k0 = kt * kGK;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      if (k0 + ak >= K) ra = z;  // K % 4 == 0: a piece is all in or out
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool ok = NK ? (n0 + bn < N && k0 + bk + 4 * h < K) : (k0 + bk < K && n0 + bn + 4 * h < N);
        if (!ok) rb[h] = z;
      }
    }
    float* a = sa[buf] + (tid >> 2) * kAStride + ak;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = ra[i];
    if (NK) {
      // B column bn, k from bk: the same row layout as A
      float* b = sb[buf] + bn * kAStride + bk;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) b[4 * h + i] = rb[h][i];
    } else {
      float* b = sb[buf] + bk * kBStride + bn;
      *(f32x4*)b = rb[0];
      *(f32x4*)(b + 4) = rb[1];
    }
  };

  f32x4 acc[2][4];
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = zero4;

  // Main loop, instantiated for the number of this wavefront's 16-row
  // subtiles that hold a row of the tile (chosen once: subtiles wholly past
  // the tile's rows run no matrix instructions, only their share of the
  // staging and the barriers).
  const int nk = (K + kGK - 1) / kGK;
  //   MSN = 0..2: that many subtiles, fixed for the loop ([K,N] weights);
  //   MSN = -1: both subtiles with the test per instruction group ([N,K]
  //   weights: the schedule the compiler makes of this form measured faster
  //   there, the fixed form faster for [K,N]).
  const bool live_rt[2] = {wm * 32 < rows, wm * 32 + 16 < rows};
  auto mainloop = [&](auto msn_tag) {
    constexpr int MSR = decltype(msn_tag)::value;
    constexpr int MSN = MSR < 0 ? 2 : MSR;
    if (nk > 0) {
      load(0);
      store(0, 0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) load(kt + 1);
      const float* a = sa[buf];
      const float* b = sb[buf];
#pragma unroll
      for (int k4 = 0; k4 < kGK / 4; ++k4) {
        // A operand: lane holds A[row col][k kq]; B operand: B[k kq][column col]
        float av[2], bv[4];
#pragma unroll
        for (int ms = 0; ms < MSN; ++ms) av[ms] = a[(wm * 32 + ms * 16 + col) * kAStride + k4 * 4 + kq];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          const int c = wn * 64 + ns * 16 + col;
          if (MSN > 0) bv[ns] = NK ? b[c * kAStride + k4 * 4 + kq] : b[(k4 * 4 + kq) * kBStride + c];
        }
#pragma unroll
        for (int ms = 0; ms < MSN; ++ms)
          if (MSR >= 0 || live_rt[ms])
#pragma unroll
            for (int ns = 0; ns < 4; ++ns)
              acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ms], bv[ns], acc[ms][ns], 0, 0, 0);
      }
      // the other buffer was last read in the previous step, finished by every
      // wavefront before the last barrier
      if (kt + 1 < nk) store(buf ^ 1, kt + 1);
      __syncthreads();
    }
  };
  const int live = min(max(rows - wm * 32, 0), 32);  // rows of this wavefront's 32
  if constexpr (NK) mainloop(std::integral_constant<int, -1>{});
  else if (live > 16) mainloop(std::integral_constant<int, 2>{});
  else if (live > 0) mainloop(std::integral_constant<int, 1>{});
  else mainloop(std::integral_constant<int, 0>{});

  // Output: lane holds rows 4 * kq + i of column col of each 16 x 16 subtile.
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    const int c = n0 + wn * 64 + ns * 16 + col;
    if (c >= N) continue;
    const float bv = g.bias ? g.bias[(long)grp * N + c] : 0.f;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = wm * 32 + ms * 16 + 4 * kq + i;
        if (rr < rows) g.out[(long)s_orow[rr] * N + c] = acc[ms][ns][i] + bv;
      }
  }
}

// Weight-streaming variant for tiles of at most 16 rows.  K is walked in
// groups of KG = 16 V: the 4 V MFMAs of a group take k = KG kg + 4 V kq + j
// (j < 4 V) in lane group kq, so V 16-byte loads of the operand row cover
// them.  Columns of MFMA block i (c = 0..15):
//   KN: n0 + 4c + i: one 16-byte load per lane and k row fetches a 256-byte
//       row segment serving all four blocks, and the results leave as
//       16-byte stores;
//   NK: n0 + 16i + c: V 16-byte loads per lane and block fetch 16 V
//       consecutive bytes of its weight row (V = 2: whole 128-byte lines per
//       four lanes).
// KSPLIT = 1: the four wavefronts of a workgroup take four 64-column strips;
// KSPLIT = 4: they take four K ranges of one strip and add their partial
// sums through LDS in wavefront order (for narrow N, to keep enough
// wavefronts streaming).  kSD groups of loads stay in flight ahead of the
// matrix instructions.  Requires K % 4 == 0 and 16-byte aligned a, w (KN:
// also N % 4 == 0 and 16-byte aligned bias and out).
template <bool NK>
struct StreamShape {
  static constexpr int V = NK ? 2 : 1;  // 16-byte vectors per lane and row per K group
  static constexpr int KG = 16 * V;     // K per group
  static constexpr int SD = NK ? 2 : 4; // groups in flight
};

template <bool NK, int KSPLIT>
__global__ void __launch_bounds__(256) qmoe_gmm_f32_rows16(const F32Gemm g, int nblk) {
  using SS = StreamShape<NK>;
  constexpr int V = SS::V, KG = SS::KG, SD = SS::SD;
  constexpr int NB = 4 * V;  // 16-byte B loads per lane and group (NK: V per block; KN: one per k row)
  const int tile = blockIdx.x / nblk;
  if (tile >= g.ntiles[0]) return;
  const int grp = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int K = g.K, N = g.N;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int n0 = KSPLIT == 1 ? (blockIdx.x % nblk) * 256 + wave * 64 : (blockIdx.x % nblk) * 64;
  if (n0 >= N) return;  // whole wavefront (whole workgroup when KSPLIT > 1): before any barrier
  const int c = lane & 15, kq = lane >> 4;
  // output rows of this lane: 4 kq + t
  int orow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) orow[t] = 4 * kq + t < rows ? gmm_orow(g, p0 + 4 * kq + t) : -1;
  // columns of this lane: KN n0 + 4c + i (all or none valid, N % 4 == 0);
  // NK n0 + 16i + c (each checked)
  bool cok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) cok[i] = (NK ? n0 + 16 * i + c : n0 + 4 * c) < N;
  if (grp >= g.G) {
    if (KSPLIT > 1 && wave > 0) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (orow[t] < 0) continue;
      float* o = g.out + (long)orow[t] * N;
      if (NK) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (cok[i]) o[n0 + 16 * i + c] = 0.f;
      } else if (cok[0]) {
        *(f32x4*)(o + n0 + 4 * c) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }
  // K groups of this wavefront: [g0, g1) of the nfull full groups; the last
  // K range also takes the tail
  const int nfull = K / KG;
  const int g0 = KSPLIT == 1 ? 0 : (int)((long)nfull * wave / KSPLIT);
  const int g1 = KSPLIT == 1 ? nfull : (int)((long)nfull * (wave + 1) / KSPLIT);
  const bool tail = nfull * KG < K && (KSPLIT == 1 || wave == KSPLIT - 1);
  const float* arow = g.a + (long)gmm_arow(g, p0 + min(c, rows - 1)) * K + 4 * V * kq;
  const float* wg = g.w + (long)grp * K * N;
  // weight pointers of this lane at k = 4 V kq (NK: one per block; KN: that k
  // row, the rows below it N apart); lanes past N re-read a valid column
  const float* wp[NK ? 4 : 1];
  if (NK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) wp[i] = wg + (long)min(n0 + 16 * i + c, N - 1) * K + 4 * V * kq;
  } else {
    wp[0] = wg + (cok[0] ? n0 + 4 * c : 0) + (long)(4 * V * kq) * N;
  }
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ra[d][v] = operand k KG kg + 4 V kq + 4 v .. + 3
  // KN: rb[d][j] = columns n0 + 4c .. + 3 at k row KG kg + 4 V kq + j
  // NK: rb[d][V i + v] = k KG kg + 4 V kq + 4 v .. + 3 of column n0 + 16 i + c
  f32x4 ra[SD][V], rb[SD][NB];
  auto load = [&](int slot, int kg) {
    const long k = (long)kg * KG;
#pragma unroll
    for (int v = 0; v < V; ++v) ra[slot][v] = *(const f32x4*)(arow + k + 4 * v);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (NK) rb[slot][b] = *(const f32x4*)(wp[b / V] + k + 4 * (b % V));
      else rb[slot][b] = *(const f32x4*)(wp[0] + (k + b) * N);
    }
  };
  auto mma = [&](int slot) {
#pragma unroll
    for (int j = 0; j < 4 * V; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float av = ra[slot][j / 4][j % 4];
        const float bv = NK ? rb[slot][V * i + j / 4][j % 4] : rb[slot][j][i];
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[i], 0, 0, 0);
      }
  };
  // Branch-free pipeline (exact load counts for the waits): past the last
  // group of the range the loads repeat it, and those values are never used.
  if (g1 > g0) {
    int kg = g0;
#pragma unroll
    for (int d = 0; d < SD; ++d) load(d, min(g0 + d, g1 - 1));
    for (; kg + SD <= g1; kg += SD) {
#pragma unroll
      for (int d = 0; d < SD; ++d) {
        mma(d);
        load(d, min(kg + SD + d, g1 - 1));
        // keep each refill right behind the matrix instructions that free
        // its registers, ahead of the next group's waits
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int d = 0; d < SD; ++d)
      if (kg + d < g1) mma(d);
  }
  if (tail) {
    // tail group: k past K reads as zero on both operands
    const int kb = nfull * KG;
    const int k0 = kb + 4 * V * kq;
#pragma unroll
    for (int j = 0; j < 4 * V; ++j) ra[0][j / 4][j % 4] = k0 + j < K ? arow[kb + j] : 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // NK: element e of vector b % V of column b / V; KN: column e of k row b
        const int j = NK ? 4 * (b % V) + e : b;
        const bool ok = k0 + j < K;
        if (NK) rb[0][b][e] = ok ? wp[b / V][kb + j] : 0.f;
        else rb[0][b][e] = ok ? wp[0][(long)(kb + j) * N + e] : 0.f;
      }
    mma(0);
  }
  if (KSPLIT > 1) {
    // partial sums of waves 1.. through LDS, added in wavefront order
    __shared__ f32x4 red[KSPLIT > 1 ? KSPLIT - 1 : 1][4][64];
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < KSPLIT - 1; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += red[w][i][lane];
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (orow[t] < 0) continue;
    float* o = g.out + (long)orow[t] * N;
    if (NK) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + 16 * i + c;
        if (cok[i]) o[n] = acc[i][t] + (g.bias ? g.bias[(long)grp * N + n] : 0.f);
      }
    } else if (cok[0]) {
      const int n = n0 + 4 * c;
      const f32x4 bv = g.bias ? *(const f32x4*)(g.bias + (long)grp * N + n) : f32x4{0.f, 0.f, 0.f, 0.f};
      *(f32x4*)(o + n) = f32x4{acc[0][t] + bv[0], acc[1][t] + bv[1], acc[2][t] + bv[2], acc[3][t] + bv[3]};
    }
  }
}

int gmm_tile_rows() { return kGM; }
int gmm_rows16_tile_rows() { return 16; }

hipError_t launch_gmm_rows16(const F32Gemm& g, bool nk, int ksplit, int max_tiles, hipStream_t st) {
  if (max_tiles <= 0 || g.N <= 0) return hipSuccess;
  if (g.K % 4 != 0 || (!nk && g.N % 4 != 0)) return hipErrorInvalidValue;
  if (ksplit != 1 && ksplit != 4) return hipErrorInvalidValue;
  const int cols = ksplit == 1 ? 256 : 64;  // columns per workgroup
  const int nblk = (g.N + cols - 1) / cols;
  const dim3 grid((unsigned)((long)max_tiles * nblk)), block(256);
  if (nk) {
    if (ksplit == 1) hipLaunchKernelGGL((qmoe_gmm_f32_rows16<true, 1>), grid, block, 0, st, g, nblk);
    else hipLaunchKernelGGL((qmoe_gmm_f32_rows16<true, 4>), grid, block, 0, st, g, nblk);
  } else {
    if (ksplit == 1) hipLaunchKernelGGL((qmoe_gmm_f32_rows16<false, 1>), grid, block, 0, st, g, nblk);
    else hipLaunchKernelGGL((qmoe_gmm_f32_rows16<false, 4>), grid, block, 0, st, g, nblk);
  }
  return hipGetLastError();
}

int gmm_rows16_ksplit(long est_tiles, int N) {
  // wavefronts streaming with one strip per wavefront; below about two
  // thousand (eight per compute unit) the K ranges are split four ways
  const long waves = est_tiles * ((N + 255) / 256) * 4;
  return waves < 2048 ? 4 : 1;
}

hipError_t launch_gmm_index(const void* idx, bool idx64, long n, int G, int* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((n + 255) / 256), block(256);
  if (idx64) hipLaunchKernelGGL(qmoe_gmm_index<int64_t>, grid, block, 0, st, (const int64_t*)idx, n, G, out);
  else hipLaunchKernelGGL(qmoe_gmm_index<int32_t>, grid, block, 0, st, (const int32_t*)idx, n, G, out);
  return hipGetLastError();
}

hipError_t launch_gmm_f32(const F32Gemm& g, bool nk, bool vec, int max_tiles, hipStream_t st) {
  if (max_tiles <= 0 || g.N <= 0) return hipSuccess;
  if (vec && (g.K % 4 != 0 || (!nk && g.N % 4 != 0))) return hipErrorInvalidValue;
  const int nblk = (g.N + kGN - 1) / kGN;
  const dim3 grid((unsigned)((long)max_tiles * nblk)), block(kGThreads);
  if (nk) {
    if (vec) hipLaunchKernelGGL((qmoe_gmm_f32<true, true>), grid, block, 0, st, g, nblk);
    else hipLaunchKernelGGL((qmoe_gmm_f32<true, false>), grid, block, 0, st, g, nblk);
  } else {
    if (vec) hipLaunchKernelGGL((qmoe_gmm_f32<false, true>), grid, block, 0, st, g, nblk);
    else hipLaunchKernelGGL((qmoe_gmm_f32<false, false>), grid, block, 0, st, g, nblk);
  }
  return hipGetLastError();
}

}  // namespace qmoe
