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
  auto load = [&](int kt) {
    const int k0 = kt * kGK;
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
  auto store = [&](int buf) {
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

  const int nk = (K + kGK - 1) / kGK;
  if (nk > 0) {
    load(0);
    store(0);
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
      for (int ms = 0; ms < 2; ++ms) av[ms] = a[(wm * 32 + ms * 16 + col) * kAStride + k4 * 4 + kq];
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const int c = wn * 64 + ns * 16 + col;
        bv[ns] = NK ? b[c * kAStride + k4 * 4 + kq] : b[(k4 * 4 + kq) * kBStride + c];
      }
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ms], bv[ns], acc[ms][ns], 0, 0, 0);
    }
    // the other buffer was last read in the previous step, finished by every
    // wavefront before the last barrier
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

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

// Weight-streaming variant for tiles of at most 16 rows.  The four MFMAs of
// one 16-deep K group take k = 16 kg + 4 kq + j (j = 0..3) in lane group kq,
// so one 16-byte load of the operand row covers them.  Columns of MFMA block
// i (c = 0..15):
//   KN: n0 + 4c + i: one 16-byte load per lane and k row fetches a 256-byte
//       row segment serving all four blocks, and the results leave as
//       16-byte stores;
//   NK: n0 + 16i + c: one 16-byte load per lane and block fetches the four
//       k of its weight row.
// kSD K groups of loads stay in flight ahead of the matrix instructions.
// Requires K % 4 == 0 and 16-byte aligned a, w (KN: also N % 4 == 0 and
// 16-byte aligned bias and out).
constexpr int kSD = 4;

template <bool NK>
__global__ void __launch_bounds__(256) qmoe_gmm_f32_rows16(const F32Gemm g, int nblk) {
  const int tile = blockIdx.x / nblk;
  if (tile >= g.ntiles[0]) return;
  const int grp = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int K = g.K, N = g.N;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x % nblk) * 256 + wave * 64;
  if (n0 >= N) return;  // whole wavefront: no barriers below
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
  const float* arow = g.a + (long)gmm_arow(g, p0 + min(c, rows - 1)) * K + 4 * kq;
  const float* wg = g.w + (long)grp * K * N;
  // weight pointers of this lane at k = 4 kq (NK: one per block; KN: k row
  // 4 kq, the rows below it N apart); lanes past N re-read a valid column
  const float* wp[NK ? 4 : 1];
  if (NK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) wp[i] = wg + (long)min(n0 + 16 * i + c, N - 1) * K + 4 * kq;
  } else {
    wp[0] = wg + (cok[0] ? n0 + 4 * c : 0) + (long)(4 * kq) * N;
  }
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nfull = K / 16;  // K groups without a tail
  // KN: rb[d][j] = columns n0 + 4c .. + 3 at k row 16 kg + 4 kq + j
  // NK: rb[d][i] = k 16 kg + 4 kq .. + 3 of column n0 + 16 i + c
  f32x4 ra[kSD], rb[kSD][4];
  auto load = [&](int slot, int kg) {
    const long k = (long)kg * 16;
    ra[slot] = *(const f32x4*)(arow + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[slot][i] = NK ? *(const f32x4*)(wp[i] + k) : *(const f32x4*)(wp[0] + (k + i) * N);
  };
  auto mma = [&](int slot) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(ra[slot][j], NK ? rb[slot][i][j] : rb[slot][j][i], acc[i], 0,
                                                      0, 0);
  };
  // Branch-free pipeline (exact load counts for the waits): past the last
  // full group the loads repeat it, and those values are never used.
  int kg = 0;
  if (nfull > 0) {
#pragma unroll
    for (int d = 0; d < kSD; ++d) load(d, min(d, nfull - 1));
    for (; kg + kSD <= nfull; kg += kSD) {
#pragma unroll
      for (int d = 0; d < kSD; ++d) {
        mma(d);
        load(d, min(kg + kSD + d, nfull - 1));
      }
    }
#pragma unroll
    for (int d = 0; d < kSD; ++d)
      if (kg + d < nfull) mma(d);
  }
  if (nfull * 16 < K) {
    // tail group: k past K reads as zero on both operands
    const int kb = nfull * 16;
    const int k0 = kb + 4 * kq;
#pragma unroll
    for (int j = 0; j < 4; ++j) ra[0][j] = k0 + j < K ? arow[kb + j] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = k0 + j < K;
        // NK: element j of column i; KN: element i of k row j (pointer of row j)
        if (NK) rb[0][i][j] = ok ? wp[i][kb + j] : 0.f;
        else rb[0][j][i] = ok ? wp[0][(long)(kb + j) * N + i] : 0.f;
      }
    mma(0);
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

hipError_t launch_gmm_rows16(const F32Gemm& g, bool nk, int max_tiles, hipStream_t st) {
  if (max_tiles <= 0 || g.N <= 0) return hipSuccess;
  if (g.K % 4 != 0 || (!nk && g.N % 4 != 0)) return hipErrorInvalidValue;
  const int nblk = (g.N + 255) / 256;
  const dim3 grid((unsigned)((long)max_tiles * nblk)), block(256);
  if (nk) hipLaunchKernelGGL(qmoe_gmm_f32_rows16<true>, grid, block, 0, st, g, nblk);
  else hipLaunchKernelGGL(qmoe_gmm_f32_rows16<false>, grid, block, 0, st, g, nblk);
  return hipGetLastError();
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
