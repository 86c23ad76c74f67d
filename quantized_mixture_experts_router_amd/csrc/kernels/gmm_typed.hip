// GroupedMatMul (ONNX operator page "GroupedMatMul - 29", Summary) in the
// page's other floating types, float16, bfloat16 and double (Type
// Constraints):
//
//   out[perm(p), n] = sum_k x[a_perm(p) / S, k] * W[g](k, n)  (+ bias[g, n])
//
// over group-sorted rows, with W[g](k, n) = w[g][k][n] (weights [G, K, N]);
// tiles of group g >= G write zero rows (indices outside [0, G)).  The rows,
// permutation and tile table come from the routing front end (route.hip),
// exactly as for float32 (gmm.hip).
//
// Arithmetic, per type:
//  * float16 / bfloat16: products on v_mfma_f32_16x16x32_f16 / _bf16 (exact
//    products of the 16-bit operands, fp32 accumulation); the bias is added
//    in fp32 and the sum rounded once to the output type (round to nearest
//    even);
//  * double: v_mfma_f64_16x16x4_f64 (fp64 products and accumulation), bias
//    added in fp64.
//
// Work decomposition: a workgroup of 4 wavefronts computes a 64-row x
// 128-column tile (2 x 2 wavefronts of 32 x 64); each K step's operand slice
// of both operands is staged in LDS, double buffered, the next step's loads
// in flight during the matrix instructions.  The 16-bit types keep the
// weight slice transposed in LDS (column-major, K contiguous), so each lane
// reads its 8 consecutive K values of a column as one 16-byte load; the
// double kernel's 16x16x4 instruction takes one K value a lane and reads the
// slice as stored.
#include <cstdlib>
#include <string>
#include <type_traits>

#include "common.hpp"
#include "launch.h"

namespace qmoe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kYM = 64;     // tile rows
constexpr int kYN = 128;    // tile columns
constexpr int kYThreads = 256;

template <typename ET>
struct Ty;
template <>
struct Ty<_Float16> {
  static constexpr int KS = 32;  // K per step: one 16x16x32 instruction
  using Frag = f16x8;
  using Acc = f32x4;
  using AccT = float;
  static __device__ __forceinline__ Acc mma(const Frag& a, const Frag& b, const Acc& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Ty<__bf16> {
  static constexpr int KS = 32;
  using Frag = bf16x8;
  using Acc = f32x4;
  using AccT = float;
  static __device__ __forceinline__ Acc mma(const Frag& a, const Frag& b, const Acc& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Ty<double> {
  static constexpr int KS = 16;  // K per step: four 16x16x4 instructions
  using Frag = double;
  using Acc = f64x4;
  using AccT = double;
  static __device__ __forceinline__ Acc mma(double a, double b, const Acc& c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
};

}  // namespace

// VEC: 16-byte loads (x and w 16-byte aligned, K and N whole 16-byte runs).
template <typename ET, bool VEC>
__global__ void __launch_bounds__(kYThreads) qmoe_gmm_typed(const TypedGemm g, int nblk) {
  using T = Ty<ET>;
  constexpr bool WIDE = sizeof(ET) == 8;      // double: 16x16x4, one K value a lane
  constexpr int KS = T::KS;
  constexpr int EV = 16 / sizeof(ET);         // elements per 16-byte load
  // LDS: A [row][k] (+ padding); B 16-bit: [column][k] (transposed), double: [k][column]
  constexpr int AST = WIDE ? KS + 1 : KS + 8;
  constexpr int BST = WIDE ? kYN + 2 : KS + 8;
  constexpr int BLEN = WIDE ? KS * BST : kYN * BST;
  __shared__ __attribute__((aligned(16))) ET sa[2][kYM * AST];
  __shared__ __attribute__((aligned(16))) ET sb[2][BLEN];
  __shared__ int s_arow[kYM];
  __shared__ int s_orow[kYM];

  const int tile = blockIdx.x / nblk;
  if (tile >= g.ntiles[0]) return;
  const int n0 = (blockIdx.x % nblk) * kYN;
  const int grp = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int K = g.K, N = g.N;
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col = lane & 15, kq = lane >> 4;
  ET* out = static_cast<ET*>(g.out);

  if (tid < kYM) {
    const int p = p0 + min(tid, rows - 1);
    s_arow[tid] = g.a_perm[p] / g.a_div;
    s_orow[tid] = g.perm[p];
  }
  __syncthreads();

  if (grp >= g.G) {  // index outside [0, G): zero rows
    for (int idx = tid; idx < rows * kYN; idx += kYThreads) {
      const int rr = idx / kYN, c = idx % kYN;
      if (n0 + c < N) out[(long)s_orow[rr] * N + n0 + c] = (ET)0.f;
    }
    return;
  }

  const ET* x = static_cast<const ET*>(g.a);
  const ET* wg = static_cast<const ET*>(g.w) + (long)grp * K * N;
  // Staging of one K step, global -> registers -> LDS.  Elements past K or
  // N read as zero; rows past the tile re-read a valid row.
  //  A: KS x 64 elements, row tid / 4, AQ = KS / 4 consecutive k from
  //     AQ * (tid % 4);
  //  B: KS x 128 elements, BQ = KS * 128 / 256 a thread, in runs of EV
  //     consecutive columns of one k row.
  constexpr int AQ = KS / 4;                 // 8 (16-bit) or 4 (double)
  constexpr int BQ = KS * kYN / kYThreads;   // 16 or 8
  constexpr int BR = BQ / EV;                // 16-byte runs a thread: 2 or 4
  const ET* arow = x + (long)s_arow[tid >> 2] * K;
  const int ak = (tid & 3) * AQ;
  ET ra[AQ];
  ET rb[BR][EV];
  // VEC: unconditional 16-byte loads (addresses clamped into the row and the
  // matrix; K and N are whole runs of EV), the pieces past K or N zeroed at
  // the LDS store, so that no load waits on a branch
  u32x4 va[AQ / EV], vb[BR];
  auto load = [&](int kt) {
    const int k0 = kt * KS;
    if constexpr (VEC) {
#pragma unroll
      for (int h = 0; h < AQ / EV; ++h) va[h] = *(const u32x4*)(arow + min(k0 + ak + h * EV, K - EV));
#pragma unroll
      for (int r = 0; r < BR; ++r) {
        const int idx = tid + r * kYThreads;
        const int k = idx / (kYN / EV), n = (idx % (kYN / EV)) * EV;
        vb[r] = *(const u32x4*)(wg + (long)min(k0 + k, K - 1) * N + min(n0 + n, N - EV));
      }
      return;
    }
#pragma unroll
    for (int h = 0; h < AQ / EV; ++h) {
      const int kk = k0 + ak + h * EV;
      if (VEC && kk + EV <= K) {
        const u32x4 v = *(const u32x4*)(arow + kk);
        const ET* e = reinterpret_cast<const ET*>(&v);
#pragma unroll
        for (int i = 0; i < EV; ++i) ra[h * EV + i] = e[i];
      } else {
#pragma unroll
        for (int i = 0; i < EV; ++i) ra[h * EV + i] = kk + i < K ? arow[kk + i] : (ET)0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < BR; ++r) {
      const int idx = tid + r * kYThreads;
      const int k = idx / (kYN / EV), n = (idx % (kYN / EV)) * EV;
      const int kk = k0 + k, nn = n0 + n;
      const ET* src = wg + (long)min(kk, K - 1) * N + nn;
      if (VEC && kk < K && nn + EV <= N) {
        const u32x4 v = *(const u32x4*)src;
        const ET* e = reinterpret_cast<const ET*>(&v);
#pragma unroll
        for (int i = 0; i < EV; ++i) rb[r][i] = e[i];
      } else {
#pragma unroll
        for (int i = 0; i < EV; ++i) rb[r][i] = (kk < K && nn + i < N) ? src[i] : (ET)0.f;
      }
    }
  };
  auto store = [&](int buf, int kt) {
    if constexpr (VEC) {
      const int k0 = kt * KS;
      const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int h = 0; h < AQ / EV; ++h) {
        const u32x4 v = k0 + ak + h * EV < K ? va[h] : z4;
        const ET* e = reinterpret_cast<const ET*>(&v);
#pragma unroll
        for (int i = 0; i < EV; ++i) ra[h * EV + i] = e[i];
      }
#pragma unroll
      for (int r = 0; r < BR; ++r) {
        const int idx = tid + r * kYThreads;
        const int k = idx / (kYN / EV), n = (idx % (kYN / EV)) * EV;
        const u32x4 v = (k0 + k < K && n0 + n < N) ? vb[r] : z4;
        const ET* e = reinterpret_cast<const ET*>(&v);
#pragma unroll
        for (int i = 0; i < EV; ++i) rb[r][i] = e[i];
      }
    }
    ET* a = sa[buf] + (tid >> 2) * AST + ak;
#pragma unroll
    for (int i = 0; i < AQ; ++i) a[i] = ra[i];
#pragma unroll
    for (int r = 0; r < BR; ++r) {
      const int idx = tid + r * kYThreads;
      const int k = idx / (kYN / EV), n = (idx % (kYN / EV)) * EV;
#pragma unroll
      for (int i = 0; i < EV; ++i) {
        if constexpr (WIDE) sb[buf][k * BST + n + i] = rb[r][i];
        else sb[buf][(n + i) * BST + k] = rb[r][i];
      }
    }
  };

  typename T::Acc acc[2][4];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = typename T::Acc{};

  const int nk = (K + KS - 1) / KS;
  if (nk > 0) {
    load(0);
    store(0, 0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
    const ET* a = sa[buf];
    const ET* b = sb[buf];
    if constexpr (WIDE) {
#pragma unroll
      for (int k4 = 0; k4 < KS / 4; ++k4) {
        // lane holds A[row col][k kq] and B[k kq][column col]
        double av[2], bv[4];
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) av[ms] = a[(wm * 32 + ms * 16 + col) * AST + k4 * 4 + kq];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) bv[ns] = b[(k4 * 4 + kq) * BST + wn * 64 + ns * 16 + col];
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = T::mma(av[ms], bv[ns], acc[ms][ns]);
      }
    } else {
      // lane holds A[row col][k 8kq .. 8kq + 7] and B[k 8kq .. 8kq + 7][column col]
      typename T::Frag af[2], bf[4];
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) af[ms] = *(const typename T::Frag*)(a + (wm * 32 + ms * 16 + col) * AST + 8 * kq);
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) bf[ns] = *(const typename T::Frag*)(b + (wn * 64 + ns * 16 + col) * BST + 8 * kq);
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = T::mma(af[ms], bf[ns], acc[ms][ns]);
    }
    if (kt + 1 < nk) store(buf ^ 1, kt + 1);
    __syncthreads();
  }

  // acc[ms][ns][i]: column wn*64 + ns*16 + col of row wm*32 + ms*16 +
  // 4*kq + i (16-bit types, f32 accumulators) or of row wm*32 + ms*16 + kq +
  // 4*i (double: the fp64 instruction leaves row kq + 4i of its 16 x 16 block
  // in register i of lane 16*kq + col)
  const ET* bias = static_cast<const ET*>(g.bias);
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    const int n = n0 + wn * 64 + ns * 16 + col;
    if (n >= N) continue;
    const typename T::AccT bv = bias ? (typename T::AccT)bias[(long)grp * N + n] : (typename T::AccT)0;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 32 + ms * 16 + (WIDE ? kq + 4 * i : 4 * kq + i);
        if (r < rows) out[(long)s_orow[r] * N + n] = (ET)(acc[ms][ns][i] + bv);
      }
  }
}

// 16-bit element types on MT-row tiles (64 or 128) with 16-byte aligned
// input and weights and K, N multiples of 8: the tile kernel above with
// deeper K steps (KS = 64: two matrix instructions a row subtile between
// barriers, 2 x 2 wavefronts of MT / 2 rows x 64 columns), loads
// two steps ahead in registers, and the weight slice transposed in registers
// instead of element by element in LDS: thread t loads rows 4kb .. 4kb + 3
// (kb = t / 16) of columns 8cb .. 8cb + 7 (cb = t % 16) of the step's
// [KS, 128] slice, regroups them into eight columns of four K values with
// byte permutes, and writes each as one 8-byte LDS store (columns of K
// contiguous, padded by 8 elements to spread the fragment reads over the
// banks).  A rows are staged as 16-byte pieces.
template <typename ET, int KS, int MT>
__global__ void __launch_bounds__(kYThreads) qmoe_gmm16_tiled(const TypedGemm g, int nblk) {
  using T = Ty<ET>;
  static_assert(sizeof(ET) == 2 && KS % 64 == 0 && (MT == 64 || MT == 128), "16-bit types, whole 64-K steps");
  constexpr int AST = KS + 8;   // LDS elements per A row and per B column
  constexpr int AH = MT / 64;   // 64-row halves of the A tile
  constexpr int AP = KS / 32;   // 16-byte A pieces per thread, step and half
  constexpr int BP = KS / 64;   // 4 x 8 B blocks per thread and step
  constexpr int MS = MT / 32;   // 16-row subtiles per wavefront
  __shared__ __attribute__((aligned(16))) ET sa[2][MT * AST];
  __shared__ __attribute__((aligned(16))) ET sb[2][kYN * AST];
  __shared__ int s_arow[MT];
  __shared__ int s_orow[MT];

  // Tile order: each XCD (workgroups are dealt round robin by linear id)
  // takes a contiguous run of work ids; work ids run over runs of GM row
  // tiles (consecutive tiles mostly share a group, hence weight columns),
  // column tile by column tile, row tile fastest.  Only the first linear ids
  // carry work, so every XCD gets its share of the real tiles.
  constexpr int GM = 8;
  const int mt = g.ntiles[0];
  const int total = mt * nblk;
  const int lin = blockIdx.x;
  if (lin >= total) return;
  const int per = total >> 3, extra = total & 7, xcd = lin & 7;
  const int wk = xcd * per + min(xcd, extra) + (lin >> 3);
  const int r0 = (wk / (GM * nblk)) * GM;
  const int gs = min(GM, mt - r0);
  const int wr = wk - r0 * nblk;
  const int tile = r0 + wr % gs;
  const int n0 = (wr / gs) * kYN;
  const int grp = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int K = g.K, N = g.N;
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col = lane & 15, kq = lane >> 4;
  ET* out = static_cast<ET*>(g.out);

  if (tid < MT) {
    const int p = p0 + min(tid, rows - 1);
    s_arow[tid] = g.a_perm[p] / g.a_div;
    s_orow[tid] = g.perm[p];
  }
  __syncthreads();

  if (grp >= g.G) {  // index outside [0, G): zero rows
    for (int idx = tid; idx < rows * kYN; idx += kYThreads) {
      const int rr = idx / kYN, c = idx % kYN;
      if (n0 + c < N) out[(long)s_orow[rr] * N + n0 + c] = (ET)0.f;
    }
    return;
  }

  const ET* x = static_cast<const ET*>(g.a);
  const ET* wg = static_cast<const ET*>(g.w) + (long)grp * K * N;
  const ET* arow[AH];
#pragma unroll
  for (int h = 0; h < AH; ++h) arow[h] = x + (long)s_arow[(tid >> 2) + 64 * h] * K;
  const int cb = tid & 15;
  const bool bcol = n0 + 8 * cb < N;  // all eight columns or none (N % 8 == 0)
  const ET* bcolp = wg + min(n0 + 8 * cb, N - 8);
  // B chunk swizzle: the 8-value K chunk c of column n sits at chunk
  // c ^ ((n / 16) % 8), so one store instruction's 64 lanes (16 column
  // blocks) spread over all banks; a fragment read's 16 columns share n / 16.
  const int bsw = (cb >> 1) & 7;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  // Loads are unconditional (addresses clamped into the row and the matrix)
  // so that the wait before a register set's LDS store counts only the loads
  // issued after it; values outside K or N become zeros when stored.
  auto load = [&](int kt, u32x4(&ra)[AH * AP], u32x4(&rb)[BP][4]) {
    const int k0 = kt * KS;
#pragma unroll
    for (int h = 0; h < AH; ++h)
#pragma unroll
      for (int q = 0; q < AP; ++q)
        ra[h * AP + q] = *(const u32x4*)(arow[h] + min(k0 + 8 * ((tid & 3) + 4 * q), K - 8));
#pragma unroll
    for (int q = 0; q < BP; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rb[q][r] = *(const u32x4*)(bcolp + (long)min(k0 + 4 * ((tid >> 4) + 16 * q) + r, K - 1) * N);
  };
  auto store = [&](int kt, int buf, const u32x4(&ra)[AH * AP], const u32x4(&rb)[BP][4]) {
    const int k0 = kt * KS;
#pragma unroll
    for (int h = 0; h < AH; ++h)
#pragma unroll
      for (int q = 0; q < AP; ++q)
        *(u32x4*)(sa[buf] + ((tid >> 2) + 64 * h) * AST + 8 * ((tid & 3) + 4 * q)) =
            k0 + 8 * ((tid & 3) + 4 * q) < K ? ra[h * AP + q] : z4;  // K % 8 == 0: a piece is all in or out
#pragma unroll
    for (int q = 0; q < BP; ++q) {
      const int kb = (tid >> 4) + 16 * q;
      u32x4 v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (bcol && k0 + 4 * kb + r < K) ? rb[q][r] : z4;
      const int koff = 8 * ((kb >> 1) ^ bsw) + 4 * (kb & 1);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        // column 8cb + c: its values in rows 0..3 are the low (c even) or
        // high (c odd) halves of dword c / 2
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(v[1][c >> 1], v[0][c >> 1], sel);
        const uint32_t hi = __builtin_amdgcn_perm(v[3][c >> 1], v[2][c >> 1], sel);
        *(u32x2*)(sb[buf] + (8 * cb + c) * AST + koff) = u32x2{lo, hi};
      }
    }
  };

  typename T::Acc acc[MS][4];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = typename T::Acc{};
  auto compute = [&](int buf) {
    const ET* a = sa[buf];
    const ET* b = sb[buf];
#pragma unroll
    for (int s = 0; s < KS / 32; ++s) {
      // lane holds A[row col][k 32s + 8kq .. + 7] and B[k ..][column col]
      typename T::Frag af[MS], bf[4];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
        af[ms] = *(const typename T::Frag*)(a + (wm * (MT / 2) + ms * 16 + col) * AST + 32 * s + 8 * kq);
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const int n = wn * 64 + ns * 16 + col;
        bf[ns] = *(const typename T::Frag*)(b + n * AST + 8 * ((4 * s + kq) ^ ((n >> 4) & 7)));
      }
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = T::mma(af[ms], bf[ns], acc[ms][ns]);
    }
  };

  // Register sets 0 and 1 hold the steps of even and odd index, loaded two
  // steps ahead of their use; the step count is rounded up to even (a step
  // past K is all zeros).
  const int nk = (K + KS - 1) / KS;
  const int nk2 = (nk + 1) & ~1;
  u32x4 ra0[AH * AP], ra1[AH * AP];
  u32x4 rb0[BP][4], rb1[BP][4];
  if (nk2 > 0) {
    load(0, ra0, rb0);
    load(1, ra1, rb1);
    store(0, 0, ra0, rb0);
    __syncthreads();
    for (int kt = 0; kt < nk2; kt += 2) {
      // the scheduling barriers keep each step's loads issued before its
      // matrix instructions
      load(kt + 2, ra0, rb0);
      __builtin_amdgcn_sched_barrier(0);
      compute(0);
      store(kt + 1, 1, ra1, rb1);
      __syncthreads();
      load(kt + 3, ra1, rb1);
      __builtin_amdgcn_sched_barrier(0);
      compute(1);
      store(kt + 2, 0, ra0, rb0);
      __syncthreads();
    }
  }

  // acc[ms][ns][i]: column wn*64 + ns*16 + col of row wm*MT/2 + ms*16 + 4*kq + i.
  // The rounded tile goes through LDS (the A buffers, free after the last
  // barrier of the K loop, or never used when K == 0) so that each output
  // row leaves as 16-byte pieces of whole 256-byte runs.
  constexpr int OST = kYN + 8;  // elements per staged row
  static_assert(MT * OST <= 2 * MT * AST, "the staged tile fits the A buffers");
  ET* so = &sa[0][0];
  const ET* bias = static_cast<const ET*>(g.bias);
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    const int cn = wn * 64 + ns * 16 + col;
    const int n = min(n0 + cn, N - 1);  // columns past N are staged, not stored
    const float bv = bias ? (float)bias[(long)grp * N + n] : 0.f;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        so[(wm * (MT / 2) + ms * 16 + 4 * kq + i) * OST + cn] = (ET)(acc[ms][ns][i] + bv);
  }
  __syncthreads();
  for (int idx = tid; idx < rows * (kYN / 8); idx += kYThreads) {
    const int r = idx / (kYN / 8), c8 = 8 * (idx % (kYN / 8));
    if (n0 + c8 < N)  // N % 8 == 0: all eight columns or none
      *(u32x4*)(out + (long)s_orow[r] * N + n0 + c8) = *(const u32x4*)(so + r * OST + c8);
  }
}

// 16-bit element types on 16-row tiles (groups averaging at most 16 rows),
// the weight streaming of gmm.hip's qmoe_gmm_f32_rows16 for [K, N] weights:
// each wavefront owns 64 columns of one tile and streams that strip of W[g]
// from HBM into matrix-core operands (no LDS, no barriers), 8 K groups of 16
// rows in flight, every 16-bit value widened to fp32 (exactly) for
// v_mfma_f32_16x16x4_f32: exact products, fp32 sums, bias added in fp32 and
// the sum rounded once to the element type (the arithmetic of the tile
// kernel above).  Lane (c, kq): columns n0 + 4c .. + 3, output rows 4kq ..
// 4kq + 3, K values 4kq .. 4kq + 3 of each group.  KSPLIT > 1: the four
// wavefronts take K ranges of the same 64 columns and add their sums through
// LDS in wavefront order.  Needs K % 4 == 0, N % 4 == 0 and 8-byte aligned
// input, weights, bias and output.
template <typename ET>
__device__ __forceinline__ float widen16(const u32x2& v, int j) {
  const uint16_t h = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
  if constexpr (std::is_same<ET, _Float16>::value) return (float)__builtin_bit_cast(_Float16, h);
  else return __builtin_bit_cast(float, (uint32_t)h << 16);
}

template <typename ET, int KSPLIT>
__global__ void __launch_bounds__(256) qmoe_gmm16_rows16(const TypedGemm g, int nblk) {
  constexpr int KG = 16, SD = 8;
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
  int orow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) orow[t] = 4 * kq + t < rows ? g.perm[p0 + 4 * kq + t] : -1;
  const bool cok = n0 + 4 * c < N;  // all four columns or none (N % 4 == 0)
  ET* out = static_cast<ET*>(g.out);
  if (grp >= g.G) {  // index outside [0, G): zero rows
    if (KSPLIT > 1 && wave > 0) return;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (orow[t] >= 0 && cok) *(u32x2*)(out + (long)orow[t] * N + n0 + 4 * c) = u32x2{0u, 0u};
    return;
  }
  const int nfull = K / KG;
  const int g0 = KSPLIT == 1 ? 0 : (int)((long)nfull * wave / KSPLIT);
  const int g1 = KSPLIT == 1 ? nfull : (int)((long)nfull * (wave + 1) / KSPLIT);
  const bool tail = nfull * KG < K && (KSPLIT == 1 || wave == KSPLIT - 1);
  const ET* arow = static_cast<const ET*>(g.a) + (long)(g.a_perm[p0 + min(c, rows - 1)] / g.a_div) * K + 4 * kq;
  // this lane's columns at k row 4 kq (lanes past N re-read column 0)
  const ET* wp = static_cast<const ET*>(g.w) + (long)grp * K * N + (cok ? n0 + 4 * c : 0) + (long)(4 * kq) * N;
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // ra[d]: operand k KG kg + 4 kq .. + 3; rb[d][j]: columns n0 + 4c .. + 3 at
  // k row KG kg + 4 kq + j (four 16-bit values each)
  u32x2 ra[SD], rb[SD][4];
  auto load = [&](int slot, int kg) {
    const long k = (long)kg * KG;
    ra[slot] = *(const u32x2*)(arow + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) rb[slot][j] = *(const u32x2*)(wp + (k + j) * N);
  };
  auto mma = [&](int slot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float av = widen16<ET>(ra[slot], j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, widen16<ET>(rb[slot][j], i), acc[i], 0, 0, 0);
    }
  };
  // branch-free pipeline as in gmm.hip (past the range's last group the
  // loads repeat it, unused)
  if (g1 > g0) {
    int kg = g0;
#pragma unroll
    for (int d = 0; d < SD; ++d) load(d, min(g0 + d, g1 - 1));
    for (; kg + SD <= g1; kg += SD) {
#pragma unroll
      for (int d = 0; d < SD; ++d) {
        mma(d);
        load(d, min(kg + SD + d, g1 - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int d = 0; d < SD; ++d)
      if (kg + d < g1) mma(d);
  }
  if (tail) {
    // tail group: k past K reads as zero on both operands (K % 4 == 0, so a
    // lane's four k are all in or all out)
    const int kb = nfull * KG;
    const bool ok = kb + 4 * kq < K;
    ra[0] = ok ? *(const u32x2*)(arow + kb) : u32x2{0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) rb[0][j] = ok ? *(const u32x2*)(wp + (long)(kb + j) * N) : u32x2{0u, 0u};
    mma(0);
  }
  if (KSPLIT > 1) {
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
  if (!cok) return;
  const int n = n0 + 4 * c;
  float bv[4] = {0.f, 0.f, 0.f, 0.f};
  if (g.bias) {
    const u32x2 b = *(const u32x2*)(static_cast<const ET*>(g.bias) + (long)grp * N + n);
#pragma unroll
    for (int i = 0; i < 4; ++i) bv[i] = widen16<ET>(b, i);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (orow[t] < 0) continue;
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = __builtin_bit_cast(uint16_t, (ET)(acc[i][t] + bv[i]));
    *(u32x2*)(out + (long)orow[t] * N + n) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  }
}

// 16-bit element types on 16-row tiles, weight streaming on the 16-bit
// matrix instruction (v_mfma_f32_16x16x32_f16 / _bf16: exact products, fp32
// sums, the arithmetic of the tile kernels) for K and N multiples of 8 and
// 16-byte aligned tensors.  Lane (c, kq) loads the 8 x 8 block of W[g] at K
// rows 8kq .. 8kq + 7 of each 32-value group and columns n0 + 8c .. + 7 (one
// 16-byte load a row) and transposes it in registers with byte permutes into
// eight operands, one per column: instruction i takes column n0 + 8c + i as
// its column c (accumulator i), so a wavefront covers 128 columns and each
// lane ends with 8 consecutive columns of rows 4kq .. 4kq + 3, stored as
// 16-byte rows.  The input rows are already 16-bit operands (lane (c, kq):
// row c, K values 8kq .. 8kq + 7).  Two K groups in flight; KSPLIT > 1 as in
// qmoe_gmm16_rows16.
template <typename ET, int KSPLIT>
__global__ void __launch_bounds__(256) qmoe_gmm16_stream(const TypedGemm g, int nblk) {
  using T = Ty<ET>;
  constexpr int KG = 32, SD = 2;
  const int tile = blockIdx.x / nblk;
  if (tile >= g.ntiles[0]) return;
  const int grp = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int K = g.K, N = g.N;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int n0 = KSPLIT == 1 ? (blockIdx.x % nblk) * 512 + wave * 128 : (blockIdx.x % nblk) * 128;
  if (n0 >= N) return;  // whole wavefront (whole workgroup when KSPLIT > 1): before any barrier
  const int c = lane & 15, kq = lane >> 4;
  int orow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) orow[t] = 4 * kq + t < rows ? g.perm[p0 + 4 * kq + t] : -1;
  const bool cok = n0 + 8 * c < N;  // all eight columns or none (N % 8 == 0)
  ET* out = static_cast<ET*>(g.out);
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  if (grp >= g.G) {  // index outside [0, G): zero rows
    if (KSPLIT > 1 && wave > 0) return;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (orow[t] >= 0 && cok) *(u32x4*)(out + (long)orow[t] * N + n0 + 8 * c) = z4;
    return;
  }
  const int nfull = K / KG;
  const int g0 = KSPLIT == 1 ? 0 : (int)((long)nfull * wave / KSPLIT);
  const int g1 = KSPLIT == 1 ? nfull : (int)((long)nfull * (wave + 1) / KSPLIT);
  const bool tail = nfull * KG < K && (KSPLIT == 1 || wave == KSPLIT - 1);
  const ET* arow = static_cast<const ET*>(g.a) + (long)(g.a_perm[p0 + min(c, rows - 1)] / g.a_div) * K + 8 * kq;
  // this lane's columns at k row 8 kq (lanes past N re-read column 0)
  const ET* wp = static_cast<const ET*>(g.w) + (long)grp * K * N + (cok ? n0 + 8 * c : 0) + (long)(8 * kq) * N;
  typename T::Acc acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = typename T::Acc{};
  // ra[d]: row c, k KG kg + 8 kq .. + 7; rb[d][r]: columns n0 + 8c .. + 7 at
  // k row KG kg + 8 kq + r
  u32x4 ra[SD], rb[SD][8];
  auto load = [&](int slot, int kg) {
    const long k = (long)kg * KG;
    ra[slot] = *(const u32x4*)(arow + k);
#pragma unroll
    for (int r = 0; r < 8; ++r) rb[slot][r] = *(const u32x4*)(wp + (k + r) * N);
  };
  auto mma = [&](const u32x4& a, const u32x4 (&b)[8]) {
    const typename T::Frag af = __builtin_bit_cast(typename T::Frag, a);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // column 8c + i: rows r are the low (i even) or high (i odd) halves of
      // dword i / 2 of b[r]
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
      u32x4 f;
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = __builtin_amdgcn_perm(b[2 * q + 1][i >> 1], b[2 * q][i >> 1], sel);
      acc[i] = T::mma(af, __builtin_bit_cast(typename T::Frag, f), acc[i]);
    }
  };
  // branch-free pipeline (past the range's last group the loads repeat it,
  // unused)
  if (g1 > g0) {
    int kg = g0;
#pragma unroll
    for (int d = 0; d < SD; ++d) load(d, min(g0 + d, g1 - 1));
    for (; kg + SD <= g1; kg += SD) {
#pragma unroll
      for (int d = 0; d < SD; ++d) {
        mma(ra[d], rb[d]);
        load(d, min(kg + SD + d, g1 - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int d = 0; d < SD; ++d)
      if (kg + d < g1) mma(ra[d], rb[d]);
  }
  if (tail) {
    // tail group: k past K reads as zero on both operands (K % 8 == 0, so a
    // lane's eight k are all in or all out)
    const int kb = nfull * KG;
    const bool ok = kb + 8 * kq < K;
    ra[0] = ok ? *(const u32x4*)(arow + kb) : z4;
#pragma unroll
    for (int r = 0; r < 8; ++r) rb[0][r] = ok ? *(const u32x4*)(wp + (long)(kb + r) * N) : z4;
    mma(ra[0], rb[0]);
  }
  if (KSPLIT > 1) {
    __shared__ f32x4 red[KSPLIT > 1 ? KSPLIT - 1 : 1][8][64];
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < KSPLIT - 1; ++w)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += red[w][i][lane];
  }
  if (!cok) return;
  const int n = n0 + 8 * c;
  float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (g.bias) {
    const u32x4 b = *(const u32x4*)(static_cast<const ET*>(g.bias) + (long)grp * N + n);
#pragma unroll
    for (int i = 0; i < 8; ++i) bv[i] = widen16<ET>(u32x2{b[(i >> 2) * 2], b[(i >> 2) * 2 + 1]}, i & 3);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (orow[t] < 0) continue;
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = __builtin_bit_cast(uint16_t, (ET)(acc[i][t] + bv[i]));
    *(u32x4*)(out + (long)orow[t] * N + n) =
        u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
}

hipError_t launch_gmm16_stream(int type, const TypedGemm& g, long est_tiles, int max_tiles, hipStream_t st) {
  if (max_tiles <= 0 || g.N <= 0) return hipSuccess;
  if (g.K % 8 != 0 || g.N % 8 != 0) return hipErrorInvalidValue;
  // one 128-column strip a wavefront; below about a thousand wavefronts
  // (four per compute unit) the K ranges are split four ways (at 1792, the
  // decode-shaped workload, whole K ranges measured 5 % faster)
  const int ksplit = est_tiles * ((g.N + 127) / 128) < 1024 ? 4 : 1;
  const int cols = ksplit == 1 ? 512 : 128;  // columns per workgroup
  const int nblk = (g.N + cols - 1) / cols;
  const dim3 grid((unsigned)((long)max_tiles * nblk)), block(256);
#define QMOE_S16(ET)                                                                                  \
  do {                                                                                                \
    if (ksplit == 1) hipLaunchKernelGGL((qmoe_gmm16_stream<ET, 1>), grid, block, 0, st, g, nblk);     \
    else hipLaunchKernelGGL((qmoe_gmm16_stream<ET, 4>), grid, block, 0, st, g, nblk);                 \
  } while (0)
  switch (type) {
    case GMM_F16: QMOE_S16(_Float16); break;
    case GMM_BF16: QMOE_S16(__bf16); break;
    default: return hipErrorInvalidValue;
  }
#undef QMOE_S16
  return hipGetLastError();
}

// double on 16-row tiles (groups averaging at most 16 rows): the same weight
// streaming with 16-byte loads (two adjacent columns of one K row a lane) on
// v_mfma_f64_16x16x4_f64 (fp64 products and sums, bias added in fp64).  A
// wavefront owns 32 columns: lane (c, kq) holds columns n0 + 2c and
// n0 + 2c + 1 (accumulators 0 and 1, each the instruction's column c) and K
// values 4kq .. 4kq + 3 of each 16-value group, one per instruction j (the
// instruction's k index kq stands for k = 4kq + j); the fp64 result leaves
// row kq + 4t of the tile in register t of lane 16kq + c.  4 K groups in
// flight.  KSPLIT > 1: the four wavefronts take K ranges of the same 32
// columns and add their sums through LDS in wavefront order.  Needs
// K % 4 == 0, N % 2 == 0 and 16-byte aligned input, weights, bias and output.
template <int KSPLIT>
__global__ void __launch_bounds__(256) qmoe_gmm64_rows16(const TypedGemm g, int nblk) {
  constexpr int KG = 16, SD = 4;
  typedef double f64x2 __attribute__((ext_vector_type(2)));
  const int tile = blockIdx.x / nblk;
  if (tile >= g.ntiles[0]) return;
  const int grp = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int K = g.K, N = g.N;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int n0 = KSPLIT == 1 ? (blockIdx.x % nblk) * 128 + wave * 32 : (blockIdx.x % nblk) * 32;
  if (n0 >= N) return;  // whole wavefront (whole workgroup when KSPLIT > 1): before any barrier
  const int c = lane & 15, kq = lane >> 4;
  int orow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) orow[t] = kq + 4 * t < rows ? g.perm[p0 + kq + 4 * t] : -1;
  const bool cok = n0 + 2 * c < N;  // both columns or none (N % 2 == 0)
  double* out = static_cast<double*>(g.out);
  if (grp >= g.G) {  // index outside [0, G): zero rows
    if (KSPLIT > 1 && wave > 0) return;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (orow[t] >= 0 && cok) *(f64x2*)(out + (long)orow[t] * N + n0 + 2 * c) = f64x2{0.0, 0.0};
    return;
  }
  const int nfull = K / KG;
  const int g0 = KSPLIT == 1 ? 0 : (int)((long)nfull * wave / KSPLIT);
  const int g1 = KSPLIT == 1 ? nfull : (int)((long)nfull * (wave + 1) / KSPLIT);
  const bool tail = nfull * KG < K && (KSPLIT == 1 || wave == KSPLIT - 1);
  const double* arow =
      static_cast<const double*>(g.a) + (long)(g.a_perm[p0 + min(c, rows - 1)] / g.a_div) * K + 4 * kq;
  // this lane's columns at k row 4 kq (lanes past N re-read column 0)
  const double* wp =
      static_cast<const double*>(g.w) + (long)grp * K * N + (cok ? n0 + 2 * c : 0) + (long)(4 * kq) * N;
  f64x4 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i] = f64x4{0.0, 0.0, 0.0, 0.0};
  // ra[d]: operand k KG kg + 4 kq .. + 3; rb[d][j]: columns n0 + 2c, + 1 at
  // k row KG kg + 4 kq + j
  f64x2 ra[SD][2], rb[SD][4];
  auto load = [&](int slot, int kg) {
    const long k = (long)kg * KG;
    ra[slot][0] = *(const f64x2*)(arow + k);
    ra[slot][1] = *(const f64x2*)(arow + k + 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) rb[slot][j] = *(const f64x2*)(wp + (k + j) * N);
  };
  auto mma = [&](int slot) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc[i] = __builtin_amdgcn_mfma_f64_16x16x4f64(ra[slot][j >> 1][j & 1], rb[slot][j][i], acc[i], 0, 0, 0);
  };
  // branch-free pipeline (past the range's last group the loads repeat it,
  // unused)
  if (g1 > g0) {
    int kg = g0;
#pragma unroll
    for (int d = 0; d < SD; ++d) load(d, min(g0 + d, g1 - 1));
    for (; kg + SD <= g1; kg += SD) {
#pragma unroll
      for (int d = 0; d < SD; ++d) {
        mma(d);
        load(d, min(kg + SD + d, g1 - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int d = 0; d < SD; ++d)
      if (kg + d < g1) mma(d);
  }
  if (tail) {
    // tail group: k past K reads as zero on both operands (K % 4 == 0, so a
    // lane's four k are all in or all out)
    const int kb = nfull * KG;
    const bool ok = kb + 4 * kq < K;
    const f64x2 z = {0.0, 0.0};
    ra[0][0] = ok ? *(const f64x2*)(arow + kb) : z;
    ra[0][1] = ok ? *(const f64x2*)(arow + kb + 2) : z;
#pragma unroll
    for (int j = 0; j < 4; ++j) rb[0][j] = ok ? *(const f64x2*)(wp + (long)(kb + j) * N) : z;
    mma(0);
  }
  if (KSPLIT > 1) {
    __shared__ f64x4 red[KSPLIT > 1 ? KSPLIT - 1 : 1][2][64];
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) red[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < KSPLIT - 1; ++w)
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i] += red[w][i][lane];
  }
  if (!cok) return;
  const int n = n0 + 2 * c;
  f64x2 bv = {0.0, 0.0};
  if (g.bias) bv = *(const f64x2*)(static_cast<const double*>(g.bias) + (long)grp * N + n);
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (orow[t] >= 0) *(f64x2*)(out + (long)orow[t] * N + n) = f64x2{acc[0][t] + bv[0], acc[1][t] + bv[1]};
}

hipError_t launch_gmm64_rows16(const TypedGemm& g, long est_tiles, int max_tiles, hipStream_t st) {
  if (max_tiles <= 0 || g.N <= 0) return hipSuccess;
  if (g.K % 4 != 0 || g.N % 2 != 0) return hipErrorInvalidValue;
  // one 32-column strip a wavefront; below about two thousand wavefronts
  // (eight per compute unit) the K ranges are split four ways
  const int ksplit = est_tiles * ((g.N + 31) / 32) < 2048 ? 4 : 1;
  const int cols = ksplit == 1 ? 128 : 32;  // columns per workgroup
  const int nblk = (g.N + cols - 1) / cols;
  const dim3 grid((unsigned)((long)max_tiles * nblk)), block(256);
  if (ksplit == 1) hipLaunchKernelGGL((qmoe_gmm64_rows16<1>), grid, block, 0, st, g, nblk);
  else hipLaunchKernelGGL((qmoe_gmm64_rows16<4>), grid, block, 0, st, g, nblk);
  return hipGetLastError();
}

hipError_t launch_gmm16_rows16(int type, const TypedGemm& g, int ksplit, int max_tiles, hipStream_t st) {
  if (max_tiles <= 0 || g.N <= 0) return hipSuccess;
  if (g.K % 4 != 0 || g.N % 4 != 0 || (ksplit != 1 && ksplit != 4)) return hipErrorInvalidValue;
  const int cols = ksplit == 1 ? 256 : 64;  // columns per workgroup
  const int nblk = (g.N + cols - 1) / cols;
  const dim3 grid((unsigned)((long)max_tiles * nblk)), block(256);
#define QMOE_R16(ET)                                                                                  \
  do {                                                                                                \
    if (ksplit == 1) hipLaunchKernelGGL((qmoe_gmm16_rows16<ET, 1>), grid, block, 0, st, g, nblk);     \
    else hipLaunchKernelGGL((qmoe_gmm16_rows16<ET, 4>), grid, block, 0, st, g, nblk);                 \
  } while (0)
  switch (type) {
    case GMM_F16: QMOE_R16(_Float16); break;
    case GMM_BF16: QMOE_R16(__bf16); break;
    default: return hipErrorInvalidValue;
  }
#undef QMOE_R16
  return hipGetLastError();
}

int gmm16_tile_rows(long R, long spread) {
  // QMOE_GMM16_TILE_ROWS = 64 or 128 forces the choice (timing comparisons)
  if (const char* v = std::getenv("QMOE_GMM16_TILE_ROWS")) {
    const std::string s(v);
    if (s == "64") return 64;
    if (s == "128") return 128;
  }
  // groups averaging at least 128 rows: 128-row tiles read each weight
  // column slice half as often
  return R >= 128 * spread ? 128 : 64;
}

hipError_t launch_gmm_typed(int type, const TypedGemm& g, bool vec, int max_tiles, hipStream_t st, int tile_rows) {
  if (max_tiles <= 0 || g.N <= 0) return hipSuccess;
  const int nblk = (g.N + kYN - 1) / kYN;
  const dim3 grid((unsigned)((long)max_tiles * nblk)), block(kYThreads);
#define QMOE_TYPED(ET)                                                                       \
  do {                                                                                       \
    if (vec) hipLaunchKernelGGL((qmoe_gmm_typed<ET, true>), grid, block, 0, st, g, nblk);   \
    else hipLaunchKernelGGL((qmoe_gmm_typed<ET, false>), grid, block, 0, st, g, nblk);      \
  } while (0)
  // 16-bit types with whole 16-byte runs of 8 K values and 8 columns: the
  // register-transposed kernel
  // register-transposed kernel, on tiles of at most tile_rows rows (64, or
  // 128 for that kernel alone)
  const bool t16 = vec && g.K % 8 == 0 && g.N % 8 == 0 && reinterpret_cast<uintptr_t>(g.out) % 16 == 0;
  if (tile_rows > kYM && !(t16 && tile_rows == 128 && (type == GMM_F16 || type == GMM_BF16)))
    return hipErrorInvalidValue;
#define QMOE_T16(ET)                                                                                  \
  do {                                                                                                \
    if (tile_rows == 128) hipLaunchKernelGGL((qmoe_gmm16_tiled<ET, 64, 128>), grid, block, 0, st, g, nblk); \
    else hipLaunchKernelGGL((qmoe_gmm16_tiled<ET, 64, 64>), grid, block, 0, st, g, nblk);            \
  } while (0)
  switch (type) {
    case GMM_F16:
      if (t16) QMOE_T16(_Float16);
      else QMOE_TYPED(_Float16);
      break;
    case GMM_BF16:
      if (t16) QMOE_T16(__bf16);
      else QMOE_TYPED(__bf16);
      break;
    case GMM_F64: QMOE_TYPED(double); break;
    default: return hipErrorInvalidValue;
  }
#undef QMOE_TYPED
#undef QMOE_T16
  return hipGetLastError();
}

}  // namespace qmoe
