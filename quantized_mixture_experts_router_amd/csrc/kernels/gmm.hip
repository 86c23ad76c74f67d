// GroupedMatMul over float32 weights (ONNX GroupedMatMul-29, Summary):
//
//   output[m, i, :] = input[m, :] @ weights[g, :, :] (+ bias[g, :]),
//   g = group_indices[m, i]
//
// The (m, i) pairs are the "slots" of the routing front end: their group
// indices are sorted into group-major order by the same histogram / scan /
// stable scatter kernels (route.hip), so that every 64-row tile multiplies
// rows of one group by that group's [K, N] matrix, read once per tile.
// Indices outside [0, G) are invalid input (the page leaves the result
// undefined); they are gathered into an extra group G whose rows are written
// as zeros, and no weight or bias outside the tensors is ever read.
//
// The tile GEMM runs on v_mfma_f32_16x16x4_f32 (fp32 operands, fp32
// accumulation): products are exact in fp32, like the definition's
// float32 arithmetic.  A workgroup of 4 wavefronts computes a 64 x 128 tile
// (2 x 2 wavefronts of 32 x 64); each 16-deep K step of both operands is
// staged in LDS (double buffered, the next step's loads in flight during the
// current step's matrix instructions).
#include "common.hpp"
#include "launch.h"

namespace qmoe {

namespace {

constexpr int kGM = 64;            // tile rows (group-sorted (m, i) pairs)
constexpr int kGN = 128;           // tile columns
constexpr int kGK = 16;            // K per step
constexpr int kGThreads = 256;
constexpr int kAStride = kGK + 1;  // LDS floats per A row (bank spread)
constexpr int kBStride = kGN + 16; // LDS floats per B row (bank spread)

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

// VEC: K and N are multiples of 4 and x, w 16-byte aligned (16-byte loads).
template <bool VEC>
__global__ void __launch_bounds__(kGThreads) qmoe_gmm_f32(const float* __restrict__ x, const float* __restrict__ w,
                                                          const float* __restrict__ bias, const int* __restrict__ perm,
                                                          const int* __restrict__ tiles, const int* __restrict__ ntiles,
                                                          int nblk, int S, int K, int N, int G,
                                                          float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float sa[2][kGM * kAStride];
  __shared__ __attribute__((aligned(16))) float sb[2][kGK * kBStride];
  __shared__ int s_slot[kGM];
  // one workgroup per (tile, 128-column block); column blocks of a tile are
  // adjacent, so they run together and share its input rows in L2
  const int tile = blockIdx.x / nblk;
  if (tile >= ntiles[0]) return;
  const int g = tiles[4 * tile + 0];
  const int p0 = tiles[4 * tile + 1];
  const int rows = tiles[4 * tile + 2];
  const int n0 = (blockIdx.x % nblk) * kGN;
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col = lane & 15, kq = lane >> 4;

  if (tid < kGM) s_slot[tid] = perm[p0 + min(tid, rows - 1)];
  __syncthreads();

  if (g >= G) {
    // invalid group index: zero rows
    for (int idx = tid; idx < rows * kGN; idx += kGThreads) {
      const int rr = idx / kGN, c = idx % kGN;
      if (n0 + c < N) out[(long)s_slot[rr] * N + n0 + c] = 0.f;
    }
    return;
  }

  // Global -> register staging of one K step.  A: row tid / 4, four k from
  // 4 * (tid % 4); B: k row tid / 16, eight columns from 8 * (tid % 16).
  // Elements past K or N are zero; rows past the tile re-read a valid row.
  const float* arow = x + (long)(s_slot[tid >> 2] / S) * K;
  const float* wg = w + (long)g * K * N;
  const int ak = (tid & 3) * 4;
  const int bk = tid >> 4, bn = (tid & 15) * 8;
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
  };
  auto store = [&](int buf) {
    float* a = sa[buf] + (tid >> 2) * kAStride + ak;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = ra[i];
    float* b = sb[buf] + bk * kBStride + bn;
    *(f32x4*)b = rb[0];
    *(f32x4*)(b + 4) = rb[1];
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
      for (int ns = 0; ns < 4; ++ns) bv[ns] = b[(k4 * 4 + kq) * kBStride + wn * 64 + ns * 16 + col];
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
    const float bv = bias ? bias[(long)g * N + c] : 0.f;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = wm * 32 + ms * 16 + 4 * kq + i;
        if (rr < rows) out[(long)s_slot[rr] * N + c] = acc[ms][ns][i] + bv;
      }
  }
}

// Weight-streaming variant for groups of at most 16 rows (16-row tiles):
// each wavefront owns a 64-column strip of one tile and streams that strip of
// the group's [K, N] weights from HBM straight into matrix-core operands, with
// no LDS and no barriers.  The 16 columns of MFMA block i are the columns
// n0 + 4c + i (c = 0..15), so one 16-byte load per lane fetches a 256-byte
// row segment serving all four blocks, and the four MFMAs of one 16-deep K
// group take k = 16 kg + 4 kq + j (j = 0..3) in lane group kq: one 16-byte
// load of the input row covers them.  kD K groups of loads stay in flight
// ahead of the matrix instructions.  Requires K % 4 == 0, N % 4 == 0 and
// 16-byte aligned x, w, bias and out.
constexpr int kSD = 4;  // K groups (16 deep) of loads in flight per wavefront

__global__ void __launch_bounds__(256) qmoe_gmm_f32_rows16(const float* __restrict__ x, const float* __restrict__ w,
                                                           const float* __restrict__ bias, const int* __restrict__ perm,
                                                           const int* __restrict__ tiles,
                                                           const int* __restrict__ ntiles, int nblk, int S, int K,
                                                           int N, int G, float* __restrict__ out) {
  const int tile = blockIdx.x / nblk;
  if (tile >= ntiles[0]) return;
  const int g = tiles[4 * tile + 0];
  const int p0 = tiles[4 * tile + 1];
  const int rows = tiles[4 * tile + 2];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x % nblk) * 256 + wave * 64;
  if (n0 >= N) return;  // whole wavefront: no barriers below
  const int c = lane & 15, kq = lane >> 4;
  const int n = n0 + 4 * c;
  const bool col_ok = n < N;  // N % 4 == 0: all four columns or none
  const int row = lane & 15;  // A operand row of this lane
  const int slot_a = perm[p0 + min(row, rows - 1)];
  if (g >= G) {
    // invalid group index: zero rows
    if (col_ok) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 4 * kq + t;
        if (r < rows) *(f32x4*)(out + (long)perm[p0 + r] * N + n) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }
  const float* arow = x + (long)(slot_a / S) * K + 4 * kq;
  // lanes past N re-read column 0 (results discarded)
  const float* wcol = w + (long)g * K * N + (col_ok ? n : 0) + (long)(4 * kq) * N;
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nfull = K / 16;  // K groups without a tail
  f32x4 ra[kSD], rb[kSD][4];
  auto load = [&](int slot, int kg) {
    const long k = (long)kg * 16;
    ra[slot] = *(const f32x4*)(arow + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) rb[slot][j] = *(const f32x4*)(wcol + (k + j) * N);
  };
  auto mma = [&](int slot) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(ra[slot][j], rb[slot][j][i], acc[i], 0, 0, 0);
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
    const int k0 = nfull * 16 + 4 * kq;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = k0 + j < K;
      ra[0][j] = ok ? arow[nfull * 16 + j] : 0.f;
      rb[0][j] = ok ? *(const f32x4*)(wcol + ((long)nfull * 16 + j) * N) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    mma(0);
  }
  if (!col_ok) return;
  const f32x4 bv = bias ? *(const f32x4*)(bias + (long)g * N + n) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r = 4 * kq + t;
    if (r < rows) {
      const f32x4 v = {acc[0][t] + bv[0], acc[1][t] + bv[1], acc[2][t] + bv[2], acc[3][t] + bv[3]};
      *(f32x4*)(out + (long)perm[p0 + r] * N + n) = v;
    }
  }
}

int gmm_tile_rows() { return kGM; }
int gmm_rows16_tile_rows() { return 16; }

hipError_t launch_gmm_rows16(const float* x, const float* w, const float* bias, const int* perm, const int* tiles,
                             const int* ntiles, int max_tiles, int S, int K, int N, int G, float* out,
                             hipStream_t st) {
  if (max_tiles <= 0 || N <= 0) return hipSuccess;
  if (K % 4 != 0 || N % 4 != 0) return hipErrorInvalidValue;
  const int nblk = (N + 255) / 256;
  const dim3 grid((unsigned)((long)max_tiles * nblk)), block(256);
  hipLaunchKernelGGL(qmoe_gmm_f32_rows16, grid, block, 0, st, x, w, bias, perm, tiles, ntiles, nblk, S, K, N, G, out);
  return hipGetLastError();
}

hipError_t launch_gmm_index(const void* idx, bool idx64, long n, int G, int* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((n + 255) / 256), block(256);
  if (idx64) hipLaunchKernelGGL(qmoe_gmm_index<int64_t>, grid, block, 0, st, (const int64_t*)idx, n, G, out);
  else hipLaunchKernelGGL(qmoe_gmm_index<int32_t>, grid, block, 0, st, (const int32_t*)idx, n, G, out);
  return hipGetLastError();
}

hipError_t launch_gmm_f32(const float* x, const float* w, const float* bias, const int* perm, const int* tiles,
                          const int* ntiles, int max_tiles, int S, int K, int N, int G, float* out, bool vec,
                          hipStream_t st) {
  if (max_tiles <= 0 || N <= 0) return hipSuccess;
  const int nblk = (N + kGN - 1) / kGN;
  const dim3 grid((unsigned)((long)max_tiles * nblk)), block(kGThreads);
  if (vec && (K % 4 != 0 || N % 4 != 0)) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL(qmoe_gmm_f32<true>, grid, block, 0, st, x, w, bias, perm, tiles, ntiles, nblk, S, K, N, G, out);
  else
    hipLaunchKernelGGL(qmoe_gmm_f32<false>, grid, block, 0, st, x, w, bias, perm, tiles, ntiles, nblk, S, K, N, G, out);
  return hipGetLastError();
}

}  // namespace qmoe
