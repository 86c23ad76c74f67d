// Operand rows of the f16 matrix-core GEMMs (see common.hpp for the layout
// and the row scaling).
//
//   qmoe_split_rows  fp32 rows -> f16 hi/lo storage groups of v * 2^e, with
//                    e from each row's largest magnitude, and e per row.  It
//                    prepares the FC1 operand rows from the layer input, and
//                    turns the FC2 operand rows that the FC1 epilogue wrote
//                    as fp32 into hi/lo groups in place.
//   qmoe_row_exp     e per fp32 row only (the weight-streaming kernels split
//                    while staging; this serves their walks over a whole row).
//   qmoe_resplit_rows hi/lo rows written with one exponent per segment (the
//                    tiled FC1 epilogue's) -> one exponent per row, in place;
//                    runs only when the epilogue flagged a row.
//
// The products these rows feed are the FC1 and FC2 sums of the QMoE WebGPU
// manifest (description; inputs[0] is float32): the scaling only changes how
// the fp32 values are carried to the matrix cores, never the sums.
#include <algorithm>

#include "common.hpp"
#include "launch.h"

namespace qmoe {

namespace {

// 32 fp32 codes [32 b, 32 b + 32) of a row of n codes (zero from n on).
__device__ __forceinline__ void load_block(const float* __restrict__ s, int b, int n, bool vec, float (&v)[32]) {
  const int c0 = 32 * b;
  if (vec && c0 + 32 <= n) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const f32x4 t = *(const f32x4*)(s + c0 + 4 * q);
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * q + c] = t[c];
    }
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) v[c] = c0 + c < n ? s[c0 + c] : 0.f;
  }
}

__device__ __forceinline__ float block_max(const float (&v)[32]) {
  float m = 0.f;
#pragma unroll
  for (int c = 0; c < 32; ++c) m = fmaxf(m, fabsf(v[c]));
  return m;
}

// Storage groups 4b .. 4b + 3 (bytes [128 b, 128 b + 128) of the row) from
// the block's fp32 codes: the same bytes the block's fp32 values occupy in a
// row of 4-byte codes, so the conversion can run in place.
template <int BITS>
__device__ __forceinline__ void store_block(uint8_t* __restrict__ d, int b, int e, const float (&v)[32]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int cg = BITS == 4 ? g : sigma8(g);  // code group held by storage group g
    float w[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) w[c] = v[8 * cg + c];
    f16x8 hi, lo;
    split_group<BITS>(w, e, hi, lo);
    uint8_t* dst = d + (long)(4 * b + g) * 32;
    *(f16x8*)dst = hi;
    *(f16x8*)(dst + 16) = lo;
  }
}

}  // namespace

// One workgroup per row.  Row r: n fp32 codes at src + r * sstride (floats),
// kp hi/lo codes (kp % 32 == 0, codes from n on are zero) at dst + r *
// dstride (bytes); exps[r] = e.  src and dst may be the same row of 4-byte
// codes (every thread reads a block before it writes that block's bytes, and
// no other thread touches them).  The first RB blocks of a thread stay in
// registers between the two passes; longer rows read the rest again.  With
// live given, rows from *live on are not in use and are skipped.
template <int BITS, int NT>
__global__ void __launch_bounds__(NT) qmoe_split_rows(const float* src, long sstride, int n, int vec, uint8_t* dst,
                                                      long dstride, int kp, int* __restrict__ exps,
                                                      const int* __restrict__ live, int* __restrict__ zero_flag) {
  constexpr int RB = 2;
  const long row = blockIdx.x;
  if (zero_flag != nullptr && row == 0 && threadIdx.x == 0) *zero_flag = 0;
  if (live != nullptr && row >= live[0]) return;
  const float* s = src + row * sstride;
  uint8_t* d = dst + row * dstride;
  const int nb = kp / 32;
  const int tid = threadIdx.x;
  float cache[RB][32];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int b = tid + i * NT;
    if (b < nb) {
      load_block(s, b, n, vec != 0, cache[i]);
      m = fmaxf(m, block_max(cache[i]));
    }
  }
  for (int b = tid + RB * NT; b < nb; b += NT) {
    float v[32];
    load_block(s, b, n, vec != 0, v);
    m = fmaxf(m, block_max(v));
  }
  m = seg_max<64>(m);
  if constexpr (NT > 64) {
    __shared__ float red[NT / 64];
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) m = fmaxf(m, red[w]);
  }
  const int e = row_exp(m);
  if (tid == 0) exps[row] = e;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int b = tid + i * NT;
    if (b < nb) store_block<BITS>(d, b, e, cache[i]);
  }
  for (int b = tid + RB * NT; b < nb; b += NT) {
    float v[32];
    load_block(s, b, n, vec != 0, v);
    store_block<BITS>(d, b, e, v);
  }
}

// One wavefront per row: exps[r] = e of the n fp32 codes at src + r * stride.
__global__ void __launch_bounds__(256) qmoe_row_exp(const float* __restrict__ src, long stride, int rows, int n,
                                                    int vec, int* __restrict__ exps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float* s = src + (long)row * stride;
  float m = 0.f;
  if (vec) {
    for (int c = 4 * lane; c + 4 <= n; c += 256) {
      const f32x4 t = *(const f32x4*)(s + c);
      m = fmaxf(fmaxf(m, fabsf(t[0])), fmaxf(fabsf(t[1]), fmaxf(fabsf(t[2]), fabsf(t[3]))));
    }
  } else {
    for (int c = lane; c < n; c += 64) m = fmaxf(m, fabsf(s[c]));
  }
  m = seg_max<64>(m);
  if (lane == 0) exps[row] = row_exp(m);
}

// A workgroup of NT threads a row (grid-stride over the rows, so that the
// launch is short when the flag is down), a storage group (8 codes) a
// thread at a time.  The elementwise rescaling keeps each group's slot
// order, and the group's segment is that of its 32-code block (segments are
// whole blocks).  Pass 1 finds the row's largest magnitude, pass 2 rewrites
// each group in place (a group is read and written by one thread only).
template <int NT>
__global__ void __launch_bounds__(NT) qmoe_resplit_rows(uint8_t* d, long stride, int n, long rows,
                                                        const int* __restrict__ seg_rows, int seg_shift,
                                                        int* __restrict__ exps, const int* __restrict__ flag,
                                                        const int* __restrict__ live) {
  if (flag[0] == 0) return;
  const long nrows = live != nullptr ? min((long)live[0], rows) : rows;
  const int ng = n / 8;
  const int tid = threadIdx.x;
  __shared__ float red[NT / 64];
  for (long row = blockIdx.x; row < nrows; row += gridDim.x) {
    uint8_t* r = d + row * stride;
    auto value = [&](int q, int sl, const f16x8& hi, const f16x8& lo) {
      return __builtin_ldexpf((float)hi[sl] + (float)lo[sl], -seg_rows[(long)((8 * q) >> seg_shift) * rows + row]);
    };
    float m = 0.f;
    for (int q = tid; q < ng; q += NT) {
      const f16x8 hi = *(const f16x8*)(r + (long)q * 32), lo = *(const f16x8*)(r + (long)q * 32 + 16);
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) m = fmaxf(m, fabsf(value(q, sl, hi, lo)));
    }
    m = seg_max<64>(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) m = fmaxf(m, red[w]);
    __syncthreads();  // red is rewritten by the next row
    const int e = row_exp(m);
    if (tid == 0) exps[row] = e;
    for (int q = tid; q < ng; q += NT) {
      uint8_t* g = r + (long)q * 32;
      const f16x8 hi = *(const f16x8*)g, lo = *(const f16x8*)(g + 16);
      f16x8 h2, l2;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        _Float16 a, b;
        split_f16(value(q, sl, hi, lo), e, a, b);
        h2[sl] = a;
        l2[sl] = b;
      }
      *(f16x8*)g = h2;
      *(f16x8*)(g + 16) = l2;
    }
  }
}

hipError_t launch_resplit_rows(int bits, uint8_t* d, long stride, int n, long rows, const int* seg_rows, int seg_shift,
                               int* exps, const int* flag, hipStream_t st, const int* live) {
  (void)bits;  // the rescaling is elementwise: the storage order of either width is kept
  if (rows <= 0) return hipSuccess;
  if (n % 32 != 0 || seg_shift < 5) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)std::min<long>(rows, 1024);
  hipLaunchKernelGGL((qmoe_resplit_rows<256>), dim3(grid), dim3(256), 0, st, d, stride, n, rows, seg_rows, seg_shift,
                     exps, flag, live);
  return hipGetLastError();
}

hipError_t launch_split_rows(int bits, const float* src, long sstride, int n, uint8_t* dst, long dstride, int kp,
                             long rows, int* exps, hipStream_t st, const int* live, int* zero_flag) {
  if (rows <= 0) return hipSuccess;
  if (kp % 32 != 0 || n > kp) return hipErrorInvalidValue;
  // 16-byte loads need 16-byte aligned rows
  const int vec = ((reinterpret_cast<uintptr_t>(src) & 15) == 0 && (sstride & 3) == 0) ? 1 : 0;
  const int nb = kp / 32;
  const dim3 grid((unsigned)rows);
  if (nb <= 128) {
    if (bits == 4) hipLaunchKernelGGL((qmoe_split_rows<4, 64>), grid, dim3(64), 0, st, src, sstride, n, vec, dst, dstride, kp, exps, live, zero_flag);
    else hipLaunchKernelGGL((qmoe_split_rows<8, 64>), grid, dim3(64), 0, st, src, sstride, n, vec, dst, dstride, kp, exps, live, zero_flag);
  } else {
    if (bits == 4) hipLaunchKernelGGL((qmoe_split_rows<4, 256>), grid, dim3(256), 0, st, src, sstride, n, vec, dst, dstride, kp, exps, live, zero_flag);
    else hipLaunchKernelGGL((qmoe_split_rows<8, 256>), grid, dim3(256), 0, st, src, sstride, n, vec, dst, dstride, kp, exps, live, zero_flag);
  }
  return hipGetLastError();
}

hipError_t launch_row_exp(const float* src, long stride, long rows, int n, int* exps, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int vec = ((reinterpret_cast<uintptr_t>(src) & 15) == 0 && (stride & 3) == 0 && (n & 3) == 0) ? 1 : 0;
  hipLaunchKernelGGL(qmoe_row_exp, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, src, stride, (int)rows, n, vec,
                     exps);
  return hipGetLastError();
}

}  // namespace qmoe
