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

#define QMOE_OPERAND_INLINE __attribute__((always_inline))

namespace qmoe {

// One workgroup of NT threads per row.  Row r: n fp32 codes at src + r *
// sstride (floats), kp hi/lo codes (kp % 32 == 0, codes from n on are zero)
// at dst + r * dstride (bytes); exps[r] = e.  Thread t takes the 4-code
// pieces t, t + NT, ... of the row, so that each load instruction of a
// wavefront reads 1 KB of it; the first RB pieces stay in registers between
// the two passes and longer rows read the rest again.  The two lanes
// holding a storage group's pieces (2j and 2j + 1, codes 0-3 and 4-7 of the
// group) swap halves, and the first writes the group's 16 bytes of hi
// parts, the second its 16 bytes of lo parts.  src and dst may be the same
// row of 4-byte codes: a storage group lies in the bytes of its own 32-code
// block, whose 8 pieces are read by 8 lanes of one wavefront in the same
// step before any of them is written.  With live given, rows from *live on
// are not in use and are skipped.
template <int BITS, int NT, int RB>
__global__ void __launch_bounds__(NT) qmoe_split_rows(const float* src, long sstride, int n, int vec, uint8_t* dst,
                                                      long dstride, int kp, int* __restrict__ exps,
                                                      const int* __restrict__ live, int* __restrict__ zero_flag) {
  const long row = blockIdx.x;
  if (zero_flag != nullptr && row == 0 && threadIdx.x == 0) *zero_flag = 0;
  if (live != nullptr && row >= live[0]) return;
  const float* s = src + row * sstride;
  uint8_t* d = dst + row * dstride;
  const int np = kp / 4;  // pieces: a whole number of storage groups and blocks
  const int tid = threadIdx.x;
  auto load = [&](int p) QMOE_OPERAND_INLINE {
    const int c0 = 4 * p;
    f32x4 v;
    if (vec && c0 + 4 <= n) {
      v = *(const f32x4*)(s + c0);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = c0 + c < n ? s[c0 + c] : 0.f;
    }
    return v;
  };
  auto vmax = [](float m, const f32x4& v) QMOE_OPERAND_INLINE {
    return fmaxf(fmaxf(m, fmaxf(fabsf(v[0]), fabsf(v[1]))), fmaxf(fabsf(v[2]), fabsf(v[3])));
  };
  f32x4 cache[RB];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int p = tid + i * NT;
    if (p < np) {
      cache[i] = load(p);
      m = vmax(m, cache[i]);
    }
  }
  for (int p = tid + RB * NT; p < np; p += NT) m = vmax(m, load(p));
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
  // piece p's part of its storage group (both lanes of a group run this
  // together: np is even and NT a multiple of 64)
  auto put = [&](int p, const f32x4& v) QMOE_OPERAND_INLINE {
    const bool odd = (p & 1) != 0;  // codes 4-7 of the group: writes the lo parts
    _Float16 h[4], l[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) split_f16(v[c], e, h[c], l[c]);
    // send the other kind: the even lane its lo parts, the odd one its hi parts
    uint32_t x[2], y[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const _Float16 a = odd ? h[2 * k] : l[2 * k], b = odd ? h[2 * k + 1] : l[2 * k + 1];
      x[k] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
      y[k] = (uint32_t)__shfl_xor((int)x[k], 1);
    }
    // the 8 codes' parts of this lane's kind, in code order
    _Float16 g8[8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const _Float16 r0 = __builtin_bit_cast(_Float16, (uint16_t)(y[k] & 0xFFFF));
      const _Float16 r1 = __builtin_bit_cast(_Float16, (uint16_t)(y[k] >> 16));
      g8[2 * k] = odd ? r0 : h[2 * k];
      g8[2 * k + 1] = odd ? r1 : h[2 * k + 1];
      g8[4 + 2 * k] = odd ? l[2 * k] : r0;
      g8[4 + 2 * k + 1] = odd ? l[2 * k + 1] : r1;
    }
    f16x8 out;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) out[sl] = g8[BITS == 4 ? perm4_of_slot(sl) : sl];
    const int q = p >> 1;                               // code group of the row
    const int sg = BITS == 4 ? (q & 3) : sigma8(q & 3);  // its storage group in the 32-code block
    *(f16x8*)(d + (long)(4 * (q >> 2) + sg) * 32 + (odd ? 16 : 0)) = out;
  };
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int p = tid + i * NT;
    if (p < np) put(p, cache[i]);
  }
  for (int p = tid + RB * NT; p < np; p += NT) put(p, load(p));
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
  const dim3 grid((unsigned)rows);
  // threads and registered pieces a row: rows up to 1024, 4096 and 16384
  // codes stay in registers between the passes
#define QMOE_SPLIT(NT, RB)                                                                                     \
  do {                                                                                                         \
    if (bits == 4)                                                                                             \
      hipLaunchKernelGGL((qmoe_split_rows<4, NT, RB>), grid, dim3(NT), 0, st, src, sstride, n, vec, dst, dstride, \
                         kp, exps, live, zero_flag);                                                           \
    else                                                                                                       \
      hipLaunchKernelGGL((qmoe_split_rows<8, NT, RB>), grid, dim3(NT), 0, st, src, sstride, n, vec, dst, dstride, \
                         kp, exps, live, zero_flag);                                                           \
  } while (0)
  if (kp <= 1024) QMOE_SPLIT(64, 4);
  else if (kp <= 4096) QMOE_SPLIT(256, 4);
  else QMOE_SPLIT(256, 16);
#undef QMOE_SPLIT
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
