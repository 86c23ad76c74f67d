// Device helpers shared by the QMoE kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Activation operand layout ("A rows").
//
// The matrix cores take f16 operands.  An fp32 activation v (scaled by a
// power of two per row, see below) is carried as two f16 values,
// hi = f16(v) and lo = f16(v - hi), so hi + lo keeps about 22 significant
// bits; each product runs twice (hi, then lo) into one fp32 accumulator.
// Weights are exact small integers in f16, so the only rounding is fp32
// accumulation and the lo residual.
//
// A row holds Kp codes (Kp a multiple of 128, zero padded).  Codes are stored
// in groups of 8: 16 bytes of hi halves then 16 bytes of lo halves, so one
// 32-byte group is what a lane feeds to one matrix instruction.  Each 32-code
// block is one matrix-instruction step; lane group g (lanes 16g..16g+15) of
// that step feeds storage group g, which holds the block's code group
//   4-bit: g            8-bit: sigma(g) = (0, 2, 1, 3)[g]
// (the order in which the weight loader's cross-lane exchange leaves packed
// bytes).  Inside a group of 8 the order follows the weight unpacker:
//   8-bit: natural order;
//   4-bit: storage slot i holds code perm4(i), i.e. pairs (0,4),(1,5),(2,6),(3,7).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int perm4_of_slot(int i) { return (i >> 1) | ((i & 1) << 2); }
__host__ __device__ constexpr int slot4_of_code(int c) { return ((c & 3) << 1) | (c >> 2); }
__host__ __device__ constexpr int sigma8(int g) { return ((g & 1) << 1) | (g >> 1); }  // an involution

// Code group (0..3 inside a 32-code block) fed by lane group g.
template <int BITS>
__device__ __forceinline__ int code_group_of_lane(int g) {
  if constexpr (BITS == 4) return g;
  else return sigma8(g);
}

// ---------------------------------------------------------------------------
// Operand row scaling.  f16 covers magnitudes from 2^-24 (subnormal spacing)
// to 65504, so the split is taken of v * 2^e, where e depends on the row (or
// on the K slice of a row that one launch reduces over): with m the row's
// largest magnitude, m * 2^e lies in [2^(kRowTop - 1), 2^kRowTop).  Then
// hi + lo carries every element to 2^-22 of itself plus 2^-(25 + kRowTop)
// of m, whatever the row's magnitude, and hi never overflows.  Scaling by a
// power of two is exact; the GEMM that consumes the row multiplies its fp32
// result for that row by 2^-e.  Rows that are all zero (or hold a NaN or an
// infinity, out of contract) take e = 0.
// ---------------------------------------------------------------------------
constexpr int kRowTop = 14;

__device__ __forceinline__ int row_exp(float m) {
  if (!(m > 0.f) || !(m <= 3.4028235e38f)) return 0;
  return kRowTop - __builtin_amdgcn_frexp_expf(m);  // m = f * 2^x, f in [0.5, 1)
}

// Split v * 2^e into f16 hi + lo (hi = f16(v * 2^e), lo = f16 of the rest).
__device__ __forceinline__ void split_f16(float v, int e, _Float16& hi, _Float16& lo) {
  const float s = __builtin_ldexpf(v, e);
  hi = (_Float16)s;
  lo = (_Float16)(s - (float)hi);
}

// Largest magnitude across the lanes of one wavefront whose lane index
// differs only in the bits below SEG (SEG a power of two up to 64).
template <int SEG>
__device__ __forceinline__ float seg_max(float v) {
#pragma unroll
  for (int o = 1; o < SEG; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Eight fp32 values of one storage group (codes in natural order
// c0 .. c0 + 7, see above) -> f16 hi and lo parts of v * 2^e in storage slot
// order.
template <int BITS>
__device__ __forceinline__ void split_group(const float (&v)[8], int e, f16x8& hi, f16x8& lo) {
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) {
    const int c = BITS == 4 ? perm4_of_slot(sl) : sl;  // code at storage slot sl
    _Float16 h, l;
    split_f16(v[c], e, h, l);
    hi[sl] = h;
    lo[sl] = l;
  }
}

// ---------------------------------------------------------------------------
// Weight unpacking: raw packed bytes -> exact f16 values (q - mid).
//
// f16 with exponent field 25 (0x6400 = 1024.0) has unit spacing on [1024,
// 2048), so OR-ing an integer q < 1024 into the mantissa gives exactly
// 1024 + q; one packed f16 subtract of (1024 + mid) leaves q - mid exactly.
// A nibble left in bits 4..7 of a half gives 1024 + 16 q, undone by a packed
// multiply-add with 1/16 (exact: powers of two).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// Bit masks used by the unpackers, held in registers: gfx9 three-operand
// instructions take no literal constants, so a mask in a VGPR lets
// (d & mask) | exponent fuse into one v_and_or_b32.
struct UnpackMasks {
  uint32_t lo, hi, exp;
};
__device__ __forceinline__ UnpackMasks unpack_masks() {
  UnpackMasks m{0x000F000Fu, 0x00F000F0u, 0x64006400u};
  asm volatile("" : "+v"(m.lo), "+v"(m.hi), "+v"(m.exp));
  return m;
}

// 8 four-bit codes of one little-endian dword (code j in bits 4j..4j+3) ->
// f16x8 in storage order (0,4,1,5,2,6,3,7), each value q - 8.
__device__ __forceinline__ f16x8 unpack4(uint32_t d, const UnpackMasks& m) {
  const f16x2 bias = {(_Float16)-1032.f, (_Float16)-1032.f};   // -(1024 + 8)
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2 bias16 = {(_Float16)-72.f, (_Float16)-72.f};     // -(64 + 8)
  const uint32_t d8 = d >> 8;
  f16x2 p0 = as_h2((d & m.lo) | m.exp) + bias;                    // codes 0, 4
  f16x2 p1 = as_h2((d & m.hi) | m.exp) * sixteenth + bias16;      // codes 1, 5
  f16x2 p2 = as_h2((d8 & m.lo) | m.exp) + bias;                   // codes 2, 6
  f16x2 p3 = as_h2((d8 & m.hi) | m.exp) * sixteenth + bias16;     // codes 3, 7
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ f16x8 unpack4(uint32_t d) { return unpack4(d, UnpackMasks{0x000F000Fu, 0x00F000F0u, 0x64006400u}); }

// 4 eight-bit codes (byte j = code j) -> two f16x2 in natural order, q - 128.
__device__ __forceinline__ void unpack8(uint32_t d, f16x2& a, f16x2& b) {
  const f16x2 bias = {(_Float16)-1152.f, (_Float16)-1152.f};   // -(1024 + 128)
  // v_perm_b32 selector bytes: 0..3 pick from src1 (d), 4..7 from src0 (0x64646464)
  a = as_h2(__builtin_amdgcn_perm(0x64646464u, d, 0x04010400u)) + bias;  // bytes 0, 1
  b = as_h2(__builtin_amdgcn_perm(0x64646464u, d, 0x04030402u)) + bias;  // bytes 2, 3
}

__device__ __forceinline__ f16x8 unpack8x2(uint32_t d0, uint32_t d1) {
  f16x2 a, b, c, e;
  unpack8(d0, a, b);
  unpack8(d1, c, e);
  f16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = e[0]; r[7] = e[1];
  return r;
}

// SwiGLU g * sigmoid(alpha g) * (u + beta) after the optional clamp limit
// (+inf: none): the gate is bounded above by limit, the linear branch to
// [-limit, limit] (the reading taken of the QMoE manifest's and the MoE
// README's swiglu_limit, which give no formula).
__device__ __forceinline__ float swiglu_act(float g, float u, float alpha, float beta, float limit) {
  g = fminf(g, limit);
  u = fminf(fmaxf(u, -limit), limit);
  return g / (1.f + expf(-alpha * g)) * (u + beta);
}

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Cross-lane exchanges between the four 16-lane row groups of a wavefront
// (gfx950 v_permlane32_swap / v_permlane16_swap).
//   swap32(x, y): lanes 32..63 of x trade places with lanes 0..31 of y.
//   swap16(x, y): rows 1 and 3 of x trade places with rows 0 and 2 of y.
__device__ __forceinline__ void swap32(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}

// 4x4 transpose of dwords across row groups: afterwards row group g holds in
// register j what row group j held in register g.
__device__ __forceinline__ void transpose4x4(u32x4& v) {
  uint32_t d0 = v[0], d1 = v[1], d2 = v[2], d3 = v[3];
  swap32(d0, d2);
  swap32(d1, d3);
  swap16(d0, d1);
  swap16(d2, d3);
  v = u32x4{d0, d1, d2, d3};
}

// Exchange of dword pairs between row groups {0,1} and {2,3}: row group g's
// registers (2,3) trade places with row group (g+2)'s registers (0,1).
__device__ __forceinline__ void swap_pairs(u32x4& v) {
  uint32_t d0 = v[0], d1 = v[1], d2 = v[2], d3 = v[3];
  swap32(d0, d2);
  swap32(d1, d3);
  v = u32x4{d0, d1, d2, d3};
}

// Wave-wide helpers.
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace qmoe
