// Activation pass of the float MoE (com.microsoft.MoE README, Attributes:
// activation_type, swiglu_fusion, activation_alpha / beta).  Four elements
// a thread (one when I is not a multiple of 4) of the activation rows
// act[p][j] (p < S sorted positions, j < I),
// from the FC1 rows h[p] (F = I or 2 I floats) and, where read, the FC3 rows
// u3[p] (I floats):
//   relu      max(h, 0)
//   gelu      h Phi(h) = h erfc(-h / sqrt 2) / 2      (exact GELU)
//   silu      h sigmoid(h)  [* u3 when FC3 is given]
//   swiglu    g sigmoid(alpha g) (u + beta), (g, u) = (h[j], u3[j]) for
//             fusion 0, (h[2j], h[2j+1]) for 1, (h[j], h[I + j]) for 2,
//             after the optional clamp limit (see swiglu_act in common.hpp)
//   identity  h
// float32 libm (erfcf, expf) throughout.
#include "common.hpp"
#include "launch.h"

namespace qmoe {

__device__ __forceinline__ float moe_sigmoid(float v) { return 1.f / (1.f + expf(-v)); }

// Activation of one element from its FC1 value v (the gate g for SwiGLU) and
// its second operand w (SwiGLU: the linear value u; SiLU with FC3: the FC3
// value; otherwise unused).
template <int ACT>
__device__ __forceinline__ float moe_act_value(float v, float w, bool has_w, float alpha, float beta, float limit) {
  if (ACT == MOE_ACT_SWIGLU) return swiglu_act(v, w, alpha, beta, limit);
  if (ACT == MOE_ACT_RELU) return fmaxf(v, 0.f);
  if (ACT == MOE_ACT_GELU) return 0.5f * v * erfcf(-v * 0.70710678118654752f);
  if (ACT == MOE_ACT_SILU) return has_w ? v * moe_sigmoid(v) * w : v * moe_sigmoid(v);
  return v;
}

// Four consecutive elements a thread (I % 4 == 0): workgroup b covers
// row b / nb, elements 1024 (b % nb) onward, with 16-byte loads and stores.
template <int ACT>
__global__ void __launch_bounds__(256) qmoe_moe_act4(const float* __restrict__ h, const float* __restrict__ u3,
                                                     int I, int F, int fusion, int nb, float alpha, float beta,
                                                     float limit, float* __restrict__ act) {
  const int p = blockIdx.x / nb;
  const int j = (blockIdx.x - p * nb) * 1024 + 4 * threadIdx.x;
  if (j >= I) return;
  const float* hp = h + (long)p * F;
  f32x4 v, w = {0.f, 0.f, 0.f, 0.f};
  const bool has_w = (ACT == MOE_ACT_SWIGLU) || (ACT == MOE_ACT_SILU && u3 != nullptr);
  if (ACT == MOE_ACT_SWIGLU && fusion == 1) {
    // interleaved (g, u) pairs: eight consecutive values
    const f32x4 a0 = *(const f32x4*)(hp + 2 * j), a1 = *(const f32x4*)(hp + 2 * j + 4);
    v = f32x4{a0[0], a0[2], a1[0], a1[2]};
    w = f32x4{a0[1], a0[3], a1[1], a1[3]};
  } else {
    v = *(const f32x4*)(hp + j);
    if (ACT == MOE_ACT_SWIGLU && fusion == 2) w = *(const f32x4*)(hp + I + j);
    else if (has_w) w = *(const f32x4*)(u3 + (long)p * I + j);
  }
  f32x4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = moe_act_value<ACT>(v[c], w[c], has_w, alpha, beta, limit);
  *(f32x4*)(act + (long)p * I + j) = r;
}

template <int ACT>
__global__ void __launch_bounds__(256) qmoe_moe_act(const float* __restrict__ h, const float* __restrict__ u3,
                                                    long S, int I, int F, int fusion, float alpha, float beta,
                                                    float limit, float* __restrict__ act) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= S * I) return;
  const long p = i / I;
  const int j = (int)(i % I);
  const float* hp = h + p * F;
  float a;
  if (ACT == MOE_ACT_SWIGLU) {
    float g, u;
    if (fusion == 0) {
      g = hp[j];
      u = u3[p * I + j];
    } else if (fusion == 1) {
      g = hp[2 * j];
      u = hp[2 * j + 1];
    } else {
      g = hp[j];
      u = hp[I + j];
    }
    a = swiglu_act(g, u, alpha, beta, limit);
  } else {
    const float v = hp[j];
    if (ACT == MOE_ACT_RELU) a = fmaxf(v, 0.f);
    else if (ACT == MOE_ACT_GELU) a = 0.5f * v * erfcf(-v * 0.70710678118654752f);
    else if (ACT == MOE_ACT_SILU) a = u3 ? v * moe_sigmoid(v) * u3[p * I + j] : v * moe_sigmoid(v);
    else a = v;
  }
  act[i] = a;
}

hipError_t launch_moe_act(int act_type, const float* h, const float* u3, long S, int I, int F, int fusion,
                          float alpha, float beta, float limit, float* act, hipStream_t st) {
  const long n = S * I;
  if (n <= 0) return hipSuccess;
  const int nb = (I + 1023) / 1024;
  const bool four = I % 4 == 0 && F % 4 == 0 && S * nb < (1L << 31);
  const dim3 grid(four ? (unsigned)(S * nb) : (unsigned)((n + 255) / 256)), block(256);
#define QMOE_MOE_ACT(A)                                                                                          \
  if (four)                                                                                                      \
    hipLaunchKernelGGL(qmoe_moe_act4<A>, grid, block, 0, st, h, u3, I, F, fusion, nb, alpha, beta, limit, act);   \
  else                                                                                                           \
    hipLaunchKernelGGL(qmoe_moe_act<A>, grid, block, 0, st, h, u3, S, I, F, fusion, alpha, beta, limit, act)
  switch (act_type) {
    case MOE_ACT_RELU: QMOE_MOE_ACT(MOE_ACT_RELU); break;
    case MOE_ACT_SWIGLU: QMOE_MOE_ACT(MOE_ACT_SWIGLU); break;
    case MOE_ACT_GELU: QMOE_MOE_ACT(MOE_ACT_GELU); break;
    case MOE_ACT_SILU: QMOE_MOE_ACT(MOE_ACT_SILU); break;
    case MOE_ACT_IDENTITY: QMOE_MOE_ACT(MOE_ACT_IDENTITY); break;
    default: return hipErrorInvalidValue;
  }
#undef QMOE_MOE_ACT
  return hipGetLastError();
}

}  // namespace qmoe
