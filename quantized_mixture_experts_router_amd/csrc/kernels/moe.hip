// Activation pass of the float MoE (com.microsoft.MoE README, Attributes:
// activation_type, swiglu_fusion, activation_alpha / beta).  One thread per
// element of the activation rows act[p][j] (p < S sorted positions, j < I),
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
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
#define QMOE_MOE_ACT(A) hipLaunchKernelGGL(qmoe_moe_act<A>, grid, block, 0, st, h, u3, S, I, F, fusion, alpha, beta, limit, act)
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
