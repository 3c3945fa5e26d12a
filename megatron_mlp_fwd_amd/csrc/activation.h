// Element-wise activations for the bf16 epilogues and the gated-MLP
// kernels, evaluated in fp32 from fp32 inputs; their results are rounded to
// bf16 by the callers.
#pragma once
#include "common.h"

namespace tpr {

// The exact-erf GELU x Phi(x) and its derivative Phi(x) + x phi(x) for the
// bf16 kernels, whose pre-activation and results are rounded to bf16.  Phi
// comes from the Abramowitz-Stegun 7.1.26 (Hastings) form of erfc,
// erfc(z) = (a1 t + ... + a5 t^5) exp(-z^2), t = 1 / (1 + p z), z >= 0, whose
// error is below 1.5e-7; evaluated in fp32 the error in Phi, gelu and gelu'
// stays below 5e-7 absolute (and below 6e-5 relative for gelu at
// 0.01 < |x| < 3), far under bf16's 2^-8.  exp(-x^2/2) is shared by erfc and
// phi.  Costs about 15 VALU operations instead of a full-precision erfcf.
struct PhiExp {
  float Phi;  // Phi(x)
  float e;    // exp(-x^2 / 2)
};
__device__ __forceinline__ PhiExp phi_exp(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  float p = fmaf(t, 1.061405429f, -1.453152027f);
  p = fmaf(t, p, 1.421413741f);
  p = fmaf(t, p, -0.284496736f);
  p = fmaf(t, p, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-0.72134752044448170f * x * x);  // 1 / (2 ln 2)
  const float q = 0.5f * p * t * e;  // Phi(-|x|)
  return PhiExp{x >= 0.f ? 1.f - q : q, e};
}

// sigma(x) and sigma'(x) for the bf16 kernels, one instance per activation:
//   GELU  x Phi(x),                      Phi(x) + x phi(x)
//   tanh  tanh(x),                       1 - tanh(x)^2
//   SiLU  x s(x), s = 1 / (1 + e^-x),    s (1 + x (1 - s))
// tanh is 1 - 2 / (e^{2|x|} + 1) with the sign of x, and below |x| = 1/8 its
// odd Taylor polynomial to x^7 (truncation error below 3e-10 relative there,
// where the exp form would lose digits to cancellation); fp32 error well
// under bf16's 2^-8 everywhere.
template <int ACT>
__device__ __forceinline__ void act_fast(float x, float& s, float& ds) {
  if constexpr (ACT == ACT_TANH) {
    const float ax = fabsf(x);
    const float e = __builtin_amdgcn_exp2f(2.8853900817779268f * ax);  // e^{2|x|}
    const float big = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
    const float x2 = x * x;
    const float small = ax * fmaf(x2, fmaf(x2, fmaf(x2, -0.053968253968253968f, 0.13333333333333333f),
                                          -0.33333333333333333f), 1.0f);
    const float t = ax < 0.125f ? small : big;
    s = copysignf(t, x);
    ds = fmaf(-t, t, 1.0f);
  } else if constexpr (ACT == ACT_SILU) {
    // e^-x overflows to inf for x < -88: then sg = 0 and s = -0.
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
    s = x * sg;
    ds = sg * fmaf(x, 1.0f - sg, 1.0f);
  } else {
    const PhiExp q = phi_exp(x);
    s = x * q.Phi;
    ds = fmaf(0.39894228040143268f * x, q.e, q.Phi);
  }
}

// The same with the activation chosen at run time (element-wise kernels).
__device__ __forceinline__ void act_eval(int act, float x, float& s, float& ds) {
  if (act == ACT_TANH)
    act_fast<ACT_TANH>(x, s, ds);
  else if (act == ACT_SILU)
    act_fast<ACT_SILU>(x, s, ds);
  else
    act_fast<ACT_GELU>(x, s, ds);
}

// The same functions at full fp32 precision (library erfc, tanh, exp) for
// the fp32 workloads, whose results are compared at fp32 tolerances.
__device__ __forceinline__ void act_eval_f32(int act, float x, float& s, float& ds) {
  if (act == ACT_TANH) {
    s = tanhf(x);
    ds = 1.0f - s * s;
  } else if (act == ACT_SILU) {
    const float sg = 1.0f / (1.0f + expf(-x));
    s = x * sg;
    ds = sg * (1.0f + x * (1.0f - sg));
  } else {
    const float Phi = 0.5f * erfcf(-0.70710678118654752f * x);
    s = x * Phi;
    ds = Phi + 0.39894228040143268f * x * expf(-0.5f * x * x);
  }
}

}  // namespace tpr
