// Elementwise epilogue math applied to fp32 GEMM accumulators.
#pragma once

#include "common.h"

namespace tpmlp {

// tanh approximation of GeLU (Hendrycks & Gimpel 2016):
//   g(y) = 0.5 y (1 + tanh(u)),  u = sqrt(2/pi) (y + 0.044715 y^3).
// Evaluated through the identity 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)),
// which needs one exponential and one reciprocal.  For y -> -inf the
// exponential overflows to +inf, the reciprocal is 0 and the result -0; for
// y -> +inf it underflows to 0 and the result is y.
constexpr float kGeluTwoScale = 1.5957691216057308f;  // 2 * sqrt(2 / pi)
constexpr float kGeluCubic = 0.044715f;

__device__ __forceinline__ float gelu_sigmoid_arg(float y)  // 2u
{
    return kGeluTwoScale * (y + kGeluCubic * y * y * y);
}

// The logistic factor 1 / (1 + exp(-2u)) uses the hardware reciprocal
// (v_rcp_f32, 1 ulp) rather than a correctly rounded division; the results
// are rounded to bf16 or compared at the fp32 tolerance, and the limits hold:
// an infinite denominator gives 0.
__device__ __forceinline__ float logistic_2u(float y)
{
    return __builtin_amdgcn_rcpf(1.0f + __expf(-gelu_sigmoid_arg(y)));
}

__device__ __forceinline__ float gelu_tanh(float y)
{
    return y * logistic_2u(y);
}

// g'(y).  With s = 1 / (1 + exp(-2u)) (so 1 + tanh(u) = 2s and
// 1 - tanh(u)^2 = 4 s (1 - s)) the derivative of y * s(2u(y)) is
//   g'(y) = s + y * s (1 - s) * 2 u'(y),   2 u'(y) = 2 sqrt(2/pi) (1 + 3 * 0.044715 y^2).
__device__ __forceinline__ float gelu_tanh_grad(float y)
{
    const float s = logistic_2u(y);
    const float du2 = kGeluTwoScale * (1.0f + 3.0f * kGeluCubic * y * y);
    return s + y * s * (1.0f - s) * du2;
}

}  // namespace tpmlp
