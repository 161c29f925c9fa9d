// tanh-GELU, the MLP activation of GPT-2 (page "Building GPT-2 from scratch",
// section on the MLP block; page "llm.c: Large Language Model Training in Pure
// C/CUDA Without Dependencies", the GELU kernel):
//   g(x) = x/2 (1 + tanh a),  a = sqrt(2/pi) (x + 0.044715 x^3).
// With s = 1 / (1 + exp(-2a)) = (1 + tanh a)/2 the same function is g = x s,
// and its derivative g' = s + 2 x s (1 - s) da/dx, da/dx = sqrt(2/pi)
// (1 + 3 * 0.044715 x^2). That form costs one exponential and one reciprocal
// on the hardware units; it is used where GELU rides in a matrix-product
// epilogue.
#pragma once

#include <hip/hip_runtime.h>

#define GELU_K 0.7978845608028654f  // sqrt(2/pi)
#define GELU_C 0.044715f
#define GELU_M2LOG2E (-2.8853900817779268f)  // -2 log2(e)

// 1 / (1 + 2^(x (c1 + c2 x^2))) with c1 = -2 log2(e) sqrt(2/pi), c2 = 0.044715 c1
__device__ __forceinline__ float gelu_sigmoid_2a(float x) {
    constexpr float c1 = GELU_M2LOG2E * GELU_K, c2 = c1 * GELU_C;
    const float u = x * fmaf(c2, x * x, c1);
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(u));
}

__device__ __forceinline__ float gelu_fast(float x) { return x * gelu_sigmoid_2a(x); }

// g' = s + (2 x da/dx) s (1 - s) with 2 da/dx = 2 sqrt(2/pi) + 6 * 0.044715
// sqrt(2/pi) x^2: x^2 shared with the sigmoid's argument, s (1 - s) one fma,
// eight VALU operations and the two hardware transcendentals.
__device__ __forceinline__ float gelu_grad_fast(float x) {
    constexpr float c1 = GELU_M2LOG2E * GELU_K, c2 = c1 * GELU_C;
    const float x2 = x * x;
    const float s = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * fmaf(c2, x2, c1)));
    const float xd = x * fmaf(6.f * GELU_C * GELU_K, x2, 2.f * GELU_K);
    return fmaf(xd, fmaf(-s, s, s), s);
}
