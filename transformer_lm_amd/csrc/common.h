// Shared device helpers for the gfx950 kernels: storage types, 16-byte vector
// access, wave64 reductions. Device code only deals in raw pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;

// ---------------------------------------------------------------- conversion
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// --------------------------------------------------------- 8-element vectors
// Every activation row length handled here is a multiple of 8 elements, and
// every row start is 16-byte aligned, so rows move in 8-element chunks: one
// 16-byte access for bf16, two for fp32.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
    typedef bf16 raw __attribute__((ext_vector_type(8)));
};
template <> struct Vec8<float> {
    typedef float raw __attribute__((ext_vector_type(8)));
};

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
    typename Vec8<T>::raw r = *reinterpret_cast<const typename Vec8<T>::raw*>(p);
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = to_f32(r[i]);
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]) {
    typename Vec8<T>::raw r;
#pragma unroll
    for (int i = 0; i < 8; i++) r[i] = from_f32<T>(v[i]);
    *reinterpret_cast<typename Vec8<T>::raw*>(p) = r;
}

// ------------------------------------------------------------ wave64 reduce
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024). `scratch` holds
// >= 16 floats of LDS. Every thread receives the total; the combination order
// is fixed, so the result is deterministic.
__device__ __forceinline__ float block_sum(float v, float* scratch) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) scratch[wid] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; i++) t += scratch[i];
    return t;
}

__device__ __forceinline__ float block_max(float v, float* scratch) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) scratch[wid] = v;
    __syncthreads();
    float t = -INFINITY;
    for (int i = 0; i < nw; i++) t = fmaxf(t, scratch[i]);
    return t;
}

static inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
