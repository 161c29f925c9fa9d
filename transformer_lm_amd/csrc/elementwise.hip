// Elementwise kernels: tanh-GELU forward/backward, fills, fp32 -> bf16 rounding.
// HBM-bound: 16-byte (8 x bf16) or 2 x 16-byte (8 x fp32) accesses per thread.
#include "gelu.h"
#include "kernels.h"

// GELU in its tanh form (the MLP activation of GPT-2):
// g(x) = x/2 (1 + tanh(a)), a = sqrt(2/pi) (x + 0.044715 x^3).
__device__ __forceinline__ float gelu(float x) {
    float a = GELU_K * (x + GELU_C * x * x * x);
    return 0.5f * x * (1.f + tanhf(a));
}

// g'(x) = (1 + tanh a)/2 + x/2 (1 - tanh^2 a) sqrt(2/pi) (1 + 3 * 0.044715 x^2)
__device__ __forceinline__ float gelu_grad(float x) {
    float a = GELU_K * (x + GELU_C * x * x * x);
    float th = tanhf(a);
    float da = GELU_K * (1.f + 3.f * GELU_C * x * x);
    return 0.5f * (1.f + th) + 0.5f * x * (1.f - th * th) * da;
}

template <typename T>
__global__ __launch_bounds__(256) void gelu_fwd_kernel(T* __restrict__ out,
                                                       const T* __restrict__ inp, int64_t n8) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8;
         i += (int64_t)gridDim.x * blockDim.x) {
        float v[8];
        load8(inp + i * 8, v);
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = gelu(v[k]);
        store8(out + i * 8, v);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void gelu_bwd_kernel(T* dinp, const T* __restrict__ inp,
                                                       const T* dout, int64_t n8) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8;
         i += (int64_t)gridDim.x * blockDim.x) {
        float x[8], d[8];
        load8(inp + i * 8, x);
        load8(dout + i * 8, d);
#pragma unroll
        for (int k = 0; k < 8; k++) d[k] = gelu_grad(x[k]) * d[k];
        store8(dinp + i * 8, d);
    }
}

static int grid_for(int64_t n_threads) {
    int64_t g = (n_threads + 255) / 256;
    return (int)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

template <typename T>
void gelu_fwd(T* out, const T* inp, int64_t n, hipStream_t st) {
    gelu_fwd_kernel<T><<<grid_for(n / 8), 256, 0, st>>>(out, inp, n / 8);
}

template <typename T>
void gelu_bwd(T* dinp, const T* inp, const T* dout, int64_t n, hipStream_t st) {
    gelu_bwd_kernel<T><<<grid_for(n / 8), 256, 0, st>>>(dinp, inp, dout, n / 8);
}

template void gelu_fwd<float>(float*, const float*, int64_t, hipStream_t);
template void gelu_fwd<bf16>(bf16*, const bf16*, int64_t, hipStream_t);
template void gelu_bwd<float>(float*, const float*, const float*, int64_t, hipStream_t);
template void gelu_bwd<bf16>(bf16*, const bf16*, const bf16*, int64_t, hipStream_t);

template <typename U>
__global__ __launch_bounds__(256) void fill_zero_kernel(U* p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

void fill_zero_f32(float* p, int64_t n, hipStream_t st) {
    if (n > 0) fill_zero_kernel<float><<<grid_for(n), 256, 0, st>>>(p, n);
}

void fill_zero_i32(int* p, int64_t n, hipStream_t st) {
    if (n > 0) fill_zero_kernel<int><<<grid_for(n), 256, 0, st>>>(p, n);
}

__global__ __launch_bounds__(256) void round_bf16_kernel(bf16* __restrict__ out,
                                                         const float* __restrict__ in,
                                                         int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        out[i] = (bf16)in[i];
}

void round_to_bf16(bf16* out, const float* in, int64_t n, hipStream_t st) {
    if (n > 0) round_bf16_kernel<<<grid_for(n), 256, 0, st>>>(out, in, n);
}
