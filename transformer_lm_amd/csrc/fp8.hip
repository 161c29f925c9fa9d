// Per-tensor E4M3 scaling and quantisation, the inputs of the FP8 matrix
// products (talk "llm.c's Origin and the Future of LLM Compilers", chapter
// "Project Roadmap, Community Forks, and LLaMA Architecture Support", names
// FP8 support; the format and recipe are the plain readings: OCP E4M3,
// s = 448 / amax(|x|) in fp32, q = E4M3(x s) rounded to nearest even).
#include "kernels.h"

#define FP8_MAX 448.0f
#define AMAX_BLOCKS 1024
typedef unsigned int q32x4 __attribute__((ext_vector_type(4)));

int64_t fp8_scale_workspace_floats() { return AMAX_BLOCKS; }

// part[b] = max |x_i| over block b's fixed set of 8-element chunks (block 0
// also takes the n % 8 tail). NaN elements are skipped by fmaxf.
__global__ __launch_bounds__(256) void fp8_amax_partial_kernel(float* __restrict__ part,
                                                               const bf16* __restrict__ x,
                                                               int64_t n) {
    __shared__ float red[16];
    float m = 0.f;
    const int64_t n8 = n / 8;
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)AMAX_BLOCKS * 256) {
        float v[8];
        load8(x + 8 * i, v);
#pragma unroll
        for (int e = 0; e < 8; e++) m = fmaxf(m, fabsf(v[e]));
    }
    if (blockIdx.x == 0)
        for (int64_t i = 8 * n8 + threadIdx.x; i < n; i += 256) m = fmaxf(m, fabsf((float)x[i]));
    m = block_max(m, red);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// *scale = 448 / amax (correctly rounded fp32 division), 1 for amax == 0
__global__ __launch_bounds__(256) void fp8_scale_final_kernel(float* __restrict__ scale,
                                                             const float* __restrict__ part) {
    __shared__ float red[16];
    float m = 0.f;
    for (int i = threadIdx.x; i < AMAX_BLOCKS; i += 256) m = fmaxf(m, part[i]);
    m = block_max(m, red);
    if (threadIdx.x == 0) scale[0] = m > 0.f ? FP8_MAX / m : 1.f;
}

void fp8_scale(float* scale, float* work, const bf16* x, int64_t n, hipStream_t st) {
    fp8_amax_partial_kernel<<<AMAX_BLOCKS, 256, 0, st>>>(work, x, n);
    fp8_scale_final_kernel<<<1, 256, 0, st>>>(scale, work);
}

// q_i = E4M3(x_i * s): one fp32 multiply, then the hardware conversion
// (v_cvt_pk_fp8_f32: round to nearest even; magnitudes above 464 give NaN,
// which a scale from fp8_scale of the same tensor never produces). 16
// elements per thread and step: two 16-byte loads, one 16-byte store.
__global__ __launch_bounds__(256) void fp8_quantize_kernel(uint8_t* __restrict__ q,
                                                           const bf16* __restrict__ x,
                                                           const float* __restrict__ scale,
                                                           int64_t n) {
    const float s = *scale;
    const int64_t n16 = n / 16;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += stride) {
        float v[16];
        load8(x + 16 * i, *reinterpret_cast<float(*)[8]>(v));
        load8(x + 16 * i + 8, *reinterpret_cast<float(*)[8]>(v + 8));
        q32x4 o;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            int p = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w] * s, v[4 * w + 1] * s, 0, false);
            p = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w + 2] * s, v[4 * w + 3] * s, p, true);
            o[w] = (uint32_t)p;
        }
        *reinterpret_cast<q32x4*>(q + 16 * i) = o;
    }
    for (int64_t i = 16 * n16 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride)
        q[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32((float)x[i] * s, 0.f, 0, false) & 0xff);
}

void fp8_quantize(uint8_t* q, const bf16* x, const float* scale, int64_t n, hipStream_t st) {
    int64_t blocks = (n / 16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    fp8_quantize_kernel<<<(int)blocks, 256, 0, st>>>(q, x, scale, n);
}
