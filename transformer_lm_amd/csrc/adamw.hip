// AdamW over the flat parameter array (page "Building GPT-2 from scratch",
// exercise A2; page "llm.c: Large Language Model Training in Pure C/CUDA
// Without Dependencies": every AdamW step in explicit kernels). One pass reads
// theta, g, m, v (fp32) and writes theta, m, v and, in bf16 mode, the bf16
// working copy: 16-byte accesses, 4 parameters per thread per iteration.
#include "kernels.h"

__device__ __forceinline__ void adamw_one(float& th, float g, float& m, float& v, float lr,
                                          float b1, float b2, float eps, float wd, float c1,
                                          float c2) {
    m = b1 * m + (1.f - b1) * g;
    v = b2 * v + (1.f - b2) * g * g;
    const float mhat = m / c1, vhat = v / c2;
    th -= lr * (mhat / (sqrtf(vhat) + eps) + wd * th);
}

#define ADAMW_GROUPS 4
// Each thread handles ADAMW_GROUPS float4 groups per iteration (16 loads in flight);
// the streams are touched once, so loads and stores bypass cache retention.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 ld_nt(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void st_nt(float* p, f32x4 x) {
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

// Gradient clipping factor: clip / ||g|| when the norm (device scalar, from
// grad_norm) exceeds clip, else 1 (also without a norm).
__device__ __forceinline__ float clip_scale(const float* gnorm, float clip) {
    if (!gnorm) return 1.f;
    const float nrm = *gnorm;
    return nrm > clip ? clip / nrm : 1.f;
}

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ theta,
                                                    const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    bf16* __restrict__ theta_bf16, int64_t n,
                                                    float lr, float b1, float b2, float eps,
                                                    float wd, float c1, float c2,
                                                    const float* __restrict__ gnorm, float clip) {
    typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const float gs = clip_scale(gnorm, clip);
    constexpr int U = ADAMW_GROUPS;
    const int64_t nq = n / (4 * U);  // groups of 4 per stream
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nq; i += stride) {
        // U groups nq*4 elements apart: every stream coalesces
        int64_t e[U];
        f32x4 th[U], gg[U], mm[U], vv[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            e[u] = (i + u * nq) * 4;
            th[u] = ld_nt(theta + e[u]);
            gg[u] = ld_nt(g + e[u]) * gs;
            mm[u] = ld_nt(m + e[u]);
            vv[u] = ld_nt(v + e[u]);
        }
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
            for (int k = 0; k < 4; k++) {
                float t = th[u][k], a = mm[u][k], b = vv[u][k];
                adamw_one(t, gg[u][k], a, b, lr, b1, b2, eps, wd, c1, c2);
                th[u][k] = t;
                mm[u][k] = a;
                vv[u][k] = b;
            }
#pragma unroll
        for (int u = 0; u < U; u++) {
            st_nt(theta + e[u], th[u]);
            st_nt(m + e[u], mm[u]);
            st_nt(v + e[u], vv[u]);
            if (theta_bf16)
                *reinterpret_cast<bf16x4*>(theta_bf16 + e[u]) =
                    bf16x4{(bf16)th[u][0], (bf16)th[u][1], (bf16)th[u][2], (bf16)th[u][3]};
        }
    }
    // tail (n % (4U) elements)
    for (int64_t i = nq * 4 * U + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
        float th = theta[i], mm = m[i], vv = v[i];
        adamw_one(th, g[i] * gs, mm, vv, lr, b1, b2, eps, wd, c1, c2);
        theta[i] = th;
        m[i] = mm;
        v[i] = vv;
        if (theta_bf16) theta_bf16[i] = (bf16)th;
    }
}

void adamw(float* theta, const float* g, float* m, float* v, bf16* theta_bf16, int64_t n,
           float lr, float b1, float b2, float eps, float wd, float c1, float c2,
           const float* gnorm, float clip, hipStream_t st) {
    int64_t blocks = (n / (4 * ADAMW_GROUPS) + 255) / 256;
    // one pass per thread up to 2^34 parameters (a grid-stride loop over a
    // capped grid measured slower: 7% at 124M, and 1.5B parameters took 6 passes)
    if (blocks > (1 << 22)) blocks = 1 << 22;
    if (blocks < 1) blocks = 1;
    adamw_kernel<<<(int)blocks, 256, 0, st>>>(theta, g, m, v, theta_bf16, n, lr, b1, b2, eps, wd,
                                              c1, c2, gnorm, clip);
}

// ---------------------------------------------------------------------------
// Global L2 norm of the gradient, the quantity that gradient clipping (page
// "Building GPT-2 from scratch", exercise table row A5) compares against its
// threshold: ||g|| = sqrt(sum_i g_i^2) over the whole flat array. Two fixed-
// shape passes keep it deterministic: GNORM_BLOCKS blocks each sum the squares
// of a fixed set of 4-float groups (thread order, then the block reduction),
// then one block adds the partials in block order.
#define GNORM_BLOCKS 1024

int64_t grad_norm_workspace_floats() { return GNORM_BLOCKS; }

__global__ __launch_bounds__(256) void grad_norm_partial_kernel(float* __restrict__ part,
                                                                const float* __restrict__ g,
                                                                int64_t n) {
    __shared__ float red[16];
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)GNORM_BLOCKS * 256;
    float s = 0.f;
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const f32x4 x = ld_nt(g + 4 * i);
        s += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
    }
    if (blockIdx.x == 0)  // tail (n % 4 elements)
        for (int64_t i = 4 * n4 + threadIdx.x; i < n; i += 256) s += g[i] * g[i];
    s = block_sum(s, red);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}

__global__ __launch_bounds__(1024) void grad_norm_final_kernel(float* __restrict__ out,
                                                               const float* __restrict__ part) {
    __shared__ float red[16];
    const float s = block_sum(part[threadIdx.x], red);  // GNORM_BLOCKS == blockDim.x
    if (threadIdx.x == 0) out[0] = sqrtf(s);
}

void grad_norm(float* out, float* part, const float* g, int64_t n, hipStream_t st) {
    grad_norm_partial_kernel<<<GNORM_BLOCKS, 256, 0, st>>>(part, g, n);
    grad_norm_final_kernel<<<1, GNORM_BLOCKS, 0, st>>>(out, part);
}
