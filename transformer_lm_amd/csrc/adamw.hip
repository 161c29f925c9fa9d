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

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ theta,
                                                    const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    bf16* __restrict__ theta_bf16, int64_t n,
                                                    float lr, float b1, float b2, float eps,
                                                    float wd, float c1, float c2) {
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 th = reinterpret_cast<float4*>(theta)[i];
        const float4 gg = reinterpret_cast<const float4*>(g)[i];
        float4 mm = reinterpret_cast<float4*>(m)[i];
        float4 vv = reinterpret_cast<float4*>(v)[i];
        adamw_one(th.x, gg.x, mm.x, vv.x, lr, b1, b2, eps, wd, c1, c2);
        adamw_one(th.y, gg.y, mm.y, vv.y, lr, b1, b2, eps, wd, c1, c2);
        adamw_one(th.z, gg.z, mm.z, vv.z, lr, b1, b2, eps, wd, c1, c2);
        adamw_one(th.w, gg.w, mm.w, vv.w, lr, b1, b2, eps, wd, c1, c2);
        reinterpret_cast<float4*>(theta)[i] = th;
        reinterpret_cast<float4*>(m)[i] = mm;
        reinterpret_cast<float4*>(v)[i] = vv;
        if (theta_bf16) {
            typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 o = {(bf16)th.x, (bf16)th.y, (bf16)th.z, (bf16)th.w};
            reinterpret_cast<bf16x4*>(theta_bf16)[i] = o;
        }
    }
    // tail (n % 4 elements)
    for (int64_t i = n4 * 4 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
        float th = theta[i], mm = m[i], vv = v[i];
        adamw_one(th, g[i], mm, vv, lr, b1, b2, eps, wd, c1, c2);
        theta[i] = th;
        m[i] = mm;
        v[i] = vv;
        if (theta_bf16) theta_bf16[i] = (bf16)th;
    }
}

void adamw(float* theta, const float* g, float* m, float* v, bf16* theta_bf16, int64_t n,
           float lr, float b1, float b2, float eps, float wd, float c1, float c2,
           hipStream_t st) {
    int64_t blocks = (n / 4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    adamw_kernel<<<(int)blocks, 256, 0, st>>>(theta, g, m, v, theta_bf16, n, lr, b1, b2, eps, wd,
                                              c1, c2);
}
