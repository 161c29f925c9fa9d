// LayerNorm forward and backward over rows of C channels (C % 8 == 0,
// C <= 2048), the operation llm.c writes out over bare float arrays (talk
// "llm.c's Origin and the Future of LLM Compilers", chapter "Deconstructing
// PyTorch Abstractions"). One wave64 per row; a lane holds up to NCH chunks of
// 8 channels (chunk k of lane l covers channels (l + 64k) * 8 .. +7) in
// registers, so a row is read from HBM once. NCH is 2 for C <= 1024 and 4
// above. Statistics and all sums are fp32.
#include "kernels.h"

#define LN_EPS 1e-5f
#define LN_ROWS_PER_BLOCK 4

// mu = mean(x); var = mean((x - mu)^2) (biased); r = 1/sqrt(var + eps);
// y = (x - mu) r w + b. Saves mu and r.
template <typename T, int NCH>
__global__ __launch_bounds__(256) void layernorm_fwd_kernel(T* __restrict__ out,
                                                            float* __restrict__ mean,
                                                            float* __restrict__ rstd,
                                                            const T* __restrict__ inp,
                                                            const T* __restrict__ w,
                                                            const T* __restrict__ b, int N,
                                                            int C) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * LN_ROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (row >= N) return;
    const T* x = inp + (int64_t)row * C;
    float v[NCH][8];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; k++) {
        const int c = (lane + 64 * k) * 8;
        if (c < C) {
            load8(x + c, v[k]);
#pragma unroll
            for (int i = 0; i < 8; i++) s += v[k][i];
        }
    }
    const float mu = wave_sum(s) / C;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; k++) {
        const int c = (lane + 64 * k) * 8;
        if (c < C)
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float d = v[k][i] - mu;
                ss += d * d;
            }
    }
    const float r = 1.f / sqrtf(wave_sum(ss) / C + LN_EPS);
#pragma unroll
    for (int k = 0; k < NCH; k++) {
        const int c = (lane + 64 * k) * 8;
        if (c < C) {
            float wv[8], bv[8], o[8];
            load8(w + c, wv);
            load8(b + c, bv);
#pragma unroll
            for (int i = 0; i < 8; i++) o[i] = (v[k][i] - mu) * r * wv[i] + bv[i];
            store8(out + (int64_t)row * C + c, o);
        }
    }
    if (lane == 0) {
        mean[row] = mu;
        rstd[row] = r;
    }
}

template <typename T>
void layernorm_fwd(T* out, float* mean, float* rstd, const T* inp, const T* w, const T* b,
                   int N, int C, hipStream_t st) {
    const int grid = ceil_div(N, LN_ROWS_PER_BLOCK);
    if (C <= 1024)
        layernorm_fwd_kernel<T, 2><<<grid, 256, 0, st>>>(out, mean, rstd, inp, w, b, N, C);
    else
        layernorm_fwd_kernel<T, 4><<<grid, 256, 0, st>>>(out, mean, rstd, inp, w, b, N, C);
}

// Backward. With xhat = (x - mu) r and g = w dy:
//   dx = r (g - mean(g) - xhat mean(g xhat))
// dw = sum_rows dy xhat and db = sum_rows dy are reduced deterministically:
// each block walks a fixed set of rows, its four waves' register sums are
// combined in wave order through LDS into one partial row per block, and a
// second kernel sums the partial rows in a fixed order.
#define LN_BWD_BLOCKS 1024

template <typename T, int NCH>
__global__ __launch_bounds__(256) void layernorm_bwd_kernel(
    T* dinp, const T* dadd, const T* __restrict__ dout, const T* __restrict__ inp,
    const T* __restrict__ w, const float* __restrict__ mean, const float* __restrict__ rstd,
    int N, int C, float* __restrict__ partials) {
    __shared__ float red[2 * 2048];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    float dw[NCH][8], db[NCH][8], wv[NCH][8];
#pragma unroll
    for (int k = 0; k < NCH; k++) {
        const int c = (lane + 64 * k) * 8;
#pragma unroll
        for (int i = 0; i < 8; i++) dw[k][i] = db[k][i] = 0.f;
        if (c < C) load8(w + c, wv[k]);
    }
    for (int row = blockIdx.x * LN_ROWS_PER_BLOCK + wid; row < N;
         row += gridDim.x * LN_ROWS_PER_BLOCK) {
        const float mu = mean[row], r = rstd[row];
        float xh[NCH][8], dy[NCH][8];
        float gs = 0.f, gxs = 0.f;
#pragma unroll
        for (int k = 0; k < NCH; k++) {
            const int c = (lane + 64 * k) * 8;
            if (c < C) {
                load8(inp + (int64_t)row * C + c, xh[k]);
                load8(dout + (int64_t)row * C + c, dy[k]);
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    xh[k][i] = (xh[k][i] - mu) * r;
                    const float g = wv[k][i] * dy[k][i];
                    gs += g;
                    gxs += g * xh[k][i];
                    dw[k][i] += dy[k][i] * xh[k][i];
                    db[k][i] += dy[k][i];
                }
            }
        }
        const float gm = wave_sum(gs) / C, gxm = wave_sum(gxs) / C;
#pragma unroll
        for (int k = 0; k < NCH; k++) {
            const int c = (lane + 64 * k) * 8;
            if (c < C) {
                float o[8];
                if (dadd) load8(dadd + (int64_t)row * C + c, o);
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const float dx = (wv[k][i] * dy[k][i] - gm - xh[k][i] * gxm) * r;
                    o[i] = dadd ? o[i] + dx : dx;
                }
                store8(dinp + (int64_t)row * C + c, o);
            }
        }
    }
    // combine the four waves in order: wave 0 stores, waves 1..3 add in turn
    for (int q = 0; q < LN_ROWS_PER_BLOCK; q++) {
        if (wid == q) {
#pragma unroll
            for (int k = 0; k < NCH; k++) {
                const int c = (lane + 64 * k) * 8;
                if (c < C)
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        red[c + i] = q == 0 ? dw[k][i] : red[c + i] + dw[k][i];
                        red[2048 + c + i] = q == 0 ? db[k][i] : red[2048 + c + i] + db[k][i];
                    }
            }
        }
        __syncthreads();
    }
    float* prow = partials + (int64_t)blockIdx.x * 2 * C;
    for (int c = threadIdx.x; c < C; c += blockDim.x) {
        prow[c] = red[c];
        prow[C + c] = red[2048 + c];
    }
}

// Sums the partial rows in two fixed-order stages. Stage 1: block (x, y) owns
// 64 columns and partial rows [y*G, (y+1)*G) (G = nblocks / LN_RED_GROUPS); its
// four row phases each sum every fourth row, then combine in phase order.
// Stage 2 sums the LN_RED_GROUPS stage-1 rows of each column in order.
#define LN_RED_GROUPS 16

// Any number of LayerNorms at once (blockIdx.z selects one): each has its
// partial rows at partials + z * LN_BWD_BLOCKS * 2C and its stage-1 rows at
// stage + z * LN_RED_GROUPS * 2C.
__global__ __launch_bounds__(256) void layernorm_bwd_reduce1_kernel(
    float* __restrict__ stage, const float* __restrict__ partials, int nblocks, int C) {
    __shared__ float red[4][64];
    partials += (int64_t)blockIdx.z * LN_BWD_BLOCKS * 2 * C;
    stage += (int64_t)blockIdx.z * LN_RED_GROUPS * 2 * C;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int j = blockIdx.x * 64 + tx;
    const int per = (nblocks + LN_RED_GROUPS - 1) / LN_RED_GROUPS;
    const int r0 = blockIdx.y * per, r1 = min(nblocks, r0 + per);
    float s = 0.f;
    if (j < 2 * C)
        for (int b = r0 + ty; b < r1; b += 4) s += partials[(int64_t)b * 2 * C + j];
    red[ty][tx] = s;
    __syncthreads();
    if (ty == 0 && j < 2 * C)
        stage[(int64_t)blockIdx.y * 2 * C + j] = ((red[0][tx] + red[1][tx]) + red[2][tx]) + red[3][tx];
}

__global__ __launch_bounds__(256) void layernorm_bwd_reduce2_kernel(const LnRedBatch b,
                                                                   const float* __restrict__ stage,
                                                                   int C) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= 2 * C) return;
    float* dw = b.t[blockIdx.y].dw;
    float* db = b.t[blockIdx.y].db;
    stage += (int64_t)blockIdx.y * LN_RED_GROUPS * 2 * C;
    float t = 0.f;
#pragma unroll
    for (int r = 0; r < LN_RED_GROUPS; r++) t += stage[(int64_t)r * 2 * C + j];
    if (j < C)
        dw[j] = t;
    else
        db[j - C] = t;
}

// workspace of `count` LayerNorms: their partial rows, then their stage-1 rows
int64_t layernorm_bwd_partials(int C, int count) {
    return (int64_t)count * (LN_BWD_BLOCKS + LN_RED_GROUPS) * 2 * C;
}

template <typename T>
void layernorm_bwd_rows(T* dinp, const T* dadd, const T* dout, const T* inp, const T* w,
                        const float* mean, const float* rstd, int N, int C, float* partials,
                        int slot, hipStream_t st) {
    int nb = ceil_div(N, LN_ROWS_PER_BLOCK);
    if (nb > LN_BWD_BLOCKS) nb = LN_BWD_BLOCKS;
    partials += (int64_t)slot * LN_BWD_BLOCKS * 2 * C;
    if (C <= 1024)
        layernorm_bwd_kernel<T, 2><<<nb, 256, 0, st>>>(dinp, dadd, dout, inp, w, mean, rstd,
                                                       N, C, partials);
    else
        layernorm_bwd_kernel<T, 4><<<nb, 256, 0, st>>>(dinp, dadd, dout, inp, w, mean, rstd,
                                                       N, C, partials);
}

void layernorm_bwd_reduce(const LnRedBatch& b, int N, int C, float* partials, int count,
                          hipStream_t st) {
    int nb = ceil_div(N, LN_ROWS_PER_BLOCK);
    if (nb > LN_BWD_BLOCKS) nb = LN_BWD_BLOCKS;
    float* stage = partials + (int64_t)count * LN_BWD_BLOCKS * 2 * C;
    layernorm_bwd_reduce1_kernel<<<dim3(ceil_div(2 * C, 64), LN_RED_GROUPS, b.count), 256, 0,
                                   st>>>(stage, partials, nb, C);
    layernorm_bwd_reduce2_kernel<<<dim3(ceil_div(2 * C, 256), b.count), 256, 0, st>>>(b, stage, C);
}

template void layernorm_fwd<float>(float*, float*, float*, const float*, const float*,
                                   const float*, int, int, hipStream_t);
template void layernorm_fwd<bf16>(bf16*, float*, float*, const bf16*, const bf16*, const bf16*,
                                  int, int, hipStream_t);
template void layernorm_bwd_rows<float>(float*, const float*, const float*, const float*,
                                        const float*, const float*, const float*, int, int, float*,
                                        int, hipStream_t);
template void layernorm_bwd_rows<bf16>(bf16*, const bf16*, const bf16*, const bf16*, const bf16*,
                                       const float*, const float*, int, int, float*, int,
                                       hipStream_t);
