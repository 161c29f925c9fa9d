// LayerNorm forward and backward over rows of C channels (C % 8 == 0,
// C <= 2048), the operation llm.c writes out over bare float arrays (talk
// "llm.c's Origin and the Future of LLM Compilers", chapter "Deconstructing
// PyTorch Abstractions"). A row belongs to one 32-lane half of a wave: lane l
// of the half holds the NCH = ceil(C / 256) chunks of 8 channels
// (l + 32k) * 8 .. +7 in registers, so a row is read from HBM once, and at
// C = 768 every lane holds exactly three chunks. Statistics and all sums are
// fp32.
#include "kernels.h"

#define LN_EPS 1e-5f
#define LN_FWD_RPH 2              // rows per half-wave in the forward kernel
#define LN_FWD_ROWS (8 * LN_FWD_RPH)  // rows per 256-thread forward block
#define LN_BWD_ROWS 8             // rows per 256-thread backward block and pass

// sum over the 32 lanes of this lane's half of the wave (fixed xor tree)
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, 32);
    return v;
}

template <typename T>
__device__ __forceinline__ void raw_to_f32(const typename Vec8<T>::raw& r, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = to_f32(r[i]);
}

// mu = mean(x); var = mean((x - mu)^2) (biased); r = 1/sqrt(var + eps);
// y = (x - mu) r w + b. Saves mu and r. Half-wave hw of the wave handles rows
// base + hw, base + hw + 2, ...; every load of those rows and of w, b is issued
// before the first reduction. Rows past N compute on zeros and store nothing.
template <typename T, int NCH>
__global__ __launch_bounds__(256) void layernorm_fwd_kernel(T* __restrict__ out,
                                                            float* __restrict__ mean,
                                                            float* __restrict__ rstd,
                                                            const T* __restrict__ inp,
                                                            const T* __restrict__ w,
                                                            const T* __restrict__ b, int N,
                                                            int C) {
    using Raw = typename Vec8<T>::raw;
    const int lane = threadIdx.x & 63, hl = lane & 31;
    const int base = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 * LN_FWD_RPH + (lane >> 5);
    Raw xr[LN_FWD_RPH][NCH], wr[NCH], br[NCH];
#pragma unroll
    for (int r = 0; r < LN_FWD_RPH; r++) {
        const int row = base + 2 * r;
#pragma unroll
        for (int k = 0; k < NCH; k++) {
            const int c = (hl + 32 * k) * 8;
            xr[r][k] = row < N && c < C ? *reinterpret_cast<const Raw*>(inp + (int64_t)row * C + c)
                                        : Raw{};
        }
    }
#pragma unroll
    for (int k = 0; k < NCH; k++) {
        const int c = (hl + 32 * k) * 8;
        wr[k] = c < C ? *reinterpret_cast<const Raw*>(w + c) : Raw{};
        br[k] = c < C ? *reinterpret_cast<const Raw*>(b + c) : Raw{};
    }
#pragma unroll
    for (int r = 0; r < LN_FWD_RPH; r++) {
        const int row = base + 2 * r;
        float v[NCH][8];
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < NCH; k++) {
            raw_to_f32<T>(xr[r][k], v[k]);
#pragma unroll
            for (int i = 0; i < 8; i++) s += v[k][i];
        }
        const float mu = half_sum(s) / C;
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < NCH; k++) {
            const int c = (hl + 32 * k) * 8;
            if (c < C)
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const float d = v[k][i] - mu;
                    ss += d * d;
                }
        }
        const float rs = 1.f / sqrtf(half_sum(ss) / C + LN_EPS);
        if (row < N) {
#pragma unroll
            for (int k = 0; k < NCH; k++) {
                const int c = (hl + 32 * k) * 8;
                if (c < C) {
                    float wv[8], bv[8], o[8];
                    raw_to_f32<T>(wr[k], wv);
                    raw_to_f32<T>(br[k], bv);
#pragma unroll
                    for (int i = 0; i < 8; i++) o[i] = (v[k][i] - mu) * rs * wv[i] + bv[i];
                    store8(out + (int64_t)row * C + c, o);
                }
            }
            if (hl == 0) {
                mean[row] = mu;
                rstd[row] = rs;
            }
        }
    }
}

template <typename T, int NCH>
static void layernorm_fwd_launch(T* out, float* mean, float* rstd, const T* inp, const T* w,
                                 const T* b, int N, int C, hipStream_t st) {
    layernorm_fwd_kernel<T, NCH><<<ceil_div(N, LN_FWD_ROWS), 256, 0, st>>>(out, mean, rstd, inp,
                                                                          w, b, N, C);
}

// chunks per lane for C channels: 1, 2, 3, 4, 6 or 8
static int ln_nch(int C) {
    const int n = (C + 255) / 256;
    return n <= 4 ? n : n <= 6 ? 6 : 8;
}

template <typename T>
void layernorm_fwd(T* out, float* mean, float* rstd, const T* inp, const T* w, const T* b,
                   int N, int C, hipStream_t st) {
    switch (ln_nch(C)) {
        case 1: layernorm_fwd_launch<T, 1>(out, mean, rstd, inp, w, b, N, C, st); break;
        case 2: layernorm_fwd_launch<T, 2>(out, mean, rstd, inp, w, b, N, C, st); break;
        case 3: layernorm_fwd_launch<T, 3>(out, mean, rstd, inp, w, b, N, C, st); break;
        case 4: layernorm_fwd_launch<T, 4>(out, mean, rstd, inp, w, b, N, C, st); break;
        case 6: layernorm_fwd_launch<T, 6>(out, mean, rstd, inp, w, b, N, C, st); break;
        default: layernorm_fwd_launch<T, 8>(out, mean, rstd, inp, w, b, N, C, st); break;
    }
}

// Backward. With xhat = (x - mu) r and g = w dy:
//   dx = r (g - mean(g) - xhat mean(g xhat))
// A row belongs to one wave: lane l holds the NCH = ceil(C / 256) chunks of 4
// channels (l + 64k) * 4 .. +3 (three per lane at C = 768). Each wave takes
// LN_BWD_RPW rows per pass (wave q of block blk: rows 8 blk + 2q, +1, then
// every 8 * gridDim.x further), with every input, output-gradient and
// added-gradient load of both rows issued before the first reduction.
// dw = sum_rows dy xhat and db = sum_rows dy are reduced deterministically:
// each lane sums its channels over its rows in row order, the four waves are
// combined in wave order through LDS into one partial row per block, and a
// second kernel sums the partial rows in a fixed order.
#define LN_BWD_BLOCKS 512
#define LN_BWD_RPW 2
static_assert(4 * LN_BWD_RPW == LN_BWD_ROWS, "four waves of LN_BWD_RPW rows per pass");

template <typename T, int NCH>
__global__ __launch_bounds__(256) void layernorm_bwd_kernel(
    T* dinp, const T* dadd, const T* __restrict__ dout, const T* __restrict__ inp,
    const T* __restrict__ w, const float* __restrict__ mean, const float* __restrict__ rstd,
    int N, int C, float* __restrict__ partials) {
    typedef T Raw4 __attribute__((ext_vector_type(4)));
    __shared__ float red[2 * 2048];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    float dw[NCH][4], db[NCH][4];
    Raw4 wr[NCH];
#pragma unroll
    for (int k = 0; k < NCH; k++) {
        const int c = (lane + 64 * k) * 4;
#pragma unroll
        for (int i = 0; i < 4; i++) dw[k][i] = db[k][i] = 0.f;
        wr[k] = c < C ? *reinterpret_cast<const Raw4*>(w + c) : Raw4{};
    }
    for (int row0 = blockIdx.x * LN_BWD_ROWS + wid * LN_BWD_RPW; row0 < N;
         row0 += gridDim.x * LN_BWD_ROWS) {
        Raw4 xr[LN_BWD_RPW][NCH], dr[LN_BWD_RPW][NCH], ar[LN_BWD_RPW][NCH];
        float mu[LN_BWD_RPW], r[LN_BWD_RPW];
#pragma unroll
        for (int q = 0; q < LN_BWD_RPW; q++) {
            const int row = row0 + q;
            const bool live = row < N;
            mu[q] = live ? mean[row] : 0.f;
            r[q] = live ? rstd[row] : 0.f;
#pragma unroll
            for (int k = 0; k < NCH; k++) {
                const int c = (lane + 64 * k) * 4;
                const bool on = live && c < C;
                const int64_t o = (int64_t)row * C + c;
                xr[q][k] = on ? *reinterpret_cast<const Raw4*>(inp + o) : Raw4{};
                dr[q][k] = on ? *reinterpret_cast<const Raw4*>(dout + o) : Raw4{};
                ar[q][k] = on && dadd ? *reinterpret_cast<const Raw4*>(dadd + o) : Raw4{};
            }
        }
#pragma unroll
        for (int q = 0; q < LN_BWD_RPW; q++) {
            const int row = row0 + q;
            float gs = 0.f, gxs = 0.f;
#pragma unroll
            for (int k = 0; k < NCH; k++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float xh = (to_f32(xr[q][k][i]) - mu[q]) * r[q], dy = to_f32(dr[q][k][i]);
                    const float g = to_f32(wr[k][i]) * dy;
                    gs += g;
                    gxs += g * xh;
                    dw[k][i] += dy * xh;
                    db[k][i] += dy;
                }
            const float gm = wave_sum(gs) / C, gxm = wave_sum(gxs) / C;
            if (row < N) {
#pragma unroll
                for (int k = 0; k < NCH; k++) {
                    const int c = (lane + 64 * k) * 4;
                    if (c < C) {
                        Raw4 o;
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const float xh = (to_f32(xr[q][k][i]) - mu[q]) * r[q];
                            const float dx =
                                (to_f32(wr[k][i]) * to_f32(dr[q][k][i]) - gm - xh * gxm) * r[q];
                            o[i] = from_f32<T>(dadd ? to_f32(ar[q][k][i]) + dx : dx);
                        }
                        *reinterpret_cast<Raw4*>(dinp + (int64_t)row * C + c) = o;
                    }
                }
            }
        }
    }
    // combine the four waves in order: wave 0 stores, waves 1..3 add in turn
    for (int q = 0; q < 4; q++) {
        if (wid == q) {
#pragma unroll
            for (int k = 0; k < NCH; k++) {
                const int c = (lane + 64 * k) * 4;
                if (c < C)
#pragma unroll
                    for (int i = 0; i < 4; i++) {
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

static int ln_bwd_blocks(int N) {
    const int nb = ceil_div(N, LN_BWD_ROWS);
    return nb < LN_BWD_BLOCKS ? nb : LN_BWD_BLOCKS;
}

template <typename T, int NCH>
static void layernorm_bwd_launch(T* dinp, const T* dadd, const T* dout, const T* inp, const T* w,
                                 const float* mean, const float* rstd, int N, int C,
                                 float* partials, hipStream_t st) {
    layernorm_bwd_kernel<T, NCH><<<ln_bwd_blocks(N), 256, 0, st>>>(dinp, dadd, dout, inp, w, mean,
                                                                   rstd, N, C, partials);
}

template <typename T>
void layernorm_bwd_rows(T* dinp, const T* dadd, const T* dout, const T* inp, const T* w,
                        const float* mean, const float* rstd, int N, int C, float* partials,
                        int slot, hipStream_t st) {
    partials += (int64_t)slot * LN_BWD_BLOCKS * 2 * C;
    switch (ln_nch(C)) {
        case 1: layernorm_bwd_launch<T, 1>(dinp, dadd, dout, inp, w, mean, rstd, N, C, partials, st); break;
        case 2: layernorm_bwd_launch<T, 2>(dinp, dadd, dout, inp, w, mean, rstd, N, C, partials, st); break;
        case 3: layernorm_bwd_launch<T, 3>(dinp, dadd, dout, inp, w, mean, rstd, N, C, partials, st); break;
        case 4: layernorm_bwd_launch<T, 4>(dinp, dadd, dout, inp, w, mean, rstd, N, C, partials, st); break;
        case 6: layernorm_bwd_launch<T, 6>(dinp, dadd, dout, inp, w, mean, rstd, N, C, partials, st); break;
        default: layernorm_bwd_launch<T, 8>(dinp, dadd, dout, inp, w, mean, rstd, N, C, partials, st); break;
    }
}

void layernorm_bwd_reduce(const LnRedBatch& b, int N, int C, float* partials, int count,
                          hipStream_t st) {
    const int nb = ln_bwd_blocks(N);
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
