// Token + position embedding (forward gather, deterministic backward scatter).
#include "kernels.h"

// One thread per 8 channels of one position.
template <typename T>
__global__ __launch_bounds__(256) void encoder_fwd_kernel(T* __restrict__ out,
                                                          const int32_t* __restrict__ tok,
                                                          const T* __restrict__ wte,
                                                          const T* __restrict__ wpe, int BT,
                                                          int Tn, int C, int V, int* err) {
    const int c8n = C / 8;
    int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (idx >= (int64_t)BT * c8n) return;
    int bt = (int)(idx / c8n), c = (int)(idx % c8n) * 8;
    int t = bt % Tn;
    int id = tok[bt];
    float v[8];
    if (id < 0 || id >= V) {
        if (c == 0) atomicOr(err, 1);
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = 0.f;
    } else {
        float a[8], b[8];
        load8(wte + (int64_t)id * C + c, a);
        load8(wpe + (int64_t)t * C + c, b);
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = a[k] + b[k];
    }
    store8(out + (int64_t)bt * C + c, v);
}

template <typename T>
void encoder_fwd(T* out, const int32_t* tok, const T* wte, const T* wpe, int B, int Tn, int C,
                 int V, int* err, hipStream_t st) {
    int64_t n = (int64_t)B * Tn * (C / 8);
    encoder_fwd_kernel<T><<<ceil_div(n, 256), 256, 0, st>>>(out, tok, wte, wpe, B * Tn, Tn, C,
                                                            V, err);
}

// dwpe[t, c] = sum_b dout[b, t, c] in increasing b; rows t >= Tn are zeroed.
template <typename T>
__global__ __launch_bounds__(256) void encoder_bwd_wpe_kernel(float* __restrict__ dwpe,
                                                              const T* __restrict__ dout, int B,
                                                              int Tn, int C, int maxT) {
    int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (idx >= (int64_t)maxT * C) return;
    int t = (int)(idx / C), c = (int)(idx % C);
    float s = 0.f;
    if (t < Tn)
        for (int b = 0; b < B; b++) s += to_f32(dout[((int64_t)b * Tn + t) * C + c]);
    dwpe[idx] = s;
}

__global__ __launch_bounds__(256) void token_count_kernel(const int32_t* __restrict__ tok,
                                                          int n, int Vp, int* count) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        int id = tok[i];
        if (id >= 0 && id < Vp) atomicAdd(&count[id], 1);
    }
}

// Exclusive scan of count[0..Vp) into offset[0..Vp] by one 1024-thread block:
// each thread scans a contiguous slice, then slice totals are scanned in LDS.
__global__ __launch_bounds__(1024) void token_scan_kernel(const int* __restrict__ count, int Vp,
                                                          int* __restrict__ offset,
                                                          int* __restrict__ cursor) {
    __shared__ int tot[1024];
    const int tid = threadIdx.x;
    const int per = (Vp + 1023) / 1024;
    const int s0 = tid * per, s1 = min(Vp, s0 + per);
    int s = 0;
    for (int i = s0; i < s1; i++) s += count[i];
    tot[tid] = s;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < 1024; i++) {
            int c = tot[i];
            tot[i] = run;
            run += c;
        }
        offset[Vp] = run;
    }
    __syncthreads();
    int run = tot[tid];
    for (int i = s0; i < s1; i++) {
        offset[i] = run;
        cursor[i] = 0;
        run += count[i];
    }
}

// Buckets positions by token (the order inside a bucket is arbitrary here; the
// summation kernel below imposes increasing position order).
__global__ __launch_bounds__(256) void token_fill_kernel(const int32_t* __restrict__ tok, int n,
                                                         int Vp, const int* __restrict__ offset,
                                                         int* cursor, int* __restrict__ bucket) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        int id = tok[i];
        if (id >= 0 && id < Vp) bucket[offset[id] + atomicAdd(&cursor[id], 1)] = i;
    }
}

// One block per (token, 256-channel slice). Each thread owns one channel and
// sums the gradient rows of the token's positions in increasing position
// order, then adds the total to dwte; the order depends only on the
// positions, so the result is deterministic. Ordering: a bucket of at most 256
// positions is ranked by counting (positions are distinct); a larger one marks
// its positions in an LDS bitmap of BT bits that every thread walks upwards.
#define ENC_SMALL 256
template <typename T>
__global__ __launch_bounds__(256) void encoder_bwd_wte_kernel(float* __restrict__ dwte,
                                                              const T* __restrict__ dout,
                                                              const int* __restrict__ offset,
                                                              const int* __restrict__ bucket,
                                                              int C, int BT) {
    extern __shared__ unsigned int enc_lds[];
    const int v = blockIdx.x, tid = threadIdx.x;
    const int b0 = offset[v], n = offset[v + 1] - b0;
    if (n == 0) return;
    const int c = blockIdx.y * blockDim.x + tid;
    float s = 0.f;
    if (n <= ENC_SMALL) {
        int* raw = reinterpret_cast<int*>(enc_lds);
        int* pos = raw + ENC_SMALL;
        int mine = tid < n ? bucket[b0 + tid] : 0;
        if (tid < n) raw[tid] = mine;
        __syncthreads();
        if (tid < n) {
            int rank = 0;
            for (int j = 0; j < n; j++) rank += raw[j] < mine;
            pos[rank] = mine;
        }
        __syncthreads();
        if (c < C)
            for (int i = 0; i < n; i++) s += to_f32(dout[(int64_t)pos[i] * C + c]);
    } else {
        const int nw = (BT + 31) / 32;
        for (int i = tid; i < nw; i += blockDim.x) enc_lds[i] = 0u;
        __syncthreads();
        for (int i = tid; i < n; i += blockDim.x) {
            int p = bucket[b0 + i];
            atomicOr(&enc_lds[p >> 5], 1u << (p & 31));
        }
        __syncthreads();
        if (c < C)
            for (int w = 0; w < nw; w++) {
                unsigned int bits = enc_lds[w];
                while (bits) {
                    int p = w * 32 + __builtin_ctz(bits);
                    bits &= bits - 1;
                    s += to_f32(dout[(int64_t)p * C + c]);
                }
            }
    }
    if (c < C) dwte[(int64_t)v * C + c] += s;
}

template <typename T>
void encoder_bwd(float* dwte, float* dwpe, const T* dout, const int32_t* tok, int B, int Tn,
                 int C, int Vp, int maxT, int* ws_count, int* ws_cursor, int* ws_offset,
                 int* ws_bucket, hipStream_t st) {
    const int n = B * Tn;
    encoder_bwd_wpe_kernel<T><<<ceil_div((int64_t)maxT * C, 256), 256, 0, st>>>(dwpe, dout, B, Tn,
                                                                                C, maxT);
    fill_zero_i32(ws_count, Vp, st);
    token_count_kernel<<<ceil_div(n, 256), 256, 0, st>>>(tok, n, Vp, ws_count);
    token_scan_kernel<<<1, 1024, 0, st>>>(ws_count, Vp, ws_offset, ws_cursor);
    token_fill_kernel<<<ceil_div(n, 256), 256, 0, st>>>(tok, n, Vp, ws_offset, ws_cursor,
                                                        ws_bucket);
    dim3 grid(Vp, ceil_div(C, 256));
    size_t lds = (size_t)((n + 31) / 32) * 4;
    if (lds < 2 * ENC_SMALL * sizeof(int)) lds = 2 * ENC_SMALL * sizeof(int);
    encoder_bwd_wte_kernel<T><<<grid, 256, lds, st>>>(dwte, dout, ws_offset, ws_bucket, C, n);
}

template void encoder_fwd<float>(float*, const int32_t*, const float*, const float*, int, int,
                                 int, int, int*, hipStream_t);
template void encoder_fwd<bf16>(bf16*, const int32_t*, const bf16*, const bf16*, int, int, int,
                                int, int*, hipStream_t);
template void encoder_bwd<float>(float*, float*, const float*, const int32_t*, int, int, int, int,
                                 int, int*, int*, int*, int*, hipStream_t);
template void encoder_bwd<bf16>(float*, float*, const bf16*, const int32_t*, int, int, int, int,
                                int, int*, int*, int*, int*, hipStream_t);
