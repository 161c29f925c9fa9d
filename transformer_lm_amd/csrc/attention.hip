// Causal multi-head self-attention on the fused qkv activations (B, T, 3C):
// per (b, h, t), s = q_t . k_t' / sqrt(hs) for t' <= t, P = softmax(s),
// y_t = sum P v_t'; the row's log-sum-exp is kept so the backward pass can
// rebuild P without storing it.
//
// This file holds the wave-per-row kernels that serve any head size that is a
// multiple of 8 up to 128, in both storage types. Softmax is computed online
// over chunks of 64 keys (one key per lane): the running maximum and sum are
// rescaled chunk by chunk, so the T x T matrix never exists in memory.
#include <type_traits>

#include "kernels.h"

#define AT_ROWS 4  // rows (waves) per block

template <typename T>
__device__ __forceinline__ float dot_row(const float* __restrict__ a_lds, const T* __restrict__ b,
                                         int hs) {
    float s = 0.f;
    for (int d = 0; d < hs; d += 8) {
        float v[8];
        load8(b + d, v);
#pragma unroll
        for (int i = 0; i < 8; i++) s += a_lds[d + i] * v[i];
    }
    return s;
}

template <typename T>
__global__ __launch_bounds__(256) void attention_fwd_rows_kernel(T* __restrict__ out,
                                                                 float* __restrict__ lse,
                                                                 const T* __restrict__ qkv,
                                                                 int Tn, int C, int NH) {
    __shared__ float qs[AT_ROWS][128];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int t = blockIdx.x * AT_ROWS + wid;
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int hs = C / NH, C3 = 3 * C;
    const float scale = 1.f / sqrtf((float)hs);
    if (t < Tn)
        for (int d = lane; d < hs; d += 64)
            qs[wid][d] = to_f32(qkv[((int64_t)b * Tn + t) * C3 + h * hs + d]);
    __syncthreads();
    if (t >= Tn) return;
    const T* kbase = qkv + (int64_t)b * Tn * C3 + C + h * hs;
    const T* vbase = kbase + C;
    float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
    for (int k0 = 0; k0 <= t; k0 += 64) {
        const int key = k0 + lane;
        float s = -INFINITY;
        if (key <= t) s = dot_row(qs[wid], kbase + (int64_t)key * C3, hs) * scale;
        const float mn = fmaxf(m, wave_max(s));
        const float p = key <= t ? expf(s - mn) : 0.f;
        const float corr = expf(m - mn);
        l = l * corr + wave_sum(p);
        acc0 *= corr;
        acc1 *= corr;
        const int nk = min(64, t - k0 + 1);
        for (int j = 0; j < nk; j++) {
            const float pj = __shfl(p, j, 64);
            const T* vr = vbase + (int64_t)(k0 + j) * C3;
            if (lane < hs) acc0 += pj * to_f32(vr[lane]);
            if (lane + 64 < hs) acc1 += pj * to_f32(vr[lane + 64]);
        }
        m = mn;
    }
    T* y = out + ((int64_t)b * Tn + t) * C + h * hs;
    if (lane < hs) y[lane] = from_f32<T>(acc0 / l);
    if (lane + 64 < hs) y[lane + 64] = from_f32<T>(acc1 / l);
    if (lane == 0) lse[(int64_t)bh * Tn + t] = m + logf(l);
}

// D_t = sum_d dy_t[d] y_t[d] = sum_t' P[t'] (dy_t . v_t'), the softmax-backward
// correction term of row t.
template <typename T>
__global__ __launch_bounds__(256) void attention_bwd_d_kernel(float* __restrict__ Dbuf,
                                                              const T* __restrict__ dout,
                                                              const T* __restrict__ out, int Tn,
                                                              int C, int NH) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int t = blockIdx.x * AT_ROWS + wid;
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int hs = C / NH;
    if (t >= Tn) return;
    const int64_t o = ((int64_t)b * Tn + t) * C + h * hs;
    float s = 0.f;
    for (int d = lane; d < hs; d += 64) s += to_f32(dout[o + d]) * to_f32(out[o + d]);
    s = wave_sum(s);
    if (lane == 0) Dbuf[(int64_t)bh * Tn + t] = s;
}

// dq_t = sum_t'<=t dS[t, t'] k_t' / sqrt(hs), with P rebuilt from the saved
// log-sum-exp and dS = P (dy_t . v_t' - D_t).
template <typename T>
__global__ __launch_bounds__(256) void attention_bwd_dq_kernel(
    T* __restrict__ dqkv, const T* __restrict__ dout, const T* __restrict__ qkv,
    const float* __restrict__ lse, const float* __restrict__ Dbuf, int Tn, int C, int NH) {
    __shared__ float qs[AT_ROWS][128];
    __shared__ float dys[AT_ROWS][128];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int t = blockIdx.x * AT_ROWS + wid;
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int hs = C / NH, C3 = 3 * C;
    const float scale = 1.f / sqrtf((float)hs);
    if (t < Tn)
        for (int d = lane; d < hs; d += 64) {
            qs[wid][d] = to_f32(qkv[((int64_t)b * Tn + t) * C3 + h * hs + d]);
            dys[wid][d] = to_f32(dout[((int64_t)b * Tn + t) * C + h * hs + d]);
        }
    __syncthreads();
    if (t >= Tn) return;
    const float lt = lse[(int64_t)bh * Tn + t], Dt = Dbuf[(int64_t)bh * Tn + t];
    const T* kbase = qkv + (int64_t)b * Tn * C3 + C + h * hs;
    const T* vbase = kbase + C;
    float dq0 = 0.f, dq1 = 0.f;
    for (int k0 = 0; k0 <= t; k0 += 64) {
        const int key = k0 + lane;
        float ds = 0.f;
        if (key <= t) {
            const float p = expf(dot_row(qs[wid], kbase + (int64_t)key * C3, hs) * scale - lt);
            const float dp = dot_row(dys[wid], vbase + (int64_t)key * C3, hs);
            ds = p * (dp - Dt);
        }
        const int nk = min(64, t - k0 + 1);
        for (int j = 0; j < nk; j++) {
            const float dsj = __shfl(ds, j, 64);
            const T* kr = kbase + (int64_t)(k0 + j) * C3;
            if (lane < hs) dq0 += dsj * to_f32(kr[lane]);
            if (lane + 64 < hs) dq1 += dsj * to_f32(kr[lane + 64]);
        }
    }
    T* dq = dqkv + ((int64_t)b * Tn + t) * C3 + h * hs;
    if (lane < hs) dq[lane] = from_f32<T>(dq0 * scale);
    if (lane + 64 < hs) dq[lane + 64] = from_f32<T>(dq1 * scale);
}

// For key row t': dv = sum_t>=t' P[t, t'] dy_t; dk = sum_t>=t' dS[t, t'] q_t / sqrt(hs).
template <typename T>
__global__ __launch_bounds__(256) void attention_bwd_dkv_kernel(
    T* __restrict__ dqkv, const T* __restrict__ dout, const T* __restrict__ qkv,
    const float* __restrict__ lse, const float* __restrict__ Dbuf, int Tn, int C, int NH) {
    __shared__ float ks[AT_ROWS][128];
    __shared__ float vs[AT_ROWS][128];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int tk = blockIdx.x * AT_ROWS + wid;
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int hs = C / NH, C3 = 3 * C;
    const float scale = 1.f / sqrtf((float)hs);
    if (tk < Tn)
        for (int d = lane; d < hs; d += 64) {
            ks[wid][d] = to_f32(qkv[((int64_t)b * Tn + tk) * C3 + C + h * hs + d]);
            vs[wid][d] = to_f32(qkv[((int64_t)b * Tn + tk) * C3 + 2 * C + h * hs + d]);
        }
    __syncthreads();
    if (tk >= Tn) return;
    const T* qbase = qkv + (int64_t)b * Tn * C3 + h * hs;
    const T* dybase = dout + (int64_t)b * Tn * C + h * hs;
    const float* lrow = lse + (int64_t)bh * Tn;
    const float* Drow = Dbuf + (int64_t)bh * Tn;
    float dk0 = 0.f, dk1 = 0.f, dv0 = 0.f, dv1 = 0.f;
    for (int q0 = tk; q0 < Tn; q0 += 64) {
        const int qi = q0 + lane;
        float p = 0.f, ds = 0.f;
        if (qi < Tn) {
            p = expf(dot_row(ks[wid], qbase + (int64_t)qi * C3, hs) * scale - lrow[qi]);
            const float dp = dot_row(vs[wid], dybase + (int64_t)qi * C, hs);
            ds = p * (dp - Drow[qi]);
        }
        const int nq = min(64, Tn - q0);
        for (int j = 0; j < nq; j++) {
            const float pj = __shfl(p, j, 64), dsj = __shfl(ds, j, 64);
            const T* qr = qbase + (int64_t)(q0 + j) * C3;
            const T* dyr = dybase + (int64_t)(q0 + j) * C;
            if (lane < hs) {
                dv0 += pj * to_f32(dyr[lane]);
                dk0 += dsj * to_f32(qr[lane]);
            }
            if (lane + 64 < hs) {
                dv1 += pj * to_f32(dyr[lane + 64]);
                dk1 += dsj * to_f32(qr[lane + 64]);
            }
        }
    }
    T* dk = dqkv + ((int64_t)b * Tn + tk) * C3 + C + h * hs;
    T* dv = dk + C;
    if (lane < hs) {
        dk[lane] = from_f32<T>(dk0 * scale);
        dv[lane] = from_f32<T>(dv0);
    }
    if (lane + 64 < hs) {
        dk[lane + 64] = from_f32<T>(dk1 * scale);
        dv[lane + 64] = from_f32<T>(dv1);
    }
}

// bf16 with head size 64 runs on the matrix cores (attention_mfma.hip); other
// head sizes and fp32 use the wave-per-row kernels above.
template <typename T>
void attention_fwd(T* out, float* lse, const T* qkv, int B, int Tn, int C, int NH,
                   hipStream_t st) {
    if constexpr (std::is_same<T, bf16>::value) {
        if (C / NH == 64 && flash_attention_fits(Tn, C)) {
            flash_attention_fwd(out, lse, qkv, B, Tn, C, NH, st);
            return;
        }
    }
    dim3 grid(ceil_div(Tn, AT_ROWS), B * NH);
    attention_fwd_rows_kernel<T><<<grid, 256, 0, st>>>(out, lse, qkv, Tn, C, NH);
}

template <typename T>
void attention_bwd(T* dqkv, const T* dout, const T* qkv, const T* out, const float* lse,
                   float* work, int B, int Tn, int C, int NH, hipStream_t st) {
    if constexpr (std::is_same<T, bf16>::value) {
        if (C / NH == 64 && flash_attention_fits(Tn, C)) {
            flash_attention_bwd(dqkv, dout, qkv, out, lse, work, B, Tn, C, NH, st);
            return;
        }
    }
    dim3 grid(ceil_div(Tn, AT_ROWS), B * NH);
    attention_bwd_d_kernel<T><<<grid, 256, 0, st>>>(work, dout, out, Tn, C, NH);
    attention_bwd_dq_kernel<T><<<grid, 256, 0, st>>>(dqkv, dout, qkv, lse, work, Tn, C, NH);
    attention_bwd_dkv_kernel<T><<<grid, 256, 0, st>>>(dqkv, dout, qkv, lse, work, Tn, C, NH);
}

template void attention_fwd<float>(float*, float*, const float*, int, int, int, int, hipStream_t);
template void attention_fwd<bf16>(bf16*, float*, const bf16*, int, int, int, int, hipStream_t);
template void attention_bwd<float>(float*, const float*, const float*, const float*,
                                   const float*, float*, int, int, int, int, hipStream_t);
template void attention_bwd<bf16>(bf16*, const bf16*, const bf16*, const bf16*, const float*,
                                  float*, int, int, int, int, hipStream_t);
