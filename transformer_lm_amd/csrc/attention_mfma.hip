// Causal attention for head size 64 in bf16 on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16), the fused online-softmax attention of page
// "llm.c: Large Language Model Training in Pure C/CUDA Without Dependencies"
// (section "Fused Attention Kernel"): scores never go to HBM; K and V tiles of
// 64 keys are staged in LDS; the backward pass rebuilds P from the saved
// log-sum-exp.
//
// Layout choices. A 32x32 MFMA accumulator gives lane l the column l%32 and
// rows 8*(v/4) + 4*(l/32) + v%4 (register v). Score tiles are computed with
// queries as columns where a kernel needs per-query statistics in one lane
// (S^T = K Q^T), and with keys as columns where it needs per-key sums (S = Q K^T).
// The MFMA reduction order inside a 16-wide k block is free as long as both
// operands use the same one, so probabilities / score gradients feed the next
// product straight from the accumulator registers: register v (0..7 of a
// half-tile) of lane group g stands for reduction index 4g + v%4 + 8*(v/4), and
// the other operand is read from a transposed LDS tile in the same order
// (two 8-byte reads).
//
// Softmax runs in base 2: x = s * log2(e) / sqrt(hs), p = exp2(x - m).
#include "kernels.h"

typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

#define HS 64
#define LDR 72          // LDS row pitch in bf16 (64 + 8 padding)
#define Q_PER_BLOCK 128 // 4 waves x 32 rows
#define KV_TILE 64
#define LOG2E 1.4426950408889634f
#define LN2 0.6931471805599453f

__device__ __forceinline__ floatx16 mfma(bf16x8 a, bf16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld16(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Two 4-element runs (reduction indices base..base+3 and base+8..base+11) of an
// LDS row, as one MFMA fragment in the accumulator-register order.
__device__ __forceinline__ bf16x8 ld_runs(const bf16* row, int base) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + base);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + base + 8);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Registers 8*hh .. 8*hh+7 of an accumulator, rounded to bf16.
__device__ __forceinline__ bf16x8 half_tile(const floatx16& a, int hh) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; i++) r[i] = (bf16)a[8 * hh + i];
    return r;
}

// Stages rows [r0, r0 + 64) of a 64-wide head slice (row stride ld) into LDS,
// row-major (rows x 64, pitch LDR) and/or transposed (64 x rows, pitch LDR).
// Rows >= nrows read as zero. 256 threads, two 8-element chunks each.
template <bool ROWMAJOR, bool TRANSPOSED>
__device__ __forceinline__ void stage64(bf16* __restrict__ rm, bf16* __restrict__ tr,
                                        const bf16* __restrict__ g, int64_t ld, int r0,
                                        int nrows, int tid) {
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int c = tid + q * 256;
        const int r = c >> 3, d = (c & 7) * 8;
        bf16x8 v = {};
        if (r0 + r < nrows) v = ld16(g + (int64_t)(r0 + r) * ld + d);
        if (ROWMAJOR) *reinterpret_cast<bf16x8*>(rm + r * LDR + d) = v;
        if (TRANSPOSED)
#pragma unroll
            for (int e = 0; e < 8; e++) tr[(d + e) * LDR + r] = v[e];
    }
}

// ---------------------------------------------------------------- forward --
// Block: 128 queries of one (b, h); wave w owns queries q0 .. q0+31, lane l the
// query q0 + l%32. Per 64-key tile: S^T (keys x queries) = K Q^T, online
// softmax per query, O^T (dims x queries) += V^T P^T.
__global__ __launch_bounds__(256) void flash_fwd_kernel(bf16* __restrict__ out,
                                                        float* __restrict__ lse,
                                                        const bf16* __restrict__ qkv, int Tn,
                                                        int C, int NH) {
    __shared__ bf16 Ks[KV_TILE * LDR];
    __shared__ bf16 Vt[HS * LDR];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5;
    const int qt = gridDim.x - 1 - blockIdx.x;  // longest rows first
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int C3 = 3 * C;
    const bf16* base = qkv + (int64_t)b * Tn * C3 + h * HS;
    const int q0 = qt * Q_PER_BLOCK + wid * 32;
    const int ql = q0 + (lane & 31);
    const float sc = LOG2E / 8.0f;  // log2(e) / sqrt(64)

    bf16x8 qf[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
        qf[kb] = ql < Tn ? ld16(base + (int64_t)ql * C3 + kb * 16 + 8 * g) : bf16x8{};
    floatx16 o[2] = {floatx16{}, floatx16{}};
    float m = -INFINITY, l = 0.f;

    const int kv_end = min(Tn, (qt + 1) * Q_PER_BLOCK);
    for (int k0 = 0; k0 < kv_end; k0 += KV_TILE) {
        __syncthreads();
        stage64<true, false>(Ks, nullptr, base + C, C3, k0, Tn, tid);
        stage64<false, true>(nullptr, Vt, base + 2 * C, C3, k0, Tn, tid);
        __syncthreads();
        if (k0 > q0 + 31 || q0 >= Tn) continue;  // every key of the tile is masked
        floatx16 s[2] = {floatx16{}, floatx16{}};
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int kb = 0; kb < 4; kb++)
                s[kt] = mfma(ld16(Ks + (32 * kt + (lane & 31)) * LDR + kb * 16 + 8 * g), qf[kb], s[kt]);
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int key = k0 + 32 * kt + 8 * (v >> 2) + 4 * g + (v & 3);
                const float x = (key <= ql && key < Tn) ? s[kt][v] * sc : -INFINITY;
                s[kt][v] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m, mx);
        const float corr = exp2f(m - mn);
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const float p = exp2f(s[kt][v] - mn);
                s[kt][v] = p;
                ps += p;
            }
        ps += __shfl_xor(ps, 32, 64);
        l = l * corr + ps;
        m = mn;
        o[0] *= corr;
        o[1] *= corr;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                const bf16x8 pb = half_tile(s[kt], hh);
                const int kk = 32 * kt + 16 * hh + 4 * g;
#pragma unroll
                for (int dt = 0; dt < 2; dt++)
                    o[dt] = mfma(ld_runs(Vt + (32 * dt + (lane & 31)) * LDR, kk), pb, o[dt]);
            }
    }
    if (ql < Tn) {
        const float inv = 1.f / l;
        bf16* orow = out + ((int64_t)b * Tn + ql) * C + h * HS;
#pragma unroll
        for (int dt = 0; dt < 2; dt++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int d = 32 * dt + 8 * r + 4 * g;
                *reinterpret_cast<bf16x4*>(orow + d) =
                    bf16x4{(bf16)(o[dt][4 * r] * inv), (bf16)(o[dt][4 * r + 1] * inv),
                           (bf16)(o[dt][4 * r + 2] * inv), (bf16)(o[dt][4 * r + 3] * inv)};
            }
        if (g == 0) lse[(int64_t)bh * Tn + ql] = (m + log2f(l)) * LN2;
    }
}

// ------------------------------------------------------------ backward dK dV --
// Block: 128 keys of one (b, h); wave w owns keys kw .. kw+31, lane l the key
// kw + l%32. Per 64-query tile (queries >= the block's first key):
// S = Q K^T and dP = dO V^T (queries x keys), P = exp2(S*c - lse2),
// dS = P (dP - D); dV^T += dO^T P; dK^T += Q^T dS.
__global__ __launch_bounds__(256) void flash_bwd_dkv_kernel(
    bf16* __restrict__ dqkv, const bf16* __restrict__ dout, const bf16* __restrict__ qkv,
    const float* __restrict__ lse, const float* __restrict__ Dbuf, int Tn, int C, int NH) {
    __shared__ bf16 Qs[KV_TILE * LDR], Qt[HS * LDR], dOs[KV_TILE * LDR], dOt[HS * LDR];
    __shared__ __attribute__((aligned(16))) float ls[KV_TILE];
    __shared__ __attribute__((aligned(16))) float Ds[KV_TILE];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5;
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int C3 = 3 * C;
    const bf16* base = qkv + (int64_t)b * Tn * C3 + h * HS;
    const bf16* dbase = dout + (int64_t)b * Tn * C + h * HS;
    const int kb0 = blockIdx.x * Q_PER_BLOCK;
    const int kw = kb0 + wid * 32;
    const int kl = kw + (lane & 31);
    const float sc = LOG2E / 8.0f;

    bf16x8 kf[4], vf[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
        kf[kb] = kl < Tn ? ld16(base + (int64_t)kl * C3 + C + kb * 16 + 8 * g) : bf16x8{};
        vf[kb] = kl < Tn ? ld16(base + (int64_t)kl * C3 + 2 * C + kb * 16 + 8 * g) : bf16x8{};
    }
    floatx16 dk[2] = {floatx16{}, floatx16{}}, dv[2] = {floatx16{}, floatx16{}};

    for (int q0 = kb0 & ~(KV_TILE - 1); q0 < Tn; q0 += KV_TILE) {
        __syncthreads();
        stage64<true, true>(Qs, Qt, base, C3, q0, Tn, tid);
        stage64<true, true>(dOs, dOt, dbase, C, q0, Tn, tid);
        if (tid < KV_TILE) {
            const int q = q0 + tid;
            ls[tid] = q < Tn ? lse[(int64_t)bh * Tn + q] * LOG2E : 0.f;
            Ds[tid] = q < Tn ? Dbuf[(int64_t)bh * Tn + q] : 0.f;
        }
        __syncthreads();
        if (kw > q0 + KV_TILE - 1 || kw >= Tn) continue;  // no query of the tile sees these keys
        floatx16 s[2] = {floatx16{}, floatx16{}}, dp[2] = {floatx16{}, floatx16{}};
#pragma unroll
        for (int qt = 0; qt < 2; qt++)
#pragma unroll
            for (int kb = 0; kb < 4; kb++) {
                const int ro = (32 * qt + (lane & 31)) * LDR + kb * 16 + 8 * g;
                s[qt] = mfma(ld16(Qs + ro), kf[kb], s[qt]);
                dp[qt] = mfma(ld16(dOs + ro), vf[kb], dp[qt]);
            }
#pragma unroll
        for (int qt = 0; qt < 2; qt++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int qo = 32 * qt + 8 * r + 4 * g;  // 4 consecutive queries
                const floatx4 l4 = *reinterpret_cast<const floatx4*>(ls + qo);
                const floatx4 d4 = *reinterpret_cast<const floatx4*>(Ds + qo);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int q = q0 + qo + e, v = 4 * r + e;
                    const float p = (kl <= q && q < Tn) ? exp2f(s[qt][v] * sc - l4[e]) : 0.f;
                    s[qt][v] = p;
                    dp[qt][v] = p * (dp[qt][v] - d4[e]);
                }
            }
#pragma unroll
        for (int qt = 0; qt < 2; qt++)
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                const bf16x8 pb = half_tile(s[qt], hh);
                const bf16x8 db = half_tile(dp[qt], hh);
                const int qq = 32 * qt + 16 * hh + 4 * g;
#pragma unroll
                for (int dt = 0; dt < 2; dt++) {
                    const int ro = (32 * dt + (lane & 31)) * LDR;
                    dv[dt] = mfma(ld_runs(dOt + ro, qq), pb, dv[dt]);
                    dk[dt] = mfma(ld_runs(Qt + ro, qq), db, dk[dt]);
                }
            }
    }
    if (kl < Tn) {
        bf16* krow = dqkv + ((int64_t)b * Tn + kl) * C3 + C + h * HS;
        bf16* vrow = krow + C;
#pragma unroll
        for (int dt = 0; dt < 2; dt++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int d = 32 * dt + 8 * r + 4 * g;
                *reinterpret_cast<bf16x4*>(krow + d) =
                    bf16x4{(bf16)(dk[dt][4 * r] * 0.125f), (bf16)(dk[dt][4 * r + 1] * 0.125f),
                           (bf16)(dk[dt][4 * r + 2] * 0.125f), (bf16)(dk[dt][4 * r + 3] * 0.125f)};
                *reinterpret_cast<bf16x4*>(vrow + d) =
                    bf16x4{(bf16)dv[dt][4 * r], (bf16)dv[dt][4 * r + 1], (bf16)dv[dt][4 * r + 2],
                           (bf16)dv[dt][4 * r + 3]};
            }
    }
}

// --------------------------------------------------------------- backward dQ --
// Block: 128 queries; wave w owns queries q0 .. q0+31, lane l the query
// q0 + l%32. Per 64-key tile: S^T = K Q^T, dP^T = V dO^T (keys x queries),
// dS^T = P^T (dP^T - D); dQ^T += K^T dS^T.
__global__ __launch_bounds__(256) void flash_bwd_dq_kernel(
    bf16* __restrict__ dqkv, const bf16* __restrict__ dout, const bf16* __restrict__ qkv,
    const float* __restrict__ lse, const float* __restrict__ Dbuf, int Tn, int C, int NH) {
    __shared__ bf16 Ks[KV_TILE * LDR], Kt[HS * LDR], Vs[KV_TILE * LDR];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5;
    const int qt = gridDim.x - 1 - blockIdx.x;
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int C3 = 3 * C;
    const bf16* base = qkv + (int64_t)b * Tn * C3 + h * HS;
    const int q0 = qt * Q_PER_BLOCK + wid * 32;
    const int ql = q0 + (lane & 31);
    const float sc = LOG2E / 8.0f;

    bf16x8 qf[4], df[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
        qf[kb] = ql < Tn ? ld16(base + (int64_t)ql * C3 + kb * 16 + 8 * g) : bf16x8{};
        df[kb] = ql < Tn ? ld16(dout + ((int64_t)b * Tn + ql) * C + h * HS + kb * 16 + 8 * g)
                         : bf16x8{};
    }
    const float l2 = ql < Tn ? lse[(int64_t)bh * Tn + ql] * LOG2E : 0.f;
    const float Dq = ql < Tn ? Dbuf[(int64_t)bh * Tn + ql] : 0.f;
    floatx16 dq[2] = {floatx16{}, floatx16{}};

    const int kv_end = min(Tn, (qt + 1) * Q_PER_BLOCK);
    for (int k0 = 0; k0 < kv_end; k0 += KV_TILE) {
        __syncthreads();
        stage64<true, true>(Ks, Kt, base + C, C3, k0, Tn, tid);
        stage64<true, false>(Vs, nullptr, base + 2 * C, C3, k0, Tn, tid);
        __syncthreads();
        if (k0 > q0 + 31 || q0 >= Tn) continue;
        floatx16 s[2] = {floatx16{}, floatx16{}}, dp[2] = {floatx16{}, floatx16{}};
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int kb = 0; kb < 4; kb++) {
                const int ro = (32 * kt + (lane & 31)) * LDR + kb * 16 + 8 * g;
                s[kt] = mfma(ld16(Ks + ro), qf[kb], s[kt]);
                dp[kt] = mfma(ld16(Vs + ro), df[kb], dp[kt]);
            }
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int key = k0 + 32 * kt + 8 * (v >> 2) + 4 * g + (v & 3);
                const float p = (key <= ql && ql < Tn) ? exp2f(s[kt][v] * sc - l2) : 0.f;
                dp[kt][v] = p * (dp[kt][v] - Dq);
            }
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                const bf16x8 db = half_tile(dp[kt], hh);
                const int kk = 32 * kt + 16 * hh + 4 * g;
#pragma unroll
                for (int dt = 0; dt < 2; dt++)
                    dq[dt] = mfma(ld_runs(Kt + (32 * dt + (lane & 31)) * LDR, kk), db, dq[dt]);
            }
    }
    if (ql < Tn) {
        bf16* qrow = dqkv + ((int64_t)b * Tn + ql) * C3 + h * HS;
#pragma unroll
        for (int dt = 0; dt < 2; dt++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int d = 32 * dt + 8 * r + 4 * g;
                *reinterpret_cast<bf16x4*>(qrow + d) =
                    bf16x4{(bf16)(dq[dt][4 * r] * 0.125f), (bf16)(dq[dt][4 * r + 1] * 0.125f),
                           (bf16)(dq[dt][4 * r + 2] * 0.125f), (bf16)(dq[dt][4 * r + 3] * 0.125f)};
            }
    }
}

void flash_attention_fwd(bf16* out, float* lse, const bf16* qkv, int B, int Tn, int C, int NH,
                         hipStream_t st) {
    dim3 grid(ceil_div(Tn, Q_PER_BLOCK), B * NH);
    flash_fwd_kernel<<<grid, 256, 0, st>>>(out, lse, qkv, Tn, C, NH);
}

// Dbuf must already hold D = rowsum(dout * out) per (b, h, t).
void flash_attention_bwd(bf16* dqkv, const bf16* dout, const bf16* qkv, const float* lse,
                         const float* Dbuf, int B, int Tn, int C, int NH, hipStream_t st) {
    dim3 grid(ceil_div(Tn, Q_PER_BLOCK), B * NH);
    flash_bwd_dkv_kernel<<<grid, 256, 0, st>>>(dqkv, dout, qkv, lse, Dbuf, Tn, C, NH);
    flash_bwd_dq_kernel<<<grid, 256, 0, st>>>(dqkv, dout, qkv, lse, Dbuf, Tn, C, NH);
}
