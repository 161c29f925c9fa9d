// Fused classifier: softmax over the real vocabulary, cross-entropy loss and
// dLoss/dlogits in one kernel per row, written over the logits in place
// (the fused cross-entropy of page "llm.c: Large Language Model Training in
// Pure C/CUDA Without Dependencies"). Padded columns v >= V take no part in
// the softmax and get a zero gradient.
#include "kernels.h"

#define CL_THREADS 1024

// One block per row: pass 1 keeps a per-thread running (max, sum of exp)
// over 8-column chunks, merged across the block; pass 2 writes
// dz = (exp(z - lse) - [v == target]) * dloss. Used for vocabularies too wide
// for the register-resident kernel below (more than 7 * 8192 columns).
template <typename T>
__global__ __launch_bounds__(CL_THREADS) void classifier_kernel(T* logits,
                                                                float* __restrict__ losses,
                                                                const int32_t* __restrict__ targets,
                                                                int V, int Vp, float dloss,
                                                                int* err, int tag) {
    __shared__ float red[16];
    const int64_t row = blockIdx.x;
    T* z = logits + row * Vp;
    const int tgt = targets[row];
    const bool ok = tgt >= 0 && tgt < V;
    float m = -INFINITY, s = 0.f;
    for (int c = threadIdx.x * 8; c < V; c += CL_THREADS * 8) {
        float v[8];
        load8(z + c, v);
        float cm = m;
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (c + i < V) cm = fmaxf(cm, v[i]);
        s *= expf(m - cm);
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (c + i < V) s += expf(v[i] - cm);
        m = cm;
    }
    const float M = block_max(m, red);
    const float S = block_sum(m == -INFINITY ? 0.f : s * expf(m - M), red);
    const float lse = M + logf(S);
    if (threadIdx.x == 0) {
        if (ok) {
            losses[row] = lse - to_f32(z[tgt]);
        } else {
            losses[row] = 0.f;
            atomicMax(err, tag);
        }
    }
    __syncthreads();  // the target logit is read before any thread overwrites it
    for (int c = threadIdx.x * 8; c < Vp; c += CL_THREADS * 8) {
        float v[8];
        load8(z + c, v);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int col = c + i;
            float d = 0.f;
            if (col < V) d = (expf(v[i] - lse) - (col == tgt ? 1.f : 0.f)) * dloss;
            v[i] = d;
        }
        store8(z + c, v);
    }
}

// Single HBM pass, one 1024-thread block per row (a 50304-column row is 7
// chunks per thread, 56 registers: two rows per CU at 8 waves per SIMD): each
// thread keeps its NCHK chunks of 8 logits in registers
// (the row is read once), runs the online (max, sum of exp) over them, and
// after the block-wide merge writes the gradients from the same registers.
// exp(x) is evaluated as 2^(x log2 e) on the hardware exponential.
#define CL_LOG2E 1.4426950408889634f

// Storage-typed chunk of 8 logits (bf16 rows stay packed in registers).
template <typename T>
struct Chunk8 {
    T x[8];
    __device__ __forceinline__ float operator[](int i) const { return to_f32(x[i]); }
    // Makes the chunk opaque to the compiler, so values converted to fp32 in
    // the first pass are not kept alive until the second (which would double
    // the registers of a bf16 row and halve the blocks per CU).
    __device__ __forceinline__ void launder() {
        typedef unsigned int u32v __attribute__((ext_vector_type(sizeof(T) * 2)));
        u32v r = *reinterpret_cast<u32v*>(x);
        asm volatile("" : "+v"(r));
        *reinterpret_cast<u32v*>(x) = r;
    }
};

// The row is read once and overwritten once: non-temporal accesses keep it
// from displacing other data in the caches.
template <typename T>
__device__ __forceinline__ Chunk8<T> load_chunk_nt(const T* p) {
    typedef unsigned int u32v __attribute__((ext_vector_type(sizeof(T) * 2)));
    Chunk8<T> c;
    *reinterpret_cast<u32v*>(c.x) = __builtin_nontemporal_load(reinterpret_cast<const u32v*>(p));
    return c;
}
template <typename T>
__device__ __forceinline__ void store8_nt(T* p, const float (&v)[8]) {
    typedef unsigned int u32v __attribute__((ext_vector_type(sizeof(T) * 2)));
    typename Vec8<T>::raw r;
#pragma unroll
    for (int i = 0; i < 8; i++) r[i] = from_f32<T>(v[i]);
    __builtin_nontemporal_store(__builtin_bit_cast(u32v, r), reinterpret_cast<u32v*>(p));
}

// Chunks wholly inside the V real columns (all but at most one per row) take
// a path without per-column tests; the chunk holding the target also yields
// the target's logit from registers, and its lane writes the row's loss.
template <typename T, int NCHK>
__global__ __launch_bounds__(CL_THREADS) void classifier_reg_kernel(
    T* logits, float* __restrict__ losses, const int32_t* __restrict__ targets, int V, int Vp,
    float dloss, int* err, int tag) {
    __shared__ float red[16];
    const int64_t row = blockIdx.x;
    T* z = logits + row * Vp;
    const int tgt = targets[row];
    const bool ok = tgt >= 0 && tgt < V;
    Chunk8<T> v[NCHK];
#pragma unroll
    for (int k = 0; k < NCHK; k++) {
        const int c = (threadIdx.x + k * CL_THREADS) * 8;
        if (c < Vp) v[k] = load_chunk_nt(z + c);
    }
    float m = -INFINITY, s = 0.f, zt = 0.f;
#pragma unroll
    for (int k = 0; k < NCHK; k++) {
        const int c = (threadIdx.x + k * CL_THREADS) * 8;
        if (c + 8 <= V) {
            float cm = fmaxf(fmaxf(fmaxf(v[k][0], v[k][1]), fmaxf(v[k][2], v[k][3])),
                             fmaxf(fmaxf(v[k][4], v[k][5]), fmaxf(v[k][6], v[k][7])));
            cm = fmaxf(cm, m);
            const float cl = cm * CL_LOG2E;
            float cs = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) cs += __builtin_amdgcn_exp2f(fmaf(v[k][i], CL_LOG2E, -cl));
            s = s * __builtin_amdgcn_exp2f((m - cm) * CL_LOG2E) + cs;
            m = cm;
        } else if (c < V) {
            float cm = m;
#pragma unroll
            for (int i = 0; i < 8; i++)
                if (c + i < V) cm = fmaxf(cm, v[k][i]);
            const float cl = cm * CL_LOG2E;
            float cs = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++)
                if (c + i < V) cs += __builtin_amdgcn_exp2f(fmaf(v[k][i], CL_LOG2E, -cl));
            s = s * __builtin_amdgcn_exp2f((m - cm) * CL_LOG2E) + cs;
            m = cm;
        }
        if (tgt >= c && tgt < c + 8) {
#pragma unroll
            for (int i = 0; i < 8; i++)
                if (tgt == c + i) zt = v[k][i];
        }
    }
#pragma unroll
    for (int k = 0; k < NCHK; k++) v[k].launder();
    const float M = block_max(m, red);
    const float S = block_sum(m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - M) * CL_LOG2E), red);
    const float lse = M + logf(S);
    // the lane holding the target column writes the loss (ok: tgt < V <= Vp)
    if (ok) {
        const int own = (tgt >> 3) % CL_THREADS;
        if ((int)threadIdx.x == own) losses[row] = lse - zt;
    } else if (threadIdx.x == 0) {
        losses[row] = 0.f;
        atomicMax(err, tag);
    }
    const float l2 = lse * CL_LOG2E;
#pragma unroll
    for (int k = 0; k < NCHK; k++) {
        const int c = (threadIdx.x + k * CL_THREADS) * 8;
        if (c + 8 <= V && !(tgt >= c && tgt < c + 8)) {
            float d[8];
#pragma unroll
            for (int i = 0; i < 8; i++)
                d[i] = __builtin_amdgcn_exp2f(fmaf(v[k][i], CL_LOG2E, -l2)) * dloss;
            store8_nt(z + c, d);
        } else if (c < Vp) {
            float d[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int col = c + i;
                d[i] = col < V ? (__builtin_amdgcn_exp2f(fmaf(v[k][i], CL_LOG2E, -l2)) -
                                  (col == tgt ? 1.f : 0.f)) *
                                     dloss
                               : 0.f;
            }
            store8_nt(z + c, d);
        }
    }
}

template <typename T>
void classifier_fwd(T* logits, float* losses, const int32_t* targets, int N, int V, int Vp,
                    float dloss, int* err, int tag, hipStream_t st) {
    const int nchk = ceil_div(Vp, 8 * CL_THREADS);
    if (nchk <= 1)
        classifier_reg_kernel<T, 1><<<N, CL_THREADS, 0, st>>>(logits, losses, targets, V, Vp, dloss, err, tag);
    else if (nchk <= 4)
        classifier_reg_kernel<T, 4><<<N, CL_THREADS, 0, st>>>(logits, losses, targets, V, Vp, dloss, err, tag);
    else if (nchk <= 7)
        classifier_reg_kernel<T, 7><<<N, CL_THREADS, 0, st>>>(logits, losses, targets, V, Vp, dloss, err, tag);
    else
        classifier_kernel<T><<<N, CL_THREADS, 0, st>>>(logits, losses, targets, V, Vp, dloss, err, tag);
}

__global__ __launch_bounds__(1024) void loss_mean_kernel(float* out, const float* __restrict__ l,
                                                         int n) {
    __shared__ float red[16];
    float s = 0.f;
    for (int i = threadIdx.x; i < n; i += blockDim.x) s += l[i];
    s = block_sum(s, red);
    if (threadIdx.x == 0) out[0] = s / n;
}

void loss_mean(float* out, const float* losses, int n, hipStream_t st) {
    loss_mean_kernel<<<1, 1024, 0, st>>>(out, losses, n);
}

template void classifier_fwd<float>(float*, float*, const int32_t*, int, int, int, float, int*,
                                    int, hipStream_t);
template void classifier_fwd<bf16>(bf16*, float*, const int32_t*, int, int, int, float, int*,
                                   int, hipStream_t);
