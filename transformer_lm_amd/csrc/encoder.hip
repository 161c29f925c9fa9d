// Token + position embedding (forward gather, deterministic backward scatter).
#include "kernels.h"

// One thread per 8 channels of one position.
template <typename T>
__global__ __launch_bounds__(256) void encoder_fwd_kernel(T* __restrict__ out,
                                                          const int32_t* __restrict__ tok,
                                                          const T* __restrict__ wte,
                                                          const T* __restrict__ wpe, int BT,
                                                          int Tn, int C, int V, int* err,
                                                          int tag) {
    const int c8n = C / 8;
    int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (idx >= (int64_t)BT * c8n) return;
    int bt = (int)(idx / c8n), c = (int)(idx % c8n) * 8;
    int t = bt % Tn;
    int id = tok[bt];
    float v[8];
    if (id < 0 || id >= V) {
        if (c == 0) atomicMax(err, tag);
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
                 int V, int* err, int tag, hipStream_t st) {
    int64_t n = (int64_t)B * Tn * (C / 8);
    encoder_fwd_kernel<T><<<ceil_div(n, 256), 256, 0, st>>>(out, tok, wte, wpe, B * Tn, Tn, C,
                                                            V, err, tag);
}

typedef float floatx4 __attribute__((ext_vector_type(4)));

// dwpe[t, c] = sum_b dout[b, t, c] in increasing b; rows t >= Tn are zeroed.
// A thread owns 8 consecutive channels (C % 8 == 0): one 16-byte (bf16) or
// 32-byte (fp32) load per batch row, all B of them issued before the sums.
template <typename T>
__global__ __launch_bounds__(256) void encoder_bwd_wpe_kernel(float* __restrict__ dwpe,
                                                              const T* __restrict__ dout, int B,
                                                              int Tn, int C, int maxT) {
    const int64_t idx8 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (idx8 * 8 >= (int64_t)maxT * C) return;
    const int t = (int)(idx8 * 8 / C), c = (int)(idx8 * 8 % C);
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (t < Tn) {
        int b = 0;
        for (; b + 8 <= B; b += 8) {
            float r[8][8];
#pragma unroll
            for (int u = 0; u < 8; u++) load8(dout + ((int64_t)(b + u) * Tn + t) * C + c, r[u]);
#pragma unroll
            for (int u = 0; u < 8; u++)
#pragma unroll
                for (int k = 0; k < 8; k++) s[k] += r[u][k];
        }
        for (; b < B; b++) {
            float r[8];
            load8(dout + ((int64_t)b * Tn + t) * C + c, r);
#pragma unroll
            for (int k = 0; k < 8; k++) s[k] += r[k];
        }
    }
    floatx4* d = reinterpret_cast<floatx4*>(dwpe + idx8 * 8);
    d[0] = floatx4{s[0], s[1], s[2], s[3]};
    d[1] = floatx4{s[4], s[5], s[6], s[7]};
}

// ---- dwte: a stable counting sort of the positions by token, then segmented
// sums over the sorted order.
//
// Positions are cut into chunks of ENC_CHUNK. For chunk c and token v,
// count[v][c] = number of positions of v in c; each position's rank among the
// positions of its token inside its chunk comes from a pairwise count in LDS.
// The exclusive scan of count in (v, c) order gives every (v, c) its first slot
// in the sorted order, so slot = scan[v][c] + rank lists each token's positions
// in increasing order. The sorted order is then cut into ranges of ENC_RANGE
// slots: a block sums each token segment inside its range in slot order. A
// segment that lies inside one range is added to dwte at once; one that
// crosses ranges leaves its per-range pieces (the piece where it starts, and
// the first piece of every later range it covers) for a fix-up block, which
// adds them in range order. Every dwte row is written by exactly one block and
// summed in a fixed order, so the result does not depend on scheduling.
#define ENC_CHUNK 256
#define ENC_SCAN 4096  // elements per scan block (1024 threads x 4)
#define ENC_RANGE 16

struct EncWs {
    int* scan;     // [Vp * nch] counts, then their per-block exclusive scan
    int* bsum;     // [nsb + 1] scan-block totals, then their exclusive scan (+ total)
    int* rank;     // [BT] rank of each position within its (token, chunk)
    int* sorted;   // [BT] positions in (token, position) order
    float* piece;  // [nr][2][C] head / tail pieces of crossing segments
    int nch, nsb, nr;
};

// Carves the workspace (256-byte aligned pieces); with ws == nullptr it only
// measures, returning the size through *bytes.
static EncWs enc_ws(void* ws, int BT, int Vp, int C, int64_t* bytes = nullptr) {
    EncWs w;
    w.nch = ceil_div(BT, ENC_CHUNK);
    const int64_t ncount = (int64_t)Vp * w.nch;
    w.nsb = ceil_div(ncount, ENC_SCAN);
    w.nr = ceil_div(BT, ENC_RANGE);
    int64_t off = 0;
    auto take = [&](int64_t n) {
        char* r = ws ? (char*)ws + off : nullptr;
        off += (n + 255) / 256 * 256;
        return r;
    };
    w.scan = (int*)take(ncount * 4);
    w.bsum = (int*)take((int64_t)(w.nsb + 1) * 4);
    w.rank = (int*)take((int64_t)BT * 4);
    w.sorted = (int*)take((int64_t)BT * 4);
    w.piece = (float*)take((int64_t)w.nr * 2 * C * 4);
    if (bytes) *bytes = off;
    return w;
}

int64_t encoder_bwd_workspace_bytes(int BT, int Vp, int C) {
    int64_t bytes = 0;
    enc_ws(nullptr, BT, Vp, C, &bytes);
    return bytes;
}

// One block per chunk: ranks inside the chunk and the chunk's token counts
// (written by the last position of each token in the chunk).
__global__ __launch_bounds__(ENC_CHUNK) void enc_rank_kernel(const int32_t* __restrict__ tok, int BT,
                                                        int Vp, int nch, int* __restrict__ count,
                                                        int* __restrict__ rank) {
    __shared__ int sh[ENC_CHUNK];
    const int c = blockIdx.x, tid = threadIdx.x;
    const int p0 = c * ENC_CHUNK, n = min(ENC_CHUNK, BT - p0);
    int v = -1;
    if (tid < n) {
        v = tok[p0 + tid];
        if (v < 0 || v >= Vp) v = -1;
    }
    sh[tid] = v;
    __syncthreads();
    if (v < 0) return;
    int before = 0, after = 0;
    for (int q = 0; q < n; q++) {
        const int u = sh[q];
        before += (u == v) & (q < tid);
        after += (u == v) & (q > tid);
    }
    rank[p0 + tid] = before;
    if (after == 0) count[(int64_t)v * nch + c] = before + 1;
}

// Exclusive scan of 1024 per-thread values across the block; returns this
// thread's prefix, and the block total through *total.
__device__ __forceinline__ int block_exclusive_scan(int x, int* lds, int* total) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    int incl = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) lds[wid] = incl;
    __syncthreads();
    if (wid == 0) {
        int w = lane < 16 ? lds[lane] : 0;
        int wi = w;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) {
            const int y = __shfl_up(wi, d, 64);
            if (lane >= d) wi += y;
        }
        if (lane < 16) lds[16 + lane] = wi - w;
        if (lane == 15) lds[32] = wi;
    }
    __syncthreads();
    const int r = lds[16 + wid] + incl - x;
    *total = lds[32];
    return r;
}

// Per-block exclusive scan of ENC_SCAN elements in place; block totals to bsum.
__global__ __launch_bounds__(1024) void enc_scan_block_kernel(int* __restrict__ a, int64_t n,
                                                              int* __restrict__ bsum) {
    __shared__ int lds[40];
    const int64_t base = (int64_t)blockIdx.x * ENC_SCAN + threadIdx.x * 4;
    int v[4];
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = base + k < n ? a[base + k] : 0;
    const int t = v[0] + v[1] + v[2] + v[3];
    int total;
    int run = block_exclusive_scan(t, lds, &total);
#pragma unroll
    for (int k = 0; k < 4; k++) {
        if (base + k < n) a[base + k] = run;
        run += v[k];
    }
    if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

// Exclusive scan of the nsb block totals by one block; bsum[nsb] = total.
__global__ __launch_bounds__(1024) void enc_scan_totals_kernel(int* __restrict__ bsum, int nsb) {
    __shared__ int lds[40];
    const int per = (nsb + 1023) / 1024;
    const int s0 = threadIdx.x * per, s1 = min(nsb, s0 + per);
    int t = 0;
    for (int i = s0; i < s1; i++) t += bsum[i];
    int total;
    int run = block_exclusive_scan(t, lds, &total);
    __syncthreads();  // every thread has read its totals before any is overwritten
    for (int i = s0; i < s1; i++) {
        const int x = bsum[i];
        bsum[i] = run;
        run += x;
    }
    if (threadIdx.x == 0) bsum[nsb] = total;
}

__global__ __launch_bounds__(256) void enc_fill_kernel(const int32_t* __restrict__ tok, int BT,
                                                       int Vp, int nch, int nsb,
                                                       const int* __restrict__ scan,
                                                       const int* __restrict__ bsum,
                                                       const int* __restrict__ rank,
                                                       int* __restrict__ sorted) {
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= BT) return;
    const int v = tok[p];
    if (v < 0 || v >= Vp) return;
    const int64_t idx = (int64_t)v * nch + p / ENC_CHUNK;
    sorted[scan[idx] + bsum[idx / ENC_SCAN] + rank[p]] = p;
}

// Sorted slot range [begin, end) of token v's positions.
struct EncSeg {
    const int* scan;
    const int* bsum;
    int nch, Vp;
    __device__ __forceinline__ int begin(int v) const {
        const int64_t idx = (int64_t)v * nch;
        return scan[idx] + bsum[idx / ENC_SCAN];
    }
    __device__ __forceinline__ int end(int v) const {
        if (v + 1 < Vp) return begin(v + 1);
        const int64_t n = (int64_t)Vp * nch;  // the sorted count is the scan total
        return bsum[(n + ENC_SCAN - 1) / ENC_SCAN];
    }
};

// Adds dout rows sorted[i0..i1) (8 channels from c8 * 8) to s, in slot order.
template <typename T>
__device__ __forceinline__ void enc_sum_rows(float (&s)[8], const T* __restrict__ dout,
                                             const int* __restrict__ sorted, int i0, int i1,
                                             int C, int c8) {
    int i = i0;
    for (; i + 8 <= i1; i += 8) {
        float r[8][8];
#pragma unroll
        for (int u = 0; u < 8; u++) load8(dout + (int64_t)sorted[i + u] * C + c8 * 8, r[u]);
#pragma unroll
        for (int u = 0; u < 8; u++)
#pragma unroll
            for (int k = 0; k < 8; k++) s[k] += r[u][k];
    }
    for (; i < i1; i++) {
        float r[8];
        load8(dout + (int64_t)sorted[i] * C + c8 * 8, r);
#pragma unroll
        for (int k = 0; k < 8; k++) s[k] += r[k];
    }
}

__device__ __forceinline__ void enc_add_row(float* __restrict__ dst, const float (&s)[8]) {
    floatx4* d = reinterpret_cast<floatx4*>(dst);
    floatx4 a = d[0], b = d[1];
    a += floatx4{s[0], s[1], s[2], s[3]};
    b += floatx4{s[4], s[5], s[6], s[7]};
    d[0] = a;
    d[1] = b;
}

// One block per range of ENC_RANGE sorted slots; thread t owns channels
// 8t.. (looping when C/8 > blockDim).
template <typename T>
__global__ __launch_bounds__(128) void enc_range_kernel(float* __restrict__ dwte,
                                                        float* __restrict__ piece,
                                                        const T* __restrict__ dout,
                                                        const int32_t* __restrict__ tok,
                                                        const int* __restrict__ sorted,
                                                        EncSeg seg, int C) {
    const int b = blockIdx.x;
    const int total = seg.end(seg.Vp - 1);
    const int lo = b * ENC_RANGE, hi = min(total, lo + ENC_RANGE);
    if (lo >= hi) return;
    for (int c8 = threadIdx.x; c8 < C / 8; c8 += blockDim.x) {
        int i = lo;
        while (i < hi) {
            const int v = tok[sorted[i]];
            const int sb = seg.begin(v), se = seg.end(v);
            const int e = max(i + 1, min(hi, se));  // always advances
            float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            enc_sum_rows(s, dout, sorted, i, e, C, c8);
            float* dst;
            if (sb >= lo && se <= hi) dst = dwte + (int64_t)v * C;        // whole segment
            else dst = piece + ((int64_t)b * 2 + (sb < lo ? 0 : 1)) * C;  // head / tail piece
            if (sb >= lo && se <= hi) enc_add_row(dst + c8 * 8, s);
            else {
                floatx4* d = reinterpret_cast<floatx4*>(dst + c8 * 8);
                d[0] = floatx4{s[0], s[1], s[2], s[3]};
                d[1] = floatx4{s[4], s[5], s[6], s[7]};
            }
            i = e;
        }
    }
}

// One block per range boundary b*ENC_RANGE: the token whose segment crosses
// it for the first time is finished here, its pieces added in range order.
__global__ __launch_bounds__(128) void enc_fix_kernel(float* __restrict__ dwte,
                                                      const float* __restrict__ piece,
                                                      const int32_t* __restrict__ tok,
                                                      const int* __restrict__ sorted, EncSeg seg,
                                                      int C) {
    const int b = blockIdx.x + 1;
    const int total = seg.end(seg.Vp - 1);
    const int cut = b * ENC_RANGE;
    if (cut >= total) return;
    const int v = tok[sorted[cut - 1]];
    if (tok[sorted[cut]] != v) return;
    const int sb = seg.begin(v), se = seg.end(v);
    if (sb < cut - ENC_RANGE) return;  // crossed an earlier boundary first
    const int bs = b - 1, be = (se - 1) / ENC_RANGE;
    for (int c8 = threadIdx.x; c8 < C / 8; c8 += blockDim.x) {
        float s[8];
        const float* t = piece + ((int64_t)bs * 2 + 1) * C + c8 * 8;
#pragma unroll
        for (int k = 0; k < 8; k++) s[k] = t[k];
        // pieces in range order, eight loads in flight at a time
        int r = bs + 1;
        for (; r + 8 <= be + 1; r += 8) {
            floatx4 h[8][2];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const floatx4* q = reinterpret_cast<const floatx4*>(piece + ((int64_t)(r + u) * 2) * C + c8 * 8);
                h[u][0] = q[0];
                h[u][1] = q[1];
            }
#pragma unroll
            for (int u = 0; u < 8; u++)
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    s[k] += h[u][0][k];
                    s[4 + k] += h[u][1][k];
                }
        }
        for (; r <= be; r++) {
            const float* h = piece + ((int64_t)r * 2) * C + c8 * 8;
#pragma unroll
            for (int k = 0; k < 8; k++) s[k] += h[k];
        }
        enc_add_row(dwte + (int64_t)v * C + c8 * 8, s);
    }
}

template <typename T>
void encoder_bwd(float* dwte, float* dwpe, const T* dout, const int32_t* tok, int B, int Tn,
                 int C, int Vp, int maxT, void* ws, hipStream_t st) {
    const int BT = B * Tn;
    encoder_bwd_wpe_kernel<T><<<ceil_div((int64_t)maxT * C / 8, 256), 256, 0, st>>>(dwpe, dout, B,
                                                                                    Tn, C, maxT);
    const EncWs w = enc_ws(ws, BT, Vp, C);
    const int64_t ncount = (int64_t)Vp * w.nch;
    fill_zero_i32(w.scan, ncount, st);
    enc_rank_kernel<<<w.nch, ENC_CHUNK, 0, st>>>(tok, BT, Vp, w.nch, w.scan, w.rank);
    enc_scan_block_kernel<<<w.nsb, 1024, 0, st>>>(w.scan, ncount, w.bsum);
    enc_scan_totals_kernel<<<1, 1024, 0, st>>>(w.bsum, w.nsb);
    enc_fill_kernel<<<ceil_div(BT, 256), 256, 0, st>>>(tok, BT, Vp, w.nch, w.nsb, w.scan, w.bsum,
                                                       w.rank, w.sorted);
    const EncSeg seg{w.scan, w.bsum, w.nch, Vp};
    enc_range_kernel<T><<<w.nr, 128, 0, st>>>(dwte, w.piece, dout, tok, w.sorted, seg, C);
    if (w.nr > 1)
        enc_fix_kernel<<<w.nr - 1, 128, 0, st>>>(dwte, w.piece, tok, w.sorted, seg, C);
}

template void encoder_fwd<float>(float*, const int32_t*, const float*, const float*, int, int,
                                 int, int, int*, int, hipStream_t);
template void encoder_fwd<bf16>(bf16*, const int32_t*, const bf16*, const bf16*, int, int, int,
                                int, int*, int, hipStream_t);
template void encoder_bwd<float>(float*, float*, const float*, const int32_t*, int, int, int, int,
                                 int, void*, hipStream_t);
template void encoder_bwd<bf16>(float*, float*, const bf16*, const int32_t*, int, int, int, int,
                                int, void*, hipStream_t);
