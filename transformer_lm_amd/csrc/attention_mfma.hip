// Causal attention for head size 64 in bf16 on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16), the fused online-softmax attention of page
// "llm.c: Large Language Model Training in Pure C/CUDA Without Dependencies"
// (section "Fused Attention Kernel"): scores never go to HBM; 64-row tiles of
// K, V (forward, dQ) or Q, dO (dK/dV) stream through a double-buffered LDS
// ring filled by direct global -> LDS loads; the backward pass rebuilds P from
// the saved log-sum-exp.
//
// Tiles keep their global layout in LDS: [64 rows][64 dims], 128-byte rows
// whose 16-byte chunks are XOR-permuted (chunk c of row r at c ^ swz(r)).
// Fragments with dims as the reduction come from one ds_read_b128; fragments
// with tile rows as the reduction (V^T, K^T, Q^T, dO^T) come from two
// ds_read_b64_tr_b16 transpose reads, which give lane o of a 16-lane group
// column c0+o of rows k0..k0+3 when lane i points at row k0 + i/4,
// columns c0 + 4*(i%4).
//
// A 32x32 accumulator gives lane l the column l%32 and rows
// 8*(v/4) + 4*(l/32) + v%4 (register v). Score tiles are computed with queries
// as columns where a kernel needs per-query statistics in one lane
// (S^T = K Q^T), and with keys as columns where it needs per-key sums
// (S = Q K^T). The reduction order inside an MFMA is free as long as both
// operands use the same one, so probabilities and score gradients feed the
// next product straight from the accumulator registers: register v (0..7 of a
// half tile) of lane group g stands for tile row 4g + v%4 + 8*(v/4), and the
// transpose reads fetch the other operand's rows in that order.
//
// Softmax runs in base 2: x = s * log2(e) / sqrt(hs), p = exp2(x - m).
//
// Launch bounds ask for 4 (forward) and 2 (dK/dV, dQ) waves per SIMD: the
// register budgets that fit keep every kernel free of spills (dQ needs under
// 170 registers and so runs 3 waves per SIMD), and the extra waves hide the
// matrix-core / exponential / LDS latencies of each wave's serial tile loop.
#include <type_traits>

#include "gemm_lds.h"

#define HS 64
#define Q_PER_BLOCK 128  // 4 waves x 32 rows
#define TILE 64          // rows of a streamed K/V or Q/dO tile
#define TILE_ELEMS (TILE * HS)
#define LOG2E 1.4426950408889634f
#define LN2 0.6931471805599453f
// The forward pass keeps its running reference maximum until a tile's maximum
// exceeds it by more than this (base 2), so probabilities stay below 2^8 and
// most tiles skip rescaling the output accumulators. O / l and the
// log-sum-exp m + log2(l) do not depend on which reference is used.
#define RESCALE_SLACK 8.0f

__device__ __forceinline__ floatx16 mfma(bf16x8 a, bf16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld16(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Chunk permutation of tile row r (8 chunks of 16 bytes, 128-byte rows, so
// even and odd rows sit on opposite halves of the 256-byte bank line). Row
// fragments read one chunk of 16 consecutive rows per 16 lanes: the 8 rows of
// each parity take 8 distinct chunks. Transpose fragments read 4 chunks of 4
// consecutive rows per 32 lanes: rows r and r+2 (same half) take opposite
// 4-chunk groups. Both reads are then free of bank conflicts.
__device__ __forceinline__ int tswz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// 2^x on the hardware exponential (no denormal rescaling: probabilities that
// small do not change a bf16 result).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer resources over the bytes at base, for the builtin and the inline-asm
// loads; the launchers keep every offset of one sequence's slice below 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ u32x4 slice_rsrc_asm(const void* base) { return raw_rsrc(base); }

// Direct loads (buffer_load ... lds) of rows r0..r0+63 of a 64-wide head
// slice (row stride ld elements, soff bytes past the resource base) into the
// LDS tile s; rows >= nrows repeat row nrows-1. 4 waves, 2 loads each. ASM
// issues them through inline asm (lds_dma16): the compiler then does not make
// the current tile's transpose reads wait for the next tile's loads, and
// tile_barrier's explicit wait is the one that covers them. Measured, the two
// backward kernels gain from it and the forward kernel runs faster with the
// builtin form.
template <bool ASM, typename Rsrc>
__device__ __forceinline__ void dma_tile(bf16* s, Rsrc rs, int soff, int ld, int r0, int nrows,
                                         int wid, int lane) {
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int blk = wid * 2 + j, ch = blk * 64 + lane;
        const int r = ch >> 3, lc = (ch & 7) ^ tswz(ch >> 3);
        const uint32_t off = (uint32_t)(min(r0 + r, nrows - 1) * ld + lc * 8) * 2u;
        if constexpr (ASM) {
            lds_dma16(rs, off, (uint32_t)soff, s + blk * 512);
        } else {
#if __HIP_DEVICE_COMPILE__
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(s + blk * 512), 16, off, soff, 0, 0);
#endif
        }
    }
}

// Fragment with tile rows r0..r0+31 as MFMA rows and dims 16kk.. as reduction.
__device__ __forceinline__ bf16x8 frag_rows(const bf16* s, int r0, int kk, int lane) {
    const int r = r0 + (lane & 31), c = 2 * kk + (lane >> 5);
    return ld16(s + r * HS + ((c ^ tswz(r)) << 3));
}

// Fragment with dims d0..d0+31 as MFMA rows and tile rows as reduction, in the
// accumulator order: lane group g takes rows base+4g..+3 and base+8+4g..+3.
__device__ __forceinline__ bf16x8 frag_dims(const bf16* s, int d0, int base, int lane) {
    const int i = lane & 15, g = lane >> 5;
    const int col = d0 + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
    const int ra = base + 4 * g + (i >> 2), rb = ra + 8;
    const bf16* pa = s + ra * HS + (((col >> 3) ^ tswz(ra)) << 3) + (col & 7);
    const bf16* pb = s + rb * HS + (((col >> 3) ^ tswz(rb)) << 3) + (col & 7);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)pa);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)pb);
    const v4i16 v[2] = {lo, hi};
    return *reinterpret_cast<const bf16x8*>(v);
}

// Lanes l and l ^ 32 combined: the swap of the upper half of one copy of x
// with the lower half of another leaves every lane holding x of lane l % 32 in
// one register and x of lane l % 32 + 32 in the other, so both lanes of a pair
// combine the same two values in the same order (no LDS round trip).
__device__ __forceinline__ void half_pair(float x, float& lo, float& hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_pair_max(float x) {
    float lo, hi;
    half_pair(x, lo, hi);
    return fmaxf(lo, hi);
}
__device__ __forceinline__ float half_pair_sum(float x) {
    float lo, hi;
    half_pair(x, lo, hi);
    return lo + hi;
}

// acc + the sum of the 8 bf16 values, exact products by one on the dot unit
// (four v_dot2_f32_bf16, accumulating in fp32).
__device__ __forceinline__ float sum_bf16x8(const bf16x8& v, float acc) {
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(bf16)1.f, (bf16)1.f};
#pragma unroll
    for (int i = 0; i < 4; i++)
        acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2 * i], v[2 * i + 1]}, one, acc, false);
    return acc;
}

// Registers 8*hh .. 8*hh+7 of an accumulator, rounded to bf16.
__device__ __forceinline__ bf16x8 half_tile(const floatx16& a, int hh) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; i++) r[i] = (bf16)a[8 * hh + i];
    return r;
}

// One-dimensional grids over (row block, b*h), ordered by decreasing causal
// work: all heads' last row blocks first. The dispatcher hands out blocks in
// index order, so long blocks start early and short ones fill in behind them.
__device__ __forceinline__ void longest_first(int& rb, int& bh, int nrb, int nblocks) {
    const int nbh = nblocks / nrb;
    rb = nrb - 1 - (int)blockIdx.x / nbh;
    bh = (int)blockIdx.x % nbh;
}

// The next tile may be requested once every wave has finished reading the
// buffer it refills; the current one is usable once this wave's loads landed
// and all waves passed the barrier.
__device__ __forceinline__ void tile_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
}

// ---------------------------------------------------------------- forward --
// Block: 128 queries of one (b, h); wave w owns queries q0 .. q0+31, lane l the
// query q0 + l%32. Per 64-key tile: S^T (keys x queries) = K Q^T, online
// softmax per query, O^T (dims x queries) += V^T P^T. Only tiles that cross
// the causal diagonal or the sequence end are masked.
__global__ __launch_bounds__(256, 4) void flash_fwd_kernel(bf16* __restrict__ out,
                                                        float* __restrict__ lse,
                                                        const bf16* __restrict__ qkv, int Tn,
                                                        int C, int NH) {
    // the tile ring lives in dynamic LDS (four 8 KB tiles)
    extern __shared__ __attribute__((aligned(16))) bf16 ring[];
    auto Ks = [&](int i) { return ring + i * TILE_ELEMS; };
    auto Vs = [&](int i) { return ring + (2 + i) * TILE_ELEMS; };
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5;
    int qt, bh;
    longest_first(qt, bh, (Tn + Q_PER_BLOCK - 1) / Q_PER_BLOCK, gridDim.x);
    const int b = bh / NH, h = bh % NH;
    const int C3 = 3 * C;
    const bf16* base = qkv + (int64_t)b * Tn * C3 + h * HS;
    const auto rs = slice_rsrc(base);
    const int q0 = qt * Q_PER_BLOCK + wid * 32;
    const int ql = q0 + (lane & 31);
    const float sc = LOG2E / 8.0f;  // log2(e) / sqrt(64)

    bf16x8 qf[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
        qf[kb] = ql < Tn ? ld16(base + (int64_t)ql * C3 + kb * 16 + 8 * g) : bf16x8{};
    floatx16 o[2] = {floatx16{}, floatx16{}};
    float m = -INFINITY, l = 0.f;

    const int ntiles = (min(Tn, (qt + 1) * Q_PER_BLOCK) + TILE - 1) / TILE;
    dma_tile<false>(Ks(0), rs, 2 * C, C3, 0, Tn, wid, lane);
    dma_tile<false>(Vs(0), rs, 4 * C, C3, 0, Tn, wid, lane);
    for (int t = 0; t < ntiles; t++) {
        const int buf = t & 1, k0 = t * TILE;
        tile_barrier();
        if (t + 1 < ntiles) {
            dma_tile<false>(Ks(buf ^ 1), rs, 2 * C, C3, k0 + TILE, Tn, wid, lane);
            dma_tile<false>(Vs(buf ^ 1), rs, 4 * C, C3, k0 + TILE, Tn, wid, lane);
        }
        if (k0 > q0 + 31 || q0 >= Tn) continue;  // every key of the tile is masked
        const bf16* kt_s = Ks(buf);
        const bf16* vt_s = Vs(buf);
        floatx16 s[2] = {floatx16{}, floatx16{}};
#pragma unroll
        for (int kb = 0; kb < 4; kb++)
#pragma unroll
            for (int kt = 0; kt < 2; kt++) s[kt] = mfma(frag_rows(kt_s, 32 * kt, kb, lane), qf[kb], s[kt]);
        if (k0 + TILE - 1 > q0 || k0 + TILE > Tn) {  // wave-uniform
#pragma unroll
            for (int kt = 0; kt < 2; kt++)
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int key = k0 + 32 * kt + 8 * (v >> 2) + 4 * g + (v & 3);
                    if (key > ql || key >= Tn) s[kt][v] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int v = 0; v < 16; v++) mx = fmaxf(mx, s[kt][v]);
        mx = half_pair_max(mx);
        // every processed tile holds a visible key for every lane, so mt is
        // finite; the reference m moves only when the tile's maximum passes it
        // by more than RESCALE_SLACK (always on a lane's first tile)
        const float mt = mx * sc;
        const bool up = mt > m + RESCALE_SLACK;
        if (__builtin_amdgcn_ballot_w64(up)) {  // wave-uniform
            const float mn = up ? mt : m;
            const float corr = exp2_fast(m - mn);
            l *= corr;
            o[0] *= corr;
            o[1] *= corr;
            m = mn;
        }
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int v = 0; v < 16; v++) s[kt][v] = exp2_fast(fmaf(s[kt][v], sc, -m));
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                const bf16x8 pb = half_tile(s[kt], hh);
                l = sum_bf16x8(pb, l);
#pragma unroll
                for (int dt = 0; dt < 2; dt++)
                    o[dt] = mfma(frag_dims(vt_s, 32 * dt, 32 * kt + 16 * hh, lane), pb, o[dt]);
            }
    }
    l = half_pair_sum(l);  // each half summed its own keys
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
// kw + l%32. Per 64-query tile (queries >= the block's first key), in two
// 32-query halves: S = Q K^T and dP = dO V^T (queries x keys),
// P = exp2(S*c - lse*log2(e)), dS = P (dP - D); dV^T += dO^T P; dK^T += Q^T dS.
// D = sum_d dO[d] O[d] per query (the softmax-backward correction of the
// row) and the row's log-sum-exp times log2(e) come from the dQ kernel, which
// runs first.
__global__ __launch_bounds__(256, 2) void flash_bwd_dkv_kernel(
    bf16* __restrict__ dqkv, const bf16* __restrict__ dout, const bf16* __restrict__ qkv,
    const float* __restrict__ Dbuf, int Tn, int C, int NH) {
    extern __shared__ __attribute__((aligned(16))) bf16 ring[];
    auto Qs = [&](int i) { return ring + i * TILE_ELEMS; };
    auto Os = [&](int i) { return ring + (2 + i) * TILE_ELEMS; };
    auto ls = [&](int i) { return reinterpret_cast<float*>(ring + 4 * TILE_ELEMS) + i * TILE; };
    auto Ds = [&](int i) { return reinterpret_cast<float*>(ring + 4 * TILE_ELEMS) + (2 + i) * TILE; };
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5;
    int kq, bh;
    longest_first(kq, bh, (Tn + Q_PER_BLOCK - 1) / Q_PER_BLOCK, gridDim.x);
    kq = (Tn + Q_PER_BLOCK - 1) / Q_PER_BLOCK - 1 - kq;  // key block 0 has the most queries
    const int b = bh / NH, h = bh % NH;
    const int C3 = 3 * C;
    const bf16* base = qkv + (int64_t)b * Tn * C3 + h * HS;
    const bf16* dbase = dout + (int64_t)b * Tn * C + h * HS;
    const auto rq = slice_rsrc_asm(base);
    const auto ro = slice_rsrc_asm(dbase);
    // the rows' base-2 log-sum-exp (written by the dQ kernel after D)
    const int64_t nrows = (int64_t)(gridDim.x / ((Tn + Q_PER_BLOCK - 1) / Q_PER_BLOCK)) * Tn;
    const auto rl = slice_rsrc_asm(wid == 2 ? Dbuf + nrows + (int64_t)bh * Tn
                                            : Dbuf + (int64_t)bh * Tn);
    const int kb0 = kq * Q_PER_BLOCK;
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

    // tile t covers queries kb0 + 64 t ..; the per-query statistics come along
    // by direct loads (wave 2: log-sum-exp, wave 3: D), one float a lane
    auto issue = [&](int t, int buf) {
        const int q0 = kb0 + t * TILE;
        dma_tile<true>(Qs(buf), rq, 0, C3, q0, Tn, wid, lane);
        dma_tile<true>(Os(buf), ro, 0, C, q0, Tn, wid, lane);
        if (wid >= 2) {
            const uint32_t off = (uint32_t)min(q0 + lane, Tn - 1) * 4u;
            lds_dma4(rl, off, 0, wid == 2 ? ls(buf) : Ds(buf));
        }
    };
    const int ntiles = (Tn - kb0 + TILE - 1) / TILE;
    if (ntiles > 0) issue(0, 0);
    for (int t = 0; t < ntiles; t++) {
        const int buf = t & 1, q0 = kb0 + t * TILE;
        tile_barrier();
        if (t + 1 < ntiles) issue(t + 1, buf ^ 1);
        if (kw > q0 + TILE - 1 || kw >= Tn) continue;  // no query of the tile sees these keys
        const bf16* qs = Qs(buf);
        const bf16* os = Os(buf);
        // the tile body, compiled once with the causal / end-of-sequence mask
        // and once without it (tiles clear of the diagonal and the end)
        auto tile = [&](auto masked) {
#pragma unroll
            for (int qt = 0; qt < 2; qt++) {
                floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
                for (int kb = 0; kb < 4; kb++) {
                    s = mfma(frag_rows(qs, 32 * qt, kb, lane), kf[kb], s);
                    dp = mfma(frag_rows(os, 32 * qt, kb, lane), vf[kb], dp);
                }
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int qo = 32 * qt + 8 * r + 4 * g;  // 4 consecutive queries
                    const floatx4 l4 = *reinterpret_cast<const floatx4*>(&ls(buf)[qo]);
                    const floatx4 d4 = *reinterpret_cast<const floatx4*>(&Ds(buf)[qo]);
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int v = 4 * r + e;
                        float p = exp2_fast(fmaf(s[v], sc, -l4[e]));
                        if constexpr (decltype(masked)::value) {
                            const int q = q0 + qo + e;
                            p = (kl <= q && q < Tn) ? p : 0.f;
                        }
                        s[v] = p;
                        dp[v] = p * (dp[v] - d4[e]);
                    }
                }
#pragma unroll
                for (int hh = 0; hh < 2; hh++) {
                    const bf16x8 pb = half_tile(s, hh);
                    const bf16x8 db = half_tile(dp, hh);
                    const int rb = 32 * qt + 16 * hh;
#pragma unroll
                    for (int dt = 0; dt < 2; dt++) {
                        dv[dt] = mfma(frag_dims(os, 32 * dt, rb, lane), pb, dv[dt]);
                        dk[dt] = mfma(frag_dims(qs, 32 * dt, rb, lane), db, dk[dt]);
                    }
                }
            }
        };
        if (q0 < kw + 31 || q0 + TILE > Tn)  // wave-uniform
            tile(std::true_type{});
        else
            tile(std::false_type{});
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
__global__ __launch_bounds__(256, 2) void flash_bwd_dq_kernel(
    bf16* __restrict__ dqkv, const bf16* __restrict__ dout, const bf16* __restrict__ qkv,
    const bf16* __restrict__ out, const float* __restrict__ lse, float* __restrict__ Dbuf, int Tn,
    int C, int NH) {
    extern __shared__ __attribute__((aligned(16))) bf16 ring[];
    auto Ks = [&](int i) { return ring + i * TILE_ELEMS; };
    auto Vs = [&](int i) { return ring + (2 + i) * TILE_ELEMS; };
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5;
    int qt, bh;
    longest_first(qt, bh, (Tn + Q_PER_BLOCK - 1) / Q_PER_BLOCK, gridDim.x);
    const int b = bh / NH, h = bh % NH;
    const int C3 = 3 * C;
    const bf16* base = qkv + (int64_t)b * Tn * C3 + h * HS;
    const auto rs = slice_rsrc_asm(base);
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
    // D = rowsum(dO o O) of this lane's query: 8-dim chunk sums (chunk 2 kb + g
    // is here), then pairs of chunks, in a fixed tree; the dK/dV kernel,
    // launched after this one, reads it from Dbuf
    float Dq = 0.f;
    {
        float cs[4];
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
            const bf16x8 o = ql < Tn ? ld16(out + ((int64_t)b * Tn + ql) * C + h * HS + kb * 16 + 8 * g)
                                     : bf16x8{};
            float t = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) t += (float)df[kb][i] * (float)o[i];
            cs[kb] = t + __shfl_xor(t, 32, 64);
        }
        Dq = (cs[0] + cs[1]) + (cs[2] + cs[3]);
        if (ql < Tn && g == 0) {
            Dbuf[(int64_t)bh * Tn + ql] = Dq;
            const int64_t nrows = (int64_t)(gridDim.x / ((Tn + Q_PER_BLOCK - 1) / Q_PER_BLOCK)) * Tn;
            Dbuf[nrows + (int64_t)bh * Tn + ql] = l2;
        }
    }
    floatx16 dq[2] = {floatx16{}, floatx16{}};

    const int ntiles = (min(Tn, (qt + 1) * Q_PER_BLOCK) + TILE - 1) / TILE;
    dma_tile<true>(Ks(0), rs, 2 * C, C3, 0, Tn, wid, lane);
    dma_tile<true>(Vs(0), rs, 4 * C, C3, 0, Tn, wid, lane);
    for (int t = 0; t < ntiles; t++) {
        const int buf = t & 1, k0 = t * TILE;
        tile_barrier();
        if (t + 1 < ntiles) {
            dma_tile<true>(Ks(buf ^ 1), rs, 2 * C, C3, k0 + TILE, Tn, wid, lane);
            dma_tile<true>(Vs(buf ^ 1), rs, 4 * C, C3, k0 + TILE, Tn, wid, lane);
        }
        if (k0 > q0 + 31 || q0 >= Tn) continue;
        const bf16* ks = Ks(buf);
        const bf16* vs = Vs(buf);
        // the tile body, compiled once with the causal / end-of-sequence mask
        // and once without it (tiles clear of the diagonal and the end)
        auto tile = [&](auto masked) {
#pragma unroll
            for (int kt = 0; kt < 2; kt++) {
                floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
                for (int kb = 0; kb < 4; kb++) {
                    s = mfma(frag_rows(ks, 32 * kt, kb, lane), qf[kb], s);
                    dp = mfma(frag_rows(vs, 32 * kt, kb, lane), df[kb], dp);
                }
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    float p = exp2_fast(fmaf(s[v], sc, -l2));
                    if constexpr (decltype(masked)::value) {
                        const int key = k0 + 32 * kt + 8 * (v >> 2) + 4 * g + (v & 3);
                        p = (key <= ql && key < Tn) ? p : 0.f;
                    }
                    dp[v] = p * (dp[v] - Dq);
                }
#pragma unroll
                for (int hh = 0; hh < 2; hh++) {
                    const bf16x8 db = half_tile(dp, hh);
#pragma unroll
                    for (int dt = 0; dt < 2; dt++)
                        dq[dt] = mfma(frag_dims(ks, 32 * dt, 32 * kt + 16 * hh, lane), db, dq[dt]);
                }
            }
        };
        if (k0 + TILE - 1 > q0 || k0 + TILE > Tn)  // wave-uniform
            tile(std::true_type{});
        else
            tile(std::false_type{});
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

// The flash kernels address one sequence's qkv slice with 32-bit buffer
// offsets.
bool flash_attention_fits(int Tn, int C) { return (int64_t)Tn * 3 * C * 2 < (int64_t(1) << 31); }

void flash_attention_fwd(bf16* out, float* lse, const bf16* qkv, int B, int Tn, int C, int NH,
                         hipStream_t st) {
    const dim3 grid(ceil_div(Tn, Q_PER_BLOCK) * B * NH);
    flash_fwd_kernel<<<grid, 256, 4 * TILE_ELEMS * sizeof(bf16), st>>>(out, lse, qkv, Tn, C, NH);
}

// work: 2*B*NH*Tn floats, written by the dQ kernel for the dK/dV kernel: the
// rows' D, then their log-sum-exp in base 2.
void flash_attention_bwd(bf16* dqkv, const bf16* dout, const bf16* qkv, const bf16* out,
                         const float* lse, float* work, int B, int Tn, int C, int NH,
                         hipStream_t st) {
    const dim3 grid(ceil_div(Tn, Q_PER_BLOCK) * B * NH);
    flash_bwd_dq_kernel<<<grid, 256, 4 * TILE_ELEMS * sizeof(bf16), st>>>(dqkv, dout, qkv, out, lse,
                                                                         work, Tn, C, NH);
    flash_bwd_dkv_kernel<<<grid, 256, 4 * TILE_ELEMS * sizeof(bf16) + 4 * TILE * sizeof(float),
                           st>>>(dqkv, dout, qkv, work, Tn, C, NH);
}
