// bf16 matrix products fed by direct global -> LDS loads (gfx950
// buffer_load_dwordx4 ... lds), for the three operand layouts of the linear
// layers, on v_mfma_f32_32x32x16_bf16 with fp32 accumulation:
//   out[i, j] = sum_p X(i, p) Y(j, p) (+ bias[j]) (+ residual[i, j]).
//
// Each load instruction of a wave writes 64 x 16 bytes to consecutive LDS
// addresses in lane order, so a tile keeps the layout it has in global memory:
//   reduction-contiguous operand (X[i*ld + p]):  LDS [rows][BK]
//   row-contiguous operand       (X[p*ld + i]):  LDS [BK][rows]
// Which global 16-byte chunk a lane fetches is XOR-permuted within its LDS
// row, so that fragment reads hit distinct banks. MFMA fragments (lane l:
// tile row l%32, 8 consecutive reduction indices 8*(l/32)..+7) come from a
// reduction-contiguous tile with one ds_read_b128, and from a row-contiguous
// tile with two ds_read_b64_tr_b16: that transpose read gives lane o of a
// 16-lane group column c0+o of rows k0..k0+3 when lane i of the group points
// at row k0 + i/4, columns c0 + 4*(i%4).
//
// Tiles sit in an S-stage LDS ring: stage k+S-1 is requested before stage k
// is computed, so the loads of S-1 stages are in flight while the matrix cores
// work, and no registers hold staged data. Waits count only the stages that
// must have landed (s_waitcnt vmcnt(N)); a plain s_barrier then publishes them
// (a __syncthreads() would also drain the later stages' loads).
//
// Requirements: the reduction length is a multiple of BK (each split's too);
// row counts of row-contiguous operands, the output width and its row stride
// are multiples of 8. Rows past the matrix edge are fetched from clamped
// addresses and their outputs discarded.
#pragma once

#include "gelu.h"
#include "gemm_mfma.h"
#include "lds_dma.h"

typedef short v4i16 __attribute__((ext_vector_type(4)));

// chunk permutation of a reduction-contiguous LDS row r (BK elements)
template <int BK>
__device__ __forceinline__ int pc_swz(int r) {
    if constexpr (BK == 64) return (r & 7) ^ ((r >> 3) & 1);
    else return (r >> 2) & 3;  // BK == 32
}

// chunk permutation of a row-contiguous LDS row k (ROWS elements). One half
// of a transpose-read fragment load reads 64 bytes at the same logical
// columns of rows k0..k0+3 (k0 % 4 == 0); the permutation moves whole 64-byte
// groups (multiples of 4 chunks) so those four land on distinct quarters of
// the 256-byte bank line: rows that start on the line's first byte cycle
// through all four quarters, rows that alternate between its halves take the
// two quarters of their half.
template <int ROWS>
__device__ __forceinline__ int rc_swz(int k) {
    static_assert(ROWS % 64 == 0, "row-contiguous tiles are whole 128-byte multiples");
    if constexpr (ROWS % 128 == 0) return 4 * (k & 3);
    else return 4 * ((k >> 1) & 1);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

#if __HIP_DEVICE_COMPILE__
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_at(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
#endif

// One operand tile (ROWS x BK) of the ring: its loads and fragment reads.
// Loads are MUBUF buffer_load ... lds: unlike the FLAT-encoded global form,
// they leave the compiler's LDS wait counting exact, so fragment reads can
// stay in flight across matrix products (see lds_dma16).
template <int ROWS, int BK, int NW, bool RC>
struct LdsOperand {
    static constexpr int CHUNKS = ROWS * BK / 8;  // 16-byte chunks per tile
    static constexpr int TOTAL = CHUNKS / 64;     // wave load instructions per tile
    static constexpr int NPW = (TOTAL + NW - 1) / NW;
    static constexpr int ELEMS = ROWS * BK;
    static_assert(TOTAL * 64 == CHUNKS, "a tile is a whole number of wave loads");

    uint32_t voff[NPW];  // this lane's byte offset from the tile origin, per load

    // Offsets for the tile whose rows start at row0; rows past the matrix edge
    // (nrows) read the last row (reduction-contiguous) or the last 8 rows
    // (row-contiguous), and their results are discarded. The last wave may
    // repeat its final chunk so that all waves issue NPW loads.
    __device__ __forceinline__ void init(int ld, int nrows, int row0, int wid, int lane) {
#pragma unroll
        for (int j = 0; j < NPW; j++) {
            const int ch = min(wid * NPW + j, TOTAL - 1) * 64 + lane;
            if (!RC) {
                constexpr int CPR = BK / 8;
                const int r = ch / CPR, lc = (ch % CPR) ^ pc_swz<BK>(ch / CPR);
                voff[j] = (uint32_t)((min(row0 + r, nrows - 1) - row0) * ld + lc * 8) * 2u;
            } else {
                constexpr int CPR = ROWS / 8;
                const int k = ch / CPR, lc = (ch % CPR) ^ rc_swz<ROWS>(ch / CPR);
                voff[j] = (uint32_t)(k * ld + min(row0 + lc * 8, nrows - 8) - row0) * 2u;
            }
        }
    }

    // Loads the tile at rows row0.., reduction k0.. into LDS at s, through
    // inline asm (ASM) or the compiler builtin (GemmLds says which launches
    // use which).
    template <bool ASM>
    __device__ __forceinline__ void load(bf16* s, const bf16* __restrict__ g, int ld, int row0,
                                         int k0, int wid) const {
        load_at<ASM>(s, RC ? g + (int64_t)k0 * ld + row0 : g + (int64_t)row0 * ld + k0, wid);
    }

    // The same, from the tile's origin at its first reduction index (base);
    // wid must be wave-uniform.
    template <bool ASM>
    __device__ __forceinline__ void load_at(bf16* s, const bf16* base, int wid) const {
        if constexpr (ASM) {
            const u32x4 rs = raw_rsrc(base);
#pragma unroll
            for (int j = 0; j < NPW; j++) {
                const int blk = min(wid * NPW + j, TOTAL - 1);
                lds_dma16(rs, voff[j], 0, s + blk * 512);
            }
        } else {
#if __HIP_DEVICE_COMPILE__
            const auto rs = buffer_at(base);
#pragma unroll
            for (int j = 0; j < NPW; j++) {
                const int blk = min(wid * NPW + j, TOTAL - 1);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void*)(s + blk * 512), 16, voff[j], 0,
                    0, 0);
            }
#endif
        }
    }

    // MFMA fragment of tile rows r0..r0+31, reduction block kk (16 wide).
    __device__ __forceinline__ static bf16x8 frag(const bf16* s, int r0, int kk, int lane) {
        if constexpr (!RC) {
            const int r = r0 + (lane & 31);
            const int c = 2 * kk + (lane >> 5);
            return *reinterpret_cast<const bf16x8*>(s + r * BK + ((c ^ pc_swz<BK>(r)) << 3));
        } else {
            const int grp = lane >> 4, i = lane & 15;
            const int col = r0 + 16 * (grp & 1) + 4 * (i & 3);
            const int k = kk * 16 + 8 * (grp >> 1) + (i >> 2);
            const bf16* p0 = s + k * ROWS + (((col >> 3) ^ rc_swz<ROWS>(k)) << 3) + (col & 7);
            const bf16* p1 =
                s + (k + 4) * ROWS + (((col >> 3) ^ rc_swz<ROWS>(k + 4)) << 3) + (col & 7);
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(p0));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(p1));
            const v4i16 v[2] = {lo, hi};
            return *reinterpret_cast<const bf16x8*>(v);
        }
    }

};

// ---------------------------------------------------------------------------
// Persistent grouped streaming kernel. A launch runs a group of products of
// one layout and epilogue ("problems": the layers' weight gradients, the
// reduction splits of one weight gradient, or a single product). Problem q
// computes
//   out_q[i, j] = sum_{p < K_q} X_q(i, p) Y_q(j, p),  i < M_q, j < N_q,
// with row strides ldx = XRC ? M : K, ldy = YRC ? N : K, ldo = N, and, when
// rowsum_q != nullptr, rowsum_q[i] = sum_p X_q(i, p) (the bias gradient of a
// weight gradient).
//
// The tiles of all problems form one list; block b walks tiles b, b + G, ...
// (G = grid size: OCC blocks per CU), each round of G tiles handed to the XCDs
// in contiguous ranges. The k-steps of a block's tiles form one stream: a load
// cursor runs S-1 stages ahead of the products, across tile boundaries, so the
// next tile's first stages load while the current tile finishes and while its
// epilogue drains.
#define GROUP_MAX 52  // the 4 weight gradients of 12 layers and the tied output head
// Cache policy of the epilogue's buffer stores. Non-temporal (nt) keeps the
// written outputs from displacing the operand panels that the L2 serves to
// the other tiles; measured in the training step, it pays for the forward
// products and the weight gradients. The input-gradient products (dX layout)
// store with the default policy: the next kernels read those gradients while
// they are still cached (step time -0.8%).
#define ST_NT 2
#define ST_POLICY(EPI, XRC, YRC, FP8) ((!(XRC) && (YRC)) ? 0 : ST_NT)
struct GemmProblem {
    const bf16* X;
    const bf16* Y;
    void* out;             // bf16 (fp32 for EPI_F32), row stride N
    bf16* out2;            // EPI_BF16_GELU: gelu(out)
    const bf16* bias;      // EPI_BF16_B / BR / GELU: added per column
    const bf16* aux;       // EPI_BF16_R / BR: residual; EPI_BF16_DGELU: pre-activation
    union {
        float* rowsum;         // or nullptr
        const float* scales;   // EPI_FP8 / EPI_FP8_B: {s_x, s_w}
    };
    int M, N, K;
};
struct GemmGroup {
    int count;
    int first_tile[GROUP_MAX + 1];  // prefix sums of the problems' tile counts
    GemmProblem p[GROUP_MAX];
};
static_assert(sizeof(GemmGroup) <= 4096, "a group travels as one kernel argument");

#if __HIP_DEVICE_COMPILE__
__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_rsrc(void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)min(bytes, (int64_t)0x7fffffff),
                                             0x00020000);
}
#endif

// Barrier after this wave's LDS reads and writes have completed. As one asm
// statement with a memory clobber, no memory access moves across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait counts. vmcnt counts a lane's vector-memory operations (loads and
// stores alike) in issue order, and "vmcnt(n)" waits until at most n are
// outstanding; any n not above the number of operations issued after the
// awaited stage's loads is safe. In steady state S-2 stages (LPS load
// instructions each) follow the awaited one; after an epilogue its NST
// buffer stores follow too, for the S-1 steps whose loads preceded them. Near
// the end of the block's stream fewer stages follow: everything is awaited.
// Inline-asm loads are invisible to the compiler, whose own waits (for the
// epilogue's bias and residual loads) then count a subset of the operations in
// flight and stay safe.
template <int BM, int BN, int BK, int WM, int WN, int GM, int S, int OCC, bool XRC, bool YRC,
          int EPI, bool ASM>
__global__ __launch_bounds__(WM* WN * 64) __attribute__((amdgpu_waves_per_eu(OCC * WM * WN / 4)))
void gemm_stream_kernel(const GemmGroup g) {
#if __HIP_DEVICE_COMPILE__  // buffer builtins exist for the device pass only
    constexpr int NW = WM * WN;
    constexpr int NT = NW * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    static_assert(FM * 32 == TM && FN * 32 == TN, "wave tiles are whole 32x32 MFMA tiles");
    static_assert(S >= 2, "ring depth");
    using XO = LdsOperand<BM, BK, NW, XRC>;
    using YO = LdsOperand<BN, BK, NW, YRC>;
    constexpr int SLOT = XO::ELEMS + YO::ELEMS;  // one ring slot: [X tile][Y tile]
    constexpr int LPS = XO::NPW + YO::NPW;       // load instructions per lane per stage
    constexpr bool FP8 = EPI == EPI_FP8 || EPI == EPI_FP8_B;
    constexpr int ST_POL = ST_POLICY(EPI, XRC, YRC, FP8);
    static_assert(!FP8 || (!XRC && !YRC), "E4M3 products: both operands reduction-contiguous");
    constexpr bool HAS_BIAS =
        EPI == EPI_BF16_B || EPI == EPI_BF16_BR || EPI == EPI_BF16_GELU || EPI == EPI_FP8_B;
    constexpr bool HAS_AUX = EPI == EPI_BF16_R || EPI == EPI_BF16_BR || EPI == EPI_BF16_DGELU;
    // buffer stores per lane per 32x32 output sub-tile, and per tile
    constexpr int SPT = EPI == EPI_F32 || EPI == EPI_BF16_GELU ? 4 : 2;
    constexpr int NST = FN * FM * SPT;
    constexpr int W_STEADY = (S - 2) * LPS;
    constexpr int W_EPI = W_STEADY + NST < 63 ? W_STEADY + NST : 63;
    static_assert(W_STEADY < 64, "vmcnt range");
    // The weight-gradient layout (both operands row-contiguous) waits for the
    // next stage's loads once the first k-step's products are issued; the
    // other layouts let those loads run until the next stage begins. Measured
    // on the grouped weight gradients of the 124M step: no early wait 4.78 ms,
    // a wait right after the loads are issued 4.24, after the first k-step's
    // products 4.12, after the second 4.42; for the forward and input-gradient
    // products every early wait was slower.
    constexpr int DRAIN_KK = (XRC && YRC) ? 0 : -1;
    constexpr int SP = 36;  // staged row stride in floats (32 + 4: spreads banks)
    static_assert(NW * 32 * SP * 4 <= SLOT * 2, "sub-tile staging fits one ring slot");
    constexpr int RSG = NT / (BM / 8);  // row sums: k groups of 16-byte column chunks
    static_assert(!XRC || (BK % RSG == 0 && RSG * BM * 4 <= SLOT * 2), "row-sum layout");
    extern __shared__ __attribute__((aligned(16))) bf16 lds_ring[];

    // wid in a scalar register: every LDS destination of the ring's loads is
    // then scalar arithmetic written straight to M0
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid % WM, wn = wid / WM;
    const int fr = lane & 31, g4 = lane >> 5;
    const int total = g.first_tile[g.count];
    const int G = gridDim.x;
    if ((int)blockIdx.x >= total) return;

    // tile of iteration `it` (XCD-contiguous ranges inside every full round)
    auto tile_at = [&](int it) {
        const int r0 = it - (int)blockIdx.x;
        if (r0 + G <= total && G % NUM_XCD == 0)
            return r0 + ((int)blockIdx.x % NUM_XCD) * (G / NUM_XCD) + (int)blockIdx.x / NUM_XCD;
        return it;
    };
    // problem q (advanced monotonically) and tile coordinates of list tile t;
    // within a problem, GM row tiles share each column of tiles
    auto decode = [&](int t, int& q, int& tm, int& tn) {
        while (q + 1 < g.count && g.first_tile[q + 1] <= t) q++;
        const GemmProblem& pr = g.p[q];
        const int nbm = (pr.M + BM - 1) / BM, nbn = (pr.N + BN - 1) / BN;
        const int lt = t - g.first_tile[q];
        const int gsz = GM * nbn, grp = lt / gsz, first = grp * GM;
        const int rows = min(GM, nbm - first), r = lt - grp * gsz;
        tm = first + r % rows;
        tn = r / rows;
    };

    // ---- load cursor: the current tile's operand origins and their advance
    // per stage stay in registers, so a stage's loads need no argument reads
    int l_it = blockIdx.x, l_kt = 0, l_q = 0, l_nk = 1;
    const bf16 *l_xb = nullptr, *l_yb = nullptr;
    int64_t l_xs = 0, l_ys = 0;
    bool l_on = true;
    XO lx;
    YO ly;
    auto l_start = [&]() {
        int tm, tn;
        decode(tile_at(l_it), l_q, tm, tn);
        const GemmProblem& p = g.p[l_q];
        const int i0 = tm * BM, j0 = tn * BN;
        const int ldx = XRC ? p.M : p.K, ldy = YRC ? p.N : p.K;
        l_nk = p.K / BK;
        l_xb = XRC ? p.X + i0 : p.X + (int64_t)i0 * ldx;
        l_yb = YRC ? p.Y + j0 : p.Y + (int64_t)j0 * ldy;
        l_xs = XRC ? (int64_t)BK * ldx : BK;
        l_ys = YRC ? (int64_t)BK * ldy : BK;
        lx.init(ldx, p.M, i0, wid, lane);
        ly.init(ldy, p.N, j0, wid, lane);
    };
    l_start();
    int issued = 0;  // stages issued so far
    auto issue = [&](int slot) {
        if (!l_on) return;
        bf16* dst = lds_ring + slot * SLOT;
        lx.template load_at<ASM>(dst, l_xb, wid);
        ly.template load_at<ASM>(dst + XO::ELEMS, l_yb, wid);
        l_xb += l_xs;
        l_yb += l_ys;
        issued++;
        if (++l_kt == l_nk) {
            l_kt = 0;
            l_it += G;
            l_on = l_it < total;
            if (l_on) l_start();
        }
    };
#pragma unroll
    for (int s = 0; s < S - 1; s++) issue(s);

    // ---- compute cursor
    int c_it = blockIdx.x, c_q = 0, c_tm, c_tn;
    decode(tile_at(c_it), c_q, c_tm, c_tn);
    int c_kt = 0, c_nk = g.p[c_q].K / BK;
    bool c_rowsum = XRC && g.p[c_q].rowsum != nullptr && c_tn == 0;
    int step = 0, epi_after = -1;  // stages issued before the last epilogue
    int slot_c = 0, slot_l = S - 1;

    floatx16 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; a++)
#pragma unroll
        for (int b = 0; b < FM; b++) acc[a][b] = floatx16{};
    // row sums: thread (rs_g, rs_c) adds chunk rs_c of k rows rs_g, rs_g + RSG, ...
    float rs[8] = {};
    const int rs_c = tid % (BM / 8), rs_g = tid / (BM / 8);

    // epilogue inputs of sub-tile st (32x32, slice fn = st / FM): this lane's
    // 8 columns of the slice (bias) and of the sub-tile's rows r, r + 16
    // (residual / pre-activation), double-buffered. Those of the first
    // sub-tile are requested with the tile's last k-step, each later one's
    // before the stores of the one before.
    const int cl = (lane & 3) * 8;
    bf16x8 biasv[2], auxv[2][2];
    auto fetch = [&](const GemmProblem& pr, int i0, int j0, int st) {
        const int fn = st / FM, fm = st % FM, buf = st & 1;
        const int j = min(j0 + wn * TN + fn * 32 + cl, pr.N - 8);
        if (HAS_BIAS && fm == 0) biasv[fn & 1] = *reinterpret_cast<const bf16x8*>(pr.bias + j);
        if (HAS_AUX)
#pragma unroll
            for (int itr = 0; itr < 2; itr++) {
                const int i = min(i0 + wm * TM + fm * 32 + ((itr * 64 + lane) >> 2), pr.M - 1);
                auxv[buf][itr] = *reinterpret_cast<const bf16x8*>(pr.aux + (int64_t)i * pr.N + j);
            }
    };

    while (true) {
        const int ahead = issued - step - 1;  // stages issued after this one
        if (ahead >= S - 2) {
            if (epi_after > step) wait_vmcnt<W_EPI>();
            else wait_vmcnt<W_STEADY>();
        } else {
            wait_vmcnt<0>();
        }
        // every wave's loads of this stage have landed, and every wave is done
        // reading the slot that the next load refills
        lds_barrier();
        const bf16* xb = lds_ring + slot_c * SLOT;
        const bf16* yb = xb + XO::ELEMS;
        // the first fragments of this stage are requested before the next
        // stage's loads, so their LDS latency overlaps the load issue
        bf16x8 a[2][FN], b[2][FM];
        auto read_frags = [&](int kk, bf16x8* af, bf16x8* bfr) {
#pragma unroll
            for (int f = 0; f < FN; f++) af[f] = YO::frag(yb, wn * TN + f * 32, kk, lane);
#pragma unroll
            for (int f = 0; f < FM; f++) bfr[f] = XO::frag(xb, wm * TM + f * 32, kk, lane);
        };
        if constexpr (!FP8) read_frags(0, a[0], b[0]);
        if ((HAS_BIAS || HAS_AUX) && c_kt + 1 == c_nk) fetch(g.p[c_q], c_tm * BM, c_tn * BN, 0);
        issue(slot_l);

        const bool do_rowsum = c_rowsum;
        if constexpr (XRC) {
            if (do_rowsum) {
#pragma unroll
                for (int k = rs_g; k < BK; k += RSG) {
                    const bf16x8 v = *reinterpret_cast<const bf16x8*>(
                        xb + k * BM + ((rs_c ^ rc_swz<BM>(k)) << 3));
#pragma unroll
                    for (int e = 0; e < 8; e++) rs[e] += (float)v[e];
                }
            }
        }
        if constexpr (FP8) {
            // E4M3: a slot row holds 2 BK codes; each 32x32x64 product takes
            // 32 bytes per lane and operand: row r0 + l%32, slot chunks
            // 4j + 2(l/32) and the one after (the same k order for both
            // operands, which is all the product needs)
            typedef int i32x8 __attribute__((ext_vector_type(8)));
            auto frag8 = [&](const bf16* sb, int r0, int j) {
                const int r = r0 + (lane & 31), c = 4 * j + 2 * (lane >> 5);
                const u32x4 lo =
                    *reinterpret_cast<const u32x4*>(sb + r * BK + ((c ^ pc_swz<BK>(r)) << 3));
                const u32x4 hi = *reinterpret_cast<const u32x4*>(
                    sb + r * BK + (((c + 1) ^ pc_swz<BK>(r)) << 3));
                return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            };
            // one set of fragments at a time (32-byte fragments, double
            // buffered, would not fit the register budget)
#pragma unroll
            for (int j = 0; j < BK / 32; j++) {
                i32x8 a[FN], b[FM];
#pragma unroll
                for (int f = 0; f < FN; f++) a[f] = frag8(yb, wn * TN + f * 32, j);
#pragma unroll
                for (int f = 0; f < FM; f++) b[f] = frag8(xb, wm * TM + f * 32, j);
#pragma unroll
                for (int fn = 0; fn < FN; fn++)
#pragma unroll
                    for (int fm = 0; fm < FM; fm++)
                        acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            a[fn], b[fm], acc[fn][fm], 0, 0, 0, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < BK / 16; kk++) {
                // fragments of step kk+1 are requested before the products of
                // step kk; the fences keep the compiler from sinking each read
                // next to its first use
                if (kk + 1 < BK / 16) read_frags(kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int fn = 0; fn < FN; fn++)
#pragma unroll
                    for (int fm = 0; fm < FM; fm++)
                        acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            a[kk & 1][fn], b[kk & 1][fm], acc[fn][fm], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (DRAIN_KK >= 0) {
                    if (kk == DRAIN_KK) wait_vmcnt<0>();
                }
            }
        }

        if (++c_kt == c_nk) {
            const GemmProblem& pr = g.p[c_q];
            // ---- epilogue of tile (c_q, c_tm, c_tn), staged through LDS (the
            // slot just consumed; the others hold the next stages) one 32x32
            // sub-tile at a time: a lane holds output row l%32 of each MFMA
            // tile and columns in runs of 4, so direct stores would write 16
            // bytes to 32 rows per instruction. Staged as fp32 rows, a sub-tile
            // leaves as 64-byte (bf16) or 128-byte (fp32) row segments; bias,
            // residual and pre-activation are applied in fp32 before the one
            // rounding.
            // Pin the accumulators to AGPRs: otherwise the bf16 epilogue's
            // conversions pull them into VGPRs for the whole kernel.
#pragma unroll
            for (int fn = 0; fn < FN; fn++)
#pragma unroll
                for (int fm = 0; fm < FM; fm++) asm volatile("" : "+a"(acc[fn][fm]));
            const int M = pr.M, N = pr.N, ldo = N;
            const int i0 = c_tm * BM, j0 = c_tn * BN;
            const float alpha = FP8 ? 1.f / (pr.scales[0] * pr.scales[1]) : 1.f;
            lds_barrier();  // every wave is done with slot_c
            float* sbase = reinterpret_cast<float*>(lds_ring + slot_c * SLOT);
            if constexpr (XRC) {
                if (do_rowsum) {
                    // partial sums of the RSG k groups, added in group order
#pragma unroll
                    for (int e = 0; e < 8; e++) sbase[rs_g * BM + rs_c * 8 + e] = rs[e];
                    lds_barrier();
                    if (tid < BM && i0 + tid < M) {
                        float t = 0.f;
                        for (int q = 0; q < RSG; q++) t += sbase[q * BM + tid];
                        pr.rowsum[i0 + tid] = t;
                    }
                    lds_barrier();
#pragma unroll
                    for (int e = 0; e < 8; e++) rs[e] = 0.f;
                }
            }
            float* stage = sbase + wid * (32 * SP);
            const int ib = i0 + wm * TM;
            constexpr int ES = EPI == EPI_F32 ? 4 : 2;
            const int64_t rows_left = min(BM, M - i0) - wm * TM;  // may be <= 0
            const int64_t span = rows_left > 0 ? rows_left * ldo * ES : 0;
            char* obase = reinterpret_cast<char*>(pr.out) + ((int64_t)ib * ldo) * ES;
            const auto rs_out = store_rsrc(obase, span);
            const auto rs_out2 =
                store_rsrc(EPI == EPI_BF16_GELU ? reinterpret_cast<char*>(pr.out2) + (int64_t)ib * ldo * 2
                                                : obase,
                           span);
#pragma unroll
            for (int st = 0; st < FN * FM; st++) {
                const int fn = st / FM, fm = st % FM;
#pragma unroll
                for (int qq = 0; qq < 4; qq++)
                    *reinterpret_cast<floatx4*>(stage + fr * SP + 8 * qq + 4 * g4) =
                        floatx4{acc[fn][fm][4 * qq], acc[fn][fm][4 * qq + 1],
                                acc[fn][fm][4 * qq + 2], acc[fn][fm][4 * qq + 3]};
                if ((HAS_BIAS || HAS_AUX) && st + 1 < FN * FM) fetch(pr, i0, j0, st + 1);
                // a wave's LDS accesses are processed in order: its reads below
                // see these writes, and the next sub-tile's writes follow them
                const int jb = j0 + wn * TN + fn * 32;
                if constexpr (EPI == EPI_F32) {
#pragma unroll
                    for (int itr = 0; itr < 4; itr++) {
                        const int idx = itr * 64 + lane, r = idx >> 3, c = (idx & 7) * 4;
                        const int j = jb + c;
                        const uint32_t off =
                            j < N ? (uint32_t)(((fm * 32 + r) * ldo + j) * 4) : 0x80000000u;
                        const floatx4 v = *reinterpret_cast<const floatx4*>(stage + r * SP + c);
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs_out,
                                                               off, 0, ST_POL);
                    }
                } else {
#pragma unroll
                    for (int itr = 0; itr < 2; itr++) {
                        const int r = (itr * 64 + lane) >> 2;
                        const int j = jb + cl;
                        const floatx4 lo = *reinterpret_cast<const floatx4*>(stage + r * SP + cl);
                        const floatx4 hi = *reinterpret_cast<const floatx4*>(stage + r * SP + cl + 4);
                        float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        if constexpr (FP8)
#pragma unroll
                            for (int e = 0; e < 8; e++) v[e] *= alpha;
                        if constexpr (HAS_BIAS)
#pragma unroll
                            for (int e = 0; e < 8; e++) v[e] += (float)biasv[fn & 1][e];
                        if constexpr (EPI == EPI_BF16_R || EPI == EPI_BF16_BR)
#pragma unroll
                            for (int e = 0; e < 8; e++) v[e] += (float)auxv[st & 1][itr][e];
                        if constexpr (EPI == EPI_BF16_DGELU)
#pragma unroll
                            for (int e = 0; e < 8; e++)
                                v[e] *= gelu_grad_fast((float)auxv[st & 1][itr][e]);
                        bf16x8 o;
#pragma unroll
                        for (int e = 0; e < 8; e++) o[e] = (bf16)v[e];
                        const uint32_t off =
                            j < N ? (uint32_t)(((fm * 32 + r) * ldo + j) * 2) : 0x80000000u;
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rs_out,
                                                               off, 0, ST_POL);
                        if constexpr (EPI == EPI_BF16_GELU) {
                            bf16x8 ga;
#pragma unroll
                            for (int e = 0; e < 8; e++) ga[e] = (bf16)gelu_fast((float)o[e]);
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ga),
                                                                   rs_out2, off, 0, ST_POL);
                        }
                    }
                }
            }
            epi_after = issued;
            c_it += G;
            if (c_it >= total) break;
            decode(tile_at(c_it), c_q, c_tm, c_tn);
            c_kt = 0;
            c_nk = g.p[c_q].K / BK;
            c_rowsum = XRC && g.p[c_q].rowsum != nullptr && c_tn == 0;
#pragma unroll
            for (int a2 = 0; a2 < FN; a2++)
#pragma unroll
                for (int b2 = 0; b2 < FM; b2++) acc[a2][b2] = floatx16{};
        }
        step++;
        slot_c = slot_c + 1 == S ? 0 : slot_c + 1;
        slot_l = slot_l + 1 == S ? 0 : slot_l + 1;
    }
#endif
}

// Launch helper for one tile shape: the grid is min(total tiles, OCC blocks
// per CU on 256 CUs). ASM selects the LDS loads' form. With builtin loads the
// compiler waits for all of them before every transpose read (it cannot tell
// which LDS bytes a read touches), so the inline-asm form is the default for
// layouts with transpose reads, whose kernels place their own waits.
template <int BM, int BN, int BK, int WM, int WN, int GM, int S, int OCC>
struct GemmLds {
    static constexpr int bm = BM, bn = BN, bk = BK, slots = OCC * 256;
    static constexpr size_t lds_bytes = (size_t)S * (BM + BN) * BK * sizeof(bf16);

    static int tiles(int M, int N) { return ceil_div(M, BM) * ceil_div(N, BN); }

    template <bool XRC, bool YRC, int EPI, bool ASM = YRC>
    static void run(const GemmGroup& g, hipStream_t st) {
        const int total = g.first_tile[g.count];
        const int grid = total < slots ? total : slots;
        gemm_stream_kernel<BM, BN, BK, WM, WN, GM, S, OCC, XRC, YRC, EPI, ASM>
            <<<grid, WM * WN * 64, lds_bytes, st>>>(g);
    }

    // Raises the kernel's dynamic-LDS limit (needed above 64 KB); call once.
    template <bool XRC, bool YRC, int EPI, bool ASM = YRC>
    static hipError_t prepare() {
        return hipFuncSetAttribute(
            (const void*)gemm_stream_kernel<BM, BN, BK, WM, WN, GM, S, OCC, XRC, YRC, EPI, ASM>,
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    }
};
