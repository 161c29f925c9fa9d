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

// Buffer resource over the bytes at base (gfx9 raw buffer, no range limit
// beyond 4 GB offsets; every offset used here stays far below that).
#if __HIP_DEVICE_COMPILE__
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_at(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
#endif

// One operand tile (ROWS x BK) of the ring: its loads and fragment reads.
// Loads are MUBUF buffer_load ... lds: unlike the FLAT-encoded global form,
// they leave the compiler's LDS wait counting exact, so fragment reads can
// stay in flight across matrix products.
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

    // Loads the tile at rows row0.., reduction k0.. into LDS at s.
    __device__ __forceinline__ void load(bf16* s, const bf16* __restrict__ g, int ld, int row0,
                                         int k0, int wid) const {
#if __HIP_DEVICE_COMPILE__  // the buffer builtins exist for the device pass only
        const bf16* base = RC ? g + (int64_t)k0 * ld + row0 : g + (int64_t)row0 * ld + k0;
        const auto rs = buffer_at(base);
#pragma unroll
        for (int j = 0; j < NPW; j++) {
            const int blk = min(wid * NPW + j, TOTAL - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(s + blk * 512), 16, voff[j], 0, 0,
                0);
        }
#endif
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

    // Element (row r, reduction index k) of the staged tile.
    __device__ __forceinline__ static float at(const bf16* s, int r, int k) {
        if constexpr (!RC)
            return (float)s[r * BK + ((((k >> 3) ^ pc_swz<BK>(r))) << 3) + (k & 7)];
        else
            return (float)s[k * ROWS + (((r >> 3) ^ rc_swz<ROWS>(k)) << 3) + (r & 7)];
    }
};

// With rowsum != nullptr, the blocks of the first column tile also sum each X
// row over their reduction range (for dW = dy^T x: the bias gradient).
// One output tile (tm, tn) over reduction split z (rows z*kchunk ..).
template <int BM, int BN, int BK, int WM, int WN, int GM, int S, bool XRC, bool YRC, int EPI>
__device__ __forceinline__ void gemm_lds_tile(
    void* __restrict__ out_, bf16* __restrict__ out2, const bf16* __restrict__ X,
    const bf16* __restrict__ Y, const bf16* __restrict__ bias, const bf16* __restrict__ residual,
    int M, int N, int K, int ldx, int ldy, int ldo, int kchunk, int64_t split_stride,
    float* __restrict__ rowsum, int64_t rowsum_stride, int tm, int tn, int z) {
    constexpr int NW = WM * WN, NT = NW * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    static_assert(FM * 32 == TM && FN * 32 == TN, "wave tiles are whole 32x32 MFMA tiles");
    using XO = LdsOperand<BM, BK, NW, XRC>;
    using YO = LdsOperand<BN, BK, NW, YRC>;
    constexpr int NPW = XO::NPW + YO::NPW;  // load instructions per wave per stage
    extern __shared__ __attribute__((aligned(16))) bf16 lds_ring[];
    bf16* Xs = lds_ring;                  // [S][BM * BK]
    bf16* Ys = lds_ring + S * XO::ELEMS;  // [S][BN * BK]

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid % WM, wn = wid / WM;
    const int i0 = tm * BM, j0 = tn * BN;
    const int kbeg = z * kchunk;
    const int nk = (min(K, kbeg + kchunk) - kbeg) / BK;

    floatx16 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; a++)
#pragma unroll
        for (int b = 0; b < FM; b++) acc[a][b] = floatx16{};

    XO xo;
    YO yo;
    xo.init(ldx, M, i0, wid, lane);
    yo.init(ldy, N, j0, wid, lane);
#pragma unroll
    for (int s = 0; s < S - 1; s++)
        if (s < nk) {
            xo.load(Xs + s * XO::ELEMS, X, ldx, i0, kbeg + s * BK, wid);
            yo.load(Ys + s * YO::ELEMS, Y, ldy, j0, kbeg + s * BK, wid);
        }

    const bool do_rowsum = rowsum != nullptr && tn == 0 && tid < BM;
    float rsum = 0.f;
    const int fr = lane & 31, g = lane >> 5;
    for (int kt = 0; kt < nk; kt++) {
        const int pending = min(S - 2, nk - 1 - kt);
        if (pending >= 3) wait_vmcnt<3 * NPW>();
        else if (pending == 2) wait_vmcnt<2 * NPW>();
        else if (pending == 1) wait_vmcnt<NPW>();
        else wait_vmcnt<0>();
        // This wave's reads of the buffer refilled below finished before its
        // last MFMA of the previous step consumed them.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        if (kt + S - 1 < nk) {
            const int sn = (kt + S - 1) % S;
            xo.load(Xs + sn * XO::ELEMS, X, ldx, i0, kbeg + (kt + S - 1) * BK, wid);
            yo.load(Ys + sn * YO::ELEMS, Y, ldy, j0, kbeg + (kt + S - 1) * BK, wid);
        }
        const bf16* xb = Xs + (kt % S) * XO::ELEMS;
        const bf16* yb = Ys + (kt % S) * YO::ELEMS;
        if (do_rowsum)
#pragma unroll 8
            for (int k = 0; k < BK; k++) rsum += XO::at(xb, tid, k);
        bf16x8 a[2][FN], b[2][FM];
        auto read_frags = [&](int kk, bf16x8* af, bf16x8* bfr) {
#pragma unroll
            for (int f = 0; f < FN; f++) af[f] = YO::frag(yb, wn * TN + f * 32, kk, lane);
#pragma unroll
            for (int f = 0; f < FM; f++) bfr[f] = XO::frag(xb, wm * TM + f * 32, kk, lane);
        };
        read_frags(0, a[0], b[0]);
#pragma unroll
        for (int kk = 0; kk < BK / 16; kk++) {
            // Fragments of step kk+1 are requested before the products of
            // step kk; the scheduling fences keep the compiler from sinking
            // each read next to its first use (which would expose the LDS
            // latency before every product).
            if (kk + 1 < BK / 16) read_frags(kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int fn = 0; fn < FN; fn++)
#pragma unroll
                for (int fm = 0; fm < FM; fm++)
                    acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        a[kk & 1][fn], b[kk & 1][fm], acc[fn][fm], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (do_rowsum && i0 + tid < M) rowsum[z * rowsum_stride + i0 + tid] = rsum;
    (void)NT;
    // Pin the accumulators to AGPRs: otherwise the bf16 epilogue's conversions
    // pull them into VGPRs for the whole kernel, and wide wave tiles spill.
#pragma unroll
    for (int fn = 0; fn < FN; fn++)
#pragma unroll
        for (int fm = 0; fm < FM; fm++) asm volatile("" : "+a"(acc[fn][fm]));

    // Epilogue through LDS, one 32-column slice of the wave tile at a time: a
    // lane holds output row i = l%32 of each 32x32 tile and columns in runs of
    // 4, so direct stores would write 16 bytes to 32 rows per instruction.
    // Staged as fp32 rows, the slice leaves as 64-byte (bf16) or 128-byte
    // (fp32) contiguous row segments; bias and residual are read the same way
    // and added in fp32 before the single rounding.
    constexpr int SP = 36;  // staged row stride in floats (32 + 4: spreads banks)
    static_assert(NW * TM * SP * 4 <= S * (BM + BN) * BK * 2, "staging fits in the ring");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();  // every wave is done reading the ring
    float* stage = reinterpret_cast<float*>(lds_ring) + wid * (TM * SP);
    const int ib = i0 + wm * TM;
#pragma unroll
    for (int fn = 0; fn < FN; fn++) {
#pragma unroll
        for (int fm = 0; fm < FM; fm++)
#pragma unroll
            for (int q = 0; q < 4; q++)
                *reinterpret_cast<floatx4*>(stage + (fm * 32 + fr) * SP + 8 * q + 4 * g) =
                    floatx4{acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                            acc[fn][fm][4 * q + 3]};
        // a wave's LDS accesses are processed in order: its reads below see
        // these writes, and the next slice's writes follow these reads
        const int jb = j0 + wn * TN + fn * 32;
        if (EPI == EPI_F32) {
#pragma unroll
            for (int it = 0; it < TM * 8 / 64; it++) {
                const int idx = it * 64 + lane, r = idx >> 3, c = (idx & 7) * 4;
                const int i = ib + r, j = jb + c;
                if (i < M && j < N)
                    *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(out_) +
                                                z * split_stride + (int64_t)i * ldo + j) =
                        *reinterpret_cast<const floatx4*>(stage + r * SP + c);
            }
        } else {
#pragma unroll
            for (int it = 0; it < TM * 4 / 64; it++) {
                const int idx = it * 64 + lane, r = idx >> 2, c = (idx & 3) * 8;
                const int i = ib + r, j = jb + c;
                if (i < M && j < N) {
                    const floatx4 lo = *reinterpret_cast<const floatx4*>(stage + r * SP + c);
                    const floatx4 hi = *reinterpret_cast<const floatx4*>(stage + r * SP + c + 4);
                    float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    if (bias) {
                        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(bias + j);
#pragma unroll
                        for (int e = 0; e < 8; e++) v[e] += (float)bv[e];
                    }
                    if (EPI == EPI_BF16 && residual) {
                        const bf16x8 rv =
                            *reinterpret_cast<const bf16x8*>(residual + (int64_t)i * ldo + j);
#pragma unroll
                        for (int e = 0; e < 8; e++) v[e] += (float)rv[e];
                    }
                    if (EPI == EPI_BF16_DGELU) {
                        const bf16x8 xv =
                            *reinterpret_cast<const bf16x8*>(residual + (int64_t)i * ldo + j);
#pragma unroll
                        for (int e = 0; e < 8; e++) v[e] *= gelu_grad_fast((float)xv[e]);
                    }
                    bf16x8 o;
#pragma unroll
                    for (int e = 0; e < 8; e++) o[e] = (bf16)v[e];
                    *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(out_) + (int64_t)i * ldo +
                                               j) = o;
                    if (EPI == EPI_BF16_GELU) {
                        bf16x8 ga;
#pragma unroll
                        for (int e = 0; e < 8; e++) ga[e] = (bf16)gelu_fast((float)o[e]);
                        *reinterpret_cast<bf16x8*>(out2 + (int64_t)i * ldo + j) = ga;
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int GM, int S, bool XRC, bool YRC, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_lds_kernel(
    void* __restrict__ out_, bf16* __restrict__ out2, const bf16* __restrict__ X,
    const bf16* __restrict__ Y, const bf16* __restrict__ bias, const bf16* __restrict__ residual,
    int M, int N, int K, int ldx, int ldy, int ldo, int kchunk, int64_t split_stride,
    float* __restrict__ rowsum, int64_t rowsum_stride) {
    int tm, tn;
    tile_of<GM>(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
    gemm_lds_tile<BM, BN, BK, WM, WN, GM, S, XRC, YRC, EPI>(
        out_, out2, X, Y, bias, residual, M, N, K, ldx, ldy, ldo, kchunk, split_stride, rowsum,
        rowsum_stride, tm, tn, blockIdx.z);
}

// A batch of independent weight-gradient products dw_p[N_p, K_p] (fp32) =
// dout_p[R, N_p]^T . inp_p[R, K_p] over the same R rows, with db_p[N_p] = the
// column sums of dout_p when db_p != nullptr, in one launch: the tiles of all
// problems form one grid (no reduction splits), handed to the XCDs in
// contiguous ranges.
#define GROUP_MAX 64
struct DwProblem {
    const bf16* dout;
    const bf16* inp;
    float* dw;
    float* db;
    int N, K;
};
struct DwGroup {
    int count, R;
    int first_tile[GROUP_MAX + 1];  // prefix sums of the problems' tile counts
    DwProblem p[GROUP_MAX];
};

template <int BM, int BN, int BK, int WM, int WN, int GM, int S>
__global__ __launch_bounds__(WM* WN * 64) void gemm_lds_dw_group_kernel(const DwGroup g) {
    const int total = g.first_tile[g.count];
    const int per = total / NUM_XCD;
    int t = blockIdx.x;
    if (t < per * NUM_XCD) t = (t % NUM_XCD) * per + t / NUM_XCD;
    int q = 0;
    while (q + 1 < g.count && g.first_tile[q + 1] <= t) q++;
    const DwProblem& pr = g.p[q];
    const int nbm = (pr.N + BM - 1) / BM, nbn = (pr.K + BN - 1) / BN;
    const int lt = t - g.first_tile[q];
    // GM-row groups walked column by column, as in tile_of
    const int gsz = GM * nbn, grp = lt / gsz, first = grp * GM;
    const int rows = min(GM, nbm - first), r = lt - grp * gsz;
    const int tm = first + r % rows, tn = r / rows;
    gemm_lds_tile<BM, BN, BK, WM, WN, GM, S, true, true, EPI_F32>(
        pr.dw, nullptr, pr.dout, pr.inp, nullptr, nullptr, pr.N, pr.K, g.R, pr.N, pr.K, pr.K,
        g.R, 0, pr.db, 0, tm, tn, 0);
}

template <int BM, int BN, int BK, int WM, int WN, int GM, int S>
struct GemmLds {
    static constexpr int bm = BM, bn = BN, bk = BK;
    static constexpr size_t lds_bytes = (size_t)S * (BM + BN) * BK * sizeof(bf16);

    template <bool XRC, bool YRC, int EPI>
    static void run(void* out, const bf16* X, const bf16* Y, const bf16* bias,
                    const bf16* residual, int M, int N, int K, int ldx, int ldy, int ldo,
                    int splits, int kchunk, int64_t split_stride, float* rowsum,
                    int64_t rowsum_stride, hipStream_t st, bf16* out2 = nullptr) {
        const int tiles = ceil_div(M, BM) * ceil_div(N, BN);
        dim3 grid(tiles, 1, splits);
        gemm_lds_kernel<BM, BN, BK, WM, WN, GM, S, XRC, YRC, EPI>
            <<<grid, WM * WN * 64, lds_bytes, st>>>(out, out2, X, Y, bias, residual, M, N, K, ldx,
                                                    ldy, ldo, kchunk, split_stride, rowsum,
                                                    rowsum_stride);
    }

    static void run_dw_group(const DwGroup& g, hipStream_t st) {
        gemm_lds_dw_group_kernel<BM, BN, BK, WM, WN, GM, S>
            <<<g.first_tile[g.count], WM * WN * 64, lds_bytes, st>>>(g);
    }

    static hipError_t prepare_dw_group() {
        return hipFuncSetAttribute((const void*)gemm_lds_dw_group_kernel<BM, BN, BK, WM, WN, GM, S>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    }

    // Raises the kernel's dynamic-LDS limit (needed above 64 KB); call once.
    template <bool XRC, bool YRC, int EPI>
    static hipError_t prepare() {
        return hipFuncSetAttribute(
            (const void*)gemm_lds_kernel<BM, BN, BK, WM, WN, GM, S, XRC, YRC, EPI>,
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    }
};
