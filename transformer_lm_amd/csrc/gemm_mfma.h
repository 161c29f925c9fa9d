// bf16 matrix-product kernel template for the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16), fp32 accumulation:
//   out[i, j] = sum_p X(i, p) Y(j, p) (+ bias[j]) (+ residual[i, j]).
//
// Operand storage: an operand is either reduction-contiguous (X[i*ld + p]) or
// row-contiguous (X[p*ld + i]). Every tile is staged into LDS
// reduction-contiguous, which is what an MFMA fragment wants: lane l reads
// 8 consecutive reduction elements (16 bytes) of tile row l % 32. A
// row-contiguous operand is transposed on the way into LDS: a thread loads
// 8 rows x 2 reduction steps (two 16-byte loads) and packs each row's pair
// into one dword with v_perm_b32 before writing it.
//
// The MFMA "row" dimension is the output column j, so each lane's
// accumulators hold runs of 4 consecutive j and stores are 8-byte (bf16) or
// 16-byte (fp32) vectors along the contiguous output dimension.
// Accumulator layout of the 32x32 product: lane l, register v holds
// (row 8*(v/4) + 4*(l/32) + v%4, column l%32).
//
// Tile order: the hardware hands consecutive workgroups to the 8 XCDs in
// turn, and each XCD has its own L2. Block ids are remapped so that each XCD
// works through one contiguous range of the tile order, and that order walks
// groups of GM row tiles column by column, so the column operand's tile is
// reused by GM consecutive tiles while it sits in that XCD's L2.
#pragma once

#include "kernels.h"

typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define LDS_PAD 8  // bf16 elements of padding per LDS row (spreads rows over banks)
#define NUM_XCD 8

template <int ROWS, int BK, int NT, bool RC>
struct Stager {
    // p-contig: one chunk = 8 consecutive p of one row (16 B)
    // row-contig: one chunk = 8 consecutive rows x 2 consecutive p (2 x 16 B)
    static constexpr int NCHUNK = RC ? (ROWS / 8) * (BK / 2) : ROWS * BK / 8;
    static constexpr int CH = (NCHUNK + NT - 1) / NT;
    static constexpr int NV = RC ? 2 : 1;
    u32x4 r[CH][NV];

    // Global -> registers for the tile at (row0, k0); rows >= nrows and
    // reduction indices >= kend read as zero.
    __device__ __forceinline__ void load(const bf16* __restrict__ g, int ld, int nrows, int kend,
                                         int row0, int k0, int tid) {
#pragma unroll
        for (int q = 0; q < CH; q++) {
            const int c = tid + q * NT;
#pragma unroll
            for (int u = 0; u < NV; u++) r[q][u] = u32x4{0u, 0u, 0u, 0u};
            if (c >= NCHUNK) continue;
            if (!RC) {
                const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
                if (row0 + row < nrows && k0 + kc < kend)
                    r[q][0] = *reinterpret_cast<const u32x4*>(g + (int64_t)(row0 + row) * ld + k0 + kc);
            } else {
                const int pp = (c % (BK / 2)) * 2, rc = (c / (BK / 2)) * 8;
                if (row0 + rc < nrows)
#pragma unroll
                    for (int u = 0; u < 2; u++)
                        if (k0 + pp + u < kend)
                            r[q][u] = *reinterpret_cast<const u32x4*>(
                                g + (int64_t)(k0 + pp + u) * ld + row0 + rc);
            }
        }
    }

    // Registers -> LDS tile [ROWS][BK + LDS_PAD], reduction-contiguous.
    __device__ __forceinline__ void store(bf16* __restrict__ s, int tid) {
#pragma unroll
        for (int q = 0; q < CH; q++) {
            const int c = tid + q * NT;
            if (c >= NCHUNK) continue;
            if (!RC) {
                const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
                *reinterpret_cast<u32x4*>(s + row * (BK + LDS_PAD) + kc) = r[q][0];
            } else {
                const int pp = (c % (BK / 2)) * 2, rc = (c / (BK / 2)) * 8;
                unsigned int* d = reinterpret_cast<unsigned int*>(s + rc * (BK + LDS_PAD) + pp);
                constexpr int DW = (BK + LDS_PAD) / 2;  // dwords per LDS row
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    // rows rc+2w (low halves) and rc+2w+1 (high halves): pair (p, p+1)
                    d[(2 * w) * DW] = __builtin_amdgcn_perm(r[q][1][w], r[q][0][w], 0x05040100u);
                    d[(2 * w + 1) * DW] = __builtin_amdgcn_perm(r[q][1][w], r[q][0][w], 0x07060302u);
                }
            }
        }
    }
};

// EPI_BF16: out bf16 = acc (+ bias) (+ residual), the terms present when
// their pointers are non-null (in the persistent kernel: neither term);
// EPI_F32: out fp32 = acc. Persistent kernel only, with the terms fixed at
// compile time: EPI_BF16_B: + bias; EPI_BF16_R: + residual; EPI_BF16_BR:
// + bias + residual; EPI_BF16_GELU: out = bf16(acc + bias), out2 =
// bf16(gelu(out)); EPI_BF16_DGELU: out = bf16(acc * gelu'(aux)) with aux the
// bf16 pre-activation. EPI_FP8 / EPI_FP8_B: both operands hold E4M3 codes
// (two per bf16 slot, K counted in slots); out bf16 = acc / (s_x s_w)
// (+ bias), with the two per-tensor scales read from device memory.
enum {
    EPI_BF16 = 0,
    EPI_F32 = 1,
    EPI_BF16_GELU = 2,
    EPI_BF16_DGELU = 3,
    EPI_BF16_B = 4,
    EPI_BF16_R = 5,
    EPI_BF16_BR = 6,
    EPI_FP8 = 7,
    EPI_FP8_B = 8
};

// Tile coordinates of block `bid` of `total` = nbm x nbn tiles (see the file
// comment): XCD-contiguous ranges, GM-row groups walked column by column.
template <int GM>
__device__ __forceinline__ void tile_of(int bid, int nbm, int nbn, int& tm, int& tn) {
    const int total = nbm * nbn;
    const int per = total / NUM_XCD;
    int t = bid;
    if (bid < per * NUM_XCD) t = (bid % NUM_XCD) * per + bid / NUM_XCD;
    const int gsz = GM * nbn;
    const int g = t / gsz, first = g * GM;
    const int rows = min(GM, nbm - first);
    const int r = t - g * gsz;
    tm = first + r % rows;
    tn = r / rows;
}

// With rowsum != nullptr, the blocks of the first output-column tile also sum
// each X row over the reduction (for dW = dy^T x that is the bias gradient,
// sum over rows of dy): the staged LDS tile is read once more per k-step.
template <int BM, int BN, int BK, int WM, int WN, int GM, bool XRC, bool YRC, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_mfma_kernel(
    void* __restrict__ out_, const bf16* __restrict__ X, const bf16* __restrict__ Y,
    const bf16* __restrict__ bias, const bf16* __restrict__ residual, int M, int N, int K,
    int ldx, int ldy, int ldo, int kchunk, int64_t split_stride, float* __restrict__ rowsum,
    int64_t rowsum_stride) {
    constexpr int NT = WM * WN * 64;
    constexpr int TPR = NT / BM;  // threads per X row for the row sums
    static_assert(TPR >= 1 && BK % (8 * TPR) == 0, "row-sum split");
    constexpr int TM = BM / WM, TN = BN / WN;  // wave tile (i extent, j extent)
    constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA tiles per wave
    constexpr int LDR = BK + LDS_PAD;
    __shared__ bf16 Xs[2][BM * LDR];
    __shared__ bf16 Ys[2][BN * LDR];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid % WM, wn = wid / WM;
    int tm, tn;
    tile_of<GM>(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
    const int i0 = tm * BM, j0 = tn * BN;
    const int kbeg = blockIdx.z * kchunk, kend = min(K, kbeg + kchunk);

    Stager<BM, BK, NT, XRC> xs;
    Stager<BN, BK, NT, YRC> ys;
    floatx16 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; a++)
#pragma unroll
        for (int b = 0; b < FM; b++) acc[a][b] = floatx16{};

    const int nk = (kend - kbeg + BK - 1) / BK;
    xs.load(X, ldx, M, kend, i0, kbeg, tid);
    ys.load(Y, ldy, N, kend, j0, kbeg, tid);
    xs.store(Xs[0], tid);
    ys.store(Ys[0], tid);
    __syncthreads();

    const int fr = lane & 31, fk = (lane >> 5) * 8;
    const bool do_rowsum = rowsum != nullptr && tn == 0 && tid < TPR * BM;
    float rsum = 0.f;
    for (int kt = 0; kt < nk; kt++) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            xs.load(X, ldx, M, kend, i0, kbeg + (kt + 1) * BK, tid);
            ys.load(Y, ldy, N, kend, j0, kbeg + (kt + 1) * BK, tid);
        }
        if (do_rowsum) {
            const bf16* p = Xs[buf] + (tid / TPR) * LDR + (tid % TPR) * (BK / TPR);
#pragma unroll
            for (int e = 0; e < BK / TPR; e += 8) {
                const bf16x8 v = *reinterpret_cast<const bf16x8*>(p + e);
#pragma unroll
                for (int u = 0; u < 8; u++) rsum += (float)v[u];
            }
        }
        const bf16* xb = Xs[buf] + (wm * TM + fr) * LDR + fk;
        const bf16* yb = Ys[buf] + (wn * TN + fr) * LDR + fk;
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8 a[FN], b[FM];
#pragma unroll
            for (int f = 0; f < FN; f++) a[f] = *reinterpret_cast<const bf16x8*>(yb + f * 32 * LDR + kk);
#pragma unroll
            for (int f = 0; f < FM; f++) b[f] = *reinterpret_cast<const bf16x8*>(xb + f * 32 * LDR + kk);
#pragma unroll
            for (int fn = 0; fn < FN; fn++)
#pragma unroll
                for (int fm = 0; fm < FM; fm++)
                    acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fn], b[fm], acc[fn][fm],
                                                                          0, 0, 0);
        }
        if (kt + 1 < nk) {
            xs.store(Xs[buf ^ 1], tid);
            ys.store(Ys[buf ^ 1], tid);
        }
        __syncthreads();
    }
    if (do_rowsum) {
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) rsum += __shfl_xor(rsum, o, 64);
        const int i = i0 + tid / TPR;
        if (tid % TPR == 0 && i < M) rowsum[blockIdx.z * rowsum_stride + i] = rsum;
    }

    // epilogue: lane holds column i = l%32 of each tile and rows j in runs of 4
#pragma unroll
    for (int fn = 0; fn < FN; fn++)
#pragma unroll
        for (int fm = 0; fm < FM; fm++) {
            const int i = i0 + wm * TM + fm * 32 + fr;
            if (i >= M) continue;
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int j = j0 + wn * TN + fn * 32 + 8 * g + 4 * (lane >> 5);
                if (j >= N) continue;
                float v0 = acc[fn][fm][4 * g], v1 = acc[fn][fm][4 * g + 1];
                float v2 = acc[fn][fm][4 * g + 2], v3 = acc[fn][fm][4 * g + 3];
                if (EPI == EPI_F32) {
                    float* o = reinterpret_cast<float*>(out_) + blockIdx.z * split_stride +
                               (int64_t)i * ldo + j;
                    *reinterpret_cast<floatx4*>(o) = floatx4{v0, v1, v2, v3};
                } else {
                    if (bias) {
                        const bf16x4 bv = *reinterpret_cast<const bf16x4*>(bias + j);
                        v0 += (float)bv[0];
                        v1 += (float)bv[1];
                        v2 += (float)bv[2];
                        v3 += (float)bv[3];
                    }
                    if (residual) {
                        const bf16x4 rv =
                            *reinterpret_cast<const bf16x4*>(residual + (int64_t)i * ldo + j);
                        v0 += (float)rv[0];
                        v1 += (float)rv[1];
                        v2 += (float)rv[2];
                        v3 += (float)rv[3];
                    }
                    bf16* o = reinterpret_cast<bf16*>(out_) + (int64_t)i * ldo + j;
                    *reinterpret_cast<bf16x4*>(o) = bf16x4{(bf16)v0, (bf16)v1, (bf16)v2, (bf16)v3};
                }
            }
        }
}

// out[e] = sum_z part[z * n + e], z in order (n % 4 == 0)
__global__ __launch_bounds__(256) void split_reduce_kernel(float* __restrict__ out,
                                                           const float* __restrict__ part,
                                                           int splits, int64_t n);

// A tile configuration and its launcher.
template <int BM, int BN, int BK, int WM, int WN, int GM>
struct GemmCfg {
    static constexpr int bm = BM, bn = BN, bk = BK, threads = WM * WN * 64;
    template <bool XRC, bool YRC, int EPI>
    static void run(void* out, const bf16* X, const bf16* Y, const bf16* bias,
                    const bf16* residual, int M, int N, int K, int ldx, int ldy, int ldo,
                    int splits, int kchunk, int64_t split_stride, float* rowsum,
                    int64_t rowsum_stride, hipStream_t st) {
        const int tiles = ceil_div(M, BM) * ceil_div(N, BN);
        dim3 grid(tiles, 1, splits);
        gemm_mfma_kernel<BM, BN, BK, WM, WN, GM, XRC, YRC, EPI><<<grid, WM * WN * 64, 0, st>>>(
            out, X, Y, bias, residual, M, N, K, ldx, ldy, ldo, kchunk, split_stride, rowsum,
            rowsum_stride);
    }
};
