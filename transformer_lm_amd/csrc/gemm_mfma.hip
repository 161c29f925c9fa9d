// bf16 matrix products on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16),
// fp32 accumulation: out[i, j] = sum_p X(i, p) Y(j, p) (+ bias[j]) (+ residual[i, j]).
//
// Operand storage: an operand is either reduction-contiguous (X[i*ld + p]) or
// row-contiguous (X[p*ld + i]). Every tile is staged into LDS
// reduction-contiguous, which is what an MFMA fragment wants: lane l reads
// 8 consecutive reduction elements (16 bytes) of tile row l % 32. A
// row-contiguous operand is transposed on the way into LDS.
//   forward  y  = x W^T      X = x  (p-contig), Y = W  (p-contig)
//   backward dx = dy W       X = dy (p-contig), Y = W  (row-contig)
//   backward dW = dy^T x     X = dy (row-contig), Y = x (row-contig)
//
// The MFMA "row" dimension is the output column j, so each lane's
// accumulators hold runs of 4 consecutive j and stores are 8-byte (bf16) or
// 16-byte (fp32) vectors along the contiguous output dimension.
// Accumulator layout of the 32x32 product: lane l, register v holds
// (row 8*(v/4) + 4*(l/32) + v%4, column l%32).
#include "kernels.h"

typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

#define LDS_PAD 8  // bf16 elements of padding per LDS row (spreads rows over banks)

template <int ROWS, int BK, int NT, bool RC>
struct Stager {
    // chunks of 8 bf16 per thread per k-tile
    static constexpr int CH = (ROWS * BK / 8 + NT - 1) / NT;
    bf16x8 r[CH];

    // Global -> registers for the tile at (row0, k0).
    __device__ __forceinline__ void load(const bf16* __restrict__ g, int ld, int nrows, int K,
                                         int row0, int k0, int tid) {
#pragma unroll
        for (int q = 0; q < CH; q++) {
            const int c = tid + q * NT;
            bf16x8 v = {};
            if (c < ROWS * BK / 8) {
                if (!RC) {  // g[row * ld + p]: chunk = 8 consecutive p of one row
                    const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
                    if (row0 + row < nrows && k0 + kc < K)
                        v = *reinterpret_cast<const bf16x8*>(g + (int64_t)(row0 + row) * ld + k0 + kc);
                } else {    // g[p * ld + row]: chunk = 8 consecutive rows of one p
                    const int p = c / (ROWS / 8), rc = (c % (ROWS / 8)) * 8;
                    if (k0 + p < K && row0 + rc < nrows)
                        v = *reinterpret_cast<const bf16x8*>(g + (int64_t)(k0 + p) * ld + row0 + rc);
                }
            }
            r[q] = v;
        }
    }

    // Registers -> LDS tile [ROWS][BK + LDS_PAD], reduction-contiguous.
    __device__ __forceinline__ void store(bf16* __restrict__ s, int tid) {
#pragma unroll
        for (int q = 0; q < CH; q++) {
            const int c = tid + q * NT;
            if (c < ROWS * BK / 8) {
                if (!RC) {
                    const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
                    *reinterpret_cast<bf16x8*>(s + row * (BK + LDS_PAD) + kc) = r[q];
                } else {
                    const int p = c / (ROWS / 8), rc = (c % (ROWS / 8)) * 8;
#pragma unroll
                    for (int e = 0; e < 8; e++) s[(rc + e) * (BK + LDS_PAD) + p] = r[q][e];
                }
            }
        }
    }
};

// EPI_BF16: out bf16 = acc (+ bias) (+ residual);  EPI_F32: out fp32 = acc.
enum { EPI_BF16 = 0, EPI_F32 = 1 };

template <int BM, int BN, int BK, int WM, int WN, bool XRC, bool YRC, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_mfma_kernel(
    void* __restrict__ out_, const bf16* __restrict__ X, const bf16* __restrict__ Y,
    const bf16* __restrict__ bias, const bf16* __restrict__ residual, int M, int N, int K,
    int ldx, int ldy, int ldo) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;  // wave tile (i extent, j extent)
    constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA tiles per wave
    constexpr int LDR = BK + LDS_PAD;
    __shared__ bf16 Xs[2][BM * LDR];
    __shared__ bf16 Ys[2][BN * LDR];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid % WM, wn = wid / WM;
    const int i0 = blockIdx.y * BM, j0 = blockIdx.x * BN;

    Stager<BM, BK, NT, XRC> xs;
    Stager<BN, BK, NT, YRC> ys;
    floatx16 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; a++)
#pragma unroll
        for (int b = 0; b < FM; b++) acc[a][b] = floatx16{};

    const int nk = (K + BK - 1) / BK;
    xs.load(X, ldx, M, K, i0, 0, tid);
    ys.load(Y, ldy, N, K, j0, 0, tid);
    xs.store(Xs[0], tid);
    ys.store(Ys[0], tid);
    __syncthreads();

    const int fr = lane & 31, fk = (lane >> 5) * 8;
    for (int kt = 0; kt < nk; kt++) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            xs.load(X, ldx, M, K, i0, (kt + 1) * BK, tid);
            ys.load(Y, ldy, N, K, j0, (kt + 1) * BK, tid);
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
                    float* o = reinterpret_cast<float*>(out_) + (int64_t)i * ldo + j;
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

template <bool XRC, bool YRC, int EPI>
static void launch(void* out, const bf16* X, const bf16* Y, const bf16* bias,
                   const bf16* residual, int M, int N, int K, int ldx, int ldy, int ldo,
                   hipStream_t st) {
    constexpr int BM = 128, BN = 128, BK = 32, WM = 2, WN = 2;
    dim3 grid(ceil_div(N, BN), ceil_div(M, BM));
    gemm_mfma_kernel<BM, BN, BK, WM, WN, XRC, YRC, EPI><<<grid, WM * WN * 64, 0, st>>>(
        out, X, Y, bias, residual, M, N, K, ldx, ldy, ldo);
}

// out[M,N] = inp[M,K] . w[N,K]^T (+ bias) (+ residual)
void gemm_bf16_fwd(bf16* out, const bf16* inp, const bf16* w, const bf16* bias,
                   const bf16* residual, int M, int K, int N, hipStream_t st) {
    launch<false, false, EPI_BF16>(out, inp, w, bias, residual, M, N, K, K, K, N, st);
}

// dinp[M,K] = dout[M,N] . w[N,K]
void gemm_bf16_bwd_dx(bf16* dinp, const bf16* dout, const bf16* w, int M, int N, int K,
                      hipStream_t st) {
    launch<false, true, EPI_BF16>(dinp, dout, w, nullptr, nullptr, M, K, N, N, K, K, st);
}

// dw[N,K] (fp32) = dout[M,N]^T . inp[M,K]
void gemm_bf16_bwd_dw(float* dw, const bf16* dout, const bf16* inp, int M, int N, int K,
                      hipStream_t st) {
    launch<true, true, EPI_F32>(dw, dout, inp, nullptr, nullptr, N, K, M, N, K, K, st);
}
