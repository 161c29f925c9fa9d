// The bf16 matrix products of the linear layers:
//   forward  y  = x W^T      X = x  (p-contig), Y = W  (p-contig)
//   backward dx = dy W       X = dy (p-contig), Y = W  (row-contig)
//   backward dW = dy^T x     X = dy (row-contig), Y = x (row-contig)
// Shapes whose reduction length is a multiple of 64 run on the persistent
// streaming direct-to-LDS kernel (gemm_lds.h); others on the register-staged kernel
// (gemm_mfma.h). A single weight gradient with few output tiles is split along
// its B*T reduction (one problem of the group per split), each split writing
// an fp32 partial that a second kernel sums in split order (deterministic);
// the weight gradients of all layers run together as one group instead. The
// bias gradient (column sums of dy) rides along in the same kernel.
#include <mutex>

#include "gemm_lds.h"

__global__ __launch_bounds__(256) void split_reduce_kernel(float* __restrict__ out,
                                                           const float* __restrict__ part,
                                                           int splits, int64_t n) {
    const int64_t i = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) * 4;
    if (i >= n) return;
    floatx4 s = *reinterpret_cast<const floatx4*>(part + i);
    for (int z = 1; z < splits; z++) s += *reinterpret_cast<const floatx4*>(part + z * n + i);
    *reinterpret_cast<floatx4*>(out + i) = s;
}

// 128x192 tiles on four waves (64x96 each) with an 80 KB two-stage ring: two
// blocks share a CU, so one block's barrier and load waits overlap the other's
// matrix products (measured: deeper rings of 32-deep stages, and 256-row tiles
// at one block per CU, are slower). 16384-row outputs of width 768, 2304 and
// 3072 make exactly 1, 3 and 4 rounds of 512 tiles.
using Cfg = GemmCfg<128, 128, 32, 2, 2, 16>;  // register-staged fallback
using Lds = GemmLds<128, 192, 64, 2, 2, 8, 2, 2>;
constexpr int LDS_BK = 64;
constexpr int BLOCK_SLOTS = Lds::slots;  // resident blocks: two per CU on 256 CUs

// The direct-to-LDS kernels use more than 64 KB of LDS; raise their limits once.
static void prepare_lds_kernels() {
    static std::once_flag once;
    std::call_once(once, [] {
        (void)Lds::prepare<false, false, EPI_BF16>();
        (void)Lds::prepare<false, false, EPI_BF16_B>();
        (void)Lds::prepare<false, false, EPI_BF16_R>();
        (void)Lds::prepare<false, false, EPI_BF16_BR>();
        (void)Lds::prepare<false, false, EPI_BF16_GELU>();
        (void)Lds::prepare<false, true, EPI_BF16>();
        (void)Lds::prepare<false, true, EPI_BF16_DGELU>();
        (void)Lds::prepare<true, true, EPI_F32>();
        (void)Lds::prepare<false, false, EPI_FP8>();
        (void)Lds::prepare<false, false, EPI_FP8_B>();
    });
}

// A group of one problem.
static GemmGroup single(const GemmProblem& p) {
    GemmGroup g;
    g.count = 1;
    g.first_tile[0] = 0;
    g.first_tile[1] = Lds::tiles(p.M, p.N);
    g.p[0] = p;
    return g;
}

// out[M,N] = inp[M,K] . w[N,K]^T (+ bias) (+ residual)
void gemm_bf16_fwd(bf16* out, const bf16* inp, const bf16* w, const bf16* bias,
                   const bf16* residual, int M, int K, int N, hipStream_t st) {
    if (K % LDS_BK == 0) {
        prepare_lds_kernels();
        const GemmGroup g = single({inp, w, out, nullptr, bias, residual, nullptr, M, N, K});
        if (bias && residual) Lds::run<false, false, EPI_BF16_BR>(g, st);
        else if (bias) Lds::run<false, false, EPI_BF16_B>(g, st);
        else if (residual) Lds::run<false, false, EPI_BF16_R>(g, st);
        else Lds::run<false, false, EPI_BF16>(g, st);
        return;
    }
    Cfg::run<false, false, EPI_BF16>(out, inp, w, bias, residual, M, N, K, K, K, N, 1, K, 0,
                                     nullptr, 0, st);
}

// out = inp . w^T + bias and out_gelu = gelu(out) (both bf16) in one pass;
// false (nothing launched) when K is not a multiple of the tile depth or
// there is no bias.
bool gemm_bf16_fwd_gelu(bf16* out, bf16* out_gelu, const bf16* inp, const bf16* w,
                        const bf16* bias, int M, int K, int N, hipStream_t st) {
    if (K % LDS_BK != 0 || !bias) return false;
    prepare_lds_kernels();
    Lds::run<false, false, EPI_BF16_GELU>(
        single({inp, w, out, out_gelu, bias, nullptr, nullptr, M, N, K}), st);
    return true;
}

// dinp[M,K] = dout[M,N] . w[N,K]
void gemm_bf16_bwd_dx(bf16* dinp, const bf16* dout, const bf16* w, int M, int N, int K,
                      hipStream_t st) {
    if (N % LDS_BK == 0) {
        prepare_lds_kernels();
        Lds::run<false, true, EPI_BF16>(
            single({dout, w, dinp, nullptr, nullptr, nullptr, nullptr, M, K, N}), st);
        return;
    }
    Cfg::run<false, true, EPI_BF16>(dinp, dout, w, nullptr, nullptr, M, K, N, N, K, K, 1, N, 0,
                                    nullptr, 0, st);
}

// dinp = (dout . w) * gelu'(pre), pre [M, K] the bf16 pre-activation; false
// (nothing launched) when N is not a multiple of the tile depth.
bool gemm_bf16_bwd_dx_dgelu(bf16* dinp, const bf16* dout, const bf16* w, const bf16* pre, int M,
                            int N, int K, hipStream_t st) {
    if (N % LDS_BK != 0) return false;
    prepare_lds_kernels();
    Lds::run<false, true, EPI_BF16_DGELU>(
        single({dout, w, dinp, nullptr, nullptr, pre, nullptr, M, K, N}), st);
    return true;
}

// Splits of the B*T reduction of a single weight gradient [N, K]. Cost model,
// in units of one block's time per reduction row: rounds of resident blocks
// times rows per split, plus the fp32 partials' HBM round trip (8 bytes per
// output per split, about 8e-5 rows each at HBM speed) and the reduce launch.
// More splits must win by 5%. At most 16 splits of at least 512 rows.
static int dw_splits(int M, int N, int K) {
    const int tiles = Lds::tiles(N, K);
    int smax = M / 512;
    if (smax > 16) smax = 16;
    int best = 1;
    double best_cost = 0.0;
    for (int s = 1; s <= (smax < 1 ? 1 : smax); s++) {
        const double rounds = ceil_div(tiles * s, BLOCK_SLOTS);
        double cost = rounds * ceil_div(M, s);
        if (s > 1) cost += 8e-5 * s * (double)N * K + 200.0;
        if (s == 1 || cost < 0.95 * best_cost) {
            best_cost = cost;
            best = s;
        }
    }
    return best;
}

int64_t gemm_dw_workspace_floats(int M, int N, int K) {
    const int s = dw_splits(M, N, K);
    return s > 1 ? (int64_t)s * N * (K + 1) : 0;
}

// dw[N,K] (fp32) = dout[M,N]^T . inp[M,K] and, if db != nullptr,
// db[N] = sum_m dout[m, :]; ws: gemm_dw_workspace_floats(M,N,K) floats
// (split partials of dw, then of db).
void gemm_bf16_bwd_dw(float* dw, float* db, const bf16* dout, const bf16* inp, int M, int N,
                      int K, float* ws, hipStream_t st) {
    const int s = dw_splits(M, N, K);
    const int kchunk = ceil_div(ceil_div(M, s), LDS_BK) * LDS_BK;
    const int splits = ceil_div(M, kchunk);
    const int64_t n = (int64_t)N * K;
    float* wsdb = ws + (int64_t)splits * n;
    if (M % LDS_BK != 0) {
        // register-staged kernel: splits along grid z
        if (splits == 1) {
            Cfg::run<true, true, EPI_F32>(dw, dout, inp, nullptr, nullptr, N, K, M, N, K, K, 1, M,
                                          0, db, 0, st);
            return;
        }
        Cfg::run<true, true, EPI_F32>(ws, dout, inp, nullptr, nullptr, N, K, M, N, K, K, splits,
                                      kchunk, n, db ? wsdb : nullptr, N, st);
    } else {
        prepare_lds_kernels();
        if (splits == 1) {
            Lds::run<true, true, EPI_F32>(
                single({dout, inp, dw, nullptr, nullptr, nullptr, db, N, K, M}), st);
            return;
        }
        // each split is one problem of the group: rows z*kchunk .. of dout and inp
        GemmGroup g;
        g.count = splits;
        g.first_tile[0] = 0;
        for (int z = 0; z < splits; z++) {
            const int rows = z + 1 < splits ? kchunk : M - z * kchunk;
            g.p[z] = GemmProblem{dout + (int64_t)z * kchunk * N, inp + (int64_t)z * kchunk * K,
                                 ws + z * n, nullptr, nullptr, nullptr,
                                 db ? wsdb + (int64_t)z * N : nullptr, N, K, rows};
            g.first_tile[z + 1] = g.first_tile[z] + Lds::tiles(N, K);
        }
        Lds::run<true, true, EPI_F32>(g, st);
    }
    split_reduce_kernel<<<ceil_div(n / 4, 256), 256, 0, st>>>(dw, ws, splits, n);
    if (db) split_reduce_kernel<<<ceil_div(N / 4, 256), 256, 0, st>>>(db, wsdb, splits, N);
}

// Grouped weight gradients (see matmul_bwd_dw_batch); false (nothing
// launched) when M is not a multiple of the tile depth.
bool gemm_bf16_bwd_dw_batch(const DwTask* tasks, int n, int M, hipStream_t st) {
    if (M % LDS_BK != 0) return false;
    prepare_lds_kernels();
    for (int t0 = 0; t0 < n; t0 += GROUP_MAX) {
        GemmGroup g;
        g.count = n - t0 < GROUP_MAX ? n - t0 : GROUP_MAX;
        g.first_tile[0] = 0;
        for (int q = 0; q < g.count; q++) {
            const DwTask& t = tasks[t0 + q];
            g.p[q] = GemmProblem{(const bf16*)t.dout, (const bf16*)t.inp, t.dw, nullptr, nullptr,
                                 nullptr, t.db, t.N, t.K, M};
            g.first_tile[q + 1] = g.first_tile[q] + Lds::tiles(t.N, t.K);
        }
        Lds::run<true, true, EPI_F32>(g, st);
    }
    return true;
}

// out[M,N] (bf16) = (qx[M,K] . qw[N,K]^T) / (scales[0] scales[1]) (+ bias[N]),
// qx and qw E4M3 codes; false (nothing launched) unless K is a multiple of
// 128 codes (one tile depth) and N of 8.
bool gemm_fp8_fwd(bf16* out, const uint8_t* qx, const uint8_t* qw, const float* scales,
                  const bf16* bias, int M, int N, int K, hipStream_t st) {
    if (K % (2 * LDS_BK) != 0 || N % 8 != 0) return false;
    prepare_lds_kernels();
    GemmProblem p{reinterpret_cast<const bf16*>(qx), reinterpret_cast<const bf16*>(qw), out,
                  nullptr, bias, nullptr, nullptr, M, N, K / 2};
    p.scales = scales;
    if (bias)
        Lds::run<false, false, EPI_FP8_B>(single(p), st);
    else
        Lds::run<false, false, EPI_FP8>(single(p), st);
    return true;
}
