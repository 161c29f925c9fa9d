// The bf16 matrix products of the linear layers:
//   forward  y  = x W^T      X = x  (p-contig), Y = W  (p-contig)
//   backward dx = dy W       X = dy (p-contig), Y = W  (row-contig)
//   backward dW = dy^T x     X = dy (row-contig), Y = x (row-contig)
// Shapes whose reduction length is a multiple of 64 run on the direct-to-LDS
// pipelined kernel (gemm_lds.h); others on the register-staged kernel
// (gemm_mfma.h). The weight gradient reduces over all B*T rows; its few output
// tiles are split along that reduction (grid z), each split writing an fp32
// partial that a second kernel sums in split order (deterministic). The bias
// gradient (column sums of dy) rides along in the same kernel.
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
// matrix products. 16384-row outputs of width 768, 2304 and 3072 make exactly
// 1, 3 and 4 rounds of 512 blocks.
using Cfg = GemmCfg<128, 128, 32, 2, 2, 16>;      // register-staged fallback
using FwdCfg = GemmLds<128, 192, 64, 2, 2, 8, 2>;  // y = x W^T and dx = dy W
using DwCfg = GemmLds<128, 192, 64, 2, 2, 8, 2>;   // dW = dy^T x
constexpr int LDS_BK = 64;
constexpr int BLOCK_SLOTS = 2 * 256;  // resident blocks: two per CU on 256 CUs

// The direct-to-LDS kernels use more than 64 KB of LDS; raise their limits once.
static void prepare_lds_kernels() {
    static std::once_flag once;
    std::call_once(once, [] {
        (void)FwdCfg::prepare<false, false, EPI_BF16>();
        (void)FwdCfg::prepare<false, false, EPI_BF16_GELU>();
        (void)FwdCfg::prepare<false, true, EPI_BF16>();
        (void)FwdCfg::prepare<false, true, EPI_BF16_DGELU>();
        (void)DwCfg::prepare<true, true, EPI_F32>();
        (void)DwCfg::prepare_dw_group();
    });
}

// out[M,N] = inp[M,K] . w[N,K]^T (+ bias) (+ residual)
void gemm_bf16_fwd(bf16* out, const bf16* inp, const bf16* w, const bf16* bias,
                   const bf16* residual, int M, int K, int N, hipStream_t st) {
    if (K % LDS_BK == 0) {
        prepare_lds_kernels();
        FwdCfg::run<false, false, EPI_BF16>(out, inp, w, bias, residual, M, N, K, K, K, N, 1, K,
                                            0, nullptr, 0, st);
        return;
    }
    Cfg::run<false, false, EPI_BF16>(out, inp, w, bias, residual, M, N, K, K, K, N, 1, K, 0,
                                     nullptr, 0, st);
}

// dinp[M,K] = dout[M,N] . w[N,K]
void gemm_bf16_bwd_dx(bf16* dinp, const bf16* dout, const bf16* w, int M, int N, int K,
                      hipStream_t st) {
    if (N % LDS_BK == 0) {
        prepare_lds_kernels();
        FwdCfg::run<false, true, EPI_BF16>(dinp, dout, w, nullptr, nullptr, M, K, N, N, K, K, 1,
                                           N, 0, nullptr, 0, st);
        return;
    }
    Cfg::run<false, true, EPI_BF16>(dinp, dout, w, nullptr, nullptr, M, K, N, N, K, K, 1, N, 0,
                                    nullptr, 0, st);
}

// out = inp . w^T + bias and out_gelu = gelu(out) (both bf16) in one pass;
// false (nothing launched) when K is not a multiple of the tile depth.
bool gemm_bf16_fwd_gelu(bf16* out, bf16* out_gelu, const bf16* inp, const bf16* w,
                        const bf16* bias, int M, int K, int N, hipStream_t st) {
    if (K % LDS_BK != 0) return false;
    prepare_lds_kernels();
    FwdCfg::run<false, false, EPI_BF16_GELU>(out, inp, w, bias, nullptr, M, N, K, K, K, N, 1, K, 0,
                                             nullptr, 0, st, out_gelu);
    return true;
}

// dinp = (dout . w) * gelu'(pre), pre [M, K] the bf16 pre-activation; false
// (nothing launched) when N is not a multiple of the tile depth.
bool gemm_bf16_bwd_dx_dgelu(bf16* dinp, const bf16* dout, const bf16* w, const bf16* pre, int M,
                            int N, int K, hipStream_t st) {
    if (N % LDS_BK != 0) return false;
    prepare_lds_kernels();
    FwdCfg::run<false, true, EPI_BF16_DGELU>(dinp, dout, w, nullptr, pre, M, K, N, N, K, K, 1, N, 0,
                                             nullptr, 0, st);
    return true;
}

// Splits of the B*T reduction of a weight gradient [N, K]. Cost model, in
// units of one block's time per reduction row: rounds of resident blocks times
// rows per split, plus the fp32 partials' HBM round trip (8 bytes per output
// per split, about 8e-5 rows each at HBM speed) and the reduce launch. More
// splits must win by 5%. At most 16 splits of at least 512 rows.
static int dw_splits(int M, int N, int K) {
    const int tiles = ceil_div(N, DwCfg::bm) * ceil_div(K, DwCfg::bn);
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
    const bool lds = M % LDS_BK == 0;
    if (lds) prepare_lds_kernels();
    auto launch = [&](void* out, int splits, int kchunk, int64_t stride, float* rs,
                      int64_t rs_stride) {
        if (lds)
            DwCfg::run<true, true, EPI_F32>(out, dout, inp, nullptr, nullptr, N, K, M, N, K, K,
                                            splits, kchunk, stride, rs, rs_stride, st);
        else
            Cfg::run<true, true, EPI_F32>(out, dout, inp, nullptr, nullptr, N, K, M, N, K, K,
                                          splits, kchunk, stride, rs, rs_stride, st);
    };
    if (s == 1) {
        launch(dw, 1, M, 0, db, 0);
        return;
    }
    const int kchunk = ceil_div(ceil_div(M, s), LDS_BK) * LDS_BK;
    const int splits = ceil_div(M, kchunk);
    const int64_t n = (int64_t)N * K;
    float* wsdb = ws + (int64_t)splits * n;
    launch(ws, splits, kchunk, n, db ? wsdb : nullptr, N);
    split_reduce_kernel<<<ceil_div(n / 4, 256), 256, 0, st>>>(dw, ws, splits, n);
    if (db) split_reduce_kernel<<<ceil_div(N / 4, 256), 256, 0, st>>>(db, wsdb, splits, N);
}

// Grouped weight gradients (see matmul_bwd_dw_batch); false (nothing
// launched) when M is not a multiple of the tile depth.
bool gemm_bf16_bwd_dw_batch(const DwTask* tasks, int n, int M, hipStream_t st) {
    if (M % LDS_BK != 0) return false;
    prepare_lds_kernels();
    for (int t0 = 0; t0 < n; t0 += GROUP_MAX) {
        DwGroup g;
        g.count = n - t0 < GROUP_MAX ? n - t0 : GROUP_MAX;
        g.R = M;
        g.first_tile[0] = 0;
        for (int q = 0; q < g.count; q++) {
            const DwTask& t = tasks[t0 + q];
            g.p[q] = DwProblem{(const bf16*)t.dout, (const bf16*)t.inp, t.dw, t.db, t.N, t.K};
            g.first_tile[q + 1] =
                g.first_tile[q] + ceil_div(t.N, DwCfg::bm) * ceil_div(t.K, DwCfg::bn);
        }
        DwCfg::run_dw_group(g, st);
    }
    return true;
}
