// Matrix products of the linear layers: forward y = x W^T + b (+ residual),
// backward dx = dy W and dW = dy^T x, and the bias gradient.
//
// This file holds the general-stride kernel that serves every layout and both
// storage types: out[i, j] = sum_p X(i, p) Y(j, p) with
// X(i, p) = X[i*sxi + p*sxp] and Y(j, p) = Y[j*syj + p*syp]; 64x64 output tiles,
// K-steps of 16 staged in LDS, fp32 accumulation, 4x4 outputs per thread.
#include <type_traits>

#include "kernels.h"

#define GT_M 64
#define GT_N 64
#define GT_K 16

template <typename TX, typename TY, typename TO, typename TR>
__global__ __launch_bounds__(256) void gemm_generic_kernel(
    TO* __restrict__ out, const TX* __restrict__ X, const TY* __restrict__ Y,
    const TR* __restrict__ bias, const TR* __restrict__ residual, int I, int J, int P,
    int64_t sxi, int64_t sxp, int64_t syj, int64_t syp, int64_t ldo) {
    __shared__ float As[GT_K][GT_M + 4];
    __shared__ float Bs[GT_K][GT_N + 4];
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const int i0 = blockIdx.y * GT_M, j0 = blockIdx.x * GT_N;
    float acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; r++)
#pragma unroll
        for (int c = 0; c < 4; c++) acc[r][c] = 0.f;

    for (int p0 = 0; p0 < P; p0 += GT_K) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int e = tid + 256 * q;
            // walk the operand along whichever index is contiguous in memory
            int il, pl;
            if (sxp == 1) {
                pl = e % GT_K;
                il = e / GT_K;
            } else {
                il = e % GT_M;
                pl = e / GT_M;
            }
            int i = i0 + il, p = p0 + pl;
            As[pl][il] = (i < I && p < P) ? to_f32(X[i * sxi + p * sxp]) : 0.f;
            int jl;
            if (syp == 1) {
                pl = e % GT_K;
                jl = e / GT_K;
            } else {
                jl = e % GT_N;
                pl = e / GT_N;
            }
            int j = j0 + jl;
            p = p0 + pl;
            Bs[pl][jl] = (j < J && p < P) ? to_f32(Y[j * syj + p * syp]) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int pl = 0; pl < GT_K; pl++) {
            float a[4], b[4];
#pragma unroll
            for (int r = 0; r < 4; r++) a[r] = As[pl][ty * 4 + r];
#pragma unroll
            for (int c = 0; c < 4; c++) b[c] = Bs[pl][tx * 4 + c];
#pragma unroll
            for (int r = 0; r < 4; r++)
#pragma unroll
                for (int c = 0; c < 4; c++) acc[r][c] += a[r] * b[c];
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int i = i0 + ty * 4 + r;
        if (i >= I) continue;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const int j = j0 + tx * 4 + c;
            if (j >= J) continue;
            float v = acc[r][c];
            if (bias) v += to_f32(bias[j]);
            if (residual) v += to_f32(residual[i * ldo + j]);
            out[i * ldo + j] = from_f32<TO>(v);
        }
    }
}

template <typename TX, typename TY, typename TO, typename TR>
static void gemm_generic(TO* out, const TX* X, const TY* Y, const TR* bias, const TR* residual,
                         int I, int J, int P, int64_t sxi, int64_t sxp, int64_t syj, int64_t syp,
                         int64_t ldo, hipStream_t st) {
    dim3 grid(ceil_div(J, GT_N), ceil_div(I, GT_M));
    gemm_generic_kernel<TX, TY, TO, TR><<<grid, 256, 0, st>>>(out, X, Y, bias, residual, I, J, P,
                                                              sxi, sxp, syj, syp, ldo);
}

// bf16 storage runs on the matrix cores (gemm_mfma.hip); fp32 storage uses the
// general-stride kernel above.
template <typename T>
void matmul_fwd(T* out, const T* inp, const T* w, const T* bias, const T* residual, int M,
                int K, int N, hipStream_t st) {
    // out[m, n] = sum_k inp[m, k] w[n, k]
    if constexpr (std::is_same<T, bf16>::value)
        gemm_bf16_fwd(out, inp, w, bias, residual, M, K, N, st);
    else
        gemm_generic<T, T, T, T>(out, inp, w, bias, residual, M, N, K, K, 1, K, 1, N, st);
}

template <typename T>
void matmul_bwd_dx(T* dinp, const T* dout, const T* w, int M, int N, int K, hipStream_t st) {
    // dinp[m, k] = sum_n dout[m, n] w[n, k]
    if constexpr (std::is_same<T, bf16>::value)
        gemm_bf16_bwd_dx(dinp, dout, w, M, N, K, st);
    else
        gemm_generic<T, T, T, T>(dinp, dout, w, nullptr, nullptr, M, K, N, N, 1, 1, K, K, st);
}

// bf16: the GELU rides in the product's epilogue when the shape allows it;
// otherwise (and for fp32) the product is followed by the elementwise kernel.
template <typename T>
void matmul_fwd_gelu(T* out, T* out_gelu, const T* inp, const T* w, const T* bias, int M, int K,
                     int N, hipStream_t st) {
    if constexpr (std::is_same<T, bf16>::value)
        if (gemm_bf16_fwd_gelu(out, out_gelu, inp, w, bias, M, K, N, st)) return;
    matmul_fwd<T>(out, inp, w, bias, nullptr, M, K, N, st);
    gelu_fwd<T>(out_gelu, out, (int64_t)M * N, st);
}

template <typename T>
void matmul_bwd_dx_dgelu(T* dinp, const T* dout, const T* w, const T* pre, int M, int N, int K,
                         hipStream_t st) {
    if constexpr (std::is_same<T, bf16>::value)
        if (gemm_bf16_bwd_dx_dgelu(dinp, dout, w, pre, M, N, K, st)) return;
    matmul_bwd_dx<T>(dinp, dout, w, M, N, K, st);
    gelu_bwd<T>(dinp, pre, dinp, (int64_t)M * K, st);
}

template <typename T>
void matmul_bwd_dw(float* dw, float* db, const T* dout, const T* inp, int M, int N, int K,
                   float* ws, float* bias_partials, hipStream_t st) {
    // dw[n, k] = sum_m dout[m, n] inp[m, k]; db[n] = sum_m dout[m, n]
    if constexpr (std::is_same<T, bf16>::value) {
        gemm_bf16_bwd_dw(dw, db, dout, inp, M, N, K, ws, st);
    } else {
        gemm_generic<T, T, float, float>(dw, dout, inp, nullptr, nullptr, N, K, M, 1, N, 1, K, K,
                                         st);
        if (db) bias_bwd<T>(db, dout, M, N, bias_partials, st);
    }
}

template <typename T>
void matmul_bwd_dw_batch(const DwTask* tasks, int n, int M, float* ws, float* bias_partials,
                         hipStream_t st) {
    if constexpr (std::is_same<T, bf16>::value)
        if (gemm_bf16_bwd_dw_batch(tasks, n, M, st)) return;
    for (int i = 0; i < n; i++)
        matmul_bwd_dw<T>(tasks[i].dw, tasks[i].db, (const T*)tasks[i].dout,
                         (const T*)tasks[i].inp, M, tasks[i].N, tasks[i].K, ws, bias_partials, st);
}

// Bias gradient db[n] = sum_m dout[m, n], deterministic two-stage column sum.
// Stage 1: a block covers 256 columns (32 threads x 8 columns, 16-byte loads)
// and BB_ROWS rows split over 8 row phases; the phases are combined in order
// through LDS into one partial row. Stage 2 sums the partial rows in order.
#define BB_ROWS 128

template <typename T>
__global__ __launch_bounds__(256) void bias_bwd_partial_kernel(float* __restrict__ partials,
                                                               const T* __restrict__ dout,
                                                               int M, int N) {
    __shared__ float red[8][256];
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const int n = blockIdx.x * 256 + tx * 8;
    const int m0 = blockIdx.y * BB_ROWS, m1 = min(M, m0 + BB_ROWS);
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (n < N)
        for (int m = m0 + ty; m < m1; m += 8) {
            float v[8];
            load8(dout + (int64_t)m * N + n, v);
#pragma unroll
            for (int k = 0; k < 8; k++) s[k] += v[k];
        }
#pragma unroll
    for (int k = 0; k < 8; k++) red[ty][tx * 8 + k] = s[k];
    __syncthreads();
    const int c = threadIdx.x, nc = blockIdx.x * 256 + c;
    if (nc < N) {
        float t = 0.f;
#pragma unroll
        for (int r = 0; r < 8; r++) t += red[r][c];
        partials[(int64_t)blockIdx.y * N + nc] = t;
    }
}

__global__ __launch_bounds__(256) void bias_bwd_reduce_kernel(float* __restrict__ db,
                                                              const float* __restrict__ partials,
                                                              int nrows, int N) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    float s = 0.f;
    for (int r = 0; r < nrows; r++) s += partials[(int64_t)r * N + n];
    db[n] = s;
}

int64_t bias_bwd_partials(int M, int N) { return (int64_t)ceil_div(M, BB_ROWS) * N; }

template <typename T>
void bias_bwd(float* db, const T* dout, int M, int N, float* partials, hipStream_t st) {
    const int nr = ceil_div(M, BB_ROWS);
    dim3 grid(ceil_div(N, 256), nr);
    bias_bwd_partial_kernel<T><<<grid, 256, 0, st>>>(partials, dout, M, N);
    bias_bwd_reduce_kernel<<<ceil_div(N, 256), 256, 0, st>>>(db, partials, nr, N);
}

#define INST(T)                                                                                \
    template void matmul_fwd<T>(T*, const T*, const T*, const T*, const T*, int, int, int,      \
                                hipStream_t);                                                  \
    template void matmul_bwd_dx<T>(T*, const T*, const T*, int, int, int, hipStream_t);         \
    template void matmul_fwd_gelu<T>(T*, T*, const T*, const T*, const T*, int, int, int,       \
                                     hipStream_t);                                             \
    template void matmul_bwd_dx_dgelu<T>(T*, const T*, const T*, const T*, int, int, int,       \
                                         hipStream_t);                                         \
    template void matmul_bwd_dw<T>(float*, float*, const T*, const T*, int, int, int, float*,  \
                                   float*, hipStream_t);                                       \
    template void bias_bwd<T>(float*, const T*, int, int, float*, hipStream_t);                \
    template void matmul_bwd_dw_batch<T>(const DwTask*, int, int, float*, float*, hipStream_t);
INST(float)
INST(bf16)
