// Host-side launchers of the gfx950 kernels. Each enqueues its kernel(s) on
// `st` and returns immediately. T is the activation storage type (float or
// bf16); all arithmetic is fp32. Shapes are validated by the caller (gpt2.hip).
#pragma once

#include "common.h"

// ---- encoder (token + position embedding) ---------------------------------
// out[b,t,:] = wte[tok[b,t],:] + wpe[t,:]; an id outside [0,V) produces a zero
// row and raises *err to at least `tag` (the caller's forward number, >= 1).
template <typename T>
void encoder_fwd(T* out, const int32_t* tok, const T* wte, const T* wpe, int B, int Tn, int C,
                 int V, int* err, int tag, hipStream_t st);
// dwte[tok[b,t],:] += dout[b,t,:] (deterministic: the positions of one token
// are summed in increasing order, in a fixed grouping); dwpe[t,:] =
// sum_b dout[b,t,:], rows >= Tn = 0. ws: encoder_bwd_workspace_bytes(B*Tn,
// Vp, C) bytes, 256-byte aligned. C % 8 == 0.
int64_t encoder_bwd_workspace_bytes(int BT, int Vp, int C);
template <typename T>
void encoder_bwd(float* dwte, float* dwpe, const T* dout, const int32_t* tok, int B, int Tn,
                 int C, int Vp, int maxT, void* ws, hipStream_t st);

// ---- LayerNorm --------------------------------------------------------------
template <typename T>
void layernorm_fwd(T* out, float* mean, float* rstd, const T* inp, const T* w, const T* b,
                   int N, int C, hipStream_t st);
// Backward in two parts. layernorm_bwd_rows: dinp = dx (+ dadd[...] when
// dadd != nullptr; dadd may alias dinp), and the per-block partial sums of
// dw, db into LayerNorm slot `slot` of the workspace. layernorm_bwd_reduce:
// the dw, db of slots 0 .. b.count-1 (task i writes slot i's sums), summed
// in a fixed order, all in two launches. partials: fp32 workspace of
// layernorm_bwd_partials(C, count) floats; every slot of one reduce has the
// same N.
#define LN_RED_MAX 128
struct LnRedTask {
    float* dw;
    float* db;
};
struct LnRedBatch {
    int count;
    LnRedTask t[LN_RED_MAX];
};
template <typename T>
void layernorm_bwd_rows(T* dinp, const T* dadd, const T* dout, const T* inp, const T* w,
                        const float* mean, const float* rstd, int N, int C, float* partials,
                        int slot, hipStream_t st);
void layernorm_bwd_reduce(const LnRedBatch& b, int N, int C, float* partials, int count,
                          hipStream_t st);
int64_t layernorm_bwd_partials(int C, int count);

// ---- matmul -----------------------------------------------------------------
// out[M,N] = inp[M,K] . w[N,K]^T (+ bias[N]) (+ residual[M,N])
template <typename T>
void matmul_fwd(T* out, const T* inp, const T* w, const T* bias, const T* residual, int M,
                int K, int N, hipStream_t st);
// dinp[M,K] = dout[M,N] . w[N,K]
// out = inp . w^T + bias, out_gelu = gelu(out)
template <typename T>
void matmul_fwd_gelu(T* out, T* out_gelu, const T* inp, const T* w, const T* bias, int M, int K,
                     int N, hipStream_t st);
// dinp[M,K] = (dout[M,N] . w[N,K]) * gelu'(pre[M,K])
template <typename T>
void matmul_bwd_dx_dgelu(T* dinp, const T* dout, const T* w, const T* pre, int M, int N, int K,
                         hipStream_t st);
template <typename T>
void matmul_bwd_dx(T* dinp, const T* dout, const T* w, int M, int N, int K, hipStream_t st);
// dw[N,K] = dout[M,N]^T . inp[M,K] (fp32, written)
template <typename T>
// and, if db != nullptr, db[N] = sum_m dout[m,:] (fp32, written).
// ws: gemm_dw_workspace_floats(M, N, K) floats (bf16 storage splits the M
// reduction); bias_partials: bias_bwd_partials(M, N) floats (fp32 storage).
void matmul_bwd_dw(float* dw, float* db, const T* dout, const T* inp, int M, int N, int K,
                   float* ws, float* bias_partials, hipStream_t st);
// the bf16 matrix-core kernels behind the three matmul entry points above
void gemm_bf16_fwd(bf16* out, const bf16* inp, const bf16* w, const bf16* bias,
                   const bf16* residual, int M, int K, int N, hipStream_t st);
void gemm_bf16_bwd_dx(bf16* dinp, const bf16* dout, const bf16* w, int M, int N, int K,
                      hipStream_t st);
bool gemm_bf16_fwd_gelu(bf16* out, bf16* out_gelu, const bf16* inp, const bf16* w,
                        const bf16* bias, int M, int K, int N, hipStream_t st);
bool gemm_bf16_bwd_dx_dgelu(bf16* dinp, const bf16* dout, const bf16* w, const bf16* pre, int M,
                            int N, int K, hipStream_t st);
void gemm_bf16_bwd_dw(float* dw, float* db, const bf16* dout, const bf16* inp, int M, int N,
                      int K, float* ws, hipStream_t st);
int64_t gemm_dw_workspace_floats(int M, int N, int K);
// db[N] = sum_m dout[m,:] (fp32, written); partials: bias_bwd_partials(M, N) floats
template <typename T>
void bias_bwd(float* db, const T* dout, int M, int N, float* partials, hipStream_t st);
int64_t bias_bwd_partials(int M, int N);

// A batch of independent weight gradients over the same M rows:
// dw_t[N_t, K_t] = dout_t[M, N_t]^T . inp_t[M, K_t] (fp32, written) and
// db_t[N_t] = sum_m dout_t[m, :] when db_t != nullptr. bf16 storage runs them
// as grouped launches of up to 52 products without reduction splits (M a
// multiple of 64); otherwise one matmul_bwd_dw per task with ws / partials.
struct DwTask {
    const void* dout;
    const void* inp;
    float* dw;
    float* db;
    int N, K;
};
template <typename T>
void matmul_bwd_dw_batch(const DwTask* tasks, int n, int M, float* ws, float* bias_partials,
                         hipStream_t st);
bool gemm_bf16_bwd_dw_batch(const DwTask* tasks, int n, int M, hipStream_t st);

// ---- attention ---------------------------------------------------------------
// Causal multi-head attention on qkv (B,T,3C): out (B,T,C), lse (B,NH,T).
template <typename T>
void attention_fwd(T* out, float* lse, const T* qkv, int B, int Tn, int C, int NH,
                   hipStream_t st);
// dqkv (B,T,3C) written; work: fp32 workspace of 2 * B * NH * Tn floats (the
// rows' D = sum dO o O, then their log-sum-exp in base 2).
template <typename T>
void attention_bwd(T* dqkv, const T* dout, const T* qkv, const T* out, const float* lse,
                   float* work, int B, int Tn, int C, int NH, hipStream_t st);

// the bf16 matrix-core kernels for head size 64 behind the two entry points
// above, used when flash_attention_fits(Tn, C)
bool flash_attention_fits(int Tn, int C);
void flash_attention_fwd(bf16* out, float* lse, const bf16* qkv, int B, int Tn, int C, int NH,
                         hipStream_t st);
void flash_attention_bwd(bf16* dqkv, const bf16* dout, const bf16* qkv, const bf16* out,
                         const float* lse, float* work, int B, int Tn, int C, int NH,
                         hipStream_t st);

// ---- elementwise --------------------------------------------------------------
template <typename T>
void gelu_fwd(T* out, const T* inp, int64_t n, hipStream_t st);
// dinp = gelu'(inp) * dout (written; dinp may alias dout)
template <typename T>
void gelu_bwd(T* dinp, const T* inp, const T* dout, int64_t n, hipStream_t st);
void fill_zero_f32(float* p, int64_t n, hipStream_t st);
void fill_zero_i32(int* p, int64_t n, hipStream_t st);
void round_to_bf16(bf16* out, const float* in, int64_t n, hipStream_t st);

// ---- classifier ----------------------------------------------------------------
// Per row n: lse over the V real columns, losses[n] = lse - z[target];
// logits overwritten by dz = (softmax - onehot) * dloss (0 on padded columns).
template <typename T>
void classifier_fwd(T* logits, float* losses, const int32_t* targets, int N, int V, int Vp,
                    float dloss, int* err, int tag, hipStream_t st);
// *out = mean of losses[0..n) (fixed summation order)
void loss_mean(float* out, const float* losses, int n, hipStream_t st);

// ---- AdamW ------------------------------------------------------------------
// gnorm: device scalar ||g|| (or nullptr: no clipping); g is scaled by
// clip / ||g|| when ||g|| > clip.
void adamw(float* theta, const float* g, float* m, float* v, bf16* theta_bf16, int64_t n,
           float lr, float b1, float b2, float eps, float wd, float c1, float c2,
           const float* gnorm, float clip, hipStream_t st);
// out[0] = sqrt(sum g_i^2), deterministic; part: grad_norm_workspace_floats().
int64_t grad_norm_workspace_floats();
void grad_norm(float* out, float* part, const float* g, int64_t n, hipStream_t st);

// ---- FP8 (E4M3) products ------------------------------------------------------
// *scale = 448 / max|x_i| (1 for an all-zero x), deterministic; work:
// fp8_scale_workspace_floats() floats. x 16-byte aligned.
int64_t fp8_scale_workspace_floats();
void fp8_scale(float* scale, float* work, const bf16* x, int64_t n, hipStream_t st);
// q_i = E4M3(x_i * *scale), round to nearest even. q, x 16-byte aligned.
void fp8_quantize(uint8_t* q, const bf16* x, const float* scale, int64_t n, hipStream_t st);
// out[M,N] (bf16) = (qx[M,K] . qw[N,K]^T) / (scales[0] scales[1]) (+ bias[N]);
// false (nothing launched) unless K % 128 == 0 and N % 8 == 0.
bool gemm_fp8_fwd(bf16* out, const uint8_t* qx, const uint8_t* qw, const float* scales,
                  const bf16* bias, int M, int N, int K, hipStream_t st);
