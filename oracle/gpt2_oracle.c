/*
 * gpt2_oracle.c -- plain CPU oracle for one GPT-2 training step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or execute this file or anything built from it. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg use it. It shares no
 * code with the GPU library.
 *
 * What it computes: the training step of GPT-2 as llm.c defines it -- page
 * "Building GPT-2 from scratch", exercise table rows A1 (forward pass "from the
 * matrix multiply up") and A2 (every gradient derived by hand, AdamW); page
 * "llm.c: Large Language Model Training in Pure C/CUDA Without Dependencies",
 * sections "Tensor Memory Layout" (flat row-major arrays) and "Exact Analytical
 * Backward Pass" (LayerNorm, MatMul and Softmax gradients); the talk "llm.c's
 * Origin and the Future of LLM Compilers", chapter "Deconstructing PyTorch
 * Abstractions" (LayerNorm forward and backward over bare float arrays).
 * The pages print no equations; every formula below is the standard
 * definition of the named operation, written out with plain loops:
 *
 *   - no blocking, no fusion, no online softmax: attention materialises the
 *     full causal T x T probability matrix;
 *   - sums run in natural index order; OpenMP only splits independent
 *     outputs between threads, so results do not depend on the thread count;
 *   - `real` is double unless built with -DREAL=float.
 *
 * Readings where the pages are silent (both the oracle and the GPU path follow
 * them): LayerNorm eps 1e-5 with the biased variance; GELU in its tanh form;
 * attention scale 1/sqrt(hs) with the diagonal kept; qkv as one (3C, C)
 * weight with row blocks [Q; K; V] and head h on columns h*hs..h*hs+hs-1 of
 * each block; weights stored (out, in) so y = x W^T + b; softmax and loss over
 * the real vocabulary V only, padded logit columns get zero gradient; loss is
 * the mean over all B*T positions; backward overwrites parameter gradients;
 * AdamW with bias correction from t = 1, eps outside the square root, decay
 * lr*wd*theta applied uniformly to the whole flat array.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared [-DREAL=float]
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef REAL
#define REAL double
#endif
typedef REAL real;

#define NUM_PARAM_TENSORS 16
#define LN_EPS 1e-5
#define ORACLE_PI 3.14159265358979323846

typedef struct {
    int V, Vp, maxT, C, L, NH, B, T;
} oracle_config;

/* ------------------------------------------------------------------------ */
/* Operations. Each follows the definition named in its comment.            */
/* ------------------------------------------------------------------------ */

/* Token + position embedding: out[b,t,:] = wte[inp[b,t],:] + wpe[t,:]. */
void oracle_encoder_forward(real* out, const int* inp, const real* wte,
                            const real* wpe, int B, int T, int C) {
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) {
            const real* we = wte + (int64_t)inp[b * T + t] * C;
            const real* pe = wpe + (int64_t)t * C;
            real* o = out + ((int64_t)b * T + t) * C;
            for (int i = 0; i < C; i++) o[i] = we[i] + pe[i];
        }
}

/* Gradient of the embedding sum: every position adds its gradient row to the
 * wte row of its token and to the wpe row of its position. */
void oracle_encoder_backward(real* dwte, real* dwpe, const real* dout,
                             const int* inp, int B, int T, int C) {
#pragma omp parallel for
    for (int i = 0; i < C; i++)
        for (int b = 0; b < B; b++)
            for (int t = 0; t < T; t++) {
                real d = dout[((int64_t)b * T + t) * C + i];
                dwte[(int64_t)inp[b * T + t] * C + i] += d;
                dwpe[(int64_t)t * C + i] += d;
            }
}

/* LayerNorm over the last axis: mu = mean(x), var = mean((x-mu)^2) (biased),
 * r = 1/sqrt(var + eps), y = (x - mu) * r * w + b. Saves mu and r. */
void oracle_layernorm_forward(real* out, real* mean, real* rstd, const real* inp,
                              const real* w, const real* b, int N, int C) {
#pragma omp parallel for
    for (int n = 0; n < N; n++) {
        const real* x = inp + (int64_t)n * C;
        real m = 0;
        for (int i = 0; i < C; i++) m += x[i];
        m = m / C;
        real v = 0;
        for (int i = 0; i < C; i++) {
            real d = x[i] - m;
            v += d * d;
        }
        v = v / C;
        real s = 1 / sqrt(v + (real)LN_EPS);
        real* o = out + (int64_t)n * C;
        for (int i = 0; i < C; i++) o[i] = (x[i] - m) * s * w[i] + b[i];
        mean[n] = m;
        rstd[n] = s;
    }
}

/* LayerNorm backward. With xhat = (x - mu) r and g = w * dy:
 *   dx = r * (g - mean(g) - xhat * mean(g * xhat))   (added into dinp)
 *   dw += sum_n dy * xhat,  db += sum_n dy. */
void oracle_layernorm_backward(real* dinp, real* dw, real* db, const real* dout,
                               const real* inp, const real* w, const real* mean,
                               const real* rstd, int N, int C) {
#pragma omp parallel for
    for (int n = 0; n < N; n++) {
        const real* x = inp + (int64_t)n * C;
        const real* dy = dout + (int64_t)n * C;
        real m = mean[n], s = rstd[n];
        real g_mean = 0, gx_mean = 0;
        for (int i = 0; i < C; i++) {
            real xhat = (x[i] - m) * s;
            real g = w[i] * dy[i];
            g_mean += g;
            gx_mean += g * xhat;
        }
        g_mean = g_mean / C;
        gx_mean = gx_mean / C;
        real* dx = dinp + (int64_t)n * C;
        for (int i = 0; i < C; i++) {
            real xhat = (x[i] - m) * s;
            real g = w[i] * dy[i];
            dx[i] += (g - g_mean - xhat * gx_mean) * s;
        }
    }
#pragma omp parallel for
    for (int i = 0; i < C; i++) {
        real sw = 0, sb = 0;
        for (int n = 0; n < N; n++) {
            real xhat = (inp[(int64_t)n * C + i] - mean[n]) * rstd[n];
            sw += dout[(int64_t)n * C + i] * xhat;
            sb += dout[(int64_t)n * C + i];
        }
        dw[i] += sw;
        db[i] += sb;
    }
}

/* Affine map with the weight stored (out, in): out[n,o] = b[o] + sum_i x[n,i] w[o,i]. */
void oracle_matmul_forward(real* out, const real* inp, const real* w,
                           const real* bias, int N, int C, int OC) {
#pragma omp parallel for
    for (int o = 0; o < OC; o++) {
        const real* wr = w + (int64_t)o * C;
        for (int n = 0; n < N; n++) {
            const real* x = inp + (int64_t)n * C;
            real acc = bias ? bias[o] : 0;
            for (int i = 0; i < C; i++) acc += x[i] * wr[i];
            out[(int64_t)n * OC + o] = acc;
        }
    }
}

/* Its gradients: dx[n,i] += sum_o dy[n,o] w[o,i]; dw[o,i] += sum_n dy[n,o] x[n,i];
 * db[o] += sum_n dy[n,o]. */
void oracle_matmul_backward(real* dinp, real* dw, real* dbias, const real* dout,
                            const real* inp, const real* w, int N, int C, int OC) {
#pragma omp parallel for
    for (int n = 0; n < N; n++) {
        real* dx = dinp + (int64_t)n * C;
        const real* dy = dout + (int64_t)n * OC;
        for (int o = 0; o < OC; o++) {
            real d = dy[o];
            const real* wr = w + (int64_t)o * C;
            for (int i = 0; i < C; i++) dx[i] += d * wr[i];
        }
    }
#pragma omp parallel for
    for (int o = 0; o < OC; o++) {
        real* dwr = dw + (int64_t)o * C;
        real sb = 0;
        for (int n = 0; n < N; n++) {
            real d = dout[(int64_t)n * OC + o];
            const real* x = inp + (int64_t)n * C;
            for (int i = 0; i < C; i++) dwr[i] += d * x[i];
            sb += d;
        }
        if (dbias) dbias[o] += sb;
    }
}

/* Causal multi-head self-attention on the fused qkv activations (B,T,3C):
 * for each (b, h, t): s[t2] = q_t . k_t2 / sqrt(hs) for t2 <= t; P = softmax(s)
 * (the row maximum is subtracted before exp); y_t = sum_t2 P[t2] v_t2.
 * att (B,NH,T,T) keeps P with zeros above the diagonal. */
void oracle_attention_forward(real* out, real* att, const real* qkv, int B, int T,
                              int C, int NH) {
    int hs = C / NH;
    int C3 = 3 * C;
    real scale = 1 / sqrt((real)hs);
#pragma omp parallel for collapse(3)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++)
            for (int t = 0; t < T; t++) {
                const real* q = qkv + ((int64_t)b * T + t) * C3 + h * hs;
                real* p = att + (((int64_t)b * NH + h) * T + t) * T;
                real mx = -INFINITY;
                for (int t2 = 0; t2 <= t; t2++) {
                    const real* k = qkv + ((int64_t)b * T + t2) * C3 + C + h * hs;
                    real s = 0;
                    for (int i = 0; i < hs; i++) s += q[i] * k[i];
                    s = s * scale;
                    p[t2] = s;
                    if (s > mx) mx = s;
                }
                real sum = 0;
                for (int t2 = 0; t2 <= t; t2++) {
                    p[t2] = exp(p[t2] - mx);
                    sum += p[t2];
                }
                for (int t2 = 0; t2 <= t; t2++) p[t2] = p[t2] / sum;
                for (int t2 = t + 1; t2 < T; t2++) p[t2] = 0;
                real* y = out + ((int64_t)b * T + t) * C + h * hs;
                for (int i = 0; i < hs; i++) {
                    real acc = 0;
                    for (int t2 = 0; t2 <= t; t2++) {
                        const real* v = qkv + ((int64_t)b * T + t2) * C3 + 2 * C + h * hs;
                        acc += p[t2] * v[i];
                    }
                    y[i] = acc;
                }
            }
}

/* Attention backward. Per (b, h, t): dP[t2] = dy_t . v_t2; dv_t2 += P[t2] dy_t;
 * softmax backward dS[t2] = P[t2] (dP[t2] - sum_t3 P[t3] dP[t3]);
 * dq_t += sum_t2 dS[t2] k_t2 / sqrt(hs); dk_t2 += dS[t2] q_t / sqrt(hs).
 * Accumulates into dqkv. Threads split (b, h); t runs in order inside. */
void oracle_attention_backward(real* dqkv, const real* dout, const real* qkv,
                               const real* att, int B, int T, int C, int NH) {
    int hs = C / NH;
    int C3 = 3 * C;
    real scale = 1 / sqrt((real)hs);
#pragma omp parallel
    {
        real* dp = (real*)malloc(sizeof(real) * T);
        real* ds = (real*)malloc(sizeof(real) * T);
#pragma omp for collapse(2)
        for (int b = 0; b < B; b++)
            for (int h = 0; h < NH; h++)
                for (int t = 0; t < T; t++) {
                    const real* p = att + (((int64_t)b * NH + h) * T + t) * T;
                    const real* dy = dout + ((int64_t)b * T + t) * C + h * hs;
                    const real* q = qkv + ((int64_t)b * T + t) * C3 + h * hs;
                    real* dq = dqkv + ((int64_t)b * T + t) * C3 + h * hs;
                    for (int t2 = 0; t2 <= t; t2++) {
                        const real* v = qkv + ((int64_t)b * T + t2) * C3 + 2 * C + h * hs;
                        real* dv = dqkv + ((int64_t)b * T + t2) * C3 + 2 * C + h * hs;
                        real acc = 0;
                        for (int i = 0; i < hs; i++) {
                            acc += dy[i] * v[i];
                            dv[i] += p[t2] * dy[i];
                        }
                        dp[t2] = acc;
                    }
                    real pdp = 0;
                    for (int t2 = 0; t2 <= t; t2++) pdp += p[t2] * dp[t2];
                    for (int t2 = 0; t2 <= t; t2++) ds[t2] = p[t2] * (dp[t2] - pdp);
                    for (int t2 = 0; t2 <= t; t2++) {
                        const real* k = qkv + ((int64_t)b * T + t2) * C3 + C + h * hs;
                        real* dk = dqkv + ((int64_t)b * T + t2) * C3 + C + h * hs;
                        for (int i = 0; i < hs; i++) {
                            dq[i] += ds[t2] * k[i] * scale;
                            dk[i] += ds[t2] * q[i] * scale;
                        }
                    }
                }
        free(dp);
        free(ds);
    }
}

/* GELU, tanh form: g(x) = x/2 (1 + tanh(a)), a = sqrt(2/pi) (x + 0.044715 x^3). */
void oracle_gelu_forward(real* out, const real* inp, int64_t N) {
    real k = sqrt(2 / (real)ORACLE_PI);
#pragma omp parallel for
    for (int64_t i = 0; i < N; i++) {
        real x = inp[i];
        real a = k * (x + (real)0.044715 * x * x * x);
        out[i] = (real)0.5 * x * (1 + tanh(a));
    }
}

/* g'(x) = (1 + tanh a)/2 + x/2 (1 - tanh^2 a) sqrt(2/pi) (1 + 3 * 0.044715 x^2);
 * dinp += g'(x) dout. */
void oracle_gelu_backward(real* dinp, const real* inp, const real* dout, int64_t N) {
    real k = sqrt(2 / (real)ORACLE_PI);
#pragma omp parallel for
    for (int64_t i = 0; i < N; i++) {
        real x = inp[i];
        real a = k * (x + (real)0.044715 * x * x * x);
        real th = tanh(a);
        real da = k * (1 + 3 * (real)0.044715 * x * x);
        real gp = (real)0.5 * (1 + th) + (real)0.5 * x * (1 - th * th) * da;
        dinp[i] += gp * dout[i];
    }
}

void oracle_residual_forward(real* out, const real* a, const real* b, int64_t N) {
#pragma omp parallel for
    for (int64_t i = 0; i < N; i++) out[i] = a[i] + b[i];
}

void oracle_residual_backward(real* da, real* db, const real* dout, int64_t N) {
#pragma omp parallel for
    for (int64_t i = 0; i < N; i++) {
        da[i] += dout[i];
        db[i] += dout[i];
    }
}

/* Softmax over the first V of Vp logit columns (padded columns get p = 0). */
void oracle_softmax_forward(real* probs, const real* logits, int N, int V, int Vp) {
#pragma omp parallel for
    for (int n = 0; n < N; n++) {
        const real* z = logits + (int64_t)n * Vp;
        real* p = probs + (int64_t)n * Vp;
        real mx = -INFINITY;
        for (int v = 0; v < V; v++)
            if (z[v] > mx) mx = z[v];
        real sum = 0;
        for (int v = 0; v < V; v++) {
            p[v] = exp(z[v] - mx);
            sum += p[v];
        }
        for (int v = 0; v < V; v++) p[v] = p[v] / sum;
        for (int v = V; v < Vp; v++) p[v] = 0;
    }
}

/* Cross-entropy per position: loss[n] = -ln p[n, target[n]]. */
void oracle_crossentropy_forward(real* losses, const real* probs, const int* targets,
                                 int N, int Vp) {
    for (int n = 0; n < N; n++) losses[n] = -log(probs[(int64_t)n * Vp + targets[n]]);
}

/* Gradient of the mean cross-entropy wrt the logits:
 * dz[n,v] = (p[n,v] - [v == target]) * dloss for v < V; 0 for padded columns. */
void oracle_crossentropy_softmax_backward(real* dlogits, const real* probs,
                                          const int* targets, real dloss, int N,
                                          int V, int Vp) {
#pragma omp parallel for
    for (int n = 0; n < N; n++) {
        const real* p = probs + (int64_t)n * Vp;
        real* dz = dlogits + (int64_t)n * Vp;
        for (int v = 0; v < V; v++) {
            real ind = (v == targets[n]) ? 1 : 0;
            dz[v] += (p[v] - ind) * dloss;
        }
    }
}

/* AdamW, step t >= 1, decoupled weight decay scaled by lr:
 * m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2; mhat = m/(1-b1^t); vhat = v/(1-b2^t);
 * theta -= lr (mhat / (sqrt(vhat) + eps) + wd theta). */
/* The same step with every gradient element multiplied by gscale first (the
 * gradient-clipping factor below; gscale = 1 is the plain step). */
void oracle_adamw_scaled(real* theta, const real* g, real* m, real* v, int64_t N, real lr,
                         real b1, real b2, real eps, real wd, int t, real gscale) {
    real c1 = 1 - pow(b1, t);
    real c2 = 1 - pow(b2, t);
#pragma omp parallel for
    for (int64_t i = 0; i < N; i++) {
        real gi = g[i] * gscale;
        m[i] = b1 * m[i] + (1 - b1) * gi;
        v[i] = b2 * v[i] + (1 - b2) * gi * gi;
        real mhat = m[i] / c1;
        real vhat = v[i] / c2;
        theta[i] -= lr * (mhat / (sqrt(vhat) + eps) + wd * theta[i]);
    }
}

void oracle_adamw(real* theta, const real* g, real* m, real* v, int64_t N, real lr,
                  real b1, real b2, real eps, real wd, int t) {
    oracle_adamw_scaled(theta, g, m, v, N, lr, b1, b2, eps, wd, t, 1);
}

/* Training infrastructure of page "Building GPT-2 from scratch", exercise
 * table row A5 ("LR schedules, grad clipping"). The page names them only;
 * these are the plain readings.
 *
 * Global gradient norm: the Euclidean norm of the whole flat gradient,
 * sqrt(sum_i g_i^2), summed in index order. */
real oracle_grad_norm(const real* g, int64_t N) {
    real s = 0;
    for (int64_t i = 0; i < N; i++) s += g[i] * g[i];
    return sqrt(s);
}

/* Learning rate at AdamW step t >= 1: linear warmup to lr_max over the first
 * `warmup` steps, then a half cosine from lr_max (at t = warmup) down to
 * lr_min (at t = total), lr_min after that. */
double oracle_lr_schedule(double lr_max, double lr_min, int warmup, int total, int t) {
    if (t <= warmup) return lr_max * t / warmup;
    double p = (double)(t - warmup) / (double)(total - warmup);
    if (p > 1) p = 1;
    return lr_min + 0.5 * (lr_max - lr_min) * (1 + cos(ORACLE_PI * p));
}

/* ------------------------------------------------------------------------ */
/* FP8 matrix products.                                                     */
/* ------------------------------------------------------------------------ */
/* The talk "llm.c's Origin and the Future of LLM Compilers", chapter
 * "Project Roadmap, Community Forks, and LLaMA Architecture Support", names
 * FP8 support as a direction and fixes nothing more. Plain readings, which the
 * GPU path follows:
 *   - format: the OCP 8-bit E4M3 format: sign, 4 exponent bits with bias 7,
 *     3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6;
 *     no infinities; codes 0x7f and 0xff are NaN; largest finite 448;
 *   - conversion of a float: round to nearest, ties to the even code, not
 *     saturating: magnitudes above 464 (the midpoint between 448 and the
 *     unrepresentable 480) give NaN;
 *   - per-tensor scaling: s = 448 / amax(|x|) computed in fp32 (s = 1 for an
 *     all-zero tensor), q = E4M3(x * s) with the product rounded to fp32
 *     first -- the precision the codes are decided in;
 *   - product: out[i][j] = (sum_k dec(qx[i][k]) dec(qw[j][k])) / (sx sw)
 *     + bias[j], the sum taken exactly (every product of two E4M3 values is a
 *     multiple of 2^-18 below 2^17, so a double sum of up to 2^18 of them is
 *     exact). */

/* Value of an E4M3 code. */
double oracle_e4m3_decode(int code) {
    const int sgn = code & 0x80, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -mag : mag;
}

/* Code of the E4M3 value nearest to y (ties to the even code), by comparison
 * with every finite non-negative code. */
int oracle_e4m3_encode(float y) {
    if (isnan(y)) return 0x7f;
    const int sgn = signbit(y) ? 0x80 : 0;
    const double a = fabs((double)y);
    if (a > 464.0) return sgn | 0x7f;
    int best = 0;
    double bd = a;  /* distance to code 0 */
    for (int c = 1; c <= 0x7e; c++) {
        const double d = fabs(a - oracle_e4m3_decode(c));
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            bd = d;
            best = c;
        }
    }
    return sgn | best;
}

/* Per-tensor scale of a tensor with largest magnitude amax. */
float oracle_fp8_scale(float amax) { return amax > 0.0f ? 448.0f / amax : 1.0f; }

/* Largest |x_i| over n floats. */
float oracle_fp8_amax(const float* x, int64_t n) {
    float m = 0.0f;
    for (int64_t i = 0; i < n; i++) m = fabsf(x[i]) > m ? fabsf(x[i]) : m;
    return m;
}

/* q_i = E4M3(x_i * s), the product rounded to fp32. */
void oracle_fp8_quantize(unsigned char* q, const float* x, int64_t n, float s) {
    for (int64_t i = 0; i < n; i++) {
        volatile float p = x[i] * s;  /* one fp32 rounding, no contraction */
        q[i] = (unsigned char)oracle_e4m3_encode(p);
    }
}

/* out[M][N] = (qx[M][K] . qw[N][K]^T) / (sx sw) + bias[N] (bias may be NULL). */
void oracle_fp8_matmul(double* out, const unsigned char* qx, const unsigned char* qw,
                       const double* bias, int M, int N, int K, float sx, float sw) {
    double dec[256];
    for (int c = 0; c < 256; c++) dec[c] = oracle_e4m3_decode(c);
    const double inv = 1.0 / ((double)sx * (double)sw);
#pragma omp parallel for
    for (int i = 0; i < M; i++)
        for (int j = 0; j < N; j++) {
            double acc = 0.0;
            for (int k = 0; k < K; k++)
                acc += dec[qx[(int64_t)i * K + k]] * dec[qw[(int64_t)j * K + k]];
            out[(int64_t)i * N + j] = acc * inv + (bias ? bias[j] : 0.0);
        }
}

/* ------------------------------------------------------------------------ */
/* The model.                                                               */
/* ------------------------------------------------------------------------ */

enum { P_WTE, P_WPE, P_LN1W, P_LN1B, P_QKVW, P_QKVB, P_ATTPROJW, P_ATTPROJB,
       P_LN2W, P_LN2B, P_FCW, P_FCB, P_FCPROJW, P_FCPROJB, P_LNFW, P_LNFB };

static void param_sizes(const oracle_config* c, int64_t s[NUM_PARAM_TENSORS]) {
    int64_t C = c->C, L = c->L;
    s[P_WTE] = (int64_t)c->Vp * C;
    s[P_WPE] = (int64_t)c->maxT * C;
    s[P_LN1W] = L * C;
    s[P_LN1B] = L * C;
    s[P_QKVW] = L * 3 * C * C;
    s[P_QKVB] = L * 3 * C;
    s[P_ATTPROJW] = L * C * C;
    s[P_ATTPROJB] = L * C;
    s[P_LN2W] = L * C;
    s[P_LN2B] = L * C;
    s[P_FCW] = L * 4 * C * C;
    s[P_FCB] = L * 4 * C;
    s[P_FCPROJW] = L * C * 4 * C;
    s[P_FCPROJB] = L * C;
    s[P_LNFW] = C;
    s[P_LNFB] = C;
}

int64_t oracle_num_params(const oracle_config* c) {
    int64_t s[NUM_PARAM_TENSORS], n = 0;
    param_sizes(c, s);
    for (int i = 0; i < NUM_PARAM_TENSORS; i++) n += s[i];
    return n;
}

/* Forward activations (and, in a second copy, their gradients). */
#define NUM_ACTS 22
static const char* ACT_NAMES[NUM_ACTS] = {
    "encoded", "ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "att", "attproj",
    "residual2", "ln2", "ln2_mean", "ln2_rstd", "fch", "fch_gelu", "fcproj",
    "residual3", "lnf", "lnf_mean", "lnf_rstd", "logits", "probs", "losses"};
enum { A_ENCODED, A_LN1, A_LN1_MEAN, A_LN1_RSTD, A_QKV, A_ATTY, A_ATT, A_ATTPROJ,
       A_RESIDUAL2, A_LN2, A_LN2_MEAN, A_LN2_RSTD, A_FCH, A_FCH_GELU, A_FCPROJ,
       A_RESIDUAL3, A_LNF, A_LNF_MEAN, A_LNF_RSTD, A_LOGITS, A_PROBS, A_LOSSES };

static void act_sizes(const oracle_config* c, int64_t s[NUM_ACTS]) {
    int64_t B = c->B, T = c->T, C = c->C, L = c->L, NH = c->NH, Vp = c->Vp;
    s[A_ENCODED] = B * T * C;
    s[A_LN1] = L * B * T * C;
    s[A_LN1_MEAN] = L * B * T;
    s[A_LN1_RSTD] = L * B * T;
    s[A_QKV] = L * B * T * 3 * C;
    s[A_ATTY] = L * B * T * C;
    s[A_ATT] = L * B * NH * T * T;
    s[A_ATTPROJ] = L * B * T * C;
    s[A_RESIDUAL2] = L * B * T * C;
    s[A_LN2] = L * B * T * C;
    s[A_LN2_MEAN] = L * B * T;
    s[A_LN2_RSTD] = L * B * T;
    s[A_FCH] = L * B * T * 4 * C;
    s[A_FCH_GELU] = L * B * T * 4 * C;
    s[A_FCPROJ] = L * B * T * C;
    s[A_RESIDUAL3] = L * B * T * C;
    s[A_LNF] = B * T * C;
    s[A_LNF_MEAN] = B * T;
    s[A_LNF_RSTD] = B * T;
    s[A_LOGITS] = B * T * Vp;
    s[A_PROBS] = B * T * Vp;
    s[A_LOSSES] = B * T;
}

typedef struct {
    oracle_config cfg;
    int64_t n_params;
    int64_t psize[NUM_PARAM_TENSORS];
    int64_t asize[NUM_ACTS];
    real *params, *grads, *m, *v;
    real* p[NUM_PARAM_TENSORS];
    real* g[NUM_PARAM_TENSORS];
    real* act[NUM_ACTS];
    real* dact[NUM_ACTS]; /* gradients of the activations (att unused) */
    int* inputs;
    int* targets;
    int have_targets;
    real mean_loss;
} oracle_model;

static void* xcalloc(int64_t n, size_t sz) {
    void* p = calloc((size_t)(n > 0 ? n : 1), sz);
    if (!p) {
        fprintf(stderr, "oracle: out of memory (%lld x %zu)\n", (long long)n, sz);
        abort();
    }
    return p;
}

int oracle_real_bytes(void) { return (int)sizeof(real); }

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int config_ok(const oracle_config* c) {
    return c->V > 0 && c->Vp >= c->V && c->maxT > 0 && c->C > 0 && c->L > 0 &&
           c->NH > 0 && c->C % c->NH == 0 && c->B > 0 && c->T > 0 && c->T <= c->maxT;
}

/* params: n_params fp32 values in the flat tensor-major layout. */
oracle_model* oracle_create(const oracle_config* cfg, const float* params) {
    if (!config_ok(cfg)) return NULL;
    oracle_model* M = (oracle_model*)xcalloc(1, sizeof(oracle_model));
    M->cfg = *cfg;
    param_sizes(cfg, M->psize);
    M->n_params = oracle_num_params(cfg);
    M->params = (real*)xcalloc(M->n_params, sizeof(real));
    M->grads = (real*)xcalloc(M->n_params, sizeof(real));
    M->m = (real*)xcalloc(M->n_params, sizeof(real));
    M->v = (real*)xcalloc(M->n_params, sizeof(real));
    int64_t off = 0;
    for (int i = 0; i < NUM_PARAM_TENSORS; i++) {
        M->p[i] = M->params + off;
        M->g[i] = M->grads + off;
        off += M->psize[i];
    }
    for (int64_t i = 0; i < M->n_params; i++) M->params[i] = (real)params[i];
    act_sizes(cfg, M->asize);
    for (int i = 0; i < NUM_ACTS; i++) {
        M->act[i] = (real*)xcalloc(M->asize[i], sizeof(real));
        M->dact[i] = (i == A_ATT) ? NULL : (real*)xcalloc(M->asize[i], sizeof(real));
    }
    M->inputs = (int*)xcalloc((int64_t)cfg->B * cfg->T, sizeof(int));
    M->targets = (int*)xcalloc((int64_t)cfg->B * cfg->T, sizeof(int));
    return M;
}

void oracle_free(oracle_model* M) {
    if (!M) return;
    free(M->params);
    free(M->grads);
    free(M->m);
    free(M->v);
    for (int i = 0; i < NUM_ACTS; i++) {
        free(M->act[i]);
        free(M->dact[i]);
    }
    free(M->inputs);
    free(M->targets);
    free(M);
}

/* Pre-LN GPT-2 forward. Returns 0, or -1 on a token outside [0, V).
 * With targets, *loss receives the mean cross-entropy over B*T positions. */
int oracle_forward(oracle_model* M, const int* inputs, const int* targets, double* loss) {
    const oracle_config* c = &M->cfg;
    int B = c->B, T = c->T, C = c->C, L = c->L, NH = c->NH, V = c->V, Vp = c->Vp;
    int64_t BT = (int64_t)B * T;
    for (int64_t i = 0; i < BT; i++) {
        if (inputs[i] < 0 || inputs[i] >= V) return -1;
        if (targets && (targets[i] < 0 || targets[i] >= V)) return -1;
    }
    memcpy(M->inputs, inputs, sizeof(int) * BT);
    M->have_targets = targets != NULL;
    if (targets) memcpy(M->targets, targets, sizeof(int) * BT);

    real** a = M->act;
    real** p = M->p;
    oracle_encoder_forward(a[A_ENCODED], inputs, p[P_WTE], p[P_WPE], B, T, C);
    for (int l = 0; l < L; l++) {
        int64_t oC = l * BT * C, o3 = l * BT * 3 * C, o4 = l * BT * 4 * C, oN = l * BT;
        const real* res = (l == 0) ? a[A_ENCODED] : a[A_RESIDUAL3] + (l - 1) * BT * C;
        oracle_layernorm_forward(a[A_LN1] + oC, a[A_LN1_MEAN] + oN, a[A_LN1_RSTD] + oN, res,
                                 p[P_LN1W] + l * C, p[P_LN1B] + l * C, (int)BT, C);
        oracle_matmul_forward(a[A_QKV] + o3, a[A_LN1] + oC, p[P_QKVW] + (int64_t)l * 3 * C * C,
                              p[P_QKVB] + l * 3 * C, (int)BT, C, 3 * C);
        oracle_attention_forward(a[A_ATTY] + oC, a[A_ATT] + (int64_t)l * B * NH * T * T,
                                 a[A_QKV] + o3, B, T, C, NH);
        oracle_matmul_forward(a[A_ATTPROJ] + oC, a[A_ATTY] + oC, p[P_ATTPROJW] + (int64_t)l * C * C,
                              p[P_ATTPROJB] + l * C, (int)BT, C, C);
        oracle_residual_forward(a[A_RESIDUAL2] + oC, res, a[A_ATTPROJ] + oC, BT * C);
        oracle_layernorm_forward(a[A_LN2] + oC, a[A_LN2_MEAN] + oN, a[A_LN2_RSTD] + oN,
                                 a[A_RESIDUAL2] + oC, p[P_LN2W] + l * C, p[P_LN2B] + l * C,
                                 (int)BT, C);
        oracle_matmul_forward(a[A_FCH] + o4, a[A_LN2] + oC, p[P_FCW] + (int64_t)l * 4 * C * C,
                              p[P_FCB] + l * 4 * C, (int)BT, C, 4 * C);
        oracle_gelu_forward(a[A_FCH_GELU] + o4, a[A_FCH] + o4, BT * 4 * C);
        oracle_matmul_forward(a[A_FCPROJ] + oC, a[A_FCH_GELU] + o4,
                              p[P_FCPROJW] + (int64_t)l * 4 * C * C, p[P_FCPROJB] + l * C,
                              (int)BT, 4 * C, C);
        oracle_residual_forward(a[A_RESIDUAL3] + oC, a[A_RESIDUAL2] + oC, a[A_FCPROJ] + oC,
                                BT * C);
    }
    oracle_layernorm_forward(a[A_LNF], a[A_LNF_MEAN], a[A_LNF_RSTD],
                             a[A_RESIDUAL3] + (L - 1) * BT * C, p[P_LNFW], p[P_LNFB], (int)BT, C);
    oracle_matmul_forward(a[A_LOGITS], a[A_LNF], p[P_WTE], NULL, (int)BT, C, Vp);
    oracle_softmax_forward(a[A_PROBS], a[A_LOGITS], (int)BT, V, Vp);
    if (targets) {
        oracle_crossentropy_forward(a[A_LOSSES], a[A_PROBS], targets, (int)BT, Vp);
        real s = 0;
        for (int64_t i = 0; i < BT; i++) s += a[A_LOSSES][i];
        M->mean_loss = s / BT;
        if (loss) *loss = (double)M->mean_loss;
    }
    return 0;
}

/* Full backward of the mean loss. Overwrites every parameter gradient.
 * Returns -1 without a preceding forward that had targets. */
int oracle_backward(oracle_model* M) {
    if (!M->have_targets) return -1;
    const oracle_config* c = &M->cfg;
    int B = c->B, T = c->T, C = c->C, L = c->L, NH = c->NH, V = c->V, Vp = c->Vp;
    int64_t BT = (int64_t)B * T;
    memset(M->grads, 0, sizeof(real) * M->n_params);
    for (int i = 0; i < NUM_ACTS; i++)
        if (M->dact[i]) memset(M->dact[i], 0, sizeof(real) * M->asize[i]);
    real** a = M->act;
    real** d = M->dact;
    real** p = M->p;
    real** g = M->g;

    oracle_crossentropy_softmax_backward(d[A_LOGITS], a[A_PROBS], M->targets,
                                         (real)1 / (real)BT, (int)BT, V, Vp);
    oracle_matmul_backward(d[A_LNF], g[P_WTE], NULL, d[A_LOGITS], a[A_LNF], p[P_WTE],
                           (int)BT, C, Vp);
    oracle_layernorm_backward(d[A_RESIDUAL3] + (L - 1) * BT * C, g[P_LNFW], g[P_LNFB],
                              d[A_LNF], a[A_RESIDUAL3] + (L - 1) * BT * C, p[P_LNFW],
                              a[A_LNF_MEAN], a[A_LNF_RSTD], (int)BT, C);
    for (int l = L - 1; l >= 0; l--) {
        int64_t oC = l * BT * C, o3 = l * BT * 3 * C, o4 = l * BT * 4 * C, oN = l * BT;
        const real* res = (l == 0) ? a[A_ENCODED] : a[A_RESIDUAL3] + (l - 1) * BT * C;
        real* dres = (l == 0) ? d[A_ENCODED] : d[A_RESIDUAL3] + (l - 1) * BT * C;
        oracle_residual_backward(d[A_RESIDUAL2] + oC, d[A_FCPROJ] + oC, d[A_RESIDUAL3] + oC,
                                 BT * C);
        oracle_matmul_backward(d[A_FCH_GELU] + o4, g[P_FCPROJW] + (int64_t)l * 4 * C * C,
                               g[P_FCPROJB] + l * C, d[A_FCPROJ] + oC, a[A_FCH_GELU] + o4,
                               p[P_FCPROJW] + (int64_t)l * 4 * C * C, (int)BT, 4 * C, C);
        oracle_gelu_backward(d[A_FCH] + o4, a[A_FCH] + o4, d[A_FCH_GELU] + o4, BT * 4 * C);
        oracle_matmul_backward(d[A_LN2] + oC, g[P_FCW] + (int64_t)l * 4 * C * C,
                               g[P_FCB] + l * 4 * C, d[A_FCH] + o4, a[A_LN2] + oC,
                               p[P_FCW] + (int64_t)l * 4 * C * C, (int)BT, C, 4 * C);
        oracle_layernorm_backward(d[A_RESIDUAL2] + oC, g[P_LN2W] + l * C, g[P_LN2B] + l * C,
                                  d[A_LN2] + oC, a[A_RESIDUAL2] + oC, p[P_LN2W] + l * C,
                                  a[A_LN2_MEAN] + oN, a[A_LN2_RSTD] + oN, (int)BT, C);
        oracle_residual_backward(dres, d[A_ATTPROJ] + oC, d[A_RESIDUAL2] + oC, BT * C);
        oracle_matmul_backward(d[A_ATTY] + oC, g[P_ATTPROJW] + (int64_t)l * C * C,
                               g[P_ATTPROJB] + l * C, d[A_ATTPROJ] + oC, a[A_ATTY] + oC,
                               p[P_ATTPROJW] + (int64_t)l * C * C, (int)BT, C, C);
        oracle_attention_backward(d[A_QKV] + o3, d[A_ATTY] + oC, a[A_QKV] + o3,
                                  a[A_ATT] + (int64_t)l * B * NH * T * T, B, T, C, NH);
        oracle_matmul_backward(d[A_LN1] + oC, g[P_QKVW] + (int64_t)l * 3 * C * C,
                               g[P_QKVB] + l * 3 * C, d[A_QKV] + o3, a[A_LN1] + oC,
                               p[P_QKVW] + (int64_t)l * 3 * C * C, (int)BT, C, 3 * C);
        oracle_layernorm_backward(dres, g[P_LN1W] + l * C, g[P_LN1B] + l * C, d[A_LN1] + oC,
                                  res, p[P_LN1W] + l * C, a[A_LN1_MEAN] + oN,
                                  a[A_LN1_RSTD] + oN, (int)BT, C);
    }
    oracle_encoder_backward(g[P_WTE], g[P_WPE], d[A_ENCODED], M->inputs, B, T, C);
    return 0;
}

void oracle_update(oracle_model* M, double lr, double b1, double b2, double eps, double wd,
                   int t) {
    oracle_adamw(M->params, M->grads, M->m, M->v, M->n_params, (real)lr, (real)b1, (real)b2,
                 (real)eps, (real)wd, t);
}

/* AdamW step t at the scheduled learning rate; with grad_clip > 0 the
 * gradient is scaled by grad_clip / ||g|| when its global norm exceeds
 * grad_clip. Returns ||g|| (0 when clipping is off). */
double oracle_update_scheduled(oracle_model* M, double lr_max, double lr_min, int warmup,
                               int total, double b1, double b2, double eps, double wd,
                               double grad_clip, int t) {
    double lr = oracle_lr_schedule(lr_max, lr_min, warmup, total, t);
    real scale = 1, norm = 0;
    if (grad_clip > 0) {
        norm = oracle_grad_norm(M->grads, M->n_params);
        if (norm > grad_clip) scale = (real)grad_clip / norm;
    }
    oracle_adamw_scaled(M->params, M->grads, M->m, M->v, M->n_params, (real)lr, (real)b1,
                        (real)b2, (real)eps, (real)wd, t, scale);
    return (double)norm;
}

/* ------------------------------------------------------------------------ */
/* Data access for the tests (all copies convert to/from double).           */
/* ------------------------------------------------------------------------ */

static void to_double(double* out, const real* in, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = (double)in[i];
}

int64_t oracle_n_params(const oracle_model* M) { return M->n_params; }
void oracle_get_params(const oracle_model* M, double* out) { to_double(out, M->params, M->n_params); }
void oracle_get_grads(const oracle_model* M, double* out) { to_double(out, M->grads, M->n_params); }
void oracle_get_m(const oracle_model* M, double* out) { to_double(out, M->m, M->n_params); }
void oracle_get_v(const oracle_model* M, double* out) { to_double(out, M->v, M->n_params); }

void oracle_set_params(oracle_model* M, const double* in) {
    for (int64_t i = 0; i < M->n_params; i++) M->params[i] = (real)in[i];
}

static int act_index(const char* name) {
    for (int i = 0; i < NUM_ACTS; i++)
        if (strcmp(name, ACT_NAMES[i]) == 0) return i;
    return -1;
}

/* Element count of a named activation, or -1. */
int64_t oracle_act_size(const oracle_model* M, const char* name) {
    int i = act_index(name);
    return i < 0 ? -1 : M->asize[i];
}

/* Copies a named activation (grad != 0: its gradient) into out. */
int oracle_get_act(const oracle_model* M, const char* name, int grad, double* out) {
    int i = act_index(name);
    if (i < 0) return -1;
    const real* src = grad ? M->dact[i] : M->act[i];
    if (!src) return -1;
    to_double(out, src, M->asize[i]);
    return 0;
}

/* Central finite differences of the mean loss for parameters
 * [start, start + count): fd[j] = (loss(theta + h e_j) - loss(theta - h e_j)) / 2h.
 * Threads split the parameters; each thread steps its own model copy. */
int oracle_fd_grads(const oracle_config* cfg, const float* params, const int* inputs,
                    const int* targets, double h, int64_t start, int64_t count, double* fd) {
    int err = 0;
#pragma omp parallel
    {
        oracle_model* M = oracle_create(cfg, params);
#pragma omp for schedule(dynamic, 16)
        for (int64_t j = start; j < start + count; j++) {
            real save = M->params[j];
            double lp = 0, lm = 0;
            M->params[j] = save + (real)h;
            if (oracle_forward(M, inputs, targets, &lp) != 0) err = -1;
            M->params[j] = save - (real)h;
            if (oracle_forward(M, inputs, targets, &lm) != 0) err = -1;
            M->params[j] = save;
            fd[j - start] = (lp - lm) / (2 * h);
        }
        oracle_free(M);
    }
    return err;
}
