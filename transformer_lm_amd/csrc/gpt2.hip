// C ABI of libgpt2.so (declared in include/gpt2.h): memory planning,
// validation, and the training step's kernel sequence on one HIP stream.
//
// The step is GPT-2 as llm.c trains it (page "Building GPT-2 from scratch",
// rows A1-A2 of its exercise table): pre-LayerNorm blocks
//   x1 = x + attproj(attention(ln1(x))),  x2 = x1 + fcproj(gelu(fc(ln2(x1)))),
// a final LayerNorm, the tied output head logits = lnf . wte^T, and the mean
// cross-entropy; then the hand-derived backward pass in reverse order and
// AdamW. All memory is planned here up front and handed in by the caller as
// two blobs (talk "llm.c's Origin and the Future of LLM Compilers": memory
// allocated in one pre-planned blob), so a step never allocates.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "gpt2.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* msg) {
    g_err = msg;
    return code;
}

int fail(int code, const std::string& msg) { return fail(code, msg.c_str()); }

enum {
    P_WTE, P_WPE, P_LN1W, P_LN1B, P_QKVW, P_QKVB, P_ATTPROJW, P_ATTPROJB,
    P_LN2W, P_LN2B, P_FCW, P_FCB, P_FCPROJW, P_FCPROJB, P_LNFW, P_LNFB, NUM_P
};

const char* const P_NAMES[NUM_P] = {"wte",  "wpe",  "ln1w",     "ln1b",     "qkvw",   "qkvb",
                                    "attprojw", "attprojb", "ln2w", "ln2b", "fcw", "fcb",
                                    "fcprojw", "fcprojb", "lnfw", "lnfb"};

// Activations and backward workspaces, in buffer order.
enum {
    A_ENCODED, A_LN1, A_LN1_MEAN, A_LN1_RSTD, A_QKV, A_ATTY, A_ATT_LSE, A_RESIDUAL2,
    A_LN2, A_LN2_MEAN, A_LN2_RSTD, A_FCH, A_FCH_GELU, A_RESIDUAL3, A_LNF, A_LNF_MEAN,
    A_LNF_RSTD, A_LOGITS, A_LOSSES, A_LOSS, A_ERR,
    W_DRES, W_DC, W_D3C, W_D4C, W_ATT_D, W_LN_PART, W_BIAS_PART, W_ENC,
    W_DW_SPLIT, A_GNORM, W_GNORM_PART, NUM_A
};

const char* const A_NAMES[NUM_A] = {
    "encoded", "ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "att_lse", "residual2",
    "ln2", "ln2_mean", "ln2_rstd", "fch", "fch_gelu", "residual3", "lnf", "lnf_mean",
    "lnf_rstd", "logits", "losses", "loss", "err",
    "dresidual", "dbuf_c", "dbuf_3c", "dbuf_4c", "att_d", "ln_partials", "bias_partials",
    "enc_work", "dw_split", "grad_norm", "gnorm_partials"};

constexpr int64_t ALIGN = 256;
int64_t align_up(int64_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
    int64_t N;
    int64_t poff[NUM_P], psize[NUM_P];
    int64_t region_off[5];
    int64_t param_bytes;
    int64_t aoff[NUM_A], abytes[NUM_A];
    int64_t act_bytes;
};

const char* check_config(const gpt2_config* c) {
    if (!c) return "config is NULL";
    if (c->dtype != GPT2_DTYPE_FP32 && c->dtype != GPT2_DTYPE_BF16) return "dtype must be 0 or 1";
    if (c->V <= 0 || c->Vp < c->V || c->Vp % 64 != 0) return "need 0 < V <= Vp, Vp % 64 == 0";
    if (c->C <= 0 || c->C % 8 != 0 || c->C > 2048) return "need C % 8 == 0 and 0 < C <= 2048";
    if (c->NH <= 0 || c->C % c->NH != 0) return "need C % NH == 0";
    int hs = c->C / c->NH;
    if (hs % 8 != 0 || hs > 128) return "need head size C/NH a multiple of 8, at most 128";
    if (c->L <= 0 || 2 * c->L + 1 > LN_RED_MAX) return "need 0 < L <= 63";
    if (c->max_T <= 0 || c->T <= 0 || c->T > c->max_T) return "need 1 <= T <= max_T";
    if (c->B <= 0) return "need B > 0";
    if ((int64_t)c->B * c->T > 524288) return "need B*T <= 524288";
    if ((int64_t)c->B * c->NH > 65535) return "need B*NH <= 65535";
    return nullptr;
}

void plan(const gpt2_config* c, Layout* lay) {
    const int64_t C = c->C, L = c->L, V = c->Vp, T = c->T, B = c->B, NH = c->NH;
    const int64_t BT = B * T;
    int64_t* s = lay->psize;
    s[P_WTE] = V * C;
    s[P_WPE] = (int64_t)c->max_T * C;
    s[P_LN1W] = s[P_LN1B] = L * C;
    s[P_QKVW] = L * 3 * C * C;
    s[P_QKVB] = L * 3 * C;
    s[P_ATTPROJW] = L * C * C;
    s[P_ATTPROJB] = L * C;
    s[P_LN2W] = s[P_LN2B] = L * C;
    s[P_FCW] = L * 4 * C * C;
    s[P_FCB] = L * 4 * C;
    s[P_FCPROJW] = L * 4 * C * C;
    s[P_FCPROJB] = L * C;
    s[P_LNFW] = s[P_LNFB] = C;
    int64_t off = 0;
    for (int i = 0; i < NUM_P; i++) {
        lay->poff[i] = off;
        off += s[i];
    }
    lay->N = off;
    const int64_t N = off;
    int64_t r = 0;
    for (int i = 0; i < 4; i++) {
        lay->region_off[i] = r;
        r = align_up(r + N * 4);
    }
    lay->region_off[4] = r;
    if (c->dtype == GPT2_DTYPE_BF16) r = align_up(r + N * 2);
    lay->param_bytes = r;

    const int64_t es = c->dtype == GPT2_DTYPE_BF16 ? 2 : 4;
    int64_t* a = lay->abytes;
    a[A_ENCODED] = BT * C * es;
    a[A_LN1] = L * BT * C * es;
    a[A_LN1_MEAN] = a[A_LN1_RSTD] = L * BT * 4;
    a[A_QKV] = L * BT * 3 * C * es;
    a[A_ATTY] = L * BT * C * es;
    a[A_ATT_LSE] = L * B * NH * T * 4;
    a[A_RESIDUAL2] = L * BT * C * es;
    a[A_LN2] = L * BT * C * es;
    a[A_LN2_MEAN] = a[A_LN2_RSTD] = L * BT * 4;
    a[A_FCH] = a[A_FCH_GELU] = L * BT * 4 * C * es;
    a[A_RESIDUAL3] = L * BT * C * es;
    a[A_LNF] = BT * C * es;
    a[A_LNF_MEAN] = a[A_LNF_RSTD] = BT * 4;
    a[A_LOGITS] = BT * V * es;
    a[A_LOSSES] = BT * 4;
    a[A_LOSS] = 4;
    a[A_ERR] = 4;
    // backward: the residual-stream gradient at every layer boundary (2L + 1
    // of them) and the per-layer qkv / fc output gradients stay resident, so
    // the weight gradients of all layers can run as one grouped product after
    // the layer loop
    a[W_DRES] = (2 * L + 1) * BT * C * es;
    a[W_DC] = BT * C * es;
    a[W_D3C] = L * BT * 3 * C * es;
    a[W_D4C] = L * BT * 4 * C * es;
    a[W_ATT_D] = 2 * B * NH * T * 4;  // attention backward's D rows and base-2 lse
    a[W_LN_PART] = layernorm_bwd_partials((int)C, (int)(2 * L + 1)) * 4;
    a[W_BIAS_PART] = bias_bwd_partials((int)BT, (int)(4 * C)) * 4;
    a[W_ENC] = encoder_bwd_workspace_bytes((int)BT, (int)V, (int)C);
    // split-reduction partials of the bf16 weight-gradient products
    int64_t dwf = 0;
    if (c->dtype == GPT2_DTYPE_BF16) {
        const int64_t shapes[5][2] = {{3 * C, C}, {C, C}, {4 * C, C}, {C, 4 * C}, {V, C}};
        for (auto& s : shapes) {
            const int64_t f = gemm_dw_workspace_floats((int)BT, (int)s[0], (int)s[1]);
            if (f > dwf) dwf = f;
        }
    }
    a[W_DW_SPLIT] = dwf * 4;
    a[A_GNORM] = 4;
    a[W_GNORM_PART] = grad_norm_workspace_floats() * 4;
    int64_t o = 0;
    for (int i = 0; i < NUM_A; i++) {
        lay->aoff[i] = o;
        o = align_up(o + a[i]);
    }
    lay->act_bytes = o;
}

// Kernel classes for timing (gpt2_timing_arm / gpt2_timing_read).
enum {
    K_ENCODER_FWD, K_LAYERNORM_FWD, K_MATMUL_FWD, K_ATTENTION_FWD, K_GELU_FWD, K_CLASSIFIER,
    K_MATMUL_BWD_DX, K_MATMUL_BWD_DW, K_GELU_BWD, K_LAYERNORM_BWD, K_ATTENTION_BWD,
    K_ENCODER_BWD, K_ADAMW, NUM_K
};
const char* const K_NAMES[NUM_K] = {
    "encoder_fwd", "layernorm_fwd", "matmul_fwd", "attention_fwd", "gelu_fwd", "classifier",
    "matmul_bwd_dx", "matmul_bwd_dw", "gelu_bwd", "layernorm_bwd", "attention_bwd",
    "encoder_bwd", "adamw"};
// 1: work is compulsory HBM bytes; 0: floating-point operations
const int K_IS_BYTES[NUM_K] = {1, 1, 0, 0, 1, 1, 0, 0, 1, 1, 0, 1, 1};

}  // namespace

struct gpt2 {
    gpt2_config cfg;
    Layout lay;
    hipStream_t st;
    char* pbuf;
    char* abuf;
    float* master;
    float* grad;
    float* m;
    float* v;
    bf16* pbf16;
    void* wp[NUM_P];   // working parameters (fp32 master or bf16 copy)
    float* gp[NUM_P];  // parameter gradients
    void* a[NUM_A];
    bool fwd_targets;
    int fwd_count;  // forwards issued so far; tags a token error with its call
    const int32_t* last_inputs;
    // timing
    bool tarm[NUM_K];
    std::vector<hipEvent_t> ev;
    std::vector<int> rec_cls;
    std::vector<double> rec_work;
    int64_t nrec;
};

namespace {

int hip_status(const char* where) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_err = std::string(where) + ": " + hipGetErrorString(e);
        return GPT2_EHIP;
    }
    return GPT2_OK;
}

// Brackets the launches in its scope with an event pair when the class is armed.
struct KScope {
    gpt2* h;
    int64_t slot;
    KScope(gpt2* h_, int cls, double work) : h(h_), slot(-1) {
        if (h->tarm[cls] && h->nrec < (int64_t)h->rec_cls.size()) {
            slot = h->nrec++;
            h->rec_cls[slot] = cls;
            h->rec_work[slot] = work;
            (void)hipEventRecord(h->ev[2 * slot], h->st);
        }
    }
    ~KScope() {
        if (slot >= 0) (void)hipEventRecord(h->ev[2 * slot + 1], h->st);
    }
};

void destroy_events(gpt2* h) {
    for (hipEvent_t e : h->ev) (void)hipEventDestroy(e);
    h->ev.clear();
    h->rec_cls.clear();
    h->rec_work.clear();
    h->nrec = 0;
    for (int k = 0; k < NUM_K; k++) h->tarm[k] = false;
}

inline double mm_flops(double M, double N, double K) { return 2.0 * M * N * K; }
inline double causal_pairs(double Tn) { return Tn * (Tn + 1) / 2; }

template <typename T>
void forward_impl(gpt2* h, const int32_t* in, const int32_t* tg) {
    const gpt2_config& c = h->cfg;
    const int B = c.B, Tn = c.T, C = c.C, L = c.L, NH = c.NH, V = c.V, Vp = c.Vp;
    const int BT = B * Tn;
    const int64_t nC = (int64_t)BT * C;
    const double es = sizeof(T);
    hipStream_t st = h->st;
    T* const* P = reinterpret_cast<T* const*>(h->wp);
    T* encoded = (T*)h->a[A_ENCODED];
    T* ln1 = (T*)h->a[A_LN1];
    float* ln1m = (float*)h->a[A_LN1_MEAN];
    float* ln1r = (float*)h->a[A_LN1_RSTD];
    T* qkv = (T*)h->a[A_QKV];
    T* atty = (T*)h->a[A_ATTY];
    float* lse = (float*)h->a[A_ATT_LSE];
    T* res2 = (T*)h->a[A_RESIDUAL2];
    T* ln2 = (T*)h->a[A_LN2];
    float* ln2m = (float*)h->a[A_LN2_MEAN];
    float* ln2r = (float*)h->a[A_LN2_RSTD];
    T* fch = (T*)h->a[A_FCH];
    T* fchg = (T*)h->a[A_FCH_GELU];
    T* res3 = (T*)h->a[A_RESIDUAL3];
    int* err = (int*)h->a[A_ERR];
    const double ln_bytes = 2.0 * nC * es + 2.0 * C * es + 8.0 * BT;
    const double attn_flops = 4.0 * B * NH * (C / NH) * causal_pairs(Tn);

    {
        KScope k(h, K_ENCODER_FWD, 3.0 * nC * es + 4.0 * BT);
        encoder_fwd<T>(encoded, in, P[P_WTE], P[P_WPE], B, Tn, C, V, err, h->fwd_count, st);
    }
    for (int l = 0; l < L; l++) {
        const T* res = l == 0 ? encoded : res3 + (l - 1) * nC;
        T* ln1_l = ln1 + l * nC;
        T* qkv_l = qkv + l * 3 * nC;
        T* atty_l = atty + l * nC;
        T* res2_l = res2 + l * nC;
        T* ln2_l = ln2 + l * nC;
        T* fch_l = fch + l * 4 * nC;
        T* fchg_l = fchg + l * 4 * nC;
        {
            KScope k(h, K_LAYERNORM_FWD, ln_bytes);
            layernorm_fwd<T>(ln1_l, ln1m + (int64_t)l * BT, ln1r + (int64_t)l * BT, res,
                             P[P_LN1W] + l * C, P[P_LN1B] + l * C, BT, C, st);
        }
        {
            KScope k(h, K_MATMUL_FWD, mm_flops(BT, 3 * C, C));
            matmul_fwd<T>(qkv_l, ln1_l, P[P_QKVW] + (int64_t)l * 3 * C * C, P[P_QKVB] + l * 3 * C,
                          nullptr, BT, C, 3 * C, st);
        }
        {
            KScope k(h, K_ATTENTION_FWD, attn_flops);
            attention_fwd<T>(atty_l, lse + (int64_t)l * B * NH * Tn, qkv_l, B, Tn, C, NH, st);
        }
        {
            KScope k(h, K_MATMUL_FWD, mm_flops(BT, C, C));
            matmul_fwd<T>(res2_l, atty_l, P[P_ATTPROJW] + (int64_t)l * C * C,
                          P[P_ATTPROJB] + l * C, res, BT, C, C, st);
        }
        {
            KScope k(h, K_LAYERNORM_FWD, ln_bytes);
            layernorm_fwd<T>(ln2_l, ln2m + (int64_t)l * BT, ln2r + (int64_t)l * BT, res2_l,
                             P[P_LN2W] + l * C, P[P_LN2B] + l * C, BT, C, st);
        }
        if (std::is_same<T, bf16>::value) {
            // bf16: the GELU is applied in the product's epilogue
            KScope k(h, K_MATMUL_FWD, mm_flops(BT, 4 * C, C));
            matmul_fwd_gelu<T>(fch_l, fchg_l, ln2_l, P[P_FCW] + (int64_t)l * 4 * C * C,
                               P[P_FCB] + l * 4 * C, BT, C, 4 * C, st);
        } else {
            {
                KScope k(h, K_MATMUL_FWD, mm_flops(BT, 4 * C, C));
                matmul_fwd<T>(fch_l, ln2_l, P[P_FCW] + (int64_t)l * 4 * C * C,
                              P[P_FCB] + l * 4 * C, nullptr, BT, C, 4 * C, st);
            }
            KScope k(h, K_GELU_FWD, 2.0 * 4 * nC * es);
            gelu_fwd<T>(fchg_l, fch_l, 4 * nC, st);
        }
        {
            KScope k(h, K_MATMUL_FWD, mm_flops(BT, C, 4 * C));
            matmul_fwd<T>(res3 + l * nC, fchg_l, P[P_FCPROJW] + (int64_t)l * 4 * C * C,
                          P[P_FCPROJB] + l * C, res2_l, BT, 4 * C, C, st);
        }
    }
    T* lnf = (T*)h->a[A_LNF];
    {
        KScope k(h, K_LAYERNORM_FWD, ln_bytes);
        layernorm_fwd<T>(lnf, (float*)h->a[A_LNF_MEAN], (float*)h->a[A_LNF_RSTD],
                         res3 + (L - 1) * nC, P[P_LNFW], P[P_LNFB], BT, C, st);
    }
    T* logits = (T*)h->a[A_LOGITS];
    {
        KScope k(h, K_MATMUL_FWD, mm_flops(BT, V, C));
        matmul_fwd<T>(logits, lnf, P[P_WTE], nullptr, nullptr, BT, C, Vp, st);
    }
    if (tg) {
        KScope k(h, K_CLASSIFIER, 2.0 * BT * (double)Vp * es + 8.0 * BT);
        float* losses = (float*)h->a[A_LOSSES];
        classifier_fwd<T>(logits, losses, tg, BT, V, Vp, 1.f / (float)BT, err, h->fwd_count, st);
        loss_mean((float*)h->a[A_LOSS], losses, BT, st);
    }
}

template <typename T>
void backward_impl(gpt2* h) {
    const gpt2_config& c = h->cfg;
    const int B = c.B, Tn = c.T, C = c.C, L = c.L, NH = c.NH, V = c.V, Vp = c.Vp;
    const int BT = B * Tn;
    const int64_t nC = (int64_t)BT * C;
    const double es = sizeof(T);
    hipStream_t st = h->st;
    T* const* P = reinterpret_cast<T* const*>(h->wp);
    float* const* G = h->gp;
    T* encoded = (T*)h->a[A_ENCODED];
    T* ln1 = (T*)h->a[A_LN1];
    float* ln1m = (float*)h->a[A_LN1_MEAN];
    float* ln1r = (float*)h->a[A_LN1_RSTD];
    T* qkv = (T*)h->a[A_QKV];
    T* atty = (T*)h->a[A_ATTY];
    float* lse = (float*)h->a[A_ATT_LSE];
    T* res2 = (T*)h->a[A_RESIDUAL2];
    T* ln2 = (T*)h->a[A_LN2];
    float* ln2m = (float*)h->a[A_LN2_MEAN];
    float* ln2r = (float*)h->a[A_LN2_RSTD];
    T* fch = (T*)h->a[A_FCH];
    T* fchg = (T*)h->a[A_FCH_GELU];
    T* res3 = (T*)h->a[A_RESIDUAL3];
    T* lnf = (T*)h->a[A_LNF];
    T* dlogits = (T*)h->a[A_LOGITS];
    T* dres = (T*)h->a[W_DRES];  // [2L + 1][BT][C]
    T* dC = (T*)h->a[W_DC];
    T* d3C_all = (T*)h->a[W_D3C];  // [L][BT][3C]
    T* d4C_all = (T*)h->a[W_D4C];  // [L][BT][4C]
    float* attD = (float*)h->a[W_ATT_D];
    float* lnp = (float*)h->a[W_LN_PART];
    float* bp = (float*)h->a[W_BIAS_PART];
    float* dws = (float*)h->a[W_DW_SPLIT];
    // LayerNorm backward reads x and dy, reads+writes (or writes) dx
    auto ln_bytes = [&](bool acc) { return (acc ? 4.0 : 3.0) * nC * es + 8.0 * BT + C * (es + 8); };
    const double attn_flops = 8.0 * B * NH * (C / NH) * causal_pairs(Tn);
    // residual-stream gradient k: 0 = dLoss/d(output of the last block), then
    // alternately d/d(x1) and d/d(input) of blocks L-1, L-2, ..., 0
    auto R = [&](int k) { return dres + (int64_t)k * nC; };
    std::vector<DwTask> dw_tasks;
    dw_tasks.reserve(4 * L + 1);
    double dw_flops = 0.0;

    // output head (tied to wte): dlnf = dz . wte now; dwte = dz^T . lnf joins
    // the layers' weight gradients in the grouped launch after the layer loop
    // (the logits buffer holds dz until then; the encoder's token gradient is
    // added to dwte after it). Every weight-gradient tile there reduces over
    // the same B*T rows, so one launch fills the GPU's rounds of resident
    // tiles better than two.
    {
        KScope k(h, K_MATMUL_BWD_DX, mm_flops(BT, C, V));
        matmul_bwd_dx<T>(dC, dlogits, P[P_WTE], BT, Vp, C, st);
    }
    dw_tasks.push_back({dlogits, lnf, G[P_WTE], nullptr, Vp, C});
    dw_flops += mm_flops(V, C, BT);
    // LayerNorm weight gradients: per-block partial sums now, one batched
    // fixed-order reduction of all 2L+1 LayerNorms after the layer loop
    LnRedBatch ln_red;
    ln_red.count = 0;
    {
        KScope k(h, K_LAYERNORM_BWD, ln_bytes(false));
        layernorm_bwd_rows<T>(R(0), nullptr, dC, res3 + (L - 1) * nC, P[P_LNFW],
                              (float*)h->a[A_LNF_MEAN], (float*)h->a[A_LNF_RSTD], BT, C, lnp,
                              ln_red.count, st);
        ln_red.t[ln_red.count++] = {G[P_LNFW], G[P_LNFB]};
    }
    for (int l = L - 1; l >= 0; l--) {
        const T* res = l == 0 ? encoded : res3 + (l - 1) * nC;
        const int64_t w4 = (int64_t)l * 4 * C * C;
        const int kx = 2 * (L - 1 - l);
        T* g2 = R(kx);      // dLoss/d(x2): the gradient of fcproj's output
        T* g1 = R(kx + 1);  // dLoss/d(x1): the gradient of attproj's output
        T* g0 = R(kx + 2);  // dLoss/d(block input)
        T* d4C = d4C_all + (int64_t)l * 4 * nC;
        T* d3C = d3C_all + (int64_t)l * 3 * nC;
        // MLP
        if (std::is_same<T, bf16>::value) {
            // bf16: gelu' is applied in the product's epilogue
            KScope k(h, K_MATMUL_BWD_DX, mm_flops(BT, 4 * C, C));
            matmul_bwd_dx_dgelu<T>(d4C, g2, P[P_FCPROJW] + w4, fch + l * 4 * nC, BT, C, 4 * C, st);
        } else {
            KScope k(h, K_MATMUL_BWD_DX, mm_flops(BT, 4 * C, C));
            matmul_bwd_dx<T>(d4C, g2, P[P_FCPROJW] + w4, BT, C, 4 * C, st);
        }
        dw_tasks.push_back({g2, fchg + l * 4 * nC, G[P_FCPROJW] + w4, G[P_FCPROJB] + l * C, C,
                            4 * C});
        if (!std::is_same<T, bf16>::value) {
            KScope k(h, K_GELU_BWD, 3.0 * 4 * nC * es);
            gelu_bwd<T>(d4C, fch + l * 4 * nC, d4C, 4 * nC, st);
        }
        {
            KScope k(h, K_MATMUL_BWD_DX, mm_flops(BT, C, 4 * C));
            matmul_bwd_dx<T>(dC, d4C, P[P_FCW] + w4, BT, 4 * C, C, st);
        }
        dw_tasks.push_back({d4C, ln2 + l * nC, G[P_FCW] + w4, G[P_FCB] + l * 4 * C, 4 * C, C});
        {
            KScope k(h, K_LAYERNORM_BWD, ln_bytes(true));
            layernorm_bwd_rows<T>(g1, g2, dC, res2 + l * nC, P[P_LN2W] + l * C,
                                  ln2m + (int64_t)l * BT, ln2r + (int64_t)l * BT, BT, C, lnp,
                                  ln_red.count, st);
            ln_red.t[ln_red.count++] = {G[P_LN2W] + l * C, G[P_LN2B] + l * C};
        }
        // attention
        const int64_t w1 = (int64_t)l * C * C, w3 = (int64_t)l * 3 * C * C;
        {
            KScope k(h, K_MATMUL_BWD_DX, mm_flops(BT, C, C));
            matmul_bwd_dx<T>(dC, g1, P[P_ATTPROJW] + w1, BT, C, C, st);
        }
        dw_tasks.push_back({g1, atty + l * nC, G[P_ATTPROJW] + w1, G[P_ATTPROJB] + l * C, C, C});
        {
            KScope k(h, K_ATTENTION_BWD, attn_flops);
            attention_bwd<T>(d3C, dC, qkv + l * 3 * nC, atty + l * nC,
                             lse + (int64_t)l * B * NH * Tn, attD, B, Tn, C, NH, st);
        }
        {
            KScope k(h, K_MATMUL_BWD_DX, mm_flops(BT, C, 3 * C));
            matmul_bwd_dx<T>(dC, d3C, P[P_QKVW] + w3, BT, 3 * C, C, st);
        }
        dw_tasks.push_back({d3C, ln1 + l * nC, G[P_QKVW] + w3, G[P_QKVB] + l * 3 * C, 3 * C, C});
        {
            KScope k(h, K_LAYERNORM_BWD, ln_bytes(true));
            layernorm_bwd_rows<T>(g0, g1, dC, res, P[P_LN1W] + l * C, ln1m + (int64_t)l * BT,
                                  ln1r + (int64_t)l * BT, BT, C, lnp, ln_red.count, st);
            ln_red.t[ln_red.count++] = {G[P_LN1W] + l * C, G[P_LN1B] + l * C};
        }
        dw_flops += mm_flops(C, 4 * C, BT) + mm_flops(4 * C, C, BT) + mm_flops(C, C, BT) +
                    mm_flops(3 * C, C, BT);
    }
    {
        KScope k(h, K_LAYERNORM_BWD, (double)ln_red.count * layernorm_bwd_partials((int)C, 1) * 4);
        layernorm_bwd_reduce(ln_red, BT, C, lnp, ln_red.count, st);
    }
    {
        KScope k(h, K_MATMUL_BWD_DW, dw_flops);
        matmul_bwd_dw_batch<T>(dw_tasks.data(), (int)dw_tasks.size(), BT, dws, bp, st);
    }
    {
        KScope k(h, K_ENCODER_BWD, nC * es + 4.0 * c.max_T * C + 8.0 * BT);
        encoder_bwd<T>(G[P_WTE], G[P_WPE], R(2 * L), h->last_inputs, B, Tn, C, Vp, c.max_T,
                       h->a[W_ENC], st);
    }
}

}  // namespace


extern "C" {

int64_t gpt2_num_params(const gpt2_config* cfg) {
    if (const char* e = check_config(cfg)) return fail(-1, e);
    Layout lay;
    plan(cfg, &lay);
    return lay.N;
}

int gpt2_num_param_tensors(void) { return NUM_P; }

int gpt2_param_table(const gpt2_config* cfg, int i, const char** name, int64_t* offset,
                     int32_t* ndim, int32_t shape[3]) {
    if (const char* e = check_config(cfg)) return fail(GPT2_ESHAPE, e);
    if (i < 0 || i >= NUM_P) return fail(GPT2_EINVAL, "tensor index out of range");
    Layout lay;
    plan(cfg, &lay);
    const int32_t C = cfg->C, L = cfg->L;
    int32_t sh[3] = {0, 0, 0}, nd = 0;
    switch (i) {
        case P_WTE: nd = 2; sh[0] = cfg->Vp; sh[1] = C; break;
        case P_WPE: nd = 2; sh[0] = cfg->max_T; sh[1] = C; break;
        case P_QKVW: nd = 3; sh[0] = L; sh[1] = 3 * C; sh[2] = C; break;
        case P_QKVB: nd = 2; sh[0] = L; sh[1] = 3 * C; break;
        case P_ATTPROJW: nd = 3; sh[0] = L; sh[1] = C; sh[2] = C; break;
        case P_FCW: nd = 3; sh[0] = L; sh[1] = 4 * C; sh[2] = C; break;
        case P_FCB: nd = 2; sh[0] = L; sh[1] = 4 * C; break;
        case P_FCPROJW: nd = 3; sh[0] = L; sh[1] = C; sh[2] = 4 * C; break;
        case P_LNFW: case P_LNFB: nd = 1; sh[0] = C; break;
        default: nd = 2; sh[0] = L; sh[1] = C; break;  // ln*, attprojb, fcprojb
    }
    if (name) *name = P_NAMES[i];
    if (offset) *offset = lay.poff[i];
    if (ndim) *ndim = nd;
    if (shape) memcpy(shape, sh, sizeof(sh));
    return GPT2_OK;
}

int64_t gpt2_param_buffer_bytes(const gpt2_config* cfg) {
    if (const char* e = check_config(cfg)) return fail(-1, e);
    Layout lay;
    plan(cfg, &lay);
    return lay.param_bytes;
}

int64_t gpt2_act_buffer_bytes(const gpt2_config* cfg) {
    if (const char* e = check_config(cfg)) return fail(-1, e);
    Layout lay;
    plan(cfg, &lay);
    return lay.act_bytes;
}

int gpt2_create(const gpt2_config* cfg, void* d_param_buf, void* d_act_buf,
                const float* h_init_params, void* hip_stream, gpt2** out) {
    if (!out) return fail(GPT2_EINVAL, "out is NULL");
    *out = nullptr;
    if (const char* e = check_config(cfg)) return fail(GPT2_ESHAPE, e);
    if (!d_param_buf || !d_act_buf) return fail(GPT2_EINVAL, "buffer pointer is NULL");
    if ((uintptr_t)d_param_buf % ALIGN || (uintptr_t)d_act_buf % ALIGN)
        return fail(GPT2_EINVAL, "buffers must be 256-byte aligned");
    gpt2* h = new gpt2();
    h->cfg = *cfg;
    plan(cfg, &h->lay);
    h->st = (hipStream_t)hip_stream;
    h->pbuf = (char*)d_param_buf;
    h->abuf = (char*)d_act_buf;
    const Layout& lay = h->lay;
    h->master = (float*)(h->pbuf + lay.region_off[GPT2_REGION_MASTER]);
    h->grad = (float*)(h->pbuf + lay.region_off[GPT2_REGION_GRAD]);
    h->m = (float*)(h->pbuf + lay.region_off[GPT2_REGION_M]);
    h->v = (float*)(h->pbuf + lay.region_off[GPT2_REGION_V]);
    const bool bf = cfg->dtype == GPT2_DTYPE_BF16;
    h->pbf16 = bf ? (bf16*)(h->pbuf + lay.region_off[GPT2_REGION_PARAM_BF16]) : nullptr;
    for (int i = 0; i < NUM_P; i++) {
        h->wp[i] = bf ? (void*)(h->pbf16 + lay.poff[i]) : (void*)(h->master + lay.poff[i]);
        h->gp[i] = h->grad + lay.poff[i];
    }
    for (int i = 0; i < NUM_A; i++) h->a[i] = h->abuf + lay.aoff[i];
    (void)hipGetLastError();  // start from a clean error state
    if (h_init_params) {
        if (hipMemcpyAsync(h->master, h_init_params, lay.N * sizeof(float),
                           hipMemcpyHostToDevice, h->st) != hipSuccess) {
            delete h;
            return fail(GPT2_EHIP, "uploading the initial parameters failed");
        }
    }
    fill_zero_f32(h->grad, lay.N, h->st);
    fill_zero_f32(h->m, lay.N, h->st);
    fill_zero_f32(h->v, lay.N, h->st);
    fill_zero_i32((int*)h->a[A_ERR], 1, h->st);
    if (bf) round_to_bf16(h->pbf16, h->master, lay.N, h->st);
    int rc = hip_status("gpt2_create");
    if (rc == GPT2_OK && hipStreamSynchronize(h->st) != hipSuccess)
        rc = fail(GPT2_EHIP, "gpt2_create: stream synchronisation failed");
    if (rc != GPT2_OK) {
        delete h;
        return rc;
    }
    *out = h;
    return GPT2_OK;
}

int gpt2_forward(gpt2* h, const int32_t* d_inputs, const int32_t* d_targets, float* h_loss) {
    if (!h || !d_inputs) return fail(GPT2_EINVAL, "handle or inputs is NULL");
    if (h_loss && !d_targets) return fail(GPT2_EINVAL, "a loss needs targets");
    if ((uintptr_t)d_inputs % 4 || (uintptr_t)d_targets % 4)
        return fail(GPT2_EINVAL, "token arrays must be 4-byte aligned");
    h->fwd_targets = false;  // until this forward has been issued cleanly
    h->fwd_count = h->fwd_count == INT32_MAX ? 1 : h->fwd_count + 1;
    if (h->cfg.dtype == GPT2_DTYPE_BF16)
        forward_impl<bf16>(h, d_inputs, d_targets);
    else
        forward_impl<float>(h, d_inputs, d_targets);
    h->last_inputs = d_inputs;
    int rc = hip_status("gpt2_forward");
    if (rc != GPT2_OK) return rc;
    h->fwd_targets = d_targets != nullptr;
    if (!h_loss) return GPT2_OK;
    float loss = 0.f;
    int err = 0;
    if (hipMemcpyAsync(&loss, h->a[A_LOSS], 4, hipMemcpyDeviceToHost, h->st) != hipSuccess ||
        hipMemcpyAsync(&err, h->a[A_ERR], 4, hipMemcpyDeviceToHost, h->st) != hipSuccess ||
        hipStreamSynchronize(h->st) != hipSuccess)
        return fail(GPT2_EHIP, "gpt2_forward: reading the loss failed");
    *h_loss = loss;
    if (err) {
        // the flag holds the number of the latest forward that saw a bad id;
        // an unchecked earlier forward is named as such
        fill_zero_i32((int*)h->a[A_ERR], 1, h->st);
        h->fwd_targets = false;
        const int now = h->fwd_count;
        return fail(GPT2_ETOKEN,
                    err == now ? std::string("a token id outside [0, V) was seen in this forward")
                               : "a token id outside [0, V) was seen in forward call " +
                                     std::to_string(err) + " (not checked then); this is call " +
                                     std::to_string(now));
    }
    return GPT2_OK;
}

int gpt2_backward(gpt2* h) {
    if (!h) return fail(GPT2_EINVAL, "handle is NULL");
    if (!h->fwd_targets) return fail(GPT2_ESTATE, "backward needs a forward with targets");
    if (h->cfg.dtype == GPT2_DTYPE_BF16)
        backward_impl<bf16>(h);
    else
        backward_impl<float>(h);
    h->fwd_targets = false;  // dlogits are consumed
    return hip_status("gpt2_backward");
}

int gpt2_update(gpt2* h, float lr, float beta1, float beta2, float eps, float weight_decay,
                int32_t step) {
    if (!h) return fail(GPT2_EINVAL, "handle is NULL");
    if (step < 1) return fail(GPT2_EINVAL, "step must be >= 1");
    const float c1 = (float)(1.0 - pow((double)beta1, (double)step));
    const float c2 = (float)(1.0 - pow((double)beta2, (double)step));
    {
        KScope k(h, K_ADAMW, (double)h->lay.N * (h->pbf16 ? 30.0 : 28.0));
        adamw(h->master, h->grad, h->m, h->v, h->pbf16, h->lay.N, lr, beta1, beta2, eps,
              weight_decay, c1, c2, nullptr, 0.f, h->st);
    }
    return hip_status("gpt2_update");
}

float gpt2_schedule_lr(const gpt2_schedule* s, int32_t step) {
    if (!s || step < 1 || s->warmup_steps < 0 || s->total_steps <= s->warmup_steps) return -1.f;
    if (step <= s->warmup_steps) return s->lr_max * (float)step / (float)s->warmup_steps;
    double p = (double)(step - s->warmup_steps) / (double)(s->total_steps - s->warmup_steps);
    if (p > 1.0) p = 1.0;
    const double pi = 3.14159265358979323846;
    return (float)(s->lr_min + 0.5 * ((double)s->lr_max - s->lr_min) * (1.0 + cos(pi * p)));
}

int gpt2_update_scheduled(gpt2* h, const gpt2_schedule* s, int32_t step) {
    if (!h || !s) return fail(GPT2_EINVAL, "handle or schedule is NULL");
    if (step < 1) return fail(GPT2_EINVAL, "step must be >= 1");
    if (s->warmup_steps < 0 || s->total_steps <= s->warmup_steps)
        return fail(GPT2_EINVAL, "schedule needs 0 <= warmup_steps < total_steps");
    const float lr = gpt2_schedule_lr(s, step);
    const float c1 = (float)(1.0 - pow((double)s->beta1, (double)step));
    const float c2 = (float)(1.0 - pow((double)s->beta2, (double)step));
    const bool clip = s->grad_clip > 0.f;
    {
        KScope k(h, K_ADAMW, (double)h->lay.N * ((h->pbf16 ? 30.0 : 28.0) + (clip ? 4.0 : 0.0)));
        float* nrm = static_cast<float*>(h->a[A_GNORM]);
        if (clip)
            grad_norm(nrm, static_cast<float*>(h->a[W_GNORM_PART]), h->grad, h->lay.N, h->st);
        adamw(h->master, h->grad, h->m, h->v, h->pbf16, h->lay.N, lr, s->beta1, s->beta2, s->eps,
              s->weight_decay, c1, c2, clip ? nrm : nullptr, s->grad_clip, h->st);
    }
    return hip_status("gpt2_update_scheduled");
}

// ---------------------------------------------------------------------------
// Checkpoints (page "Building GPT-2 from scratch", exercise table row A5:
// bit-exact checkpoint resume). The training state is the master parameters
// and both AdamW moments plus the step; the bf16 working copy is a function
// of the master parameters and gradients are rebuilt by every backward pass.
// Host image: a 128-byte header, then master, m and v (N fp32 each).
namespace {
constexpr char CKPT_MAGIC[8] = {'G', 'P', 'T', '2', 'C', 'K', 'P', '1'};
constexpr int CKPT_HEADER = 128;
struct CkptHeader {
    char magic[8];
    uint32_t version, header_bytes;
    gpt2_config cfg;
    int32_t pad0;
    int64_t N, step;
};
static_assert(sizeof(CkptHeader) <= CKPT_HEADER, "checkpoint header");

bool same_model(const gpt2_config& a, const gpt2_config& b) {
    return a.V == b.V && a.Vp == b.Vp && a.max_T == b.max_T && a.C == b.C && a.L == b.L &&
           a.NH == b.NH && a.dtype == b.dtype;
}
}  // namespace

int64_t gpt2_checkpoint_bytes(const gpt2_config* cfg) {
    const int64_t n = gpt2_num_params(cfg);
    return n < 0 ? -1 : CKPT_HEADER + 3 * n * (int64_t)sizeof(float);
}

int gpt2_checkpoint_save(gpt2* h, int64_t step, void* host_buf, int64_t bytes) {
    if (!h || !host_buf) return fail(GPT2_EINVAL, "handle or host_buf is NULL");
    const int64_t need = gpt2_checkpoint_bytes(&h->cfg);
    if (bytes < need) return fail(GPT2_EINVAL, "host_buf is smaller than gpt2_checkpoint_bytes()");
    CkptHeader hd;
    memset(&hd, 0, sizeof(hd));
    memcpy(hd.magic, CKPT_MAGIC, 8);
    hd.version = 1;
    hd.header_bytes = CKPT_HEADER;
    hd.cfg = h->cfg;
    hd.N = h->lay.N;
    hd.step = step;
    char* out = static_cast<char*>(host_buf);
    memset(out, 0, CKPT_HEADER);
    memcpy(out, &hd, sizeof(hd));
    const size_t nb = (size_t)h->lay.N * sizeof(float);
    const float* src[3] = {h->master, h->m, h->v};
    for (int i = 0; i < 3; i++)
        if (hipMemcpyAsync(out + CKPT_HEADER + i * nb, src[i], nb, hipMemcpyDeviceToHost, h->st) !=
            hipSuccess)
            return fail(GPT2_EHIP, "gpt2_checkpoint_save: copy to the host failed");
    if (hipStreamSynchronize(h->st) != hipSuccess)
        return fail(GPT2_EHIP, "gpt2_checkpoint_save: stream synchronisation failed");
    return hip_status("gpt2_checkpoint_save");
}

int gpt2_checkpoint_load(gpt2* h, const void* host_buf, int64_t bytes, int64_t* step) {
    if (!h || !host_buf) return fail(GPT2_EINVAL, "handle or host_buf is NULL");
    if (bytes < CKPT_HEADER) return fail(GPT2_EINVAL, "checkpoint shorter than its header");
    CkptHeader hd;
    memcpy(&hd, host_buf, sizeof(hd));
    if (memcmp(hd.magic, CKPT_MAGIC, 8) != 0 || hd.version != 1 || hd.header_bytes != CKPT_HEADER)
        return fail(GPT2_EINVAL, "not a checkpoint of this format");
    if (!same_model(hd.cfg, h->cfg) || hd.N != h->lay.N)
        return fail(GPT2_ESHAPE, "checkpoint of a different model or precision");
    if (bytes < gpt2_checkpoint_bytes(&h->cfg)) return fail(GPT2_EINVAL, "checkpoint truncated");
    const char* in = static_cast<const char*>(host_buf);
    const size_t nb = (size_t)h->lay.N * sizeof(float);
    float* dst[3] = {h->master, h->m, h->v};
    for (int i = 0; i < 3; i++)
        if (hipMemcpyAsync(dst[i], in + CKPT_HEADER + i * nb, nb, hipMemcpyHostToDevice, h->st) !=
            hipSuccess)
            return fail(GPT2_EHIP, "gpt2_checkpoint_load: copy to the device failed");
    fill_zero_f32(h->grad, h->lay.N, h->st);
    if (h->pbf16) round_to_bf16(h->pbf16, h->master, h->lay.N, h->st);
    h->fwd_targets = false;
    if (hipStreamSynchronize(h->st) != hipSuccess)
        return fail(GPT2_EHIP, "gpt2_checkpoint_load: stream synchronisation failed");
    if (step) *step = hd.step;
    return hip_status("gpt2_checkpoint_load");
}

int gpt2_region(gpt2* h, int which, void** d_ptr) {
    if (!h || !d_ptr) return fail(GPT2_EINVAL, "handle or d_ptr is NULL");
    if (which < 0 || which > 4) return fail(GPT2_EINVAL, "unknown region");
    if (which == GPT2_REGION_PARAM_BF16 && h->cfg.dtype != GPT2_DTYPE_BF16)
        return fail(GPT2_EINVAL, "no bf16 region in fp32 mode");
    *d_ptr = h->pbuf + h->lay.region_off[which];
    return GPT2_OK;
}

int gpt2_act(gpt2* h, const char* name, void** d_ptr, int64_t* bytes) {
    if (!h || !name) return fail(GPT2_EINVAL, "handle or name is NULL");
    for (int i = 0; i < NUM_A; i++)
        if (strcmp(name, A_NAMES[i]) == 0) {
            if (d_ptr) *d_ptr = h->a[i];
            if (bytes) *bytes = h->lay.abytes[i];
            return GPT2_OK;
        }
    return fail(GPT2_EINVAL, "unknown activation name");
}

int gpt2_timing_arm(gpt2* h, const char* prefix, int32_t max_launches) {
    if (!h) return fail(GPT2_EINVAL, "handle is NULL");
    destroy_events(h);
    if (!prefix) return GPT2_OK;
    if (max_launches <= 0) return fail(GPT2_EINVAL, "max_launches must be > 0");
    h->ev.resize(2 * (size_t)max_launches);
    for (auto& e : h->ev)
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            destroy_events(h);
            return fail(GPT2_EHIP, "hipEventCreate failed");
        }
    h->rec_cls.assign(max_launches, 0);
    h->rec_work.assign(max_launches, 0.0);
    const size_t n = strlen(prefix);
    for (int k = 0; k < NUM_K; k++) h->tarm[k] = strncmp(K_NAMES[k], prefix, n) == 0;
    return GPT2_OK;
}

int gpt2_timing_classes(void) { return NUM_K; }

int gpt2_timing_read(gpt2* h, int i, const char** name, int64_t* launches, double* total_ms,
                     double* work, int32_t* work_is_bytes) {
    if (!h) return fail(GPT2_EINVAL, "handle is NULL");
    if (i < 0 || i >= NUM_K) return fail(GPT2_EINVAL, "class index out of range");
    if (hipStreamSynchronize(h->st) != hipSuccess) return fail(GPT2_EHIP, "synchronisation failed");
    int64_t n = 0;
    double ms = 0.0, wk = 0.0;
    for (int64_t r = 0; r < h->nrec; r++) {
        if (h->rec_cls[r] != i) continue;
        float t = 0.f;
        if (hipEventElapsedTime(&t, h->ev[2 * r], h->ev[2 * r + 1]) != hipSuccess)
            return fail(GPT2_EHIP, "hipEventElapsedTime failed");
        n++;
        ms += t;
        wk += h->rec_work[r];
    }
    if (name) *name = K_NAMES[i];
    if (launches) *launches = n;
    if (total_ms) *total_ms = ms;
    if (work) *work = wk;
    if (work_is_bytes) *work_is_bytes = K_IS_BYTES[i];
    return GPT2_OK;
}

void gpt2_free(gpt2* h) {
    if (!h) return;
    destroy_events(h);
    delete h;
}

const char* gpt2_last_error(void) { return g_err.c_str(); }

// ---- FP8 (E4M3) products ------------------------------------------------------

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int64_t gpt2_fp8_scale_workspace_bytes(void) { return fp8_scale_workspace_floats() * 4; }

int gpt2_fp8_scale(float* scale, void* work, const void* x, int64_t n, void* hip_stream) {
    if (!scale || !work || (!x && n > 0)) return fail(GPT2_EINVAL, "null pointer");
    if (n < 0) return fail(GPT2_EINVAL, "negative size");
    if (!aligned16(x) || ((uintptr_t)work & 255)) return fail(GPT2_EINVAL, "misaligned pointer");
    fp8_scale(scale, (float*)work, (const bf16*)x, n, (hipStream_t)hip_stream);
    return hip_status("gpt2_fp8_scale");
}

int gpt2_fp8_quantize(uint8_t* q, const void* x, const float* scale, int64_t n,
                      void* hip_stream) {
    if (!scale || ((!q || !x) && n > 0)) return fail(GPT2_EINVAL, "null pointer");
    if (n < 0) return fail(GPT2_EINVAL, "negative size");
    if (!aligned16(q) || !aligned16(x)) return fail(GPT2_EINVAL, "misaligned pointer");
    if (n == 0) return GPT2_OK;
    fp8_quantize(q, (const bf16*)x, scale, n, (hipStream_t)hip_stream);
    return hip_status("gpt2_fp8_quantize");
}

int gpt2_fp8_matmul(void* out, const uint8_t* qx, const uint8_t* qw, const float* scales,
                    const void* bias, int32_t M, int32_t N, int32_t K, void* hip_stream) {
    if (!out || !qx || !qw || !scales) return fail(GPT2_EINVAL, "null pointer");
    if (!aligned16(out) || !aligned16(qx) || !aligned16(qw) || !aligned16(bias))
        return fail(GPT2_EINVAL, "misaligned pointer");
    if (M <= 0 || N <= 0 || K <= 0) return fail(GPT2_ESHAPE, "M, N, K must be positive");
    if (K % 128 != 0 || N % 8 != 0)
        return fail(GPT2_ESHAPE, "K must be a multiple of 128 and N of 8");
    if (!gemm_fp8_fwd((bf16*)out, qx, qw, scales, (const bf16*)bias, M, N, K,
                      (hipStream_t)hip_stream))
        return fail(GPT2_ESHAPE, "unsupported shape");
    return hip_status("gpt2_fp8_matmul");
}

int gpt2_attention_forward(void* out, float* lse, const void* qkv, int32_t B, int32_t T,
                           int32_t C, int32_t NH, int32_t dtype, void* hip_stream) {
    if (!out || !lse || !qkv) return fail(GPT2_EINVAL, "null pointer");
    if (!aligned16(out) || !aligned16(qkv) || !aligned16(lse))
        return fail(GPT2_EINVAL, "misaligned pointer");
    if (dtype != GPT2_DTYPE_FP32 && dtype != GPT2_DTYPE_BF16)
        return fail(GPT2_EINVAL, "dtype must be 0 or 1");
    if (B <= 0 || T <= 0 || C <= 0 || NH <= 0)
        return fail(GPT2_ESHAPE, "B, T, C, NH must be positive");
    if (C % 8 != 0 || C > 2048 || C % NH != 0 || (C / NH) % 8 != 0 || C / NH > 128)
        return fail(GPT2_ESHAPE, "need C % 8 == 0, C <= 2048, head size C/NH a multiple of 8, at most 128");
    if ((int64_t)B * T > 524288 || (int64_t)B * NH > 65535)
        return fail(GPT2_ESHAPE, "need B*T <= 524288 and B*NH <= 65535");
    const hipStream_t st = (hipStream_t)hip_stream;
    if (dtype == GPT2_DTYPE_BF16)
        attention_fwd<bf16>((bf16*)out, lse, (const bf16*)qkv, B, T, C, NH, st);
    else
        attention_fwd<float>((float*)out, lse, (const float*)qkv, B, T, C, NH, st);
    return hip_status("gpt2_attention_forward");
}

// Validation shared by the attention backward entry points.
static int attention_bwd_args(const void* dqkv, const void* dout, const void* qkv, const void* out,
                              const float* lse, int32_t B, int32_t T, int32_t C, int32_t NH,
                              int32_t dtype) {
    if (!dqkv || !dout || !qkv || !out || !lse) return fail(GPT2_EINVAL, "null pointer");
    if (!aligned16(dqkv) || !aligned16(dout) || !aligned16(qkv) || !aligned16(out) ||
        !aligned16(lse))
        return fail(GPT2_EINVAL, "misaligned pointer");
    if (dtype != GPT2_DTYPE_FP32 && dtype != GPT2_DTYPE_BF16)
        return fail(GPT2_EINVAL, "dtype must be 0 or 1");
    if (B <= 0 || T <= 0 || C <= 0 || NH <= 0)
        return fail(GPT2_ESHAPE, "B, T, C, NH must be positive");
    if (C % 8 != 0 || C > 2048 || C % NH != 0 || (C / NH) % 8 != 0 || C / NH > 128)
        return fail(GPT2_ESHAPE, "need C % 8 == 0, C <= 2048, head size C/NH a multiple of 8, at most 128");
    if ((int64_t)B * T > 524288 || (int64_t)B * NH > 65535)
        return fail(GPT2_ESHAPE, "need B*T <= 524288 and B*NH <= 65535");
    return GPT2_OK;
}

static void attention_bwd_launch(void* dqkv, float* work, const void* dout, const void* qkv,
                                 const void* out, const float* lse, int B, int T, int C, int NH,
                                 int dtype, hipStream_t st) {
    if (dtype == GPT2_DTYPE_BF16)
        attention_bwd<bf16>((bf16*)dqkv, (const bf16*)dout, (const bf16*)qkv, (const bf16*)out, lse,
                            work, B, T, C, NH, st);
    else
        attention_bwd<float>((float*)dqkv, (const float*)dout, (const float*)qkv,
                             (const float*)out, lse, work, B, T, C, NH, st);
}

// Scratch of gpt2_attention_backward_noalloc: the rows' D values and base-2
// log-sum-exp, 2*B*NH*T floats at most. A file-scope device array: each GPU the library runs on
// holds one copy until the process ends. Host code never uses the array's
// name as an address; it uses the per-device address hipGetSymbolAddress
// returns, looked up once per device with that device current.
#define NOALLOC_SCRATCH_FLOATS (1 << 20)
#define NOALLOC_MAX_DEVICES 64
static __device__ __align__(256) float scratch[NOALLOC_SCRATCH_FLOATS];
static std::mutex g_scratch_mu;
static float* g_scratch_ptr[NOALLOC_MAX_DEVICES];

// Address of the current device's scratch (looked up on its first use).
static int scratch_of_current_device(float** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(GPT2_EHIP, "hipGetDevice failed");
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
        return fail(GPT2_EINVAL, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(GPT2_EHIP, "hipGetSymbolAddress(scratch) failed");
        }
        g_scratch_ptr[dev] = static_cast<float*>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return GPT2_OK;
}

int gpt2_attention_backward_noalloc(void* dqkv, const void* dout, const void* qkv,
                                    const void* out, const float* lse, int32_t B, int32_t T,
                                    int32_t C, int32_t NH, int32_t dtype, void* hip_stream) {
    int rc = attention_bwd_args(dqkv, dout, qkv, out, lse, B, T, C, NH, dtype);
    if (rc != GPT2_OK) return rc;
    const int64_t need = 2 * (int64_t)B * NH * T;
    if (need > NOALLOC_SCRATCH_FLOATS)
        return fail(GPT2_ESHAPE, "2*B*NH*T = " + std::to_string(need) +
                                     " exceeds the static scratch of " +
                                     std::to_string(NOALLOC_SCRATCH_FLOATS) + " floats");
    const hipStream_t st = (hipStream_t)hip_stream;
    if (st) {
        int cur = -1, sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(st, &sdev) != hipSuccess)
            return fail(GPT2_EHIP, "querying the stream's device failed");
        if (cur != sdev)
            return fail(GPT2_EINVAL, "the stream belongs to a device other than the current one");
    }
    float* work = nullptr;
    rc = scratch_of_current_device(&work);
    if (rc != GPT2_OK) return rc;
    attention_bwd_launch(dqkv, work, dout, qkv, out, lse, B, T, C, NH, dtype, st);
    return hip_status("gpt2_attention_backward_noalloc");
}

int gpt2_attention_backward(void* dqkv, float* work, const void* dout, const void* qkv,
                            const void* out, const float* lse, int32_t B, int32_t T, int32_t C,
                            int32_t NH, int32_t dtype, void* hip_stream) {
    const int rc = attention_bwd_args(dqkv, dout, qkv, out, lse, B, T, C, NH, dtype);
    if (rc != GPT2_OK) return rc;
    if (!work) return fail(GPT2_EINVAL, "null pointer");
    if (!aligned16(work)) return fail(GPT2_EINVAL, "misaligned pointer");
    attention_bwd_launch(dqkv, work, dout, qkv, out, lse, B, T, C, NH, dtype,
                         (hipStream_t)hip_stream);
    return hip_status("gpt2_attention_backward");
}

}  // extern "C"
