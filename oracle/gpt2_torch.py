"""The same GPT-2 training step as oracle/gpt2_oracle.c, written over PyTorch
CPU tensors, for model and batch sizes that the plain C loops cannot step in
reasonable time (the 124M model at B=16, T=1024 for 20 steps; the 350M and
1.5B shapes at full depth and batch).

TEST INFRASTRUCTURE ONLY. Only the test suite, the scripts that write the
stored expected values under tests/golden/, the smoke check and the
benchmark's CPU-baseline leg may use it; the product path never does. It
shares no code with the GPU library and reads only the bytes that
transformer_lm_amd.synth writes.

What differs from the C file is the form, not the arithmetic:
  - every matrix product is one call of the library's matrix multiply (a
    step the definition names, so a library primitive may take it); its
    summation order is the library's, so results agree with the C file up to
    rounding, not bit for bit;
  - the attention probabilities are not kept between the forward and the
    backward: the backward recomputes them from the saved qkv with the same
    formula (this keeps the 1.5B shape inside host memory);
  - GELU of the fc output is recomputed in the backward for the same reason.
Everything else is the plain definition, step for step in the order of the C
file: LayerNorm with the biased variance and eps = 1e-5 inside the root
(talk "llm.c's Origin and the Future of LLM Compilers", chapter
"Deconstructing PyTorch Abstractions"); the fused [Q; K; V] weight, causal
softmax attention with scale 1/sqrt(hs) materialised as full T x T score
matrices per sequence; tanh GELU; softmax and cross-entropy over the real
vocabulary only with zero gradient in the padded columns; the mean loss over
all B*T positions; the hand-derived gradients of each operation (page
"llm.c: Large Language Model Training in Pure C/CUDA Without Dependencies",
section "Exact Analytical Backward Pass"); AdamW with bias correction from
t = 1, eps outside the root and decay lr*wd*theta over the whole flat array
(page "Building GPT-2 from scratch", exercise table row A2).

Precision: float32 by default -- the bf16 training step is compared with the
fp32 oracle -- or float64 (dtype=torch.float64), in which the tests pin it to
the C oracle's double build element by element.
"""
import math

import numpy as np
import torch

LN_EPS = 1e-5
GELU_K = math.sqrt(2.0 / math.pi)
GELU_C = 0.044715


def _param_shapes(w):
    C, L = w.C, w.L
    return [("wte", (w.Vp, C)), ("wpe", (w.max_T, C)),
            ("ln1w", (L, C)), ("ln1b", (L, C)),
            ("qkvw", (L, 3 * C, C)), ("qkvb", (L, 3 * C)),
            ("attprojw", (L, C, C)), ("attprojb", (L, C)),
            ("ln2w", (L, C)), ("ln2b", (L, C)),
            ("fcw", (L, 4 * C, C)), ("fcb", (L, 4 * C)),
            ("fcprojw", (L, C, 4 * C)), ("fcprojb", (L, C)),
            ("lnfw", (C,)), ("lnfb", (C,))]


def _views(flat, w):
    out, off = {}, 0
    for name, shape in _param_shapes(w):
        n = math.prod(shape)
        out[name] = flat[off:off + n].view(*shape)
        off += n
    assert off == flat.numel()
    return out


# ---------------------------------------------------------------------------
# Operations (each the definition named in its docstring)
# ---------------------------------------------------------------------------

def layernorm_forward(x, weight, bias):
    """mu = mean(x), var = mean((x - mu)^2), r = 1/sqrt(var + eps),
    y = (x - mu) r weight + bias; returns y, mu, r."""
    mu = x.mean(dim=-1, keepdim=True)
    d = x - mu
    var = (d * d).mean(dim=-1, keepdim=True)
    r = 1.0 / torch.sqrt(var + LN_EPS)
    return d * r * weight + bias, mu, r


def layernorm_backward(dy, x, weight, mu, r):
    """With xhat = (x - mu) r and g = weight * dy:
    dx = r (g - mean(g) - xhat mean(g xhat)); dweight = sum_n dy xhat;
    dbias = sum_n dy."""
    xhat = (x - mu) * r
    g = weight * dy
    gm = g.mean(dim=-1, keepdim=True)
    gxm = (g * xhat).mean(dim=-1, keepdim=True)
    dx = (g - gm - xhat * gxm) * r
    return dx, (dy * xhat).sum(dim=0), dy.sum(dim=0)


def matmul_forward(x, weight, bias):
    """y = x weight^T + bias with weight stored (out, in)."""
    y = x @ weight.t()
    if bias is not None:
        y += bias
    return y


def matmul_backward(dy, x, weight):
    """dx = dy weight; dweight = dy^T x; dbias = sum_n dy."""
    return dy @ weight, dy.t() @ x, dy.sum(dim=0)


def gelu_forward(u):
    """g(u) = u/2 (1 + tanh(a)), a = sqrt(2/pi) (u + 0.044715 u^3)."""
    a = GELU_K * (u + GELU_C * u * u * u)
    return 0.5 * u * (1.0 + torch.tanh(a))


def gelu_backward(u, dy):
    """g'(u) dy with g'(u) = (1 + tanh a)/2 + u/2 (1 - tanh^2 a) sqrt(2/pi) (1 + 3 * 0.044715 u^2)."""
    a = GELU_K * (u + GELU_C * u * u * u)
    th = torch.tanh(a)
    da = GELU_K * (1.0 + 3.0 * GELU_C * u * u)
    return (0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * da) * dy


def _heads(qkv_b, C, NH):
    """(T, 3C) rows of one sequence -> q, k, v as (NH, T, hs)."""
    T = qkv_b.shape[0]
    hs = C // NH
    q = qkv_b[:, :C].reshape(T, NH, hs).transpose(0, 1)
    k = qkv_b[:, C:2 * C].reshape(T, NH, hs).transpose(0, 1)
    v = qkv_b[:, 2 * C:].reshape(T, NH, hs).transpose(0, 1)
    return q, k, v


def attention_probs(q, k):
    """Causal softmax of the scaled scores of one sequence, all heads:
    s[t, t2] = q_t . k_t2 / sqrt(hs) for t2 <= t; P = exp(s - max_t2 s) / sum
    over t2 <= t; P = 0 above the diagonal."""
    T, hs = q.shape[1], q.shape[2]
    s = (q @ k.transpose(1, 2)) * (1.0 / math.sqrt(hs))
    mask = torch.ones(T, T, dtype=torch.bool).triu_(1)
    s.masked_fill_(mask, -math.inf)
    s -= s.amax(dim=-1, keepdim=True)
    p = torch.exp(s)
    p /= p.sum(dim=-1, keepdim=True)
    return p


def attention_forward(qkv, B, T, C, NH):
    """y_t = sum_{t2 <= t} P[t, t2] v_t2 per head; qkv (B*T, 3C) -> y (B*T, C)."""
    y = torch.empty(B * T, C, dtype=qkv.dtype)
    for b in range(B):
        q, k, v = _heads(qkv[b * T:(b + 1) * T], C, NH)
        yb = attention_probs(q, k) @ v                     # (NH, T, hs)
        y[b * T:(b + 1) * T] = yb.transpose(0, 1).reshape(T, C)
    return y


def attention_backward(dy, qkv, B, T, C, NH):
    """dP = dy v^T; dv = P^T dy; dS = P (dP - rowsum(P dP)); dq = dS k / sqrt(hs);
    dk = dS^T q / sqrt(hs). P is recomputed from qkv. Returns dqkv (B*T, 3C)."""
    hs = C // NH
    scale = 1.0 / math.sqrt(hs)
    dqkv = torch.empty(B * T, 3 * C, dtype=qkv.dtype)
    for b in range(B):
        q, k, v = _heads(qkv[b * T:(b + 1) * T], C, NH)
        p = attention_probs(q, k)
        dyb = dy[b * T:(b + 1) * T].reshape(T, NH, hs).transpose(0, 1)
        dp = dyb @ v.transpose(1, 2)
        dv = p.transpose(1, 2) @ dyb
        ds = p * (dp - (p * dp).sum(dim=-1, keepdim=True))
        dq = (ds @ k) * scale
        dk = (ds.transpose(1, 2) @ q) * scale
        rows = dqkv[b * T:(b + 1) * T]
        rows[:, :C] = dq.transpose(0, 1).reshape(T, C)
        rows[:, C:2 * C] = dk.transpose(0, 1).reshape(T, C)
        rows[:, 2 * C:] = dv.transpose(0, 1).reshape(T, C)
    return dqkv


def softmax_over_vocab_(logits, V):
    """In place: row softmax over the first V columns; padded columns -> 0."""
    z = logits[:, :V]
    z -= z.amax(dim=-1, keepdim=True)
    torch.exp(z, out=z)
    z /= z.sum(dim=-1, keepdim=True)
    logits[:, V:] = 0
    return logits


def adamw_(theta, g, m, v, lr, b1, b2, eps, wd, t):
    """m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2; mhat = m/(1-b1^t);
    vhat = v/(1-b2^t); theta -= lr (mhat/(sqrt(vhat) + eps) + wd theta).
    Walks the flat arrays in slices to bound the temporaries."""
    c1 = 1.0 - b1 ** t
    c2 = 1.0 - b2 ** t
    n = theta.numel()
    step = 1 << 24
    for i in range(0, n, step):
        th, gi, mi, vi = theta[i:i + step], g[i:i + step], m[i:i + step], v[i:i + step]
        mi.mul_(b1).add_(gi, alpha=1.0 - b1)
        vi.mul_(b2).add_(gi * gi, alpha=1.0 - b2)
        upd = (mi / c1) / (torch.sqrt(vi / c2) + eps) + wd * th
        th.sub_(lr * upd)


# ---------------------------------------------------------------------------
# The model
# ---------------------------------------------------------------------------

class TorchOracle:
    """One model: forward (mean loss), backward (overwrites all parameter
    gradients), update (AdamW step t), as the GPU step has them."""

    def __init__(self, w, params, dtype=torch.float32, threads=None):
        if threads:
            torch.set_num_threads(int(threads))
        self.w = w
        self.dtype = dtype
        params = np.ascontiguousarray(params, dtype=np.float32)
        assert params.size == sum(math.prod(s) for _, s in _param_shapes(w))
        if dtype == torch.float32:
            self.theta = torch.from_numpy(params.copy())
        else:
            self.theta = torch.from_numpy(params).to(dtype)
        self.grad = torch.zeros_like(self.theta)
        self.m = torch.zeros_like(self.theta)
        self.v = torch.zeros_like(self.theta)
        self.p = _views(self.theta, w)
        self.g = _views(self.grad, w)
        self.saved = None

    def forward(self, inputs, targets):
        w = self.w
        B, T = inputs.shape
        C, L, NH, V = w.C, w.L, w.NH, w.V
        BT = B * T
        tok = torch.from_numpy(np.ascontiguousarray(inputs, np.int64)).reshape(-1)
        tgt = torch.from_numpy(np.ascontiguousarray(targets, np.int64)).reshape(-1)
        if int(tok.min()) < 0 or int(tok.max()) >= V or int(tgt.min()) < 0 or \
                int(tgt.max()) >= V:
            raise ValueError("token id outside [0, V)")
        p = self.p
        # encoder: x0[b, t] = wte[tok] + wpe[t]
        pos = torch.arange(T).repeat(B)
        x = p["wte"][tok] + p["wpe"][pos]
        layers = []
        for l in range(L):
            ln1, mu1, r1 = layernorm_forward(x, p["ln1w"][l], p["ln1b"][l])
            qkv = matmul_forward(ln1, p["qkvw"][l], p["qkvb"][l])
            atty = attention_forward(qkv, B, T, C, NH)
            res2 = x + matmul_forward(atty, p["attprojw"][l], p["attprojb"][l])
            ln2, mu2, r2 = layernorm_forward(res2, p["ln2w"][l], p["ln2b"][l])
            fch = matmul_forward(ln2, p["fcw"][l], p["fcb"][l])
            res3 = res2 + matmul_forward(gelu_forward(fch), p["fcprojw"][l], p["fcprojb"][l])
            layers.append(dict(x=x, ln1=ln1, mu1=mu1, r1=r1, qkv=qkv, atty=atty, res2=res2,
                               ln2=ln2, mu2=mu2, r2=r2, fch=fch))
            x = res3
        lnf, muf, rf = layernorm_forward(x, p["lnfw"], p["lnfb"])
        probs = softmax_over_vocab_(matmul_forward(lnf, p["wte"], None), V)
        losses = -torch.log(probs[torch.arange(BT), tgt])
        self.saved = dict(tok=tok, tgt=tgt, B=B, T=T, layers=layers, xL=x, lnf=lnf, muf=muf,
                          rf=rf, probs=probs)
        self.losses = losses.double().numpy()
        return float(losses.double().mean())

    def backward(self):
        if self.saved is None:
            raise RuntimeError("backward needs a forward with targets")
        s, w, p, g = self.saved, self.w, self.p, self.g
        B, T = s["B"], s["T"]
        C, L, NH, V = w.C, w.L, w.NH, w.V
        BT = B * T
        self.grad.zero_()
        # d(mean loss)/dz = (P - onehot) / BT over the real vocabulary, 0 beyond
        dz = s.pop("probs")
        dz[torch.arange(BT), s["tgt"]] -= 1.0
        dz[:, :V] *= 1.0 / BT
        dlnf, dwte_head, _ = matmul_backward(dz, s["lnf"], p["wte"])
        del dz
        g["wte"] += dwte_head
        del dwte_head
        dx, dw_, db_ = layernorm_backward(dlnf, s["xL"], p["lnfw"], s["muf"], s["rf"])
        g["lnfw"] += dw_
        g["lnfb"] += db_
        for l in range(L - 1, -1, -1):
            a = s["layers"][l]
            # x3 = x2 + fcproj(gelu(fc(ln2(x2))))
            gl = gelu_forward(a["fch"])
            dgelu, dW, db = matmul_backward(dx, gl, p["fcprojw"][l])
            g["fcprojw"][l] += dW
            g["fcprojb"][l] += db
            del gl
            dfch = gelu_backward(a["fch"], dgelu)
            del dgelu
            dln2, dW, db = matmul_backward(dfch, a["ln2"], p["fcw"][l])
            g["fcw"][l] += dW
            g["fcb"][l] += db
            del dfch
            dres2, dw_, db_ = layernorm_backward(dln2, a["res2"], p["ln2w"][l], a["mu2"], a["r2"])
            g["ln2w"][l] += dw_
            g["ln2b"][l] += db_
            dx = dx + dres2
            # x2 = x + attproj(attention(qkv(ln1(x))))
            datty, dW, db = matmul_backward(dx, a["atty"], p["attprojw"][l])
            g["attprojw"][l] += dW
            g["attprojb"][l] += db
            dqkv = attention_backward(datty, a["qkv"], B, T, C, NH)
            del datty
            dln1, dW, db = matmul_backward(dqkv, a["ln1"], p["qkvw"][l])
            g["qkvw"][l] += dW
            g["qkvb"][l] += db
            del dqkv
            dres, dw_, db_ = layernorm_backward(dln1, a["x"], p["ln1w"][l], a["mu1"], a["r1"])
            g["ln1w"][l] += dw_
            g["ln1b"][l] += db_
            dx = dx + dres
            s["layers"][l] = None
        # encoder: each position adds its row to its token's and its position's rows
        g["wte"].index_add_(0, s["tok"], dx)
        g["wpe"][:T] += dx.view(B, T, C).sum(dim=0)
        self.saved = None

    def update(self, lr, b1, b2, eps, wd, t):
        adamw_(self.theta, self.grad, self.m, self.v, lr, b1, b2, eps, wd, int(t))

    def params(self):
        """A float64 copy of the parameters."""
        return self.theta.to(torch.float64, copy=True).numpy()

    def grads(self):
        """A float64 copy of the last backward's gradients."""
        return self.grad.to(torch.float64, copy=True).numpy()
