"""Pins for the oracle's individual operations, CPU only.

Each operation is checked against something other than itself: a closed form,
an invariant, brute force, or an independent library routine (PyTorch's CPU
float64 kernels and autograd) computing the same defined quantity. The oracle is
the double-precision build unless a test says otherwise.
"""
import ctypes as ct
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.wrapper import ptr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = ct.c_double
I = ct.c_int


def _rng(seed):
    return np.random.default_rng(seed)


def _c(a, dtype=np.float64):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ encoder --

@pytest.mark.parametrize("prec", ["f64", "f32"])
def test_encoder_forward_is_exact_gather_add(prec, oracle_lib, oracle_lib32):
    lib = oracle_lib if prec == "f64" else oracle_lib32
    dt = np.float64 if prec == "f64" else np.float32
    ctype = D if prec == "f64" else ct.c_float
    r = _rng(1)
    B, T, C, V = 3, 5, 8, 11
    wte = _c(r.normal(size=(V, C)), dt)
    wpe = _c(r.normal(size=(7, C)), dt)
    tok = _c(r.integers(0, V, size=(B, T)), np.int32)
    out = np.zeros((B, T, C), dt)
    lib.oracle_encoder_forward(ptr(out, ctype), ptr(tok, I), ptr(wte, ctype), ptr(wpe, ctype), B, T, C)
    expect = wte[tok] + wpe[None, :T]          # one IEEE add per element
    assert np.array_equal(out, expect)


def test_encoder_backward_scatter(oracle_lib):
    r = _rng(2)
    B, T, C, V = 2, 6, 4, 5
    tok = _c(r.integers(0, V, size=(B, T)), np.int32)
    tok[0, 0] = tok[1, 3] = 2                  # repeated ids must accumulate
    dout = _c(r.normal(size=(B, T, C)))
    dwte = np.zeros((V, C))
    dwpe = np.zeros((8, C))
    oracle_lib.oracle_encoder_backward(ptr(dwte, D), ptr(dwpe, D), ptr(dout, D), ptr(tok, I), B, T, C)
    ewte = np.zeros((V, C))
    np.add.at(ewte, tok.reshape(-1), dout.reshape(-1, C))
    assert np.allclose(dwte, ewte, rtol=0, atol=1e-14)
    assert np.allclose(dwpe[:T], dout.sum(0), rtol=0, atol=1e-14)
    assert not dwpe[T:].any()                   # rows past T get no gradient


# ---------------------------------------------------------------- layernorm --

def _ln_fwd(lib, x, w, b):
    N, C = x.shape
    out = np.zeros_like(x)
    mean = np.zeros(N)
    rstd = np.zeros(N)
    lib.oracle_layernorm_forward(ptr(out, D), ptr(mean, D), ptr(rstd, D), ptr(x, D), ptr(w, D),
                                 ptr(b, D), N, C)
    return out, mean, rstd


def test_layernorm_forward_closed_form(oracle_lib):
    r = _rng(3)
    N, C = 16, 48
    x = _c(r.normal(loc=3.0, scale=2.0, size=(N, C)))
    y, mean, rstd = _ln_fwd(oracle_lib, x, np.ones(C), np.zeros(C))
    var = x.var(axis=1)                          # biased
    assert np.abs(y.mean(axis=1)).max() < 1e-12
    # "unit variance" up to eps: var(y) = var / (var + eps)
    assert np.allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12, atol=0)
    assert np.allclose(mean, x.mean(axis=1), rtol=1e-13)
    assert np.allclose(rstd, 1 / np.sqrt(var + 1e-5), rtol=1e-13)


def test_layernorm_forward_matches_torch(oracle_lib):
    r = _rng(4)
    N, C = 10, 32
    x, w, b = _c(r.normal(size=(N, C))), _c(r.normal(size=C)), _c(r.normal(size=C))
    y, _, _ = _ln_fwd(oracle_lib, x, w, b)
    ref = F.layer_norm(torch.from_numpy(x), (C,), torch.from_numpy(w), torch.from_numpy(b), eps=1e-5)
    assert np.allclose(y, ref.numpy(), rtol=0, atol=1e-12)


def test_layernorm_backward(oracle_lib):
    r = _rng(5)
    N, C = 12, 40
    x, w, b = _c(r.normal(size=(N, C))), _c(r.normal(size=C)), _c(r.normal(size=C))
    dy = _c(r.normal(size=(N, C)))
    y, mean, rstd = _ln_fwd(oracle_lib, x, w, b)
    dx = _c(r.normal(size=(N, C)))               # backward adds into dx
    dx0 = dx.copy()
    dw = np.zeros(C)
    db = np.zeros(C)
    oracle_lib.oracle_layernorm_backward(ptr(dx, D), ptr(dw, D), ptr(db, D), ptr(dy, D), ptr(x, D),
                                         ptr(w, D), ptr(mean, D), ptr(rstd, D), N, C)
    tx = torch.from_numpy(x).requires_grad_()
    tw = torch.from_numpy(w).requires_grad_()
    tb = torch.from_numpy(b).requires_grad_()
    F.layer_norm(tx, (C,), tw, tb, eps=1e-5).backward(torch.from_numpy(dy))
    assert np.allclose(dx - dx0, tx.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dw, tw.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(db, tb.grad.numpy(), rtol=0, atol=1e-12)
    # invariants per row: sum dx = 0; sum dx * xhat = O(eps)
    g = dx - dx0
    xhat = (x - mean[:, None]) * rstd[:, None]
    assert np.abs(g.sum(1)).max() < 1e-12
    assert np.abs((g * xhat).sum(1)).max() < 1e-4 * np.abs(g).max()


# ------------------------------------------------------------------- matmul --

def test_matmul_forward_brute_force(oracle_lib):
    r = _rng(6)
    N, C, OC = 7, 9, 5
    x, w, b = _c(r.normal(size=(N, C))), _c(r.normal(size=(OC, C))), _c(r.normal(size=OC))
    out = np.zeros((N, OC))
    oracle_lib.oracle_matmul_forward(ptr(out, D), ptr(x, D), ptr(w, D), ptr(b, D), N, C, OC)
    brute = np.array([[b[o] + sum(x[n, i] * w[o, i] for i in range(C)) for o in range(OC)]
                      for n in range(N)])
    assert np.allclose(out, brute, rtol=0, atol=1e-13)
    out2 = np.zeros((N, OC))
    oracle_lib.oracle_matmul_forward(ptr(out2, D), ptr(x, D), ptr(w, D), None, N, C, OC)
    assert np.allclose(out2, x @ w.T, rtol=0, atol=1e-13)   # NULL bias: no bias


def test_matmul_backward_autograd(oracle_lib):
    r = _rng(7)
    N, C, OC = 6, 10, 4
    x, w, b = _c(r.normal(size=(N, C))), _c(r.normal(size=(OC, C))), _c(r.normal(size=OC))
    dy = _c(r.normal(size=(N, OC)))
    dx, dw, db = np.zeros((N, C)), np.zeros((OC, C)), np.zeros(OC)
    oracle_lib.oracle_matmul_backward(ptr(dx, D), ptr(dw, D), ptr(db, D), ptr(dy, D), ptr(x, D),
                                      ptr(w, D), N, C, OC)
    tx, tw, tb = (torch.from_numpy(a).requires_grad_() for a in (x, w, b))
    F.linear(tx, tw, tb).backward(torch.from_numpy(dy))
    for mine, ref in ((dx, tx), (dw, tw), (db, tb)):
        assert np.allclose(mine, ref.grad.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- attention --

def _attn(lib, qkv, B, T, C, NH):
    out = np.zeros((B, T, C))
    att = np.zeros((B, NH, T, T))
    lib.oracle_attention_forward(ptr(out, D), ptr(att, D), ptr(qkv, D), B, T, C, NH)
    return out, att


def _torch_attn(qkv, B, T, C, NH):
    hs = C // NH
    q, k, v = qkv.split(C, dim=2)
    q, k, v = (a.view(B, T, NH, hs).transpose(1, 2) for a in (q, k, v))
    y = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    return y.transpose(1, 2).reshape(B, T, C)


def test_attention_forward_matches_torch_and_rows_sum_to_one(oracle_lib):
    r = _rng(8)
    B, T, C, NH = 2, 9, 24, 3
    qkv = _c(r.normal(size=(B, T, 3 * C)))
    y, att = _attn(oracle_lib, qkv, B, T, C, NH)
    ref = _torch_attn(torch.from_numpy(qkv), B, T, C, NH)
    assert np.allclose(y, ref.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(att.sum(-1), 1.0, rtol=0, atol=1e-13)
    assert not np.triu(att, k=1).any()             # causal: nothing above the diagonal


def test_attention_closed_forms(oracle_lib):
    r = _rng(9)
    B, C, NH = 2, 16, 2
    # T = 1: the only key is the query itself, y = v.
    qkv = _c(r.normal(size=(B, 1, 3 * C)))
    y, _ = _attn(oracle_lib, qkv, B, 1, C, NH)
    assert np.allclose(y, qkv[:, :, 2 * C:], rtol=0, atol=1e-15)
    # q = 0: uniform weights over the causal prefix, y_t = mean(v_0..v_t).
    T = 7
    qkv = _c(r.normal(size=(B, T, 3 * C)))
    qkv[:, :, :C] = 0
    y, _ = _attn(oracle_lib, qkv, B, T, C, NH)
    v = qkv[:, :, 2 * C:]
    expect = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    assert np.allclose(y, expect, rtol=0, atol=1e-13)


def test_attention_is_causal(oracle_lib):
    r = _rng(10)
    B, T, C, NH = 1, 8, 8, 2
    qkv = _c(r.normal(size=(B, T, 3 * C)))
    y1, _ = _attn(oracle_lib, qkv, B, T, C, NH)
    qkv2 = qkv.copy()
    qkv2[:, 5:] = r.normal(size=(B, T - 5, 3 * C))
    y2, _ = _attn(oracle_lib, qkv2, B, T, C, NH)
    assert np.array_equal(y1[:, :5], y2[:, :5])


def test_attention_backward_autograd(oracle_lib):
    r = _rng(11)
    B, T, C, NH = 2, 6, 12, 3
    qkv = _c(r.normal(size=(B, T, 3 * C)))
    dy = _c(r.normal(size=(B, T, C)))
    _, att = _attn(oracle_lib, qkv, B, T, C, NH)
    dqkv = np.zeros_like(qkv)
    oracle_lib.oracle_attention_backward(ptr(dqkv, D), ptr(dy, D), ptr(qkv, D), ptr(att, D),
                                         B, T, C, NH)
    tq = torch.from_numpy(qkv).requires_grad_()
    _torch_attn(tq, B, T, C, NH).backward(torch.from_numpy(dy))
    assert np.allclose(dqkv, tq.grad.numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------- gelu --

def test_gelu_identities_and_torch(oracle_lib):
    x = _c(np.linspace(-6, 6, 1001))
    y = np.zeros_like(x)
    ym = np.zeros_like(x)
    oracle_lib.oracle_gelu_forward(ptr(y, D), ptr(x, D), x.size)
    xn = _c(-x)
    oracle_lib.oracle_gelu_forward(ptr(ym, D), ptr(xn, D), x.size)
    assert np.allclose(y - ym, x, rtol=0, atol=1e-14)     # g(x) - g(-x) = x
    assert y[500] == 0.0                                   # g(0) = 0
    ref = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.allclose(y, ref, rtol=0, atol=1e-14)


def test_gelu_backward_fd_and_autograd(oracle_lib):
    x = _c(np.linspace(-5, 5, 401))
    dout = np.ones_like(x)
    dx = np.zeros_like(x)
    oracle_lib.oracle_gelu_backward(ptr(dx, D), ptr(x, D), ptr(dout, D), x.size)
    h = 1e-6
    yp, ym = np.zeros_like(x), np.zeros_like(x)
    xp, xm = _c(x + h), _c(x - h)
    oracle_lib.oracle_gelu_forward(ptr(yp, D), ptr(xp, D), x.size)
    oracle_lib.oracle_gelu_forward(ptr(ym, D), ptr(xm, D), x.size)
    assert np.allclose(dx, (yp - ym) / (2 * h), rtol=0, atol=1e-8)
    tx = torch.from_numpy(x.copy()).requires_grad_()
    F.gelu(tx, approximate="tanh").sum().backward()
    assert np.allclose(dx, tx.grad.numpy(), rtol=0, atol=1e-13)


# --------------------------------------------------------------- classifier --

def _golden_lnv():
    out = {}
    with open(os.path.join(GOLDEN, "uniform_logits.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                v, val = line.split()
                out[int(v)] = float(val)
    return out


@pytest.mark.parametrize("V,Vp", [(64, 64), (61, 64), (2, 64), (50257, 50304)])
def test_uniform_logits_give_ln_v(oracle_lib, V, Vp):
    N = 3
    logits = np.zeros((N, Vp))
    probs = np.zeros((N, Vp))
    oracle_lib.oracle_softmax_forward(ptr(probs, D), ptr(logits, D), N, V, Vp)
    tg = _c([0, V - 1, V // 2], np.int32)
    losses = np.zeros(N)
    oracle_lib.oracle_crossentropy_forward(ptr(losses, D), ptr(probs, D), ptr(tg, I), N, Vp)
    assert np.allclose(losses, _golden_lnv()[V], rtol=2e-12, atol=0)
    assert not probs[:, V:].any()


def test_classifier_matches_torch_and_invariants(oracle_lib):
    r = _rng(12)
    N, V, Vp = 9, 61, 64
    logits = _c(r.normal(scale=3.0, size=(N, Vp)))
    tg = _c(r.integers(0, V, size=N), np.int32)
    probs = np.zeros((N, Vp))
    oracle_lib.oracle_softmax_forward(ptr(probs, D), ptr(logits, D), N, V, Vp)
    losses = np.zeros(N)
    oracle_lib.oracle_crossentropy_forward(ptr(losses, D), ptr(probs, D), ptr(tg, I), N, Vp)
    dz = np.zeros((N, Vp))
    oracle_lib.oracle_crossentropy_softmax_backward(ptr(dz, D), ptr(probs, D), ptr(tg, I), 1.0 / N,
                                                    N, V, Vp)
    tz = torch.from_numpy(logits[:, :V].copy()).requires_grad_()
    ref = F.cross_entropy(tz, torch.from_numpy(tg).long(), reduction="none")
    assert np.allclose(losses, ref.detach().numpy(), rtol=0, atol=1e-12)
    ref.mean().backward()
    assert np.allclose(dz[:, :V], tz.grad.numpy(), rtol=0, atol=1e-14)
    assert not dz[:, V:].any()                       # padded columns: zero gradient
    assert np.allclose(probs.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.abs(dz.sum(1)).max() < 1e-15           # sum_v dlogits = 0


def test_two_class_reduces_to_logistic_loss(oracle_lib):
    z = _c([[0.3, -1.2], [2.0, 0.5]])
    tg = _c([0, 1], np.int32)
    probs = np.zeros_like(z)
    oracle_lib.oracle_softmax_forward(ptr(probs, D), ptr(z, D), 2, 2, 2)
    losses = np.zeros(2)
    oracle_lib.oracle_crossentropy_forward(ptr(losses, D), ptr(probs, D), ptr(tg, I), 2, 2)
    margin = np.array([z[0, 0] - z[0, 1], z[1, 1] - z[1, 0]])
    assert np.allclose(losses, np.log1p(np.exp(-margin)), rtol=1e-14)


# -------------------------------------------------------------------- adamw --

def _adamw(lib, theta, g, m, v, lr, b1, b2, eps, wd, t):
    lib.oracle_adamw(ptr(theta, D), ptr(g, D), ptr(m, D), ptr(v, D), theta.size, lr, b1, b2, eps,
                     wd, t)


def test_adamw_step1_and_step2_closed_forms(oracle_lib):
    r = _rng(13)
    n = 5
    th0 = _c(r.normal(size=n))
    g1 = _c(r.normal(size=n))
    g2 = _c(r.normal(size=n))
    lr, b1, b2, eps, wd = 1e-2, 0.9, 0.999, 1e-8, 0.1
    th, m, v = th0.copy(), np.zeros(n), np.zeros(n)
    _adamw(oracle_lib, th, g1, m, v, lr, b1, b2, eps, wd, 1)
    # t = 1: mhat = g, vhat = g^2, so the step is lr * (g / (|g| + eps) + wd * theta)
    assert np.allclose(th, th0 - lr * (g1 / (np.abs(g1) + eps) + wd * th0), rtol=0, atol=1e-15)
    assert np.allclose(m, (1 - b1) * g1, rtol=1e-15)
    assert np.allclose(v, (1 - b2) * g1 * g1, rtol=1e-15)
    th1 = th.copy()
    _adamw(oracle_lib, th, g2, m, v, lr, b1, b2, eps, wd, 2)
    m2 = b1 * (1 - b1) * g1 + (1 - b1) * g2
    v2 = b2 * (1 - b2) * g1 ** 2 + (1 - b2) * g2 ** 2
    step = (m2 / (1 - b1 ** 2)) / (np.sqrt(v2 / (1 - b2 ** 2)) + eps)
    assert np.allclose(th, th1 - lr * (step + wd * th1), rtol=0, atol=1e-15)


def test_adamw_matches_torch_optim(oracle_lib):
    r = _rng(14)
    n = 64
    th0 = _c(r.normal(size=n))
    grads = [_c(r.normal(size=n)) for _ in range(4)]
    lr, b1, b2, eps, wd = 6e-4, 0.9, 0.999, 1e-8, 0.1
    th, m, v = th0.copy(), np.zeros(n), np.zeros(n)
    p = torch.nn.Parameter(torch.from_numpy(th0.copy()))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    for t, g in enumerate(grads, start=1):
        _adamw(oracle_lib, th, g, m, v, lr, b1, b2, eps, wd, t)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
    assert np.allclose(th, p.detach().numpy(), rtol=0, atol=1e-14)


def test_constants_used_by_the_oracle():
    """GELU's sqrt(2/pi) and the LN eps, as the readings fix them."""
    src = open(os.path.join(os.path.dirname(__file__), "..", "oracle", "gpt2_oracle.c")).read()
    assert "#define LN_EPS 1e-5" in src
    assert "0.044715" in src
    assert math.isclose(float(src.split("#define ORACLE_PI ")[1].split()[0]), math.pi, rel_tol=1e-16)


# ------------------------------------------- LR schedule and gradient norm --
# Page "Building GPT-2 from scratch", exercise table row A5, names LR schedules
# and gradient clipping without formulas; the oracle takes the plain readings
# (linear warmup then half-cosine decay; global L2 norm, scaled down to the
# threshold). These pins fix special values and shapes of those readings.

def test_grad_norm_pins(oracle_lib):
    n = 1000
    assert oracle_lib.oracle_grad_norm(ptr(_c(np.full(n, -3.0)), D), n) == pytest.approx(
        3.0 * math.sqrt(n), rel=1e-15)
    e = np.zeros(n)
    e[417] = -2.5
    assert oracle_lib.oracle_grad_norm(ptr(_c(e), D), n) == 2.5
    assert oracle_lib.oracle_grad_norm(ptr(_c(np.zeros(n)), D), n) == 0.0
    g = _c(_rng(21).normal(size=12345))
    assert oracle_lib.oracle_grad_norm(ptr(g, D), g.size) == pytest.approx(
        np.linalg.norm(g), rel=1e-13)


def test_scaled_adamw_carries_the_scaled_gradient(oracle_lib):
    """With beta1 = 0 the first moment is the (scaled) gradient itself; with
    scale 1 the step equals the plain AdamW step bit for bit."""
    r = _rng(22)
    n = 50
    th0, g = _c(r.normal(size=n)), _c(r.normal(size=n))
    th, m, v = th0.copy(), np.zeros(n), np.zeros(n)
    oracle_lib.oracle_adamw_scaled(ptr(th, D), ptr(g, D), ptr(m, D), ptr(v, D), n, 1e-3, 0.0,
                                   0.999, 1e-8, 0.0, 1, 0.25)
    assert np.array_equal(m, 0.25 * g)
    assert np.allclose(v, 0.001 * (0.25 * g) ** 2, rtol=1e-14)
    th1, m1, v1 = th0.copy(), np.zeros(n), np.zeros(n)
    th2, m2, v2 = th0.copy(), np.zeros(n), np.zeros(n)
    oracle_lib.oracle_adamw_scaled(ptr(th1, D), ptr(g, D), ptr(m1, D), ptr(v1, D), n, 1e-3, 0.9,
                                   0.999, 1e-8, 0.1, 3, 1.0)
    _adamw(oracle_lib, th2, g, m2, v2, 1e-3, 0.9, 0.999, 1e-8, 0.1, 3)
    assert np.array_equal(th1, th2) and np.array_equal(m1, m2) and np.array_equal(v1, v2)


def test_clipping_matches_torch_clip_grad_norm(oracle_lib):
    """torch.nn.utils.clip_grad_norm_ scales by max_norm / (norm + 1e-6), capped at
    1; the oracle's reading has no 1e-6, so the two agree to ~1e-6 relative."""
    r = _rng(23)
    n = 300
    th0 = _c(r.normal(size=n))
    g = _c(r.normal(size=n) * 3)
    for max_norm in (0.5, 1e6):
        norm = oracle_lib.oracle_grad_norm(ptr(g, D), n)
        scale = max_norm / norm if norm > max_norm else 1.0
        th, m, v = th0.copy(), np.zeros(n), np.zeros(n)
        oracle_lib.oracle_adamw_scaled(ptr(th, D), ptr(g, D), ptr(m, D), ptr(v, D), n, 1e-3, 0.9,
                                       0.999, 1e-8, 0.1, 1, scale)
        p = torch.nn.Parameter(torch.from_numpy(th0.copy()))
        p.grad = torch.from_numpy(g.copy())
        tn = torch.nn.utils.clip_grad_norm_([p], max_norm)
        assert float(tn) == pytest.approx(norm, rel=1e-13)
        assert np.allclose(m, 0.1 * p.grad.numpy(), rtol=2e-6, atol=0)


def _lr(lib, t, lr_max=6e-4, lr_min=6e-5, warmup=100, total=1100):
    return lib.oracle_lr_schedule(lr_max, lr_min, warmup, total, t)


def test_lr_schedule_special_points(oracle_lib):
    lib = oracle_lib
    # linear warmup: lr_max / warmup at t = 1, half at t = warmup / 2, lr_max at warmup
    assert _lr(lib, 1) == pytest.approx(6e-6, rel=1e-15)
    assert _lr(lib, 50) == pytest.approx(3e-4, rel=1e-15)
    assert _lr(lib, 100) == pytest.approx(6e-4, rel=1e-15)
    # cosine: midpoint halfway between lr_max and lr_min, end and beyond at lr_min
    assert _lr(lib, 600) == pytest.approx(3.3e-4, rel=1e-14)
    assert _lr(lib, 1100) == pytest.approx(6e-5, rel=1e-14)
    assert _lr(lib, 5000) == pytest.approx(6e-5, rel=1e-14)
    # symmetric about the midpoint, non-increasing, and flat where it starts
    # (second order in the progress p: a linear decay would drop 1e-3 here)
    lrs = [_lr(lib, t) for t in range(100, 1101)]
    assert all(a >= b for a, b in zip(lrs, lrs[1:]))
    for k in (1, 137, 400):
        assert _lr(lib, 100 + k) + _lr(lib, 1100 - k) == pytest.approx(6.6e-4, rel=1e-13)
    drop = (6e-4 - _lr(lib, 101)) / (6e-4 - 6e-5)
    assert drop == pytest.approx((math.pi * 1e-3) ** 2 / 4, rel=1e-3)
    # no warmup: the cosine starts at step 0, so step 5 of 10 is the midpoint
    assert lib.oracle_lr_schedule(1e-3, 0.0, 0, 10, 5) == pytest.approx(5e-4, rel=1e-14)
    assert lib.oracle_lr_schedule(1e-3, 0.0, 0, 10, 10) == pytest.approx(0.0, abs=1e-20)


def test_library_schedule_matches_the_oracle(oracle_lib):
    """gpt2_schedule_lr (host code of the library) against the oracle."""
    from transformer_lm_amd import gpt2
    s = gpt2.Schedule(6e-4, 6e-5, 100, 1100, 0.9, 0.95, 1e-8, 0.1, 1.0)
    for t in (1, 2, 37, 99, 100, 101, 350, 600, 1099, 1100, 1500):
        assert gpt2.schedule_lr(s, t) == pytest.approx(_lr(oracle_lib, t), rel=2e-7, abs=1e-12)
    with pytest.raises(gpt2.GPT2Error):
        gpt2.schedule_lr(gpt2.Schedule(6e-4, 6e-5, 10, 10, 0.9, 0.95, 1e-8, 0.1, 1.0), 1)
