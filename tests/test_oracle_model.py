"""Pins for the oracle's whole training step, CPU only.

- every parameter gradient against central finite differences of the loss
  (double build, all 28,544 parameters of the tiny model and its padded-vocab
  variant);
- the forward composition and its gradients against an independent PyTorch
  float64 model built from library ops and differentiated by autograd;
- closed forms (uniform logits give ln V) and invariants (causality, padded
  rows stay zero, thread-count independence);
- several AdamW steps against torch.optim.AdamW.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.wrapper import Oracle, fd_grads
from transformer_lm_amd import synth
from transformer_lm_amd.workloads import WORKLOADS, param_offsets


def _setup(name, **kw):
    w = WORKLOADS[name]
    if kw:
        w = w.with_batch(**kw)
    p = synth.init_params(w)
    x, y = synth.split_batch(synth.tokens(w)[0])
    return w, p, x, y


def _per_tensor(w, flat):
    return {n: flat[off:off + int(np.prod(s))] for n, (off, s) in param_offsets(w).items()}


@pytest.mark.slow
@pytest.mark.parametrize("name", ["tiny", "tiny_pad"])
def test_every_gradient_matches_finite_differences(oracle_lib, name):
    w, p, x, y = _setup(name)
    o = Oracle(w, p)
    o.forward(x, y)
    o.backward()
    g = o.grads()
    fd = fd_grads(w, p, x, y, h=1e-5)
    for tname, ga in _per_tensor(w, g).items():
        gf = _per_tensor(w, fd)[tname]
        bound = 1e-6 * max(1.0, np.abs(ga).max())
        assert np.abs(gf - ga).max() <= bound, tname
    # gradients are not trivially zero
    assert np.abs(g).max() > 1e-2


class TorchGPT2:
    """GPT-2 as a composition of PyTorch library ops (float64), for
    cross-checking the oracle's forward and, via autograd, its backward."""

    def __init__(self, w, flat):
        self.w = w
        self.flat = torch.tensor(flat, dtype=torch.float64, requires_grad=True)

    def t(self, name):
        off, shape = param_offsets(self.w)[name]
        n = int(np.prod(shape))
        return self.flat[off:off + n].view(*shape)

    def loss(self, x, y):
        w = self.w
        B, T, C, NH = x.shape[0], x.shape[1], w.C, w.NH
        hs = C // NH
        xt = torch.from_numpy(x).long()
        h = self.t("wte")[xt] + self.t("wpe")[:T][None]
        for l in range(w.L):
            a = F.layer_norm(h, (C,), self.t("ln1w")[l], self.t("ln1b")[l], eps=1e-5)
            qkv = F.linear(a, self.t("qkvw")[l], self.t("qkvb")[l])
            q, k, v = (u.view(B, T, NH, hs).transpose(1, 2) for u in qkv.split(C, dim=2))
            att = F.scaled_dot_product_attention(q, k, v, is_causal=True)
            att = att.transpose(1, 2).reshape(B, T, C)
            h = h + F.linear(att, self.t("attprojw")[l], self.t("attprojb")[l])
            a = F.layer_norm(h, (C,), self.t("ln2w")[l], self.t("ln2b")[l], eps=1e-5)
            u = F.gelu(F.linear(a, self.t("fcw")[l], self.t("fcb")[l]), approximate="tanh")
            h = h + F.linear(u, self.t("fcprojw")[l], self.t("fcprojb")[l])
        h = F.layer_norm(h, (C,), self.t("lnfw"), self.t("lnfb"), eps=1e-5)
        logits = F.linear(h, self.t("wte"))[..., :w.V]
        return F.cross_entropy(logits.reshape(-1, w.V), torch.from_numpy(y).long().reshape(-1))


@pytest.mark.parametrize("name", ["tiny", "tiny_pad"])
def test_forward_and_backward_match_torch_composition(oracle_lib, name):
    w, p, x, y = _setup(name)
    o = Oracle(w, p)
    loss = o.forward(x, y)
    o.backward()
    m = TorchGPT2(w, p.astype(np.float64))
    ref = m.loss(x, y)
    ref.backward()
    assert abs(loss - ref.item()) < 1e-12
    assert np.allclose(o.grads(), m.flat.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.slow
def test_gpt2_124m_shape_matches_torch_composition(oracle_lib):
    """The 124M shape at a short sequence: loss and a sample of gradients."""
    w, p, x, y = _setup("gpt2_124m_fp32", B=1, T=8)
    o = Oracle(w, p, threads=8)
    loss = o.forward(x, y)
    o.backward()
    g = o.grads()
    m = TorchGPT2(w, p.astype(np.float64))
    ref = m.loss(x, y)
    ref.backward()
    assert abs(loss - ref.item()) < 1e-10
    gr = m.flat.grad.numpy()
    for name, (off, shape) in param_offsets(w).items():
        n = int(np.prod(shape))
        a, b = g[off:off + n], gr[off:off + n]
        assert np.abs(a - b).max() <= 1e-9 * max(1.0, np.abs(b).max()), name


@pytest.mark.parametrize("name", ["tiny", "tiny_pad"])
def test_zero_embedding_gives_ln_v(oracle_lib, name):
    w, p, x, y = _setup(name)
    off, shape = param_offsets(w)["wte"]
    p = p.copy()
    p[off:off + int(np.prod(shape))] = 0
    loss = Oracle(w, p).forward(x, y)
    assert abs(loss - np.log(w.V)) < 1e-12


def test_causality_of_the_whole_model(oracle_lib):
    w, p, x, y = _setup("tiny")
    o = Oracle(w, p)
    o.forward(x, y)
    l1 = o.act("losses").reshape(w.B, w.T)
    x2, y2 = x.copy(), y.copy()
    x2[:, 10:] = (x2[:, 10:] + 7) % w.V
    o.forward(x2, y2)
    l2 = o.act("losses").reshape(w.B, w.T)
    assert np.array_equal(l1[:, :10], l2[:, :10])
    assert not np.array_equal(l1[:, 10:], l2[:, 10:])


def test_padded_rows_stay_zero_and_unused_wpe_rows_get_no_gradient(oracle_lib):
    w, p, x, y = _setup("tiny_pad")
    w = w.with_batch(steps=3)
    o = Oracle(w, p)
    toks = synth.tokens(w)
    offs = param_offsets(w)
    for t in range(3):
        xi, yi = synth.split_batch(toks[t])
        o.forward(xi, yi)
        o.backward()
        g = _per_tensor(w, o.grads())
        assert not g["wte"].reshape(w.Vp, w.C)[w.V:].any()
        assert not g["wpe"].reshape(w.max_T, w.C)[w.T:].any()
        o.update(1e-3, 0.9, 0.999, 1e-8, 0.1, t + 1)
    off, _ = offs["wte"]
    wte = o.params()[off:off + w.Vp * w.C].reshape(w.Vp, w.C)
    assert not wte[w.V:].any()


def test_results_do_not_depend_on_thread_count(oracle_lib):
    w, p, x, y = _setup("tiny")
    res = []
    for th in (1, 5):
        o = Oracle(w, p, threads=th)
        loss = o.forward(x, y)
        o.backward()
        res.append((loss, o.grads()))
    oracle_lib.oracle_set_threads(8)
    assert res[0][0] == res[1][0]
    assert np.array_equal(res[0][1], res[1][1])


def test_multi_step_training_matches_torch_adamw(oracle_lib):
    w, p, _, _ = _setup("tiny")
    w = w.with_batch(steps=3)
    toks = synth.tokens(w)
    o = Oracle(w, p)
    m = TorchGPT2(w, p.astype(np.float64))
    opt = torch.optim.AdamW([m.flat], lr=1e-2, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.1)
    for t in range(3):
        x, y = synth.split_batch(toks[t])
        loss = o.forward(x, y)
        o.backward()
        o.update(1e-2, 0.9, 0.999, 1e-8, 0.1, t + 1)
        opt.zero_grad()
        ref = m.loss(x, y)
        ref.backward()
        opt.step()
        assert abs(loss - ref.item()) < 1e-11
    assert np.allclose(o.params(), m.flat.detach().numpy(), rtol=0, atol=1e-12)


def test_scheduled_clipped_training_matches_torch(oracle_lib):
    """Three scheduled steps with the gradient clipped every step against
    torch: clip_grad_norm_ (whose extra 1e-6 in the divisor is the only
    difference) and AdamW at the schedule's learning rate."""
    w, p, _, _ = _setup("tiny")
    w = w.with_batch(steps=3)
    toks = synth.tokens(w)
    o = Oracle(w, p)
    m = TorchGPT2(w, p.astype(np.float64))
    opt = torch.optim.AdamW([m.flat], lr=1e-2, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.1)
    lr_max, lr_min, warmup, total, clip = 1e-2, 1e-3, 2, 5, 0.05
    for t in range(1, 4):
        x, y = synth.split_batch(toks[t - 1])
        o.forward(x, y)
        o.backward()
        norm = o.update_scheduled(lr_max, lr_min, warmup, total, 0.9, 0.999, 1e-8, 0.1, clip, t)
        opt.zero_grad()
        m.loss(x, y).backward()
        tn = torch.nn.utils.clip_grad_norm_([m.flat], clip)
        # equal at step 1; later steps see parameters that moved by torch's
        # slightly different scale
        assert norm == pytest.approx(float(tn), rel=1e-12 if t == 1 else 1e-7) and norm > clip
        for grp in opt.param_groups:
            grp["lr"] = oracle_lib.oracle_lr_schedule(lr_max, lr_min, warmup, total, t)
        opt.step()
    assert np.allclose(o.params(), m.flat.detach().numpy(), rtol=0, atol=1e-7)


def test_backward_without_targets_is_an_error(oracle_lib):
    w, p, x, _ = _setup("tiny")
    o = Oracle(w, p)
    o.forward(x)
    with pytest.raises(RuntimeError):
        o.backward()


def test_out_of_range_token_is_rejected(oracle_lib):
    w, p, x, y = _setup("tiny_pad")
    x = x.copy()
    x[0, 0] = w.V                     # a padded id is not a token
    with pytest.raises(ValueError):
        Oracle(w, p).forward(x, y)


def test_nan_poisoned_parameter_gives_a_non_finite_loss(oracle_lib):
    """A NaN in a parameter that the step reads (a LayerNorm gain of the first
    block) propagates: the loss and the gradients are NaN; no error code,
    since nothing about the call is invalid."""
    w, p, x, y = _setup("tiny")
    off, _ = param_offsets(w)["ln1w"]
    p = p.copy()
    p[off + 3] = np.nan
    o = Oracle(w, p)
    assert np.isnan(o.forward(x, y))
    o.backward()
    assert np.isnan(o.grads()).any()
