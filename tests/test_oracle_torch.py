"""Pins for oracle/gpt2_torch.py, the large-configuration form of the oracle,
and for the trajectories it wrote under tests/golden/. CPU only.

- In float64 it must agree with the C oracle (itself pinned by finite
  differences of every parameter, closed forms and an autograd composition)
  element by element: losses, per-position losses, every gradient and the
  parameters after AdamW steps with weight decay, on the tiny model and its
  padded-vocabulary variant, and on the 124M shape at a short sequence.
- In float32 (the precision the stored trajectories use) it must meet the
  fp32 contract against the double C oracle on the 124M shape.
- The stored trajectories: written by the current oracle source, from the
  current generator's inputs, self-consistent, and (124M) the stored
  per-position losses of one sequence equal the C oracle's own forward of it.
"""
import hashlib
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.gpt2_torch import TorchOracle
from oracle.wrapper import Oracle
from transformer_lm_amd import synth
from transformer_lm_amd.workloads import WORKLOADS, param_offsets

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _run_both(w, steps, dtype, threads=8):
    p = synth.init_params(w)
    toks = synth.tokens(w, steps=steps)
    c = Oracle(w, p, threads=threads)
    t = TorchOracle(w, p, dtype=dtype)
    out = []
    for s in range(steps):
        x, y = synth.split_batch(toks[s])
        lc, lt = c.forward(x, y), t.forward(x, y)
        pc, pt = c.act("losses"), t.losses.copy()
        c.backward()
        t.backward()
        out.append((lc, lt, pc, pt, c.grads(), t.grads()))
        c.update(w.lr, w.beta1, w.beta2, w.eps, 0.1, s + 1)
        t.update(w.lr, w.beta1, w.beta2, w.eps, 0.1, s + 1)
    return out, c.params(), t.params()


@pytest.mark.parametrize("name", ["tiny", "tiny_pad"])
def test_float64_matches_c_oracle_over_three_steps(oracle_lib, name):
    w = WORKLOADS[name]
    steps, pc, pt = _run_both(w, 3, torch.float64)
    for lc, lt, plc, plt, gc, gt in steps:
        assert abs(lc - lt) <= 1e-13 * abs(lc)
        assert np.abs(plc - plt).max() <= 1e-12
        assert np.abs(gc - gt).max() <= 1e-13 * np.abs(gc).max()
    assert np.abs(pc - pt).max() <= 1e-12


@pytest.mark.slow
def test_float64_matches_c_oracle_at_124m_shape(oracle_lib):
    w = WORKLOADS["gpt2_124m_fp32"].with_batch(B=1, T=16)
    steps, _, _ = _run_both(w, 1, torch.float64)
    lc, lt, _, _, gc, gt = steps[0]
    assert abs(lc - lt) <= 1e-12 * abs(lc)
    for name, (off, shape) in param_offsets(w).items():
        n = math.prod(shape)
        a, b = gc[off:off + n], gt[off:off + n]
        assert np.abs(a - b).max() <= 1e-10 * max(np.abs(a).max(), 1e-30), name


@pytest.mark.slow
def test_float32_meets_the_fp32_contract_at_124m_shape(oracle_lib):
    """The float32 form against the double C oracle: loss relative error
    <= 1e-5 and per-tensor max|dg| / max|g| <= 1e-3 (the fp32 contract)."""
    w = WORKLOADS["gpt2_124m_fp32"].with_batch(B=2, T=64)
    steps, _, _ = _run_both(w, 1, torch.float32)
    lc, lt, plc, plt, gc, gt = steps[0]
    assert abs(lc - lt) <= 1e-5 * abs(lc)
    assert np.abs(plc - plt).max() <= 1e-4
    for name, (off, shape) in param_offsets(w).items():
        n = math.prod(shape)
        a, b = gc[off:off + n], gt[off:off + n]
        assert np.abs(a - b).max() <= 1e-3 * np.abs(a).max(), name


def test_finite_differences_of_the_float64_form():
    """Central differences of the loss for a few parameters of every tensor
    of the tiny model against the float64 form's own gradient."""
    w = WORKLOADS["tiny_pad"]
    p = synth.init_params(w)
    x, y = synth.split_batch(synth.tokens(w)[0])
    t = TorchOracle(w, p, dtype=torch.float64)
    t.forward(x, y)
    t.backward()
    g = t.grads()
    h = 1e-5
    for k, (name, (off, shape)) in enumerate(param_offsets(w).items()):
        n = math.prod(shape)
        u = synth.uniform(500 + k, 0, 3)
        for j in sorted({off + min(int(v * n), n - 1) for v in u}):
            th = t.theta[j].item()
            t.theta[j] = th + h
            lp = t.forward(x, y)
            t.theta[j] = th - h
            lm = t.forward(x, y)
            t.theta[j] = th
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[j]) <= 1e-7 * max(1.0, abs(g[j])), (name, j)


# ---- the stored trajectories --------------------------------------------------

def _golden(name):
    path = os.path.join(GOLDEN, f"trajectory_{name}.json")
    if not os.path.exists(path):
        pytest.fail(f"{path} missing: run tests/golden/make_trajectories.py {name}")
    with open(path) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["gpt2_124m", "gpt2_350m", "gpt2_1558m"])
def test_trajectory_is_current_and_consistent(name):
    gold = _golden(name)
    w = WORKLOADS[name]
    with open(os.path.join(ROOT, "oracle", "gpt2_torch.py"), "rb") as f:
        assert gold["oracle_sha256"] == hashlib.sha256(f.read()).hexdigest()
    toks = synth.tokens(w)
    assert gold["inputs_sha256"]["tokens"] == hashlib.sha256(toks.tobytes()).hexdigest()
    if name == "gpt2_124m":   # the others take longer to regenerate than to check here
        p = synth.init_params(w)
        assert gold["inputs_sha256"]["params"] == hashlib.sha256(p.tobytes()).hexdigest()
    assert len(gold["losses"]) == w.steps
    assert all(np.isfinite(gold["losses"]))
    # step 1 from the initial weights is near ln V: the logits start with
    # variance about C * 0.02^2 (unit-variance LayerNorm output against
    # N(0, 0.02^2) embedding rows), which lifts the mean loss above ln V by
    # about half that; twice the estimate bounds it. Training lowers the loss.
    excess = gold["losses"][0] - math.log(w.V)
    assert -0.05 <= excess <= w.C * 0.02 ** 2, excess
    # the updates move the model (at 350M and 1.5B the loss first jumps up:
    # AdamW's first steps move every parameter by about lr)
    assert max(abs(v - gold["losses"][0]) for v in gold["losses"][1:]) > 0.5
    pos = np.asarray(gold["step1_position_losses"])
    assert pos.size == w.BT
    assert abs(pos.mean() - gold["losses"][0]) <= 1e-5
    for k, (tname, (off, shape)) in enumerate(param_offsets(w).items()):
        e = gold["step1_grads"][tname]
        idx, val = np.asarray(e["idx"]), np.asarray(e["val"])
        assert idx.size == val.size and idx.size >= min(64, math.prod(shape))
        assert np.abs(val).max() == pytest.approx(e["max_abs"], rel=1e-6)
        assert np.linalg.norm(val) <= e["norm"] * (1 + 1e-6)


@pytest.mark.slow
def test_trajectory_124m_positions_match_the_c_oracle(oracle_lib):
    """Step-1 losses of the first sequence depend on that sequence alone: the
    C oracle (float build, plain loops) run on it reproduces the stored
    per-position losses of the 124M trajectory to float32 accuracy."""
    gold = _golden("gpt2_124m")
    w = WORKLOADS["gpt2_124m"]
    p = synth.init_params(w)
    x, y = synth.split_batch(synth.tokens(w, steps=1)[0])
    ws = w.with_batch(B=1, steps=1)
    o = Oracle(ws, p, precision="f32", threads=8)
    o.forward(x[:1], y[:1])
    got = o.act("losses")
    ref = np.asarray(gold["step1_position_losses"][:w.T])
    assert np.abs(got - ref).max() <= 2e-4


# ---- the bf16-storage variant (oracle/gpt2_torch_bf16.py) -----------------------

def test_bf16_storage_variant_without_rounding_is_the_float32_oracle(monkeypatch):
    """With its roundings replaced by the identity (and a float32 working
    copy), the variant computes what TorchOracle computes, over three steps
    with weight decay: only the form of the loss (log-sum-exp minus the target
    logit instead of the log of the normalised probability) and of the
    attention normalisation differ, so the two agree to float32 rounding."""
    import oracle.gpt2_torch_bf16 as ob
    monkeypatch.setattr(ob, "r16", lambda t: t)
    monkeypatch.setattr(ob.TorchOracleBF16Storage, "_refresh",
                        lambda self: (setattr(self, "work", self.theta.clone()),
                                      setattr(self, "pw", ob._views(self.work, self.w))))
    for name in ("tiny", "tiny_pad"):
        w = WORKLOADS[name]
        p = synth.init_params(w)
        toks = synth.tokens(w, steps=3)
        a, b = TorchOracle(w, p), ob.TorchOracleBF16Storage(w, p)
        for s in range(3):
            x, y = synth.split_batch(toks[s])
            la, lb = a.forward(x, y), b.forward(x, y)
            assert abs(la - lb) <= 1e-6 * abs(la)
            a.backward()
            b.backward()
            ga, gb = a.grads(), b.grads()
            assert np.abs(ga - gb).max() <= 1e-5 * np.abs(ga).max()
            a.update(1e-3, 0.9, 0.999, 1e-8, 0.1, s + 1)
            b.update(1e-3, 0.9, 0.999, 1e-8, 0.1, s + 1)
        # AdamW divides by |g|: an entry whose gradient is within rounding of
        # zero may move by up to 2 lr per step; all others agree closely
        dth = np.abs(a.params() - b.params())
        assert np.percentile(dth, 99) <= 1e-7 and dth.max() <= 3 * 2 * 1e-3


def test_bf16_storage_variant_rounds_where_a_bf16_step_stores():
    """With rounding: the working copy and the stored activations are bf16
    values (their float32 bits have zero low halves), and the step stays
    within the bf16 contract of the float32 oracle (loss 2e-2, cosine 0.99)
    while differing from it (so the roundings are applied)."""
    from oracle.gpt2_torch_bf16 import TorchOracleBF16Storage
    w = WORKLOADS["tiny_pad"]
    p = synth.init_params(w)
    x, y = synth.split_batch(synth.tokens(w)[0])
    a, b = TorchOracle(w, p), TorchOracleBF16Storage(w, p)
    la, lb = a.forward(x, y), b.forward(x, y)
    for key in ("ln1", "qkv", "atty", "res2", "fch"):
        bits = b.saved["layers"][0][key].numpy().view(np.uint32)
        assert not (bits & 0xFFFF).any(), key
    assert 0 < abs(la - lb) <= 2e-2
    a.backward()
    b.backward()
    ga, gb = a.grads(), b.grads()
    for name, (off, shape) in param_offsets(w).items():
        n = math.prod(shape)
        u, v = ga[off:off + n], gb[off:off + n]
        if np.abs(u).max() > 0:
            assert np.dot(u, v) / (np.linalg.norm(u) * np.linalg.norm(v)) >= 0.99, name
    assert np.abs(ga - gb).max() > 0


@pytest.mark.parametrize("name,kind", [("gpt2_350m", "bf16storage"),
                                       ("gpt2_1558m", "bf16storage"), ("gpt2_350m", "bf16init")])
def test_variant_trajectory_is_current_and_consistent(name, kind):
    """The stored variant trajectories (bf16 storage; the bf16-rounded start)
    were written by the current oracle sources from the same inputs as the
    fp32 trajectory, and start where it starts."""
    path = os.path.join(GOLDEN, f"trajectory_{name}_{kind}.json")
    if not os.path.exists(path):
        pytest.fail(f"{path} missing: run tests/golden/make_trajectories.py --{kind[:4]}-"
                    f"{kind[4:]} {name}")
    with open(path) as f:
        var = json.load(f)
    gold = _golden(name)
    w = WORKLOADS[name]
    with open(os.path.join(ROOT, "oracle", "gpt2_torch.py"), "rb") as f:
        assert var["oracle_sha256"] == hashlib.sha256(f.read()).hexdigest()
    if kind == "bf16storage":
        with open(os.path.join(ROOT, "oracle", "gpt2_torch_bf16.py"), "rb") as f:
            assert var["variant_sha256"] == hashlib.sha256(f.read()).hexdigest()
    assert var["inputs_sha256"] == gold["inputs_sha256"]
    assert len(var["losses"]) == w.steps and all(np.isfinite(var["losses"]))
    # step 1 reads identical inputs up to bf16 rounding: within the bf16 contract
    assert abs(var["losses"][0] - gold["losses"][0]) <= 2e-2
