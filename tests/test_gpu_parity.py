"""GPU parity: the HIP training step through the C ABI against the CPU oracle,
on the same seeded parameters and tokens.

Tolerances (the training-step contract): encoder gather bit-exact; fp32 mode
loss relative error <= 1e-5 and per-tensor max|dg|/max|g_ref| <= 1e-3; bf16
mode loss within 2e-2 absolute and per-tensor gradient cosine >= 0.99.
Reduced-depth variants of the 350M and 1.5B shapes keep their per-layer shapes
(C, NH, head size) at sizes the oracle steps in seconds.
"""
from dataclasses import replace

import numpy as np
import pytest

from parity import (bf16_round, check_bf16, check_fp32, cosine, gpu_steps, oracle_steps,
                    per_tensor, rel_err, say)
from transformer_lm_amd import synth
from transformer_lm_amd.workloads import WORKLOADS, param_offsets

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    oracle.build(force=False)
    from transformer_lm_amd import build
    if not build.is_built():
        build.build()


def _inputs(w, steps=None):
    return synth.init_params(w), synth.tokens(w, steps=steps)


# ---------------------------------------------------------------- encoder --

@pytest.mark.parametrize("name,dtype", [("tiny", "fp32"), ("gpt2_124m_fp32", "fp32"),
                                        ("tiny", "bf16"), ("gpt2_124m", "bf16")])
def test_encoder_forward_is_bit_exact(name, dtype):
    import torch
    from transformer_lm_amd import gpt2
    w = replace(WORKLOADS[name], dtype=dtype)
    if name == "gpt2_124m":
        w = w.with_batch(B=2, T=256)
    p, toks = _inputs(w, steps=1)
    x, y = synth.split_batch(toks[0])
    say(f"encoder {name} {dtype} B={w.B} T={w.T}")
    m = gpt2.GPT2(gpt2.config(w), p)
    m.forward(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda())
    got = m.act("encoded").float().cpu().numpy().reshape(w.B, w.T, w.C)
    offs = param_offsets(w)
    wte = p[offs["wte"][0]:][: w.Vp * w.C].reshape(w.Vp, w.C)
    wpe = p[offs["wpe"][0]:][: w.max_T * w.C].reshape(w.max_T, w.C)
    if dtype == "fp32":
        from oracle.wrapper import Oracle
        o = Oracle(w, p, precision="f32")
        o.forward(x, y)
        expect = o.act("encoded").astype(np.float32).reshape(w.B, w.T, w.C)
    else:
        # one fp32 add of the two bf16 embeddings, rounded to bf16
        expect = bf16_round(bf16_round(wte)[x] + bf16_round(wpe)[None, :w.T])
    assert np.array_equal(got, expect)


# -------------------------------------------------------------- fp32 step --

@pytest.mark.parametrize("name", ["tiny", "tiny_pad", "gpt2_124m_fp32"])
def test_fp32_step_matches_oracle(name):
    w = WORKLOADS[name]
    p, toks = _inputs(w)
    say(f"fp32 step {name}")
    gpu = gpu_steps(w, p, toks, 1)
    ref = oracle_steps(w, p, toks, 1)
    rep = check_fp32(w, gpu, ref)
    say({k: f"{v:.2e}" for k, v in rep.items()})
    # after the update: m and v are linear / quadratic in g
    assert rel_err(gpu["m"], ref["m"]) <= 1e-3
    assert rel_err(gpu["v"], ref["v"]) <= 2e-3
    # theta: at t = 1 the step is lr * g / (|g| + eps), which may flip for
    # near-zero gradients; elsewhere it must agree to well under lr
    g = ref["grads"][1]
    dth = np.abs(gpu["params"] - ref["params"])
    small = np.zeros_like(g, dtype=bool)
    for n, gt in per_tensor(w, g).items():
        off, s = param_offsets(w)[n]
        small[off:off + gt.size] = np.abs(gt) < 1e-3 * np.abs(gt).max()
    assert dth[small].max(initial=0) <= 2 * w.lr
    assert dth[~small].max() <= 1e-4 * w.lr + 1e-6 * np.abs(ref["params"]).max()


@pytest.mark.parametrize("name", ["tiny", "gpt2_124m_fp32"])
def test_fp32_scheduled_clipped_step_matches_oracle(name):
    """The scheduled update with gradient clipping active: warmup puts the
    first step at lr_max / 4; the threshold is a tenth of the gradient norm,
    so m and v carry the clipped gradient; the device norm matches the
    oracle's."""
    from oracle.wrapper import Oracle
    w = WORKLOADS[name]
    p, toks = _inputs(w)
    x, y = synth.split_batch(toks[0])
    o = Oracle(w, p)
    o.forward(x, y)
    o.backward()
    norm = float(np.linalg.norm(o.grads()))
    sched = {"lr_max": 4 * w.lr, "lr_min": 0.1 * w.lr, "warmup": 4, "total": 20,
             "grad_clip": 0.1 * norm}
    lr = w.lr  # 4 lr * 1 / 4 at step 1
    say(f"fp32 scheduled step {name}: |g| = {norm:.4e}, clip {sched['grad_clip']:.4e}")
    gpu = gpu_steps(w, p, toks, 1, sched=sched)
    ref = oracle_steps(w, p, toks, 1, sched=sched)
    check_fp32(w, gpu, ref)
    assert abs(gpu["norms"][0] - ref["norms"][0]) <= 1e-4 * ref["norms"][0]
    assert abs(ref["norms"][0] - norm) <= 1e-12 * norm
    assert rel_err(gpu["m"], ref["m"]) <= 1e-3
    assert rel_err(gpu["v"], ref["v"]) <= 2e-3
    # m holds (1 - b1) times the clipped gradient: its norm is (1 - b1) * clip
    assert abs(np.linalg.norm(gpu["m"]) - (1 - w.beta1) * sched["grad_clip"]) <= \
        1e-4 * sched["grad_clip"]
    # theta: the step is lr * g' / (|g'| + eps) with g' the clipped gradient,
    # ten times smaller than g, so eps weighs ten times more: elements below a
    # hundredth of their tensor's largest gradient only need to stay within lr
    g = ref["grads"][1]
    dth = np.abs(gpu["params"] - ref["params"])
    small = np.zeros_like(g, dtype=bool)
    for n, gt in per_tensor(w, g).items():
        off, s = param_offsets(w)[n]
        small[off:off + gt.size] = np.abs(gt) < 1e-2 * np.abs(gt).max()
    assert dth[small].max(initial=0) <= 2 * lr
    assert dth[~small].max() <= 1e-4 * lr + 1e-6 * np.abs(ref["params"]).max()


def test_fp32_step_skewed_tokens():
    """Tokens drawn almost all from a few ids: one token's positions span many
    of the summation ranges of the embedding backward (and two position
    chunks), so its pieces go through the in-order fix-up."""
    w = replace(WORKLOADS["tiny"], name="tiny_skewed", B=40, T=32, token_dist="zipf", zipf_s=4.0,
                steps=1)
    p, toks = _inputs(w)
    x, _ = synth.split_batch(toks[0])
    counts = np.bincount(x.ravel(), minlength=w.V)
    say(f"fp32 step tiny_skewed: B*T={w.B * w.T}, largest bucket {counts.max()}")
    assert counts.max() > 20 * 32  # spans more than 20 ranges of 32 positions
    gpu = gpu_steps(w, p, toks, 1)
    ref = oracle_steps(w, p, toks, 1)
    rep = check_fp32(w, gpu, ref)
    say({k: f"{v:.2e}" for k, v in rep.items()})


@pytest.mark.parametrize("name", ["tiny", "gpt2_124m_fp32"])
def test_fp32_intermediates_match_oracle(name):
    """Forward activations in dependency order: the first to fail is the bug."""
    import torch
    from oracle.wrapper import Oracle
    from transformer_lm_amd import gpt2
    w = WORKLOADS[name]
    p, toks = _inputs(w)
    x, y = synth.split_batch(toks[0])
    say(f"fp32 intermediates {name}")
    m = gpt2.GPT2(gpt2.config(w), p)
    xd, yd = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
    m.forward(xd)                       # no targets: the logits stay
    torch.cuda.synchronize()
    o = Oracle(w, p)
    o.forward(x, y)
    for act in ("encoded", "ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "residual2", "ln2",
                "fch", "fch_gelu", "residual3", "lnf", "logits"):
        got = m.act(act).double().cpu().numpy()
        ref = o.act(act)
        e = rel_err(got[: ref.size], ref)
        say(f"  {act}: {e:.2e}")
        assert e <= 1e-4, act
    m.forward(xd, yd)
    losses = m.act("losses").double().cpu().numpy()
    assert rel_err(losses, o.act("losses")) <= 1e-5
    dz = m.act("logits").double().cpu().numpy().reshape(w.BT, w.Vp)
    assert not dz[:, w.V:].any()                              # padded columns
    assert np.abs(dz.sum(1)).max() <= 1e-6 / w.BT * 100       # sum_v dlogits = 0


@pytest.mark.parametrize("B,T", [(2, 200), (1, 64)])
def test_bf16_intermediates_match_oracle(B, T):
    """bf16 forward activations of the 124M shape against the fp64 oracle, in
    dependency order. T=200 leaves ragged query/key tiles and a ragged GEMM
    row count. bf16 storage bounds the agreement: cosine >= 0.999 per tensor."""
    import torch
    from oracle.wrapper import Oracle
    from transformer_lm_amd import gpt2
    w = WORKLOADS["gpt2_124m"].with_batch(B=B, T=T, steps=1)
    p, toks = _inputs(w)
    x, y = synth.split_batch(toks[0])
    say(f"bf16 intermediates 124M B={B} T={T}")
    m = gpt2.GPT2(gpt2.config(w), p)
    m.forward(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    o = Oracle(w, p, threads=16)
    o.forward(x, y)
    for act in ("encoded", "ln1", "qkv", "atty", "residual2", "ln2", "fch", "fch_gelu",
                "residual3", "lnf", "logits"):
        got = m.act(act).double().cpu().numpy()
        ref = o.act(act)
        got = got[: ref.size]
        c = cosine(got, ref)
        say(f"  {act}: cos {c:.6f} rel {rel_err(got, ref):.2e}")
        assert c >= 0.999, act
    lse = m.act("att_lse").double().cpu().numpy()
    att = o.act("att").reshape(w.L, B, w.NH, T, T)
    qkv = o.act("qkv").reshape(w.L, B, T, 3 * w.C)
    # log-sum-exp of layer 0 from the oracle's scores, recomputed here in float64
    q = qkv[0, :, :, :w.C].reshape(B, T, w.NH, 64).transpose(0, 2, 1, 3)
    k = qkv[0, :, :, w.C:2 * w.C].reshape(B, T, w.NH, 64).transpose(0, 2, 1, 3)
    s = q @ k.transpose(0, 1, 3, 2) / 8.0
    s = np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)
    ref_lse = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
    got_lse = lse[: B * w.NH * T].reshape(B, w.NH, T)
    assert np.abs(got_lse - ref_lse).max() < 0.05
    del att


# -------------------------------------------------------------- bf16 step --

def _bf16_cases():
    return [
        ("tiny_bf16", replace(WORKLOADS["tiny"], dtype="bf16", steps=3)),
        ("tiny_pad_bf16", replace(WORKLOADS["tiny_pad"], dtype="bf16", steps=2)),
        ("gpt2_124m_B2T96", WORKLOADS["gpt2_124m"].with_batch(B=2, T=96, steps=2)),
        ("gpt2_350m_L2_B1T128", replace(WORKLOADS["gpt2_350m"], L=2, B=1, T=128, steps=2)),
        ("gpt2_1558m_L2_B1T64", replace(WORKLOADS["gpt2_1558m"], L=2, B=1, T=64, steps=2)),
        # degenerate and ragged: one-token sequences (attention over a single
        # key, 3 GEMM rows), and B*T = 130 (not a multiple of the 64-row
        # reduction depth: the weight gradients take the register-staged path)
        ("gpt2_124m_L2_B3T1", replace(WORKLOADS["gpt2_124m"], L=2, B=3, T=1, steps=2)),
        ("gpt2_124m_L2_B1T130", replace(WORKLOADS["gpt2_124m"], L=2, B=1, T=130, steps=2)),
    ]


@pytest.mark.parametrize("case", _bf16_cases(), ids=[c[0] for c in _bf16_cases()])
def test_bf16_steps_match_oracle(case):
    name, w = case
    p, toks = _inputs(w)
    say(f"bf16 steps {name} ({w.steps} steps)")
    gpu = gpu_steps(w, p, toks, w.steps)
    ref = oracle_steps(w, p, toks, w.steps, threads=16)
    rep = check_bf16(w, gpu, ref)
    say({k: (f"{v:.4f}") for k, v in rep.items()})


def test_bf16_gelu_gradient_epilogue():
    """The fcproj input-gradient product applies GELU' of the stored
    pre-activation in its epilogue: per layer, d4C = (g2 W_fcproj) * gelu'(fch)
    against the same formula in float64 on the GPU's own bf16 inputs. The
    products are exact and summed in fp32, gelu' is evaluated in fp32, and the
    result is rounded to bf16 (2^-9): |gpu - ref| <= 2^-8 |ref| +
    1e-4 max|ref| per layer, cosine >= 0.99999. A gelu' off by a percent fails."""
    import torch
    from transformer_lm_amd import gpt2
    w = replace(WORKLOADS["gpt2_124m"], L=2, B=2, T=64, steps=1)
    p, toks = _inputs(w)
    x, y = synth.split_batch(toks[0])
    say("bf16 gelu' epilogue 124M L=2 B=2 T=64")
    m = gpt2.GPT2(gpt2.config(w), p)
    m.forward(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda())
    m.backward()
    torch.cuda.synchronize()
    BT, C, L = w.BT, w.C, w.L
    dres = m.act("dresidual").double().cpu().numpy()[: (2 * L + 1) * BT * C].reshape(
        2 * L + 1, BT, C)
    d4c = m.act("dbuf_4c").double().cpu().numpy()[: L * BT * 4 * C].reshape(L, BT, 4 * C)
    fch = m.act("fch").double().cpu().numpy()[: L * BT * 4 * C].reshape(L, BT, 4 * C)
    off, shape = param_offsets(w)["fcprojw"]
    wbf = m.region(gpt2.REGION_PARAM_BF16).double().cpu().numpy()
    Wfp = wbf[off:off + int(np.prod(shape))].reshape(L, C, 4 * C)
    k = np.sqrt(2.0 / np.pi)
    for l in range(L):
        g2 = dres[2 * (L - 1 - l)]          # dLoss/d(fcproj output) of layer l
        u = fch[l]
        a = k * (u + 0.044715 * u ** 3)
        th = np.tanh(a)
        gp = 0.5 * (1 + th) + 0.5 * u * (1 - th * th) * k * (1 + 3 * 0.044715 * u * u)
        ref = (g2 @ Wfp[l]) * gp
        got = d4c[l]
        mx = np.abs(ref).max()
        err = np.abs(got - ref)
        c = cosine(got.ravel(), ref.ravel())
        say(f"  layer {l}: max|d|/max|ref| {err.max() / mx:.2e}, cos {c:.7f}")
        assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-4 * mx).all(), l
        assert c >= 0.99999, l


def test_steps_are_deterministic():
    w = WORKLOADS["gpt2_124m"].with_batch(B=2, T=128, steps=1)
    p, toks = _inputs(w)
    say("determinism 124M bf16 B=2 T=128")
    a = gpu_steps(w, p, toks, 1, want=("params",))
    b = gpu_steps(w, p, toks, 1, want=("params",))
    assert a["losses"] == b["losses"]
    assert np.array_equal(a["grads"][1], b["grads"][1])
    assert np.array_equal(a["params"], b["params"])


@pytest.mark.parametrize("name", ["tiny", "gpt2_124m_B2T96"])
def test_checkpoint_resume_is_bit_exact(name):
    """Four steps straight through against two steps, a checkpoint, a fresh
    handle (started from other parameters) restored from it, and the last two
    steps on the same tokens: losses, parameters, moments and the bf16 copy
    agree bit for bit."""
    import torch
    from transformer_lm_amd import gpt2
    w = WORKLOADS["tiny"] if name == "tiny" else WORKLOADS["gpt2_124m"].with_batch(B=2, T=96)
    w = w.with_batch(steps=4)
    p, toks = _inputs(w)
    say(f"checkpoint resume {name}")

    def run(model, steps, losses):
        for s in steps:
            x, y = synth.split_batch(toks[s])
            losses.append(model.forward(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()))
            model.backward()
            model.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, s + 1)

    def state(model):
        regs = [gpt2.REGION_MASTER, gpt2.REGION_M, gpt2.REGION_V]
        if model.bf16:
            regs.append(gpt2.REGION_PARAM_BF16)
        return [model.region(r).cpu().clone() for r in regs]

    ref_losses, res_losses = [], []
    a = gpt2.GPT2(gpt2.config(w), p)
    run(a, range(4), ref_losses)
    ref = state(a)
    b = gpt2.GPT2(gpt2.config(w), p)
    run(b, range(2), res_losses)
    image = b.checkpoint(2)
    del b
    c = gpt2.GPT2(gpt2.config(w), synth.init_params(w) * 0.5)
    assert c.restore(image) == 2
    run(c, range(2, 4), res_losses)
    assert res_losses == ref_losses
    for x, y in zip(state(c), ref):
        assert torch.equal(x, y)
    # a foreign or mismatched image is refused
    with pytest.raises(gpt2.GPT2Error) as e:
        c.restore(image[:100])
    assert e.value.code == gpt2.GPT2_EINVAL
    bad = image.copy()
    bad[0] ^= 1
    with pytest.raises(gpt2.GPT2Error) as e:
        c.restore(bad)
    assert e.value.code == gpt2.GPT2_EINVAL
    other = gpt2.GPT2(gpt2.config(WORKLOADS["tiny_pad"]), synth.init_params(WORKLOADS["tiny_pad"]))
    with pytest.raises(gpt2.GPT2Error) as e:
        other.restore(image)
    assert e.value.code == gpt2.GPT2_ESHAPE


def test_nan_poisoned_parameter_gives_a_non_finite_loss():
    """A NaN in a parameter the step reads gives a NaN loss and NaN gradients
    through the ABI (as the oracle's own definition does), with no error code
    and no fault; a fresh handle on clean parameters then steps normally."""
    import torch
    from transformer_lm_amd import gpt2
    for dtype in ("fp32", "bf16"):
        w = replace(WORKLOADS["tiny"], dtype=dtype)
        p, toks = _inputs(w)
        x, y = synth.split_batch(toks[0])
        say(f"nan-poisoned parameter tiny {dtype}")
        off, _ = param_offsets(w)["ln1w"]
        bad = p.copy()
        bad[off + 3] = np.nan
        m = gpt2.GPT2(gpt2.config(w), bad)
        loss = m.forward(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda())
        assert np.isnan(loss)
        m.backward()
        m.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1)
        torch.cuda.synchronize()
        assert torch.isnan(m.region(gpt2.REGION_GRAD)).any()
        m.close()
        ok = gpt2.GPT2(gpt2.config(w), p)
        assert np.isfinite(ok.forward(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()))


def test_error_paths():
    import torch
    from transformer_lm_amd import gpt2
    w = WORKLOADS["tiny_pad"]
    p, toks = _inputs(w)
    x, y = synth.split_batch(toks[0])
    say("error paths tiny_pad")
    m = gpt2.GPT2(gpt2.config(w), p)
    with pytest.raises(gpt2.GPT2Error) as e:
        m.backward()
    assert e.value.code == gpt2.GPT2_ESTATE
    bad = x.copy()
    bad[1, 3] = w.V                   # a padded column is not a token
    with pytest.raises(gpt2.GPT2Error) as e:
        m.forward(torch.from_numpy(bad).cuda(), torch.from_numpy(y).cuda())
    assert e.value.code == gpt2.GPT2_ETOKEN
    # after GPT2_ETOKEN the backward is refused until the next forward
    with pytest.raises(gpt2.GPT2Error) as e:
        m.backward()
    assert e.value.code == gpt2.GPT2_ESTATE
    # the flag is cleared: a valid step afterwards succeeds
    loss = m.forward(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda())
    assert np.isfinite(loss)
    m.backward()
    m.update(1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    # a bad id in a forward that does not read the loss is reported by the
    # next checked forward, which names the unchecked call
    m.forward(torch.from_numpy(bad).cuda(), torch.from_numpy(y).cuda(), want_loss=False)
    m.backward()
    with pytest.raises(gpt2.GPT2Error) as e:
        m.forward(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda())
    assert e.value.code == gpt2.GPT2_ETOKEN
    assert "forward call 3 (not checked then); this is call 4" in str(e.value)
    loss = m.forward(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda())
    assert np.isfinite(loss)
    with pytest.raises(gpt2.GPT2Error) as e:
        m.update(1e-3, 0.9, 0.999, 1e-8, 0.0, 0)
    assert e.value.code == gpt2.GPT2_EINVAL
