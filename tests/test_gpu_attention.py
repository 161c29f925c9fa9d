"""GPU parity of causal self-attention on its own (gpt2_attention_forward,
the kernels the training step runs) against the CPU oracle, on inputs whose
score profiles drive the forward kernel's online softmax through every
branch: scores that climb by more than 2^8 (base 2) per 64-key tile, one
step of that size after 128 keys of comparable weight, a climb below the
step size, and plain random scores (transformer_lm_amd.synth.attention_qkv).

Bars. bf16 (matrix-core kernel): the probabilities are rounded to bf16 for
the product with V and the row sums add the same rounded values, so each
output is a convex combination of the values whose weights are off by at
most 2^-9 relatively, then rounded to bf16: |gpu - ref| <= 2^-7 max|v| +
2^-8 |ref| per head, and the log-sum-exp within 5e-3 (2^-9 on the row sum,
fp32 elsewhere). fp32 (row kernels): 1e-4 max|v| and 1e-4 on the
log-sum-exp."""
import numpy as np
import pytest

from parity import say
from transformer_lm_amd import synth
from oracle import wrapper as ow

pytestmark = pytest.mark.gpu
NH, HS = 4, 64
LOG2E = 1.4426950408889634


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _scores(x, B, T):
    """Scaled causal scores (B, NH, T, T) in float64, -inf above the diagonal."""
    C = NH * HS
    q = x[:, :, :C].reshape(B, T, NH, HS).transpose(0, 2, 1, 3)
    k = x[:, :, C:2 * C].reshape(B, T, NH, HS).transpose(0, 2, 1, 3)
    s = q @ k.transpose(0, 1, 3, 2) / 8.0
    return np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)


def _late_rescales(s, head):
    """Queries of one head whose 64-key tile maxima (base 2) pass the running
    reference by more than 2^8 after their first tile: the inputs must reach
    the forward kernel's rescaling branch there."""
    T = s.shape[-1]
    count = 0
    for b in range(s.shape[0]):
        for t in range(T):
            m = None
            for k0 in range(0, t + 1, 64):
                tm = s[b, head, t, k0:min(k0 + 64, t + 1)].max() * LOG2E
                if m is None:
                    m = tm
                elif tm > m + 8:
                    m, count = tm, count + 1
    return count


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,T", [(2, 300), (1, 1024), (1, 1), (3, 64)])
def test_attention_forward_matches_oracle(dtype, B, T):
    import torch
    from transformer_lm_amd import gpt2
    say(f"attention forward {dtype} B={B} T={T} NH={NH}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(synth.attention_qkv(B, T, NH)).to(tdt)
    xin = x.double().numpy()                          # the values the GPU reads
    ref, _ = ow.attention_forward(xin, NH)
    s = _scores(xin, B, T)
    mx = s.max(-1, keepdims=True)
    ref_lse = (np.log(np.exp(s - mx).sum(-1, keepdims=True)) + mx)[..., 0]
    if dtype == "bf16" and T == 300:
        for h in range(3):
            assert _late_rescales(s, h) > 0, h

    xd = x.cuda()
    out = torch.empty(B, T, NH * HS, dtype=tdt, device="cuda")
    lse = torch.empty(B, NH, T, dtype=torch.float32, device="cuda")
    gpt2.attention_forward(out, lse, xd, NH)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    got_lse = lse.double().cpu().numpy()

    v = xin[:, :, 2 * NH * HS:]
    for h in range(NH):
        sl = slice(h * HS, (h + 1) * HS)
        vmax = np.abs(v[:, :, sl]).max()
        err = np.abs(got[:, :, sl] - ref[:, :, sl])
        if dtype == "bf16":
            tol = 2.0 ** -7 * vmax + 2.0 ** -8 * np.abs(ref[:, :, sl])
            ltol = 5e-3
        else:
            tol = 1e-4 * vmax
            ltol = 1e-4
        lerr = np.abs(got_lse[:, h] - ref_lse[:, h]).max()
        say(f"  head {h}: out err/tol {(err / tol).max():.3f}, lse err {lerr:.2e}")
        assert (err <= tol).all(), h
        assert lerr <= ltol, h


def _backward_bound(x, dy, B, T):
    """Per-element bound on |gpu - ref| for the bf16 attention backward,
    first order in the roundings it makes (each at most 2^-9 relative; 2^-8
    is used for margin). With P, dS the exact probabilities and score
    gradients, s = 1/sqrt(hs):
      - D = sum_d dO O is formed from the bf16 output O, whose error (P
        rounded for the product with V, O stored in bf16) is at most
        2^-8 sum_t' P |v|; so dD_t <= 2^-8 sum_d |dO_t,d| (sum_t' P_t,t' |v_t',d|);
      - dq = s dS k: dS rounded to bf16 before the product, D's error times
        P, and the output rounding:
        2^-8 s |dS| |k| + s dD (P |k|) + 2^-8 |dq|;
      - dk = s dS^T q likewise: 2^-8 s |dS|^T |q| + s (dD P)^T |q| + 2^-8 |dk|;
      - dv = P^T dO: P rounded to bf16: 2^-8 P^T |dO| + 2^-8 |dv|.
    Rows whose keys are nearly equal make dq a sum that cancels almost
    entirely, so the bound is per element, not relative to dq itself."""
    C = NH * HS
    sc = 1.0 / np.sqrt(HS)
    bound = np.zeros((B, T, 3 * C))
    for b in range(B):
        for h in range(NH):
            sl = slice(h * HS, (h + 1) * HS)
            q, k, v = (x[b, :, i * C:(i + 1) * C][:, sl] for i in range(3))
            do = dy[b][:, sl]
            s = q @ k.T * sc
            s = np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)
            p = np.exp(s - s.max(-1, keepdims=True))
            p /= p.sum(-1, keepdims=True)
            o = p @ v
            dp = do @ v.T
            ds = p * (dp - (do * o).sum(-1, keepdims=True))
            dD = 2.0 ** -8 * (np.abs(do) * (p @ np.abs(v))).sum(-1, keepdims=True)
            dq, dk, dv = sc * ds @ k, sc * ds.T @ q, p.T @ do
            e = 2.0 ** -8
            bound[b, :, sl] = e * sc * np.abs(ds) @ np.abs(k) + sc * dD * (p @ np.abs(k)) + \
                e * np.abs(dq)
            bound[b, :, C:][:, sl] = e * sc * np.abs(ds).T @ np.abs(q) + \
                sc * (dD * p).T @ np.abs(q) + e * np.abs(dk)
            bound[b, :, 2 * C:][:, sl] = e * p.T @ np.abs(do) + e * np.abs(dv)
    return bound


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,T", [(1, 1024), (2, 300), (1, 1), (3, 64)])
def test_attention_backward_matches_oracle(dtype, B, T):
    """gpt2_attention_backward (the kernels the training step runs) against
    the oracle's softmax backward on the same inputs, at up to T = 1024.

    Bars. bf16: every element within the first-order rounding bound of
    _backward_bound (+ 1e-6). fp32 (row kernels): |gpu - ref| <= 1e-4
    max|ref| (+ 1e-6) per head and q / k / v block. The crafted heads make
    the keys of neighbouring positions nearly equal, so dq cancels almost
    entirely there: cosine is reported, not required."""
    import torch
    from transformer_lm_amd import gpt2
    say(f"attention backward {dtype} B={B} T={T} NH={NH}")
    C = NH * HS
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(synth.attention_qkv(B, T, NH)).to(tdt)
    dy = torch.from_numpy(synth.attention_dout(B, T, C)).to(tdt)
    xin, dyin = x.double().numpy(), dy.double().numpy()
    ref = ow.attention_backward(xin, dyin, NH)

    xd, dyd = x.cuda(), dy.cuda()
    out = torch.empty(B, T, C, dtype=tdt, device="cuda")
    lse = torch.empty(B, NH, T, dtype=torch.float32, device="cuda")
    dqkv = torch.full((B, T, 3 * C), float("nan"), dtype=tdt, device="cuda")
    work = torch.empty(2 * B * NH * T, dtype=torch.float32, device="cuda")
    gpt2.attention_forward(out, lse, xd, NH)
    gpt2.attention_backward(dqkv, work, dyd, xd, out, lse, NH)
    torch.cuda.synchronize()
    got = dqkv.double().cpu().numpy()
    assert np.isfinite(got).all()
    bound = _backward_bound(xin, dyin, B, T) if dtype == "bf16" else None
    for part, name in enumerate("qkv"):
        for h in range(NH):
            sl = slice(part * C + h * HS, part * C + (h + 1) * HS)
            r, gg = ref[:, :, sl], got[:, :, sl]
            m = np.abs(r).max()
            err = np.abs(gg - r)
            c = float(np.dot(gg.ravel(), r.ravel()) /
                      max(np.linalg.norm(gg) * np.linalg.norm(r), 1e-300))
            if dtype == "bf16":
                bd = bound[:, :, sl] + 1e-6
                say(f"  d{name} head {h}: max|d|/max|ref| {err.max() / max(m, 1e-30):.2e}, "
                    f"err/bound {(err / bd).max():.3f}, cos {c:.6f}")
                assert (err <= bd).all(), (name, h)
            else:
                say(f"  d{name} head {h}: max|d|/max|ref| {err.max() / max(m, 1e-30):.2e}")
                assert err.max() <= 1e-4 * m + 1e-6, (name, h)


def test_attention_forward_rejects_bad_shapes():
    import torch
    from transformer_lm_amd import gpt2
    x = torch.zeros(1, 8, 3 * 120, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(1, 8, 120, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, 2, 8, dtype=torch.float32, device="cuda")
    with pytest.raises(gpt2.GPT2Error):
        gpt2.attention_forward(out, lse, x, 2)         # head size 60
