"""The step of oracle/gpt2_torch.py with bf16 storage: a second, independent
model of what a bf16 training step computes, used to size how far rounding
alone moves a multi-step loss trajectory.

TEST INFRASTRUCTURE ONLY (the same rules as oracle/gpt2_torch.py: only the
test suite and the scripts under tests/golden/ use it; it shares no code with
the GPU library).

The arithmetic is the float32 oracle's, operation for operation; what is
added is a rounding to bf16 (nearest, ties to even) wherever the bf16 step of
the pages keeps a tensor in bf16 (page "llm.c: Large Language Model Training
in Pure C/CUDA Without Dependencies", its mixed-precision feature: bf16
parameters and activations, fp32 master weights and optimiser state):
  - the working copy of the parameters that the forward and backward read
    (refreshed from the fp32 master after every update);
  - every activation a layer writes: the encoder output, LayerNorm outputs,
    qkv, the attention output (and the attention probabilities and score
    gradients before their products), the residual stream after each
    addition, the fc output and its GELU, the final LayerNorm output, the
    logits and their gradient;
  - every activation gradient the backward writes (each layer's input
    gradients and the residual-stream gradient after each addition).
Parameter gradients, LayerNorm statistics, softmax sums, the loss and
AdamW's state stay float32, as do all sums inside an operation.

Its summation orders are the library's matrix multiply's, not the GPU
kernels': it is a second bf16 implementation, not a copy of the GPU's.
"""
import math

import numpy as np
import torch

from oracle.gpt2_torch import (TorchOracle, _heads, _views, adamw_, gelu_backward,
                               gelu_forward, layernorm_backward, layernorm_forward,
                               matmul_backward, matmul_forward)


def r16(t):
    """t rounded to the nearest bf16 value (ties to even), kept as float32."""
    return t.to(torch.bfloat16).to(torch.float32)


def _probs_bf16(q, k):
    """Causal softmax of one sequence's scaled scores (all heads), as float32
    sums of the probabilities rounded to bf16: returns (P_bf16 / l, P_bf16, l)
    where l is the row sum of the rounded probabilities."""
    T, hs = q.shape[1], q.shape[2]
    s = (q @ k.transpose(1, 2)) * (1.0 / math.sqrt(hs))
    mask = torch.ones(T, T, dtype=torch.bool).triu_(1)
    s.masked_fill_(mask, -math.inf)
    s -= s.amax(dim=-1, keepdim=True)
    pb = r16(torch.exp(s))
    lsum = pb.sum(dim=-1, keepdim=True)
    return pb / lsum, pb, lsum


def attention_forward_bf16(qkv, B, T, C, NH):
    """y = (P_bf16 V) / l per head, rounded to bf16."""
    y = torch.empty(B * T, C)
    for b in range(B):
        q, k, v = _heads(qkv[b * T:(b + 1) * T], C, NH)
        _, pb, lsum = _probs_bf16(q, k)
        y[b * T:(b + 1) * T] = ((pb @ v) / lsum).transpose(0, 1).reshape(T, C)
    return r16(y)


def attention_backward_bf16(dy, qkv, B, T, C, NH):
    """The oracle's attention backward with P and dS rounded to bf16 before
    their products and dqkv rounded to bf16."""
    hs = C // NH
    scale = 1.0 / math.sqrt(hs)
    dqkv = torch.empty(B * T, 3 * C)
    for b in range(B):
        q, k, v = _heads(qkv[b * T:(b + 1) * T], C, NH)
        p, _, _ = _probs_bf16(q, k)
        dyb = dy[b * T:(b + 1) * T].reshape(T, NH, hs).transpose(0, 1)
        dp = dyb @ v.transpose(1, 2)
        dv = r16(p).transpose(1, 2) @ dyb
        ds = r16(p * (dp - (p * dp).sum(dim=-1, keepdim=True)))
        dq = (ds @ k) * scale
        dk = (ds.transpose(1, 2) @ q) * scale
        rows = dqkv[b * T:(b + 1) * T]
        rows[:, :C] = dq.transpose(0, 1).reshape(T, C)
        rows[:, C:2 * C] = dk.transpose(0, 1).reshape(T, C)
        rows[:, 2 * C:] = dv.transpose(0, 1).reshape(T, C)
    return r16(dqkv)


class TorchOracleBF16Storage(TorchOracle):
    """TorchOracle (float32) with bf16 storage as listed in the module text."""

    def __init__(self, w, params, threads=None):
        super().__init__(w, params, dtype=torch.float32, threads=threads)
        self._refresh()

    def _refresh(self):
        # the working copy is held in bf16 (half the host memory of a float32
        # copy); _P widens the slices an operation reads
        self.work = self.theta.to(torch.bfloat16)
        self.pw = _views(self.work, self.w)

    def _P(self, name, l=None):
        t = self.pw[name] if l is None else self.pw[name][l]
        return t.to(torch.float32)

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
        P = self._P
        pos = torch.arange(T).repeat(B)
        x = r16(P("wte")[tok] + P("wpe")[pos])
        layers = []
        for l in range(L):
            ln1, mu1, r1 = layernorm_forward(x, P("ln1w", l), P("ln1b", l))
            ln1 = r16(ln1)
            qkv = r16(matmul_forward(ln1, P("qkvw", l), P("qkvb", l)))
            atty = attention_forward_bf16(qkv, B, T, C, NH)
            res2 = r16(x + matmul_forward(atty, P("attprojw", l), P("attprojb", l)))
            ln2, mu2, r2 = layernorm_forward(res2, P("ln2w", l), P("ln2b", l))
            ln2 = r16(ln2)
            fch = r16(matmul_forward(ln2, P("fcw", l), P("fcb", l)))
            gl = r16(gelu_forward(fch))
            res3 = r16(res2 + matmul_forward(gl, P("fcprojw", l), P("fcprojb", l)))
            layers.append(dict(x=x, ln1=ln1, mu1=mu1, r1=r1, qkv=qkv, atty=atty, res2=res2,
                               ln2=ln2, mu2=mu2, r2=r2, fch=fch))
            x = res3
        lnf, muf, rf = layernorm_forward(x, P("lnfw"), P("lnfb"))
        lnf = r16(lnf)
        z = r16(matmul_forward(lnf, P("wte"), None))[:, :V]
        z = z - z.amax(dim=-1, keepdim=True)
        e = torch.exp(z)
        probs = torch.zeros(BT, w.Vp)
        probs[:, :V] = e / e.sum(dim=-1, keepdim=True)
        losses = torch.logsumexp(z, dim=-1) - z[torch.arange(BT), tgt]
        self.saved = dict(tok=tok, tgt=tgt, B=B, T=T, layers=layers, xL=x, lnf=lnf, muf=muf,
                          rf=rf, probs=probs)
        self.losses = losses.double().numpy()
        return float(losses.double().mean())

    def backward(self):
        if self.saved is None:
            raise RuntimeError("backward needs a forward with targets")
        s, w, g = self.saved, self.w, self.g
        P = self._P
        B, T = s["B"], s["T"]
        C, L, NH, V = w.C, w.L, w.NH, w.V
        BT = B * T
        self.grad.zero_()
        dz = s.pop("probs")
        dz[torch.arange(BT), s["tgt"]] -= 1.0
        dz[:, :V] *= 1.0 / BT
        dz = r16(dz)
        dlnf, dwte_head, _ = matmul_backward(dz, s["lnf"], P("wte"))
        del dz
        g["wte"] += dwte_head
        del dwte_head
        dlnf = r16(dlnf)
        dx, dw_, db_ = layernorm_backward(dlnf, s["xL"], P("lnfw"), s["muf"], s["rf"])
        dx = r16(dx)
        g["lnfw"] += dw_
        g["lnfb"] += db_
        for l in range(L - 1, -1, -1):
            a = s["layers"][l]
            gl = r16(gelu_forward(a["fch"]))
            dgelu, dW, db = matmul_backward(dx, gl, P("fcprojw", l))
            g["fcprojw"][l] += dW
            g["fcprojb"][l] += db
            del gl
            dfch = r16(gelu_backward(a["fch"], dgelu))
            del dgelu
            dln2, dW, db = matmul_backward(dfch, a["ln2"], P("fcw", l))
            g["fcw"][l] += dW
            g["fcb"][l] += db
            del dfch
            dln2 = r16(dln2)
            dres2, dw_, db_ = layernorm_backward(dln2, a["res2"], P("ln2w", l), a["mu2"], a["r2"])
            g["ln2w"][l] += dw_
            g["ln2b"][l] += db_
            dx = r16(dx + dres2)
            datty, dW, db = matmul_backward(dx, a["atty"], P("attprojw", l))
            g["attprojw"][l] += dW
            g["attprojb"][l] += db
            dqkv = attention_backward_bf16(r16(datty), a["qkv"], B, T, C, NH)
            del datty
            dln1, dW, db = matmul_backward(dqkv, a["ln1"], P("qkvw", l))
            g["qkvw"][l] += dW
            g["qkvb"][l] += db
            del dqkv
            dln1 = r16(dln1)
            dres, dw_, db_ = layernorm_backward(dln1, a["x"], P("ln1w", l), a["mu1"], a["r1"])
            g["ln1w"][l] += dw_
            g["ln1b"][l] += db_
            dx = r16(dx + dres)
            s["layers"][l] = None
        g["wte"].index_add_(0, s["tok"], dx)
        g["wpe"][:T] += dx.view(B, T, C).sum(dim=0)
        self.saved = None

    def update(self, lr, b1, b2, eps, wd, t):
        adamw_(self.theta, self.grad, self.m, self.v, lr, b1, b2, eps, wd, int(t))
        self._refresh()
