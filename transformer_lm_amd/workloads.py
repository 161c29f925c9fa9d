"""The GPT-2 training-step workloads: model shapes, batch shapes, optimiser
constants and input seeds.

These are plain data. The model is GPT-2 as llm.c trains it (page "Building
GPT-2 from scratch", exercise table rows A1 "Forward pass" and A2 "Backprop and
AdamW"): pre-LayerNorm blocks, a tanh-GELU MLP of width 4C, tied token
embedding / output head, AdamW over one flat parameter array.

Five workloads are defined, from a tiny fp32 model that a plain CPU
implementation steps in milliseconds up to the 1.5B-parameter shape, plus a
tiny variant whose vocabulary (61) is padded to 64 columns.
"""
from dataclasses import dataclass, replace
import math


@dataclass(frozen=True)
class Workload:
    name: str
    V: int          # real vocabulary size
    Vp: int         # padded vocabulary size (rows of wte, columns of logits)
    max_T: int      # rows of wpe
    C: int          # channels
    L: int          # layers
    NH: int         # heads
    B: int          # batch
    T: int          # sequence length (<= max_T)
    steps: int      # consecutive optimiser steps
    dtype: str      # "fp32" or "bf16" (bf16: fp32 master weights and moments)
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    token_dist: str  # "uniform" or "zipf"
    token_seed: int
    param_seed: int
    zipf_s: float = 1.1

    @property
    def hs(self):
        return self.C // self.NH

    @property
    def BT(self):
        return self.B * self.T

    def num_params(self):
        return sum(n for _, _, n in param_shapes(self))

    def flops_per_token(self):
        """Dense forward+backward FLOPs per trained token: 6 x (matmul
        parameters used per token) plus causal attention (Q.K^T and P.V, each
        averaged over the causal half, forward and twice in backward)."""
        C, L, V, T = self.C, self.L, self.V, self.T
        return 6 * (12 * L * C * C + C * V) + 6 * L * T * C

    def with_batch(self, B=None, T=None, steps=None):
        kw = {}
        if B is not None:
            kw["B"] = B
        if T is not None:
            kw["T"] = T
        if steps is not None:
            kw["steps"] = steps
        return replace(self, **kw)


def param_shapes(w):
    """Tensor-major flat layout of the parameter array: (name, shape, count),
    in storage order. Weights are stored (out, in) row-major; the fused qkv
    weight holds the row blocks [Q; K; V]."""
    C, L = w.C, w.L
    shapes = [
        ("wte", (w.Vp, C)),
        ("wpe", (w.max_T, C)),
        ("ln1w", (L, C)), ("ln1b", (L, C)),
        ("qkvw", (L, 3 * C, C)), ("qkvb", (L, 3 * C)),
        ("attprojw", (L, C, C)), ("attprojb", (L, C)),
        ("ln2w", (L, C)), ("ln2b", (L, C)),
        ("fcw", (L, 4 * C, C)), ("fcb", (L, 4 * C)),
        ("fcprojw", (L, C, 4 * C)), ("fcprojb", (L, C)),
        ("lnfw", (C,)), ("lnfb", (C,)),
    ]
    return [(n, s, math.prod(s)) for n, s in shapes]


def param_offsets(w):
    """name -> (offset in elements, shape)."""
    out, off = {}, 0
    for n, s, cnt in param_shapes(w):
        out[n] = (off, s)
        off += cnt
    return out


def pad_vocab(V, multiple=64):
    return ((V + multiple - 1) // multiple) * multiple


_TINY = Workload(
    name="tiny", V=64, Vp=64, max_T=32, C=32, L=2, NH=4, B=4, T=16, steps=1,
    dtype="fp32", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
    token_dist="uniform", token_seed=1001, param_seed=2001)

WORKLOADS = {
    # fp32, one full step; uniform tokens.
    "tiny": _TINY,
    # the same with a vocabulary of 61 padded to 64 columns.
    "tiny_pad": replace(_TINY, name="tiny_pad", V=61, Vp=64,
                        token_seed=1006, param_seed=2006),
    # GPT-2 124M shape, fp32, one step, short sequences.
    "gpt2_124m_fp32": Workload(
        name="gpt2_124m_fp32", V=50257, Vp=50304, max_T=1024, C=768, L=12,
        NH=12, B=4, T=64, steps=1, dtype="fp32", lr=1e-3, beta1=0.9,
        beta2=0.999, eps=1e-8, weight_decay=0.0, token_dist="zipf",
        token_seed=1002, param_seed=2002),
    # GPT-2 124M, bf16 with fp32 master weights and moments: the timed workload.
    "gpt2_124m": Workload(
        name="gpt2_124m", V=50257, Vp=50304, max_T=1024, C=768, L=12, NH=12,
        B=16, T=1024, steps=20, dtype="bf16", lr=6e-4, beta1=0.9, beta2=0.999,
        eps=1e-8, weight_decay=0.1, token_dist="zipf", token_seed=1003,
        param_seed=2003),
    "gpt2_350m": Workload(
        name="gpt2_350m", V=50257, Vp=50304, max_T=1024, C=1024, L=24, NH=16,
        B=8, T=1024, steps=10, dtype="bf16", lr=6e-4, beta1=0.9, beta2=0.999,
        eps=1e-8, weight_decay=0.1, token_dist="zipf", token_seed=1004,
        param_seed=2004),
    "gpt2_1558m": Workload(
        name="gpt2_1558m", V=50257, Vp=50304, max_T=1024, C=1600, L=48, NH=25,
        B=4, T=1024, steps=5, dtype="bf16", lr=6e-4, beta1=0.9, beta2=0.999,
        eps=1e-8, weight_decay=0.1, token_dist="zipf", token_seed=1005,
        param_seed=2005),
}
