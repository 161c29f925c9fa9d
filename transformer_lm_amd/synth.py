"""Seeded synthetic inputs for the GPT-2 training step: initial parameters and
token batches.

Both the CPU oracle and the GPU path read the bytes written here; this module
holds none of the model's arithmetic.

Random source: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style: word i of the stream
with seed s is mix64(s + (i + 1) * 0x9E3779B97F4A7C15). Uniform doubles take
the top 53 bits. Normals come from the Box-Muller transform on word pairs
(2p, 2p+1): element 2p takes the cosine branch, 2p+1 the sine branch.

Parameter initialisation (GPT-2 as llm.c trains it): wte rows < V, wpe, qkvw,
fcw ~ N(0, 0.02); attprojw and fcprojw ~ N(0, 0.02 / sqrt(2L)); biases 0;
LayerNorm gains 1, shifts 0; padded wte rows (>= V) are 0. The normal stream is
indexed by flat position in the parameter array, so any slice can be
regenerated on its own.

FP8 product operands (fp8_operands): an activation block x[M, K] ~ N(0, 1)
(the scale of LayerNorm outputs that feed the products), a weight w[N, K] ~
N(0, 0.02) and a bias b[N] ~ N(0, 0.02), from three seeds derived from one.

Tokens: uniform integers on [0, V) or a bounded Zipf law
P(k) = (k+1)^-s / H over k in [0, V), drawn by inverse CDF on a float64
cumulative table (smallest k with CDF(k) > u). Each optimiser step draws a
fresh (B, T+1) block; inputs are [:, :T] and targets [:, 1:].
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .workloads import param_offsets

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def splitmix64(seed, start, count):
    """Words start .. start+count-1 of the SplitMix64 stream for `seed`."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed) + idx * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def uniform(seed, start, count):
    """Doubles in [0, 1) from words start .. start+count-1."""
    w = splitmix64(seed, start, count)
    return (w >> np.uint64(11)).astype(np.float64) * (1.0 / (1 << 53))


def normal(seed, start, count):
    """Standard normals for stream elements start .. start+count-1 (float64).

    Element e uses the word pair (2*(e//2), 2*(e//2)+1)."""
    if count <= 0:
        return np.zeros(0, np.float64)
    p0 = start // 2
    p1 = (start + count - 1) // 2 + 1
    u = uniform(seed, 2 * p0, 2 * (p1 - p0)).reshape(-1, 2)
    r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))      # 1-u in (0, 1]
    th = 2.0 * math.pi * u[:, 1]
    z = np.empty((p1 - p0, 2), np.float64)
    z[:, 0] = r * np.cos(th)
    z[:, 1] = r * np.sin(th)
    z = z.reshape(-1)
    off = start - 2 * p0
    return z[off:off + count]


def _fill_normal(out, seed, flat_start, std):
    """out[i] = std * normal element (flat_start + i), in chunks (bounded
    memory) spread over threads; every element depends only on its index, so
    the bytes do not depend on the thread count."""
    n = out.size

    def chunk(c0):
        c1 = min(n, c0 + _CHUNK)
        out[c0:c1] = (std * normal(seed, flat_start + c0, c1 - c0)).astype(np.float32)

    starts = range(0, n, _CHUNK)
    if len(starts) <= 1:
        for c0 in starts:
            chunk(c0)
        return
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1, len(starts))) as ex:
        list(ex.map(chunk, starts))


def init_params(w, seed=None):
    """The initial flat fp32 parameter array for workload `w`."""
    seed = w.param_seed if seed is None else seed
    offs = param_offsets(w)
    n = w.num_params()
    p = np.zeros(n, np.float32)
    std = 0.02
    proj_std = 0.02 / math.sqrt(2 * w.L)
    for name, (off, shape) in offs.items():
        cnt = int(np.prod(shape))
        view = p[off:off + cnt]
        if name == "wte":
            _fill_normal(view[: w.V * w.C], seed, off, std)
        elif name in ("wpe", "qkvw", "fcw"):
            _fill_normal(view, seed, off, std)
        elif name in ("attprojw", "fcprojw"):
            _fill_normal(view, seed, off, proj_std)
        elif name in ("ln1w", "ln2w", "lnfw"):
            view[:] = 1.0
        # biases and LayerNorm shifts stay 0
    return p


def zipf_cdf(V, s):
    """Float64 cumulative table of the bounded Zipf law over [0, V)."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def tokens(w, seed=None, steps=None):
    """int32 array (steps, B, T+1) of token ids for workload `w`."""
    seed = w.token_seed if seed is None else seed
    steps = w.steps if steps is None else steps
    n = steps * w.B * (w.T + 1)
    u = uniform(seed, 0, n)
    if w.token_dist == "uniform":
        ids = np.minimum(np.floor(u * w.V), w.V - 1)
    elif w.token_dist == "zipf":
        ids = np.minimum(np.searchsorted(zipf_cdf(w.V, w.zipf_s), u, side="right"),
                         w.V - 1)
    else:
        raise ValueError(f"unknown token distribution {w.token_dist!r}")
    return ids.astype(np.int32).reshape(steps, w.B, w.T + 1)


def split_batch(tok_step):
    """(B, T+1) block -> (inputs (B, T), targets (B, T)), both C-contiguous."""
    return (np.ascontiguousarray(tok_step[:, :-1]),
            np.ascontiguousarray(tok_step[:, 1:]))


def fp8_operands(M, N, K, seed=20240):
    """(x[M, K], w[N, K], b[N]) float32 for the FP8 products."""
    x = np.empty(M * K, np.float32)
    w = np.empty(N * K, np.float32)
    b = np.empty(N, np.float32)
    _fill_normal(x, seed, 0, 1.0)
    _fill_normal(w, seed + 1, 0, 0.02)
    _fill_normal(b, seed + 2, 0, 0.02)
    return x.reshape(M, K), w.reshape(N, K), b


def attention_qkv(B, T, NH, seed=31337):
    """Fused (B, T, 3C) float32 attention inputs, head size 64, whose scaled
    scores q_t . k_t' / 8 follow a per-head key profile f(t') plus small
    noise: head 0 rises by 0.1 per key, head 1 steps up by 6.25 at key 128,
    head 2 rises by 0.055 per key (q_t = 4e + 0.25 n, k_t' = 2 f(t') e +
    0.25 n' with e the unit vector of equal entries); other heads draw plain
    N(0, 1) queries and keys. Values ~ N(0, 1)."""
    hs = 64
    n = np.empty(B * T * 3 * NH * hs, np.float32)
    _fill_normal(n, seed, 0, 1.0)
    n = n.reshape(B, T, 3, NH, hs)
    qkv = n.copy()
    e = np.full(hs, 1.0 / 8.0, np.float32)
    t = np.arange(T, dtype=np.float32)
    profiles = (0.1 * t, np.where(t >= 128, 6.25, 0.0).astype(np.float32), 0.055 * t)
    for h, f in enumerate(profiles[:NH]):
        qkv[:, :, 0, h] = 4.0 * e + 0.25 * n[:, :, 0, h]
        qkv[:, :, 1, h] = 2.0 * f[None, :, None] * e + 0.25 * n[:, :, 1, h]
    return qkv.reshape(B, T, 3 * NH * hs)


def attention_dout(B, T, C, seed=31338):
    """Output gradient (B, T, C) float32 ~ N(0, 1) for the attention backward."""
    d = np.empty(B * T * C, np.float32)
    _fill_normal(d, seed, 0, 1.0)
    return d.reshape(B, T, C)
