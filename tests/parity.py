"""Helpers for the GPU-vs-oracle parity tests: run the same seeded step on
both sides and compare with the tolerances of the training-step contract.

fp32 mode: loss relative error <= 1e-5; per parameter tensor
max|g - g_ref| / max|g_ref| <= 1e-3. bf16 mode (fp32 master weights): loss
within 2e-2 absolute of the fp32-or-better oracle; per-tensor gradient cosine
similarity >= 0.99.
"""
import sys

import numpy as np

from transformer_lm_amd import synth
from transformer_lm_amd.workloads import param_offsets

FP32_LOSS_REL = 1e-5
FP32_GRAD_REL = 1e-3
BF16_LOSS_ABS = 2e-2
BF16_GRAD_COS = 0.99


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def per_tensor(w, flat):
    return {n: flat[off:off + int(np.prod(s))] for n, (off, s) in param_offsets(w).items()}


def rel_err(a, ref):
    m = np.abs(ref).max()
    d = np.abs(a - ref).max()
    return d / m if m > 0 else d


def cosine(a, b):
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    if na == 0 or nb == 0:
        return 0.0
    return float(np.dot(a, b) / (na * nb))


def gpu_steps(w, params, toks, steps, keep_grads_at=(1,), want=("params", "m", "v"), sched=None):
    """Runs `steps` training steps through the C ABI; returns per-step losses,
    the gradients after the listed steps (fp64 numpy) and the final regions.
    sched (dict: lr_max, lr_min, warmup, total, grad_clip) switches to the
    scheduled, clipped update and records the gradient norm of each step."""
    import torch
    from transformer_lm_amd import gpt2
    model = gpt2.GPT2(gpt2.config(w), params)
    out = {"losses": [], "grads": {}, "norms": []}
    for s in range(steps):
        x, y = synth.split_batch(toks[s])
        xd = torch.from_numpy(x).cuda()
        yd = torch.from_numpy(y).cuda()
        out["losses"].append(model.forward(xd, yd))
        model.backward()
        if s + 1 in keep_grads_at:
            out["grads"][s + 1] = model.region(gpt2.REGION_GRAD).double().cpu().numpy()
        if sched is None:
            model.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, s + 1)
        else:
            model.update_scheduled(schedule_struct(w, sched), s + 1)
            out["norms"].append(float(model.act("grad_norm")[0].item()))
    torch.cuda.synchronize()
    if "params" in want:
        out["params"] = model.region(gpt2.REGION_MASTER).double().cpu().numpy()
    if "m" in want:
        out["m"] = model.region(gpt2.REGION_M).double().cpu().numpy()
    if "v" in want:
        out["v"] = model.region(gpt2.REGION_V).double().cpu().numpy()
    out["model"] = model
    return out


def schedule_struct(w, sched):
    from transformer_lm_amd import gpt2
    return gpt2.Schedule(sched["lr_max"], sched["lr_min"], sched["warmup"], sched["total"],
                         w.beta1, w.beta2, w.eps, w.weight_decay, sched["grad_clip"])


def oracle_steps(w, params, toks, steps, keep_grads_at=(1,), precision="f64", threads=None,
                 sched=None):
    from oracle.wrapper import Oracle
    o = Oracle(w, params, precision=precision, threads=threads)
    out = {"losses": [], "grads": {}, "norms": []}
    for s in range(steps):
        x, y = synth.split_batch(toks[s])
        out["losses"].append(o.forward(x, y))
        o.backward()
        if s + 1 in keep_grads_at:
            out["grads"][s + 1] = o.grads()
        if sched is None:
            o.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, s + 1)
        else:
            out["norms"].append(o.update_scheduled(
                sched["lr_max"], sched["lr_min"], sched["warmup"], sched["total"], w.beta1,
                w.beta2, w.eps, w.weight_decay, sched["grad_clip"], s + 1))
    out["params"] = o.params()
    out["m"] = o.m()
    out["v"] = o.v()
    out["oracle"] = o
    return out


def check_fp32(w, gpu, ref, step=1):
    """Asserts the fp32-mode tolerances; returns a report dict."""
    rep = {}
    for s, (lg, lr_) in enumerate(zip(gpu["losses"], ref["losses"]), 1):
        rel = abs(lg - lr_) / abs(lr_)
        rep[f"loss_rel_step{s}"] = rel
        assert rel <= FP32_LOSS_REL, (s, lg, lr_)
    gg, gr = per_tensor(w, gpu["grads"][step]), per_tensor(w, ref["grads"][step])
    for name in gr:
        e = rel_err(gg[name], gr[name])
        rep[f"grad_{name}"] = e
        assert e <= FP32_GRAD_REL, (name, e)
    return rep


def check_bf16(w, gpu, ref, step=1):
    rep = {}
    for s, (lg, lr_) in enumerate(zip(gpu["losses"], ref["losses"]), 1):
        d = abs(lg - lr_)
        rep[f"loss_abs_step{s}"] = d
        assert d <= BF16_LOSS_ABS, (s, lg, lr_)
    gg, gr = per_tensor(w, gpu["grads"][step]), per_tensor(w, ref["grads"][step])
    for name in gr:
        c = cosine(gg[name], gr[name])
        rep[f"cos_{name}"] = c
        assert c >= BF16_GRAD_COS, (name, c)
    return rep


def bf16_round(x):
    """Round float32 values to bfloat16 (nearest, ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)
