"""Training throughput of the GPT-2 124M step (bf16, fp32 master weights and
AdamW moments, B=16, T=1024) on one MI355X, through the C ABI.

One step = the upload of the step's tokens from pinned host memory (2 x 64 KB)
+ forward with the mean loss read back + backward + AdamW update, on seeded
synthetic Zipf(1.1) tokens; parameters and activations are resident in HBM.
Prints one JSON line: tokens/s over the K timed steps (and the median and
minimum per-step time), MFU against the bf16 dense peak, every kernel class
against its roofline (HIP events in a profiled warmup step), the dominant
kernel measured again inside the timed steps, and the CPU oracle timed on a
bounded sample of the same workload.

The dominant kernel is the single kernel with the most time per step: among
the classes whose every timed launch is one kernel of one symbol
(SINGLE_KERNEL_CLASSES), the one with the largest time. At 124M that is the
grouped weight-gradient launch, one gemm_stream_kernel launch per step for
the weight gradients of all layers and the output head; the forward products
are five kernels (one per epilogue) and appear, like every class, in
"classes".

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-fp8]

A second object, "fp8_matmul", measures the FP8 (E4M3) products on the same
model's forward shapes (not part of the training step, which stays bf16).
"""
import argparse
import json
import os
import sys
import time
from dataclasses import replace

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA, published
# classes timed as launches of a single kernel symbol (the others group
# several kernels: the products' epilogue variants, the attention backward's
# two kernels, the LayerNorm backward and its reductions, the classifier and
# the loss mean, the encoder backward's sort)
SINGLE_KERNEL_CLASSES = {
    "matmul_bwd_dw": "gemm_stream_kernel<128, 192, 64, 2, 2, 8, 2, 2, true, true, 1, true>",
    "attention_fwd": "flash_fwd_kernel",
    "adamw": "adamw_kernel",
    "layernorm_fwd": "layernorm_fwd_kernel",
}
PEAK_FP8_FLOPS = 5.0e15    # MI355X dense fp8 MFMA, published
PEAK_HBM_BYTES = 8.0e12    # MI355X HBM3E, published
WORKLOAD = "gpt2_124m"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def recorded_traffic(cls):
    """HBM bytes per launch of kernel class `cls` as the FETCH_SIZE / WRITE_SIZE
    counter passes recorded them, or None when the kernel sources have changed
    since (the recorded figures no longer describe the kernels that ran)."""
    from transformer_lm_amd.prof_summary import source_sha
    path = os.path.join(ROOT, "profiles", "gpt2_124m_bf16_B16_T1024_class_traffic.txt")
    if not os.path.exists(path):
        return None
    sha, rows = None, {}
    for line in open(path):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "source_sha256":
            sha = f[1]
        elif len(f) == 3:
            rows[f[0]] = (float(f[1]), float(f[2]))
    if sha != source_sha() or cls not in rows:
        return None
    return {"fetch_bytes": round(rows[cls][0]), "write_bytes": round(rows[cls][1]),
            "bytes": round(rows[cls][0] + rows[cls][1])}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_step_seconds(w, threads, precision="f32n"):
    """Seconds of one training step (forward with loss, backward, AdamW) of the
    oracle on workload w's first batch."""
    from oracle.wrapper import Oracle
    from transformer_lm_amd import synth
    p = synth.init_params(w)
    x, y = synth.split_batch(synth.tokens(w, steps=1)[0])
    o = Oracle(w, p, precision=precision, threads=threads)
    t0 = time.perf_counter()
    o.forward(x, y)
    o.backward()
    o.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1)
    dt = time.perf_counter() - t0
    used = o.lib.oracle_get_threads()
    o.close()
    return dt, used


def cpu_baseline(w, T_sample=1024, single_thread=True):
    """The oracle as it stands (plain loops; OpenMP over independent outputs),
    built in single precision with -O2 -march=native -fopenmp
    -ffp-contract=off and no fast math, timed on this host:
      - value: one training step of the same model on one sequence of T_sample
        tokens, on every thread the process may use (OMP_NUM_THREADS if set);
      - single_thread: one step of the tiny model (B=4, T=16) and of the 124M
        model at B=4, T=64 on one thread."""
    import oracle
    from transformer_lm_amd.workloads import WORKLOADS
    oracle.build(force=True, precisions=("f32n",))
    threads = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    ws = w.with_batch(B=1, T=T_sample, steps=1)
    dt, used = _oracle_step_seconds(replace(ws, dtype="fp32"), threads)
    out = {"value": round(ws.BT / dt, 2), "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": f"one training step (forward with loss, backward, AdamW) of the same "
                     f"124M model on 1 sequence of {T_sample} tokens: fp32 oracle built -O2 "
                     f"-march=native -fopenmp -ffp-contract=off, {used} threads, {dt:.1f} s",
           "cpu_model": _cpu_model(), "nproc": os.cpu_count()}
    if single_thread:
        st = {}
        for name in ("tiny", "gpt2_124m_fp32"):
            wn = WORKLOADS[name]
            d1, _ = _oracle_step_seconds(wn, 1)
            st[name] = {"B": wn.B, "T": wn.T, "tokens_per_s": round(wn.BT / d1, 2),
                        "step_s": round(d1, 3)}
        out["single_thread"] = st
    return out


def fp8_leg(torch, gpt2, synth, M=16384, C=768, V=50304, reps=10):
    """The FP8 (E4M3) products on the forward shapes of the 124M model at
    M = B*T rows: per-tensor scale and quantisation of the operands, then the
    product with a bf16 output, timed with events on the launch stream."""
    shapes = {"qkv": (3 * C, C), "attproj": (C, C), "fc": (4 * C, C), "fcproj": (C, 4 * C),
              "lm_head": (V, C)}
    stream = torch.cuda.current_stream()
    work = torch.empty(gpt2.fp8_scale_workspace_bytes(), dtype=torch.uint8, device="cuda")

    def timed(fn):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    per, tot_fl, tot_ms = {}, 0.0, 0.0
    q_rate = s_rate = None
    for name, (N, K) in shapes.items():
        x, wt, b = synth.fp8_operands(M, N, K, seed=N + K)
        xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
        wd = torch.from_numpy(wt).cuda().to(torch.bfloat16)
        bd = torch.from_numpy(b).cuda().to(torch.bfloat16)
        scales = torch.empty(4, dtype=torch.float32, device="cuda")
        qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        qw = torch.empty((N, K), dtype=torch.uint8, device="cuda")
        gpt2.fp8_scale(scales[0:], work, xd)
        gpt2.fp8_quantize(qx, xd, scales[0:])
        gpt2.fp8_scale(scales[1:], work, wd)
        gpt2.fp8_quantize(qw, wd, scales[1:])
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        use_bias = name != "lm_head"
        ms = timed(lambda: gpt2.fp8_matmul(out, qx, qw, scales, bd if use_bias else None))
        fl = 2.0 * M * N * K
        per[name] = {"N": N, "K": K, "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1)}
        tot_fl += fl
        tot_ms += ms
        if name == "qkv":   # operand preparation, on the activation block [M, C]
            ms_s = timed(lambda: gpt2.fp8_scale(scales[0:], work, xd))
            ms_q = timed(lambda: gpt2.fp8_quantize(qx, xd, scales[0:]))
            s_rate = 2.0 * xd.numel() / (ms_s * 1e-3) / 1e9
            q_rate = 3.0 * xd.numel() / (ms_q * 1e-3) / 1e9
        del xd, wd, bd, qx, qw, out
    torch.cuda.empty_cache()
    achieved = tot_fl / (tot_ms * 1e-3)
    lm = per["lm_head"]
    return {
        "workload": f"E4M3 products of the 124M forward shapes at {M} rows (qkv, attproj, "
                    f"fc, fcproj with bias; lm_head), per-tensor scales, bf16 output",
        "per_shape": per,
        "roofline": {"kernel": "fp8_matmul", "bound": "mfma",
                     "achieved": round(achieved / 1e12, 1), "peak": PEAK_FP8_FLOPS / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_FLOPS, 4),
                     "lm_head_frac": round(lm["tflops"] * 1e12 / PEAK_FP8_FLOPS, 4)},
        "scale_gb_s": round(s_rate, 1), "quantize_gb_s": round(q_rate, 1),
    }


def class_table(prof):
    """Per kernel class, from one event-timed step: launches, ms per step, the
    algorithmic work rate and its fraction of the class's roofline."""
    out = {}
    for k, (n, ms, wk, isb) in sorted(prof.items(), key=lambda kv: -kv[1][1]):
        rate = wk / (ms * 1e-3)
        peak = PEAK_HBM_BYTES if isb else PEAK_BF16_FLOPS
        out[k] = {"launches": n, "ms_per_step": round(ms, 4),
                  "achieved": round(rate / (1e9 if isb else 1e12), 1),
                  "unit": "GB/s" if isb else "TFLOP/s", "bound": "hbm" if isb else "mfma",
                  "frac": round(rate / peak, 4)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 (E4M3) products' measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the step is a single-GPU hot path with no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    from transformer_lm_amd import gpt2, synth
    from transformer_lm_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    total = args.warmup + args.steps
    log(f"[bench] {w.name}: B={w.B} T={w.T} C={w.C} L={w.L} dtype={w.dtype}; "
        f"{args.warmup} warmup + {args.steps} timed steps")
    params = synth.init_params(w)
    toks = synth.tokens(w, steps=max(total, 1))
    # every step's tokens wait in pinned host memory; each step uploads its
    # inputs and targets (2 x B*T int32) before the forward, as a data loader
    # feeding the step would
    host_in = [torch.from_numpy(np.ascontiguousarray(toks[s][:, :-1])).pin_memory()
               for s in range(total)]
    host_tg = [torch.from_numpy(np.ascontiguousarray(toks[s][:, 1:])).pin_memory()
               for s in range(total)]
    dev_in = torch.empty((w.B, w.T), dtype=torch.int32, device="cuda")
    dev_tg = torch.empty((w.B, w.T), dtype=torch.int32, device="cuda")
    model = gpt2.GPT2(gpt2.config(w), params)
    del params
    stream = model.stream
    losses = []

    def step(s):
        with torch.cuda.stream(stream):
            dev_in.copy_(host_in[s], non_blocking=True)
            dev_tg.copy_(host_tg[s], non_blocking=True)
        losses.append(model.forward(dev_in, dev_tg))   # reads the loss (synchronises)
        model.backward()
        model.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, s + 1)

    # warmup: one step (the second, if there are two) records every kernel
    # class with HIP events, for the per-class table and the dominant class
    pidx = 1 if args.warmup >= 2 else 0
    prof = {}
    for s in range(args.warmup):
        if s == pidx:
            model.timing_arm("", 8192)
        step(s)
        if s == pidx:
            prof = model.timing_read()
            model.timing_arm(None)
    torch.cuda.synchronize()
    classes = class_table(prof)
    singles = [k for k in classes if k in SINGLE_KERNEL_CLASSES]
    dominant = singles[0] if singles else (next(iter(classes)) if classes else "matmul")
    for k, c in classes.items():
        log(f"[bench] warmup profile {k:15s} {c['launches']:4d} launches "
            f"{c['ms_per_step']:9.3f} ms  {c['achieved']:8.1f} {c['unit']} "
            f"({100 * c['frac']:.1f}% of peak)")

    # timed region: K steps between synchronisations; an event at every step
    # boundary on the handle's stream gives the per-step times, and events
    # bracket the dominant kernel's launches
    model.timing_arm(dominant, 4096)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, s in enumerate(range(args.warmup, total)):
        evs[i].record(stream)
        step(s)
    evs[-1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    dom = model.timing_read().get(dominant)

    ms_per_step = wall * 1e3 / max(args.steps, 1)
    tok_s = w.BT * args.steps / wall
    mfu = tok_s * w.flops_per_token() / PEAK_BF16_FLOPS
    med = float(np.median(step_ms)) if step_ms else None
    mn = float(np.min(step_ms)) if step_ms else None
    log(f"[bench] {ms_per_step:.2f} ms/step (per-step events: median {med:.2f}, min {mn:.2f}), "
        f"{tok_s:,.0f} tokens/s, MFU {100 * mfu:.2f}%")
    log("[bench] loss per step: " + " ".join(f"{v:.4f}" for v in losses))

    roofline = None
    if dom:
        n, ms, wk, isb = dom
        achieved = wk / (ms * 1e-3)
        peak = PEAK_HBM_BYTES if isb else PEAK_BF16_FLOPS
        unit_div = 1e9 if isb else 1e12
        tr = recorded_traffic(dominant) if w.name == WORKLOAD else None
        roofline = {"kernel": dominant, "symbol": SINGLE_KERNEL_CLASSES.get(dominant),
                    "bound": "hbm" if isb else "mfma",
                    "achieved": round(achieved / unit_div, 2), "peak": peak / unit_div,
                    "unit": "GB/s" if isb else "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": tr["bytes"] if tr else None,
                    "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                    "traffic_fetch_write": [tr["fetch_bytes"], tr["write_bytes"]] if tr else None,
                    "launches": n, "avg_launch_ms": round(ms / n, 4)}

    fp8 = None
    if not args.no_fp8:
        fp8 = fp8_leg(torch, gpt2, synth)
        log("[bench] fp8 products: " + ", ".join(
            f"{k} {v['tflops']:.0f}" for k, v in fp8["per_shape"].items()) +
            f" TFLOP/s; all {fp8['roofline']['achieved']:.0f} TFLOP/s "
            f"({100 * fp8['roofline']['frac']:.1f}% of fp8 peak); quantise "
            f"{fp8['quantize_gb_s']:.0f} GB/s, scale {fp8['scale_gb_s']:.0f} GB/s")

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w)
        log(f"[bench] cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads "
            f"({cpu['cpu_model']}); single thread: " +
            ", ".join(f"{k} {v['tokens_per_s']:.1f} tokens/s"
                      for k, v in cpu.get("single_thread", {}).items()))

    out = {
        "metric": "train tokens/s, GPT-2 124M bf16 B=16 T=1024, 1 MI355X; MFU %",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "ms_per_step_median": round(med, 3) if med is not None else None,
        "ms_per_step_min": round(mn, 3) if mn is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded Zipf(1.1) tokens over 50257 ids, seeded N(0,0.02) init; "
                "each step uploads its tokens from pinned host memory and reads its loss",
        "config": {"workload": f"GPT-2 124M training step (forward, backward, AdamW), bf16 "
                               f"activations with fp32 master weights and moments, "
                               f"B={w.B} T={w.T}",
                   "global_batch": w.B, "seq_len": w.T, "parallelism": "single GPU"},
        "mfu": round(mfu, 4),
        "flops_per_token": w.flops_per_token(),
        "losses": [round(v, 4) for v in losses[args.warmup:]],
        "roofline": roofline,
        "classes": classes,
        "cpu_baseline": cpu,
        "fp8_matmul": fp8,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
