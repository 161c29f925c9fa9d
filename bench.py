"""Training throughput of the GPT-2 124M step (bf16, fp32 master weights and
AdamW moments, B=16, T=1024) on one MI355X, through the C ABI.

One step = forward (with the mean loss) + backward + AdamW update, on seeded
synthetic Zipf(1.1) tokens, inputs resident in HBM before timing starts.
Prints one JSON line: tokens/s, MFU against the bf16 dense peak, the dominant
kernel class against its roofline (HIP-event durations measured in the timed
steps), and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-fp8]

A second object, "fp8_matmul", measures the FP8 (E4M3) products on the same
model's forward shapes (not part of the training step, which stays bf16).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA, published
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


def cpu_baseline(w, T_sample=1024):
    """The oracle (fp64, plain loops, OpenMP over independent outputs) on one
    sequence of T_sample tokens of the same model: one full training step."""
    import oracle
    from oracle.wrapper import Oracle
    from transformer_lm_amd import synth
    oracle.build(force=False)
    ws = w.with_batch(B=1, T=T_sample, steps=1)
    p = synth.init_params(ws)
    x, y = synth.split_batch(synth.tokens(ws)[0])
    threads = len(os.sched_getaffinity(0))
    o = Oracle(ws, p, threads=threads)
    t0 = time.perf_counter()
    o.forward(x, y)
    o.backward()
    o.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1)
    dt = time.perf_counter() - t0
    cores = o.lib.oracle_get_threads()
    o.close()
    return {"value": ws.BT / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"one training step (fwd+bwd+AdamW) of the same 124M model on 1 sequence "
                      f"of {T_sample} tokens, fp64 oracle, {dt:.1f} s"}


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
    dev_in = [torch.from_numpy(np.ascontiguousarray(toks[s][:, :-1])).cuda() for s in range(total)]
    dev_tg = [torch.from_numpy(np.ascontiguousarray(toks[s][:, 1:])).cuda() for s in range(total)]
    model = gpt2.GPT2(gpt2.config(w), params)
    stream = model.stream
    loss_dev = torch.zeros(total, dtype=torch.float32, device="cuda")
    loss_view = model.act("loss")

    def step(s):
        model.forward(dev_in[s], dev_tg[s], want_loss=False)
        loss_dev[s].copy_(loss_view[0])
        model.backward()
        model.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, s + 1)

    # warmup: one step (the second, if there are two) records every kernel
    # class to find the dominant one
    pidx = 1 if args.warmup >= 2 else 0
    for s in range(args.warmup):
        if s == pidx:
            model.timing_arm("", 8192)
        step(s)
        if s == pidx:
            prof = model.timing_read()
            model.timing_arm(None)
    torch.cuda.synchronize()
    if args.warmup == 0:
        prof = {}
    dominant = max(prof, key=lambda k: prof[k][1]) if prof else "matmul"
    for k, (n, ms, wk, isb) in sorted(prof.items(), key=lambda kv: -kv[1][1]):
        rate = wk / (ms * 1e-3) / (1e9 if isb else 1e12)
        log(f"[bench] warmup profile {k:15s} {n:4d} launches {ms:9.3f} ms  "
            f"{rate:8.1f} {'GB/s' if isb else 'TFLOP/s'}")

    # timed region: events bracket only the dominant class's launches
    model.timing_arm(dominant, 4096)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for s in range(args.warmup, total):
        step(s)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    dom = model.timing_read().get(dominant)
    losses = loss_dev.cpu().tolist()

    ms_per_step = wall * 1e3 / max(args.steps, 1)
    tok_s = w.BT * args.steps / wall
    mfu = tok_s * w.flops_per_token() / PEAK_BF16_FLOPS
    log(f"[bench] {ms_per_step:.2f} ms/step (events {gpu_ms / max(args.steps, 1):.2f}), "
        f"{tok_s:,.0f} tokens/s, MFU {100 * mfu:.2f}%")
    log("[bench] loss per step: " + " ".join(f"{v:.4f}" for v in losses))

    roofline = None
    if dom:
        n, ms, wk, isb = dom
        achieved = wk / (ms * 1e-3)
        peak = PEAK_HBM_BYTES if isb else PEAK_BF16_FLOPS
        unit_div = 1e9 if isb else 1e12
        tr = recorded_traffic(dominant) if w.name == WORKLOAD else None
        roofline = {"kernel": dominant, "bound": "hbm" if isb else "mfma",
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
        log(f"[bench] cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    out = {
        "metric": "train tokens/s, GPT-2 124M bf16 B=16 T=1024, 1 MI355X; MFU %",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded Zipf(1.1) tokens over 50257 ids, seeded N(0,0.02) init",
        "config": {"workload": f"GPT-2 124M training step (forward, backward, AdamW), bf16 "
                               f"activations with fp32 master weights and moments, "
                               f"B={w.B} T={w.T}",
                   "global_batch": w.B, "seq_len": w.T, "parallelism": "single GPU"},
        "mfu": round(mfu, 4),
        "flops_per_token": w.flops_per_token(),
        "loss_first_last": [round(losses[0], 4), round(losses[-1], 4)] if losses else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fp8_matmul": fp8,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
