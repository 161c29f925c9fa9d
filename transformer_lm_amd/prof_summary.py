"""Summaries of rocprofv3 output for the training step (measurement tooling).

    python -m transformer_lm_amd.prof_summary stats  <kernel_stats.csv> [steps]
    python -m transformer_lm_amd.prof_summary traffic <fetch counter_collection.csv>
                                                      <write counter_collection.csv>
    python -m transformer_lm_amd.prof_summary class-traffic <fetch csv> <write csv> <steps> <L>
    python -m transformer_lm_amd.prof_summary fp8 <kernel_trace.csv>

`stats` prints each kernel's launches, total and average duration, and the
launches grouped into the kernel classes the library's event timing reports.
`traffic` prints FETCH_SIZE / WRITE_SIZE per dispatch (KiB) averaged per kernel,
and scales them by the ratio measured on the plain device copy of known size
that `bench.py --calibrate-copy` runs (1 GiB read + 1 GiB written).
`class-traffic` prints the same scaled bytes per launch of each kernel class,
with the SHA-256 of the kernel sources, in the form bench.py reads.
"""
import csv
import re
import sys
from collections import defaultdict

# kernel symbol (substring) -> library timing class
CLASSES = [
    (r"gemm_stream_kernel<[^>]*false, false, [78], ", "fp8_matmul"),
    (r"fp8_", "fp8_prepare"),
    (r"gemm_(lds|mfma|persistent|stream)_kernel<[^>]*false, false", "matmul_fwd"),
    (r"gemm_(lds|mfma|persistent|stream)_kernel<[^>]*false, true", "matmul_bwd_dx"),
    (r"gemm_(lds|mfma|persistent|stream)_kernel<[^>]*true, true", "matmul_bwd_dw"),
    (r"split_reduce_kernel", "matmul_bwd_dw"),
    (r"flash_fwd_kernel|attention_fwd_rows", "attention_fwd"),
    (r"flash_bwd|attention_bwd", "attention_bwd"),
    (r"layernorm_fwd", "layernorm_fwd"),
    (r"layernorm_bwd", "layernorm_bwd"),
    (r"gelu_fwd", "gelu_fwd"),
    (r"gelu_bwd", "gelu_bwd"),
    (r"classifier|loss_mean", "classifier"),
    (r"encoder_fwd", "encoder_fwd"),
    (r"encoder_bwd|token_|enc_(rank|scan|fill|range|fix)", "encoder_bwd"),
    (r"fill_zero_kernel<int>", "encoder_bwd"),
    (r"adamw|grad_norm", "adamw"),
]


def kclass(name):
    for pat, cls in CLASSES:
        if re.search(pat, name):
            return cls
    return "other"


def short(name, n=90):
    return name if len(name) <= n else name[:n - 3] + "..."


def stats(path, steps=None):
    rows = list(csv.DictReader(open(path)))
    out = []
    by_class = defaultdict(lambda: [0, 0.0])
    out.append(f"{'kernel':92s} {'calls':>6s} {'total ms':>10s} {'avg us':>9s} {'%':>6s}")
    for r in rows:
        name = r["Name"]
        calls = int(r["Calls"])
        tot = float(r["TotalDurationNs"]) / 1e6
        avg = float(r["AverageNs"]) / 1e3
        pct = float(r["Percentage"])
        out.append(f"{short(name):92s} {calls:6d} {tot:10.3f} {avg:9.2f} {pct:6.2f}")
        c = by_class[kclass(name)]
        c[0] += calls
        c[1] += tot
    out.append("")
    div = f" per step ({steps} profiled steps)" if steps else ""
    out.append(f"by class{div}: {'calls':>6s} {'total ms':>10s}")
    for cls, (calls, tot) in sorted(by_class.items(), key=lambda kv: -kv[1][1]):
        if steps:
            out.append(f"  {cls:18s} {calls / steps:8.1f} {tot / steps:10.3f}")
        else:
            out.append(f"  {cls:18s} {calls:8d} {tot:10.3f}")
    return "\n".join(out)


def _per_kernel(path, counter):
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def traffic(fetch_path, write_path, copy_bytes=1 << 30):
    f = _per_kernel(fetch_path, "FETCH_SIZE")
    w = _per_kernel(write_path, "WRITE_SIZE")

    def copy_kib(vals):
        for k, v in vals.items():
            if "copyBuffer" in k or "copy" in k.lower() and "elementwise" in k:
                return max(v)
        return None

    cf, cw = copy_kib(f), copy_kib(w)
    sf = copy_bytes / (cf * 1024) if cf else float("nan")
    sw = copy_bytes / (cw * 1024) if cw else float("nan")
    out = [f"copy calibration: {copy_bytes} B read and written; FETCH_SIZE reads "
           f"{cf} KiB (scale {sf:.4f}), WRITE_SIZE reads {cw} KiB (scale {sw:.4f})", "",
           f"{'kernel':92s} {'n':>4s} {'fetch MB':>10s} {'write MB':>10s} (per dispatch, scaled)"]
    for k in sorted(set(f) | set(w), key=lambda k: -(sum(f.get(k, [0])) / max(1, len(f.get(k, [1]))))):
        fv, wv = f.get(k, []), w.get(k, [])
        fm = sum(fv) / len(fv) * 1024 * sf / 1e6 if fv else float("nan")
        wm = sum(wv) / len(wv) * 1024 * sw / 1e6 if wv else float("nan")
        out.append(f"{short(k):92s} {max(len(fv), len(wv)):4d} {fm:10.2f} {wm:10.2f}")
    return "\n".join(out)


def source_sha():
    """SHA-256 over the kernel sources (csrc/*), in name order."""
    import glob
    import hashlib
    import os
    h = hashlib.sha256()
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for p in sorted(glob.glob(os.path.join(here, "*"))):
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()


# timed launches of each class in one training step (L layers); the weight
# gradients of all layers and the output head run as one timed group
def launches_per_step(L):
    return {"matmul_fwd": 4 * L + 1, "matmul_bwd_dx": 4 * L + 1, "matmul_bwd_dw": 1,
            "attention_fwd": L, "attention_bwd": L, "layernorm_fwd": 2 * L + 1,
            "layernorm_bwd": 2 * L + 2, "gelu_fwd": L, "gelu_bwd": L, "classifier": 1,
            "encoder_fwd": 1, "encoder_bwd": 1, "adamw": 1}


def class_traffic(fetch_path, write_path, steps, L, copy_bytes=1 << 30):
    """Scaled HBM bytes per launch of each timing class, from `steps` steps."""
    f = _per_kernel(fetch_path, "FETCH_SIZE")
    w = _per_kernel(write_path, "WRITE_SIZE")
    cf = max(v for k, v in ((k, max(v)) for k, v in f.items()) if "copyBuffer" in k)
    cw = max(v for k, v in ((k, max(v)) for k, v in w.items()) if "copyBuffer" in k)
    sf, sw = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    per = launches_per_step(L)
    tot = defaultdict(lambda: [0.0, 0.0])
    for k, v in f.items():
        tot[kclass(k)][0] += sum(v) * 1024 * sf
    for k, v in w.items():
        tot[kclass(k)][1] += sum(v) * 1024 * sw
    out = {}
    for cls, n in per.items():
        fb, wb = tot.get(cls, (0.0, 0.0))
        out[cls] = {"fetch_bytes": fb / (steps * n), "write_bytes": wb / (steps * n)}
    return {"fetch_scale": sf, "write_scale": sw, "classes": out}


# the FP8 products bench.py times: per shape, 2 warmup + `reps` timed launches,
# in this order (the lm-head without bias: its own kernel instantiation)
FP8_SHAPES = ("qkv", "attproj", "fc", "fcproj", "lm_head")


def fp8_products(trace_path, reps=10, warm=2):
    """Average kernel-trace duration of each FP8 product's timed launches."""
    rows = [r for r in csv.DictReader(open(trace_path))
            if kclass(r["Kernel_Name"]) == "fp8_matmul"]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = len(rows) // len(FP8_SHAPES)
    out = [f"{'product':10s} {'launches':>8s} {'avg us (timed)':>15s}"]
    for i, name in enumerate(FP8_SHAPES):
        grp = rows[i * per:(i + 1) * per][warm:warm + reps]
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in grp]
        out.append(f"{name:10s} {len(d):8d} {sum(d) / max(len(d), 1):15.2f}")
    return "\n".join(out)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2], int(sys.argv[3]) if len(sys.argv) > 3 else None))
    elif sys.argv[1] == "fp8":
        print(fp8_products(sys.argv[2]))
    elif sys.argv[1] == "traffic":
        print(traffic(sys.argv[2], sys.argv[3]))
    elif sys.argv[1] == "class-traffic":
        res = class_traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), int(sys.argv[5]))
        print(f"# fetch scale {res['fetch_scale']:.4f}, write scale {res['write_scale']:.4f}")
        print(f"source_sha256 {source_sha()}")
        print(f"# {'class':16s} {'fetch_bytes':>14s} {'write_bytes':>15s}")
        for cls, v in res["classes"].items():
            print(f"{cls:18s} {v['fetch_bytes']:14.0f} {v['write_bytes']:15.0f}")
    else:
        raise SystemExit(__doc__)
