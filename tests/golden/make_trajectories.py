"""Writes tests/golden/trajectory_<workload>.json for the bf16 training
workloads at their full sizes: what the fp32 oracle (oracle/gpt2_torch.py)
computes on the seeded inputs of transformer_lm_amd.synth.

Calls only oracle/ (plus the input generator); no value here comes from the
GPU library. Run from the repository root:

    python tests/golden/make_trajectories.py gpt2_124m gpt2_350m gpt2_1558m

Stored per workload:
  - the mean loss of every optimiser step (20, 10 and 5 steps);
  - the loss of every position at step 1 (identical parameters on both sides);
  - per parameter tensor at step 1: the Euclidean norm and the largest
    magnitude of the gradient, and a sample of gradient entries -- the 64
    largest in magnitude plus up to 448 drawn uniformly from a seeded stream
    (seed 7000 + tensor number) -- with their flat indices inside the tensor;
  - SHA-256 of the oracle source that made them and of the input bytes
    (initial parameters, tokens) it read.

With --bf16-init it writes trajectory_<workload>_bf16init.json instead: the
same oracle and batches started from the initial parameters rounded to bf16
(round to nearest, ties to even), per-step losses only. The distance between
the two oracle trajectories measures how far a perturbation of bf16 rounding
size carries the loss at each step, i.e. where the trajectory is sensitive
to rounding.

With --bf16-storage it writes trajectory_<workload>_bf16storage.json: the
trajectory of oracle/gpt2_torch_bf16.py, the same step with bf16 storage
(parameters' working copy, activations and activation gradients rounded to
bf16; fp32 master weights, optimiser state and sums), per-step losses only.
Its distance from the fp32 trajectory is how far a bf16 step drifts by
rounding alone.
"""
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from oracle.gpt2_torch import TorchOracle  # noqa: E402
from oracle.gpt2_torch_bf16 import TorchOracleBF16Storage  # noqa: E402
from transformer_lm_amd import synth  # noqa: E402
from transformer_lm_amd.workloads import WORKLOADS, param_offsets  # noqa: E402

ORACLE_SOURCE = "oracle/gpt2_torch.py"
N_TOP = 64
N_UNIFORM = 448


def file_hash(rel):
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def oracle_hash():
    return file_hash(ORACLE_SOURCE)


def input_hashes(params, toks):
    return {"params": hashlib.sha256(params.tobytes()).hexdigest(),
            "tokens": hashlib.sha256(toks.tobytes()).hexdigest()}


def sample_indices(g, tensor_number):
    """Flat indices: the N_TOP largest |g| and up to N_UNIFORM uniform draws."""
    n = g.size
    top = np.argsort(-np.abs(g), kind="stable")[:min(N_TOP, n)]
    u = synth.uniform(7000 + tensor_number, 0, N_UNIFORM)
    uni = np.minimum(np.floor(u * n).astype(np.int64), n - 1)
    return np.unique(np.concatenate([top, uni]))


def round_to_bf16(a):
    """float32 array rounded to the nearest bf16 value (ties to even), as float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def perturbed_trajectory(name, threads=None, kind="bf16init"):
    w = WORKLOADS[name]
    t0 = time.time()
    params = synth.init_params(w)
    toks = synth.tokens(w)
    if kind == "bf16init":
        o = TorchOracle(w, round_to_bf16(params), dtype=torch.float32, threads=threads)
        what = "initial parameters rounded to bf16"
        src = ORACLE_SOURCE + ", float32"
    else:
        o = TorchOracleBF16Storage(w, params, threads=threads)
        what = "bf16 storage (oracle/gpt2_torch_bf16.py)"
        src = "oracle/gpt2_torch_bf16.py over " + ORACLE_SOURCE
    out = {"workload": name, "steps": w.steps, "perturbation": what, "oracle": src,
           "oracle_sha256": oracle_hash(), "variant_sha256": file_hash("oracle/gpt2_torch_bf16.py"),
           "inputs_sha256": input_hashes(params, toks), "losses": []}
    del params
    for s in range(w.steps):
        x, y = synth.split_batch(toks[s])
        loss = o.forward(x, y)
        out["losses"].append(round(loss, 7))
        o.backward()
        o.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, s + 1)
        print(f"{name} ({kind}) step {s + 1}/{w.steps}: loss {loss:.6f} "
              f"({time.time() - t0:.0f} s)", flush=True)
    out["oracle_seconds"] = round(time.time() - t0, 1)
    path = os.path.join(ROOT, "tests", "golden", f"trajectory_{name}_{kind}.json")
    with open(path, "w") as f:
        json.dump(out, f, separators=(",", ":"))
        f.write("\n")
    print(f"wrote {path}", flush=True)


def trajectory(name, threads=None):
    w = WORKLOADS[name]
    t0 = time.time()
    params = synth.init_params(w)
    toks = synth.tokens(w)
    o = TorchOracle(w, params, dtype=torch.float32, threads=threads)
    out = {"workload": name, "B": w.B, "T": w.T, "C": w.C, "L": w.L, "NH": w.NH, "V": w.V,
           "Vp": w.Vp, "steps": w.steps, "lr": w.lr, "weight_decay": w.weight_decay,
           "oracle": ORACLE_SOURCE + ", float32", "oracle_sha256": oracle_hash(),
           "inputs_sha256": input_hashes(params, toks), "losses": []}
    del params
    for s in range(w.steps):
        x, y = synth.split_batch(toks[s])
        loss = o.forward(x, y)
        out["losses"].append(round(loss, 7))
        if s == 0:
            out["step1_position_losses"] = [round(float(v), 6) for v in o.losses]
        o.backward()
        if s == 0:
            grads = {}
            g = o.grads()
            for k, (tname, (off, shape)) in enumerate(param_offsets(w).items()):
                gt = g[off:off + math.prod(shape)]
                idx = sample_indices(gt, k)
                grads[tname] = {"norm": float(np.linalg.norm(gt)),
                                "max_abs": float(np.abs(gt).max()),
                                "idx": [int(i) for i in idx],
                                "val": [float("%.8e" % gt[i]) for i in idx]}
            out["step1_grads"] = grads
            del g
        o.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, s + 1)
        print(f"{name} step {s + 1}/{w.steps}: loss {loss:.6f} ({time.time() - t0:.0f} s)",
              flush=True)
    out["oracle_seconds"] = round(time.time() - t0, 1)
    path = os.path.join(ROOT, "tests", "golden", f"trajectory_{name}.json")
    with open(path, "w") as f:
        json.dump(out, f, separators=(",", ":"))
        f.write("\n")
    print(f"wrote {path}", flush=True)


if __name__ == "__main__":
    args = sys.argv[1:]
    fn = trajectory
    for flag, kind in (("--bf16-init", "bf16init"), ("--bf16-storage", "bf16storage")):
        if flag in args:
            args.remove(flag)
            fn = lambda n, k=kind: perturbed_trajectory(n, kind=k)  # noqa: E731
    for n in args or ("gpt2_124m", "gpt2_350m", "gpt2_1558m"):
        fn(n)
