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
from transformer_lm_amd import synth  # noqa: E402
from transformer_lm_amd.workloads import WORKLOADS, param_offsets  # noqa: E402

ORACLE_SOURCE = "oracle/gpt2_torch.py"
N_TOP = 64
N_UNIFORM = 448


def oracle_hash():
    with open(os.path.join(ROOT, ORACLE_SOURCE), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


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
    for n in sys.argv[1:] or ("gpt2_124m", "gpt2_350m", "gpt2_1558m"):
        trajectory(n)
