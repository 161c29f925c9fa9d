"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a
driver (tests/csrc/oracle_step_main.c) built with the oracle by gcc runs three
training steps of the tiny model and of its padded-vocabulary variant, a few
finite differences and a refused out-of-range token. The sanitized run must
report nothing and print the same losses as the ordinary float build would
(double precision here, so the losses match the ctypes oracle to the last
printed digit). CPU only."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.wrapper import Oracle
from transformer_lm_amd import synth
from transformer_lm_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    out = str(tmp_path_factory.mktemp("asan") / "oracle_step_main")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-ffp-contract=off"] + SANITIZE + [
        os.path.join(ROOT, "oracle", "gpt2_oracle.c"),
        os.path.join(ROOT, "tests", "csrc", "oracle_step_main.c"), "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


@pytest.mark.parametrize("name", ["tiny", "tiny_pad"])
def test_oracle_step_is_clean_under_sanitizers(driver, tmp_path, name):
    w = WORKLOADS[name].with_batch(steps=3)
    p = synth.init_params(w)
    toks = synth.tokens(w)
    pf, tf = tmp_path / "params.f32", tmp_path / "tokens.i32"
    p.astype(np.float32).tofile(pf)
    toks.astype(np.int32).tofile(tf)
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([driver, str(w.V), str(w.Vp), str(w.max_T), str(w.C), str(w.L),
                        str(w.NH), str(w.B), str(w.T), str(w.steps), str(pf), str(tf)],
                       capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    got = [float(l.split()[2]) for l in r.stdout.splitlines() if l.startswith("loss")]
    o = Oracle(w, p)
    ref = []
    for s in range(w.steps):
        x, y = synth.split_batch(toks[s])
        ref.append(o.forward(x, y))
        o.backward()
        o.update(1e-3, 0.9, 0.999, 1e-8, 0.1, s + 1)
    assert got == ref
