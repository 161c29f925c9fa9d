"""Host-side tooling: bench.py's single-GPU contract and the profile
summariser's kernel classes (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_profile_classes():
    from transformer_lm_amd.prof_summary import kclass, launches_per_step
    g = "void gemm_stream_kernel<128, 192, 64, 2, 2, 8, 2, 2, {}>(GemmGroup)"
    assert kclass(g.format("false, false, 4, false")) == "matmul_fwd"
    assert kclass(g.format("false, true, 3, true")) == "matmul_bwd_dx"
    assert kclass(g.format("true, true, 1, false")) == "matmul_bwd_dw"
    assert kclass(g.format("false, false, 7, false")) == "fp8_matmul"
    assert kclass(g.format("false, false, 8, false")) == "fp8_matmul"
    assert kclass("fp8_quantize_kernel(unsigned char*, __bf16 const*, float const*, long)") == \
        "fp8_prepare"
    assert kclass("flash_bwd_dq_kernel(...)") == "attention_bwd"
    assert kclass("adamw_kernel(float*, ...)") == "adamw"
    per = launches_per_step(12)
    assert per["matmul_fwd"] == 49 and per["matmul_bwd_dw"] == 1
