"""gpt2_attention_backward_noalloc (static per-GPU scratch, no workspace, no
allocation) against gpt2_attention_backward (caller workspace) through the C
ABI: the same kernels on the same inputs, so the results must be identical
bit for bit. Two calls in a row, the second with a smaller input (the scratch
keeps the first call's D values, which the second must not read), in bf16
(matrix-core kernels) and fp32 (row kernels); then a size beyond the scratch
is refused without a launch."""
import numpy as np
import pytest

from parity import say
from transformer_lm_amd import synth

pytestmark = pytest.mark.gpu
HS = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_lm_amd import build
    if not build.is_built():
        build.build()


def _inputs(B, T, NH, tdt):
    import torch
    C = NH * HS
    x = torch.from_numpy(synth.attention_qkv(B, T, NH)).to(tdt).cuda()
    dy = torch.from_numpy(synth.attention_dout(B, T, C)).to(tdt).cuda()
    return x, dy


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_matches_workspace_entry_point(dtype):
    import torch
    from transformer_lm_amd import gpt2
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for B, T, NH in ((2, 1024, 12), (1, 300, 4)):
        say(f"no-alloc attention backward {dtype} B={B} T={T} NH={NH}")
        C = NH * HS
        x, dy = _inputs(B, T, NH, tdt)
        out = torch.empty(B, T, C, dtype=tdt, device="cuda")
        lse = torch.empty(B, NH, T, dtype=torch.float32, device="cuda")
        gpt2.attention_forward(out, lse, x, NH)
        ref = torch.full((B, T, 3 * C), float("nan"), dtype=tdt, device="cuda")
        work = torch.empty(2 * B * NH * T, dtype=torch.float32, device="cuda")
        gpt2.attention_backward(ref, work, dy, x, out, lse, NH)
        got = torch.full((B, T, 3 * C), float("nan"), dtype=tdt, device="cuda")
        gpt2.attention_backward_noalloc(got, dy, x, out, lse, NH)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(ref).all())
        assert torch.equal(got, ref)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    import torch
    from transformer_lm_amd import gpt2
    B, T, NH = 33, 1024, 16          # 2*B*NH*T = 1081344 > 2^20
    C = NH * HS
    a = torch.empty(16, dtype=torch.uint8, device="cuda").data_ptr()
    rc = gpt2._lib.gpt2_attention_backward_noalloc(a, a, a, a, a, B, T, C, NH,
                                                   gpt2.DTYPE_BF16, None)
    assert rc == gpt2.GPT2_ESHAPE
    assert "static scratch" in gpt2.last_error()
