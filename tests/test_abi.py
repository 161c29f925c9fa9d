"""The C-ABI library: it loads, exports every entry point include/gpt2.h
declares, and its host-side planning and validation behave. No kernel runs."""
import ctypes as ct
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def g():
    from transformer_lm_amd import build
    if not build.is_built():
        build.build()
    from transformer_lm_amd import gpt2
    return gpt2


def declared_functions():
    src = open(os.path.join(ROOT, "include", "gpt2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt2_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported(g):
    names = declared_functions()
    assert len(names) == 28
    lib = ct.CDLL(g.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(g.EXPORTS) == names


def test_param_layout_matches_the_generator(g):
    from transformer_lm_amd.workloads import WORKLOADS, param_offsets
    for name in ("tiny", "tiny_pad", "gpt2_124m", "gpt2_350m", "gpt2_1558m"):
        w = WORKLOADS[name]
        cfg = g.config(w)
        assert g.num_params(cfg) == w.num_params()
        offs = param_offsets(w)
        tab = g.param_table(cfg)
        assert [t[0] for t in tab] == list(offs)
        for tname, off, shape in tab:
            assert (off, shape) == offs[tname], tname


def test_buffer_sizes(g):
    from transformer_lm_amd.workloads import WORKLOADS
    w = WORKLOADS["gpt2_124m"]
    cfg = g.config(w)
    n = w.num_params()
    pb = g.param_buffer_bytes(cfg)
    assert 18 * n <= pb <= 18 * n + 5 * 256          # 4 fp32 regions + bf16 copy
    ab = g.act_buffer_bytes(cfg)
    BT, C, L = w.BT, w.C, w.L
    # the bf16 activations alone: 14 C-wide rows per layer-position + the logits
    assert ab > 2 * (L * BT * 14 * C + BT * w.Vp)
    assert ab < 12e9                                  # well inside 288 GB of HBM
    w32 = WORKLOADS["tiny"]
    assert g.param_buffer_bytes(g.config(w32)) >= 16 * w32.num_params()
    # checkpoint image: 128-byte header + master, m, v
    assert g._lib.gpt2_checkpoint_bytes(ct.byref(cfg)) == 128 + 12 * n


@pytest.mark.parametrize("field,value", [("C", 30), ("NH", 5), ("Vp", 60), ("T", 64),
                                         ("dtype", 7), ("C", 4096), ("B", 0)])
def test_invalid_configs_are_rejected(g, field, value):
    from transformer_lm_amd.workloads import WORKLOADS
    cfg = g.config(WORKLOADS["tiny"])
    setattr(cfg, field, value)
    with pytest.raises(g.GPT2Error) as e:
        g.num_params(cfg)
    assert e.value.code == g.GPT2_ESHAPE
    assert g.last_error()


def test_create_rejects_null_and_misaligned_buffers(g):
    from transformer_lm_amd.workloads import WORKLOADS
    cfg = g.config(WORKLOADS["tiny"])
    h = ct.c_void_p()
    rc = g._lib.gpt2_create(ct.byref(cfg), None, None, None, None, ct.byref(h))
    assert rc == g.GPT2_EINVAL and not h.value
    rc = g._lib.gpt2_create(ct.byref(cfg), 0x1004, 0x2000, None, None, ct.byref(h))
    assert rc == g.GPT2_EINVAL and "aligned" in g.last_error()


def test_null_handle_calls_fail_cleanly(g):
    assert g._lib.gpt2_backward(None) == g.GPT2_EINVAL
    assert g._lib.gpt2_update(None, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1) == g.GPT2_EINVAL
    assert g._lib.gpt2_forward(None, None, None, None) == g.GPT2_EINVAL
    s = g.Schedule(6e-4, 6e-5, 10, 100, 0.9, 0.95, 1e-8, 0.1, 1.0)
    assert g._lib.gpt2_update_scheduled(None, ct.byref(s), 1) == g.GPT2_EINVAL
    assert g._lib.gpt2_schedule_lr(None, 1) == -1.0
    assert g._lib.gpt2_schedule_lr(ct.byref(s), 0) == -1.0
    assert g._lib.gpt2_checkpoint_save(None, 1, None, 0) == g.GPT2_EINVAL
    assert g._lib.gpt2_checkpoint_load(None, None, 0, None) == g.GPT2_EINVAL
    g._lib.gpt2_free(None)


def test_fp8_entry_points_validate_before_launching(g):
    lib = g._lib
    a = 1 << 20                                      # 16-byte aligned, never dereferenced
    assert g.fp8_scale_workspace_bytes() >= 4
    assert lib.gpt2_fp8_scale(None, a, a, 10, None) == g.GPT2_EINVAL
    assert lib.gpt2_fp8_scale(a, a, a, -1, None) == g.GPT2_EINVAL
    assert lib.gpt2_fp8_scale(a, a, a + 2, 10, None) == g.GPT2_EINVAL      # x misaligned
    assert lib.gpt2_fp8_quantize(None, a, a, 10, None) == g.GPT2_EINVAL
    assert lib.gpt2_fp8_quantize(a + 8, a, a, 10, None) == g.GPT2_EINVAL  # q misaligned
    assert lib.gpt2_fp8_quantize(a, a, a, 0, None) == g.GPT2_OK           # empty: no launch
    mm = lib.gpt2_fp8_matmul
    assert mm(None, a, a, a, None, 8, 8, 128, None) == g.GPT2_EINVAL
    assert mm(a, a, a, None, None, 8, 8, 128, None) == g.GPT2_EINVAL
    assert mm(a, a + 4, a, a, None, 8, 8, 128, None) == g.GPT2_EINVAL
    assert mm(a, a, a, a, a + 2, 8, 8, 128, None) == g.GPT2_EINVAL        # bias misaligned
    assert mm(a, a, a, a, None, 8, 8, 100, None) == g.GPT2_ESHAPE         # K % 128
    assert mm(a, a, a, a, None, 8, 12, 128, None) == g.GPT2_ESHAPE        # N % 8
    assert mm(a, a, a, a, None, 0, 8, 128, None) == g.GPT2_ESHAPE
    assert g.last_error()


def test_attention_entry_point_validates_before_launching(g):
    att = g._lib.gpt2_attention_forward
    a = 1 << 20                                      # 16-byte aligned, never dereferenced
    bf16 = g.DTYPE_BF16
    assert att(None, a, a, 1, 8, 128, 2, bf16, None) == g.GPT2_EINVAL
    assert att(a, None, a, 1, 8, 128, 2, bf16, None) == g.GPT2_EINVAL
    assert att(a, a, a + 2, 1, 8, 128, 2, bf16, None) == g.GPT2_EINVAL     # qkv misaligned
    assert att(a, a, a, 1, 8, 128, 2, 7, None) == g.GPT2_EINVAL            # dtype
    assert att(a, a, a, 0, 8, 128, 2, bf16, None) == g.GPT2_ESHAPE
    assert att(a, a, a, 1, 0, 128, 2, bf16, None) == g.GPT2_ESHAPE
    assert att(a, a, a, 1, 8, 120, 2, bf16, None) == g.GPT2_ESHAPE         # head size 60
    assert att(a, a, a, 1, 8, 512, 2, bf16, None) == g.GPT2_ESHAPE         # head size 256
    assert att(a, a, a, 1, 8, 128, 3, bf16, None) == g.GPT2_ESHAPE         # C % NH
    assert att(a, a, a, 1024, 1024, 128, 2, bf16, None) == g.GPT2_ESHAPE   # B*T
    assert g.last_error()


def test_attention_backward_entry_point_validates_before_launching(g):
    att = g._lib.gpt2_attention_backward
    a = 1 << 20                                      # 16-byte aligned, never dereferenced
    bf16 = g.DTYPE_BF16
    assert att(None, a, a, a, a, a, 1, 8, 128, 2, bf16, None) == g.GPT2_EINVAL
    assert att(a, None, a, a, a, a, 1, 8, 128, 2, bf16, None) == g.GPT2_EINVAL   # no workspace
    assert att(a, a, a, a, a, None, 1, 8, 128, 2, bf16, None) == g.GPT2_EINVAL
    assert att(a, a, a + 2, a, a, a, 1, 8, 128, 2, bf16, None) == g.GPT2_EINVAL  # dout misaligned
    assert att(a, a, a, a, a, a, 1, 8, 128, 2, 5, None) == g.GPT2_EINVAL         # dtype
    assert att(a, a, a, a, a, a, 0, 8, 128, 2, bf16, None) == g.GPT2_ESHAPE
    assert att(a, a, a, a, a, a, 1, 8, 120, 2, bf16, None) == g.GPT2_ESHAPE      # head size 60
    assert att(a, a, a, a, a, a, 1024, 1024, 128, 2, bf16, None) == g.GPT2_ESHAPE  # B*T
    assert g.last_error()


def test_noalloc_attention_backward_validates_before_launching(g):
    att = g._lib.gpt2_attention_backward_noalloc
    a = 1 << 20                                      # 16-byte aligned, never dereferenced
    bf16 = g.DTYPE_BF16
    assert att(None, a, a, a, a, 1, 8, 128, 2, bf16, None) == g.GPT2_EINVAL
    assert att(a, a, a, a, a + 4, 1, 8, 128, 2, bf16, None) == g.GPT2_EINVAL   # lse misaligned
    assert att(a, a, a, a, a, 1, 8, 128, 2, 9, None) == g.GPT2_EINVAL          # dtype
    assert att(a, a, a, a, a, 1, 8, 120, 2, bf16, None) == g.GPT2_ESHAPE       # head size 60
    # beyond the static scratch: 2*B*NH*T = 2 * 33 * 16 * 1024 > 2^20
    assert att(a, a, a, a, a, 33, 1024, 1024, 16, bf16, None) == g.GPT2_ESHAPE
    assert "static scratch" in g.last_error()
