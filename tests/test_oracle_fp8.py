"""Pins of the oracle's FP8 (E4M3) functions against what fixes them
independently of its code: the OCP E4M3 definition (values of named codes),
torch's own float -> float8_e4m3fn conversion (a library routine, compared on
a sweep that covers every rounding boundary), exhaustive round trips, and an
exact integer matrix product for the scaled products. The pages only name FP8
support (talk "llm.c's Origin and the Future of LLM Compilers", chapter
"Project Roadmap, Community Forks, and LLaMA Architecture Support")."""
import math

import numpy as np
import pytest
import torch

from oracle import wrapper as ow


def test_named_codes_follow_the_e4m3_definition():
    # sign | exponent (bias 7) | 3 mantissa bits; exponent 0 = subnormals m/8 * 2^-6
    cases = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0x3c: 1.5, 0x7e: 448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x0f: 1.875 * 2.0 ** -6,
             0xb8: -1.0, 0xfe: -448.0, 0x77: 240.0, 0x6f: 120.0}
    for code, val in cases.items():
        assert ow.e4m3_decode([code])[0] == val, hex(code)
    assert math.isnan(ow.e4m3_decode([0x7f])[0]) and math.isnan(ow.e4m3_decode([0xff])[0])
    assert math.copysign(1.0, ow.e4m3_decode([0x80])[0]) == -1.0


def test_encode_ties_go_to_the_even_code():
    x = np.array([1.0625, 1.1875, 1.0 + 1e-6, 2.0 ** -10, 1.5 * 2.0 ** -10, 456.0, 464.0,
                  464.5, 472.0, -1.0625], np.float32)
    want = [0x38, 0x3a, 0x38, 0x00, 0x01, 0x7e, 0x7e, 0x7f, 0x7f, 0xb8]
    assert [int(c) for c in ow.e4m3_encode(x)] == want


def test_encode_matches_torch_float8_e4m3fn():
    vals = ow.e4m3_decode(np.arange(0x7f))
    pts = []
    for lo, hi in zip(vals[:-1], vals[1:]):
        mid = 0.5 * (lo + hi)
        pts += [lo, mid, lo + 0.25 * (hi - lo), lo + 0.75 * (hi - lo),
                np.nextafter(np.float32(mid), np.float32(0)),
                np.nextafter(np.float32(mid), np.float32(1e9))]
    rng = np.random.default_rng(7)
    pts += list(rng.uniform(-460, 460, 4000)) + list(rng.normal(0, 1e-2, 2000))
    pts += [448.0, 463.99, 464.0, 470.0, 1e6, 1e-30, 0.0]
    x = np.array(pts + [-p for p in pts], np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = ow.e4m3_encode(x)
    # the two NaN codes of one sign are the same value; compare codes otherwise
    assert np.array_equal(got, ref)


def test_every_finite_code_round_trips():
    codes = [c for c in range(256) if c not in (0x7f, 0xff)]
    vals = ow.e4m3_decode(codes).astype(np.float32)
    assert [int(c) for c in ow.e4m3_encode(vals)] == codes


def test_scale_maps_the_largest_magnitude_to_448():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 3.0, 5000).astype(np.float32)
    x[123] = -11.5
    amax = ow.fp8_amax(x)
    assert amax == np.float32(np.abs(x).max())
    s = ow.fp8_scale(amax)
    assert s == np.float32(448.0) / np.float32(amax)
    q = ow.fp8_quantize(x, s)
    i = int(np.argmax(np.abs(x)))
    assert q[i] in (0x7e, 0xfe)
    assert not np.isnan(ow.e4m3_decode(q)).any()          # nothing overflows
    assert ow.fp8_scale(0.0) == 1.0
    assert (ow.fp8_quantize(np.zeros(17, np.float32), 1.0) == 0).all()


def test_quantize_rounds_the_fp32_product():
    # x * s is rounded to fp32 before the code is chosen: a product whose exact
    # value sits just past a tie but rounds onto it in fp32 takes the tie rule
    x = np.array([1.0625 * (1 + 2.0 ** -30)], np.float32)   # == 1.0625 in fp32
    assert ow.fp8_quantize(x, 1.0)[0] == 0x38


@pytest.mark.parametrize("M,N,K", [(5, 7, 16), (33, 40, 128), (3, 8, 300)])
def test_scaled_product_equals_exact_integer_product(M, N, K):
    # codes of the integers -8..8 and of halves: scaled by 2 they are integers,
    # so the product is an exact int64 matrix product
    ints = {0x00: 0, 0x30: 1, 0x38: 2, 0x3c: 3, 0x40: 4, 0x42: 5, 0x44: 6, 0x46: 7,
            0x48: 8, 0x4a: 10, 0x4c: 12, 0x50: 16}
    codes = np.array(list(ints), np.uint8)
    twice = np.array([ints[c] for c in codes], np.int64)  # 2 * value
    rng = np.random.default_rng(M * N + K)
    ix = rng.integers(0, len(codes), (M, K))
    iw = rng.integers(0, len(codes), (N, K))
    sx = rng.choice([1, -1], (M, K))
    sw = rng.choice([1, -1], (N, K))
    qx = (codes[ix] | np.where(sx < 0, 0x80, 0)).astype(np.uint8)
    qw = (codes[iw] | np.where(sw < 0, 0x80, 0)).astype(np.uint8)
    qx[qx == 0x80] = 0
    qw[qw == 0x80] = 0
    X = twice[ix] * sx
    W = twice[iw] * sw
    exact = (X @ W.T)                                     # = 4 * value product
    bias = rng.normal(size=N)
    scx, scw = np.float32(3.5), np.float32(0.75)
    got = ow.fp8_matmul(qx, qw, scx, scw, bias)
    want = exact / 4.0 / (float(scx) * float(scw)) + bias
    assert np.allclose(got, want, rtol=1e-15, atol=1e-12)
    assert np.allclose(ow.fp8_matmul(qx, qw, 1.0, 1.0), exact / 4.0, rtol=0, atol=0)
