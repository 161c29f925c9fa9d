"""The seeded input generator: determinism, layout and distributions."""
import math

import numpy as np

from transformer_lm_amd import synth
from transformer_lm_amd.workloads import WORKLOADS, param_offsets


def test_splitmix64_reference_words():
    # SplitMix64 from seed 0: the first outputs as published with the algorithm
    # (Steele, Lea & Flood 2014; also the seeding generator of xoshiro).
    w = synth.splitmix64(0, 0, 3)
    assert [int(v) for v in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_slices_agree():
    a = synth.normal(7, 0, 100)
    b = synth.normal(7, 37, 20)
    assert np.array_equal(a[37:57], b)
    u = synth.uniform(7, 0, 50)
    assert np.array_equal(u[10:20], synth.uniform(7, 10, 10))
    assert u.min() >= 0 and u.max() < 1


def test_normal_moments():
    z = synth.normal(3, 0, 400_000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01


def test_init_layout_and_scales():
    w = WORKLOADS["tiny_pad"]
    p = synth.init_params(w)
    assert p.dtype == np.float32 and p.size == w.num_params() == 28544
    offs = param_offsets(w)

    def t(n):
        off, s = offs[n]
        return p[off:off + int(np.prod(s))].reshape(s)
    assert not t("wte")[w.V:].any()                      # padded rows are zero
    assert np.all(t("ln1w") == 1) and np.all(t("lnfw") == 1)
    assert not t("qkvb").any() and not t("lnfb").any()
    assert abs(t("fcw").std() - 0.02) < 0.002
    assert abs(t("fcprojw").std() - 0.02 / math.sqrt(2 * w.L)) < 0.001
    assert np.array_equal(p, synth.init_params(w))       # deterministic


def test_param_count_124m():
    assert WORKLOADS["gpt2_124m"].num_params() == 124_475_904
    assert WORKLOADS["gpt2_350m"].num_params() == 354_871_296
    assert WORKLOADS["gpt2_1558m"].num_params() == 1_557_686_400


def test_uniform_tokens():
    w = WORKLOADS["tiny"]
    t = synth.tokens(w)
    assert t.shape == (1, 4, 17) and t.dtype == np.int32
    assert t.min() >= 0 and t.max() < w.V
    x, y = synth.split_batch(t[0])
    assert np.array_equal(x[:, 1:], y[:, :-1])


def test_zipf_tokens_follow_the_law():
    w = WORKLOADS["gpt2_124m"].with_batch(steps=2)
    t = synth.tokens(w)
    assert t.shape == (2, 16, 1025)
    assert t.min() >= 0 and t.max() < w.V
    H = np.sum(np.arange(1, w.V + 1, dtype=np.float64) ** -1.1)
    p0 = 1.0 / H
    frac0 = (t == 0).mean()
    n = t.size
    assert abs(frac0 - p0) < 4 * math.sqrt(p0 * (1 - p0) / n)
    assert abs(H - 7.196944) < 1e-5
    assert not np.array_equal(t[0], t[1])                # fresh block per step
