"""Seeded input generators (CPU only): determinism, rounding, distributions."""
import numpy as np
import pytest

import la_inputs


def test_determinism_and_offsets(inputs_lib):
    a = la_inputs.normal(7, 1, (1000,), "fp32")
    b = la_inputs.normal(7, 1, (1000,), "fp32", nthreads=3)
    assert np.array_equal(a, b)
    c = la_inputs.normal(7, 1, (600,), "fp32", offset=400)
    assert np.array_equal(a[400:], c)
    assert not np.array_equal(a, la_inputs.normal(7, 2, (1000,), "fp32"))
    assert not np.array_equal(a, la_inputs.normal(8, 1, (1000,), "fp32"))


def test_bf16_round_to_nearest_even(inputs_lib):
    """The bf16 stream is the fp32 stream rounded to nearest even (checked with
    an independent numpy rounding of the same fp32 values)."""
    f = la_inputs.normal(11, 0, (200000,), "fp32", scale=0.1)
    h = la_inputs.normal(11, 0, (200000,), "bf16", scale=0.1)
    u = f.view(np.uint32).astype(np.uint64)
    lower = u >> 16
    rem = u & 0xFFFF
    up = (rem > 0x8000) | ((rem == 0x8000) & ((lower & 1) == 1))
    ref = (lower + up).astype(np.uint16)
    assert np.array_equal(h, ref)
    # explicit halfway cases through the C helper
    lib = la_inputs._load()
    for bits, exp in [(0x3F808000, 0x3F80), (0x3F818000, 0x3F82), (0x3F808001, 0x3F81), (0x3F807FFF, 0x3F80)]:
        x = np.array([bits], dtype=np.uint32).view(np.float32)[0]
        assert lib.lagen_f32_to_bf16(float(x)) == exp


def test_normal_moments(inputs_lib):
    x = la_inputs.normal(3, 0, (2_000_000,), "fp32").astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.var() - 1.0) < 5e-3
    assert abs(np.mean(x ** 4) - 3.0) < 3e-2  # Gaussian kurtosis
    assert abs(np.mean(x > 1.0) - 0.158655) < 2e-3


def test_ternary(inputs_lib):
    t = la_inputs.ternary(5, 0, (30000,), "fp32")
    assert set(np.unique(t).tolist()) == {-1.0, 0.0, 1.0}
    tb = la_inputs.ternary(5, 0, (30000,), "bf16")
    assert np.array_equal(la_inputs.bf16_bits_to_f32(tb), t)


def test_doc_lengths_recipe(inputs_lib):
    cu = la_inputs.doc_lengths(103, 131072, 512, 32768)
    lens = np.diff(cu)
    assert cu[0] == 0 and cu[-1] == 131072
    assert np.all(lens[:-1] >= 512) and np.all(lens[:-1] < 32768)
    assert 1 <= lens[-1] < 32768
    # log-uniform: log-lengths of many draws spread evenly over [ln 512, ln 32768)
    many = np.diff(la_inputs.doc_lengths(1, 50_000_000, 512, 32768))[:-1]
    z = (np.log(many) - np.log(512)) / (np.log(32768) - np.log(512))
    hist = np.histogram(z, bins=8, range=(0, 1))[0] / len(z)
    assert np.all(np.abs(hist - 0.125) < 0.02)


def test_workload_shapes(inputs_lib):
    w = la_inputs.prefill_inputs("tiny_fp32")
    assert w["q"].shape == (256, 2, 16) and w["q"].dtype == np.float32
    assert np.array_equal(w["cu"], [0, 256])
    x = w["q"].astype(np.float64)
    assert abs(x.var() - 1 / 16) < 0.01


def test_decode_state_sampler_matches_direct_sums(inputs_lib):
    """The Bartlett sampler draws K^T V for n rows of N(0, I/d) without the n d^2
    sum.  Compare its moments with direct sums of outer products: entries have
    mean 0 and variance n/d^2, and E[S S^T] = (n/d) I."""
    d, n, pairs = 16, 4096, 64
    fixed = np.full(pairs, n, dtype=np.int64)
    S = la_inputs.decode_states(9, 1, pairs, d, 1024, 1 << 20, fixed_n=fixed).astype(np.float64)
    rng = np.random.default_rng(0)
    direct = np.empty_like(S)
    for p in range(pairs):
        K = rng.standard_normal((n, d)) / np.sqrt(d)
        V = rng.standard_normal((n, d)) / np.sqrt(d)
        direct[p] = K.T @ V
    for X in (S, direct):
        var = X.var() / (n / d ** 2)
        assert abs(X.mean()) < 0.05 * np.sqrt(n) / d
        assert abs(var - 1.0) < 0.06
        SS = np.einsum("pij,pkj->ik", X, X) / pairs
        assert np.allclose(np.diag(SS), n / d, rtol=0.1)
        off = SS - np.diag(np.diag(SS))
        assert np.max(np.abs(off)) < 0.15 * n / d
    # fourth moment of the entries agrees between the two routes (sums of
    # products are not Gaussian at small n; this checks the Wishart part)
    k4 = lambda X: np.mean(X ** 4) / np.mean(X ** 2) ** 2
    assert abs(k4(S) - k4(direct)) < 0.15


def test_decode_state_prefix_lengths(inputs_lib):
    n = la_inputs.prefix_lengths(105, 256, 1024, 1 << 20)
    assert n.min() >= 1024 and n.max() < (1 << 20)
    S = la_inputs.decode_states(105, 2, 3, 8, 1024, 1 << 20)
    assert S.shape == (6, 8, 8) and np.all(np.isfinite(S))
    S2 = la_inputs.decode_states(105, 2, 3, 8, 1024, 1 << 20, nthreads=1)
    assert np.array_equal(S, S2)


def test_decode_state_sampler_small_prefix(inputs_lib):
    """n just above d exercises chi-square shapes below 1 (boosted gamma draws);
    entries keep variance n/d^2.  n < d is rejected."""
    d, n, pairs = 8, 9, 4000
    S = la_inputs.decode_states(4, 1, pairs, d, 1, 2, fixed_n=np.full(pairs, n)).astype(np.float64)
    assert np.all(np.isfinite(S))
    assert abs(S.var() / (n / d ** 2) - 1.0) < 0.05
    with pytest.raises(ValueError):
        la_inputs.decode_states(4, 1, 2, 8, 1, 2, fixed_n=np.array([7, 9]))
