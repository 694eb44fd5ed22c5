"""Pins of the oracle's single-GPU parts of the FP8 gradient all-reduce ("FP8-LM: Training FP8 Large Language
Models", Section 3.4: automatic scaling factor mu, Eq. 3, and the shared scaling factor, Eq. 4-6).
The overflow counts and mu decisions below are worked out by hand from the rule (halve mu when more than 0.001 % of
the codes sit at the format's maximum, else grow it by 2^(1/1000)); the codes reduce to the per-tensor cast at scale
mu, and the requantize to identities of the (pinned) codec."""
import numpy as np
import pytest

import oracle

F32 = np.float32


def _grad_with_saturating(n, k, big):
    g = np.full(n, 0.25, np.float32)
    g[1::2] = -0.125
    g[np.arange(k) * 7] = big * (1 - 2 * (np.arange(k) % 2))       # k values of magnitude `big`, alternating sign
    return oracle.bf16_from_f32(g)


@pytest.mark.parametrize("k,halve", [(0, False), (2, False), (3, True), (50, True)])
def test_overflow_ratio_threshold(k, halve):
    n = 200_000                                                    # 1e-5 * n = 2 codes
    g = _grad_with_saturating(n, k, 600.0)
    q, cnt, s, mu_next = oracle.autoscale_cast(g, 1.0, oracle.E4M3)
    assert cnt == k
    assert s == F32(1.0)
    assert mu_next == (F32(0.5) if halve else F32(2.0 ** (1 / 1000)))


def test_codes_are_the_per_tensor_cast_at_scale_mu_and_e5m2_max():
    rng = np.random.default_rng(12)
    g = oracle.bf16_from_f32((rng.standard_normal(5000) * 1e-3).astype(np.float32)).reshape(50, 100)
    mu = F32(3.0e4)
    q, cnt, s, _ = oracle.autoscale_cast(g, float(mu), oracle.E5M2)
    _, _, q_pt, _ = oracle.pertensor_quantize(g, oracle.E5M2, scale_in=float(mu), want_qt=False)
    assert np.array_equal(q, q_pt.reshape(-1))
    assert cnt == int(np.sum((q & 0x7F) == 0x7B))


def test_requantize_identities():
    codes = np.arange(256, dtype=np.uint8)
    finite = ~np.isnan(oracle.fp8_value(codes, oracle.E4M3))
    same = oracle.requantize_shared(codes, oracle.E4M3, 0.37, 0.37, oracle.E4M3)
    assert np.array_equal(same[finite], codes[finite])              # s_g = s_i: every finite code comes back
    half = oracle.requantize_shared(codes, oracle.E4M3, 2.0, 1.0, oracle.E4M3)
    v = oracle.fp8_value(codes, oracle.E4M3)
    assert np.array_equal(half[finite], oracle.fp8_encode(v[finite] / 2.0, oracle.E4M3))
    to5 = oracle.requantize_shared(codes, oracle.E4M3, 1.0, 1.0, oracle.E5M2)
    assert np.array_equal(to5[finite], oracle.fp8_encode(v[finite], oracle.E5M2))
    assert oracle.min_scale(np.array([3.0, 0.5, 2.0], np.float32)) == F32(0.5)
