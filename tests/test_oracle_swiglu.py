"""Pins of the oracle's fused SwiGLU + MX row quantize ("OLMo-core MoE, Section 11: MXFP8 Training", Section 11.4.1):
the fixed fp32 exponential against the true exponential, the SwiGLU value against float64 arithmetic and its limits,
and the fused quantize against the fp32-input MX quantize (pinned separately) of the SwiGLU values."""
import math

import numpy as np

import oracle


def _ulp(t: float) -> float:
    return math.ldexp(1.0, math.frexp(t)[1] - 24)


def test_exp_against_true_exponential():
    xs = np.concatenate([np.linspace(-87.0, 88.0, 20001), np.linspace(-1.0, 1.0, 2001)]).astype(np.float32)
    worst = 0.0
    for x in xs:
        t = math.exp(float(x))
        worst = max(worst, abs(float(oracle.exp_f32(float(x))) - t) / _ulp(t))
    assert worst <= 4.0, worst
    assert oracle.exp_f32(0.0) == 1.0
    assert oracle.exp_f32(200.0) == np.inf and oracle.exp_f32(-200.0) == 0.0
    assert np.isnan(oracle.exp_f32(float("nan")))


def test_swiglu_values_and_limits():
    rng = np.random.default_rng(8)
    g = (rng.standard_normal(4000) * 3).astype(np.float32)
    u = (rng.standard_normal(4000) * 3).astype(np.float32)
    for a, b in zip(g, u):
        ref = float(a) / (1.0 + math.exp(-float(a))) * float(b)
        got = float(oracle.swiglu_f32(float(a), float(b)))
        assert abs(got - ref) <= 8 * _ulp(abs(ref)) + 1e-30, (a, b, got, ref)
    assert oracle.swiglu_f32(0.0, 5.0) == 0.0 and oracle.swiglu_f32(3.0, 0.0) == 0.0
    assert oracle.swiglu_f32(100.0, 1.5) == np.float32(150.0)          # silu(g) -> g for large g
    assert oracle.swiglu_f32(-100.0, 2.0) == 0.0                        # silu(g) -> -0 for very negative g


def test_fused_quantize_is_mx_quantize_of_swiglu_values():
    rng = np.random.default_rng(9)
    rows, F = 64, 96
    c = oracle.bf16_from_f32((rng.standard_normal((rows, 2 * F)) * 2).astype(np.float32))
    cf = oracle.bf16_to_f32(c).reshape(rows, 2 * F)
    for rule in (oracle.RCEIL, oracle.FLOOR):
        q, s, h = oracle.swiglu_mx_quantize(c, rule, want_h=True)
        expect_h = np.array([[oracle.swiglu_f32(float(cf[r, j]), float(cf[r, F + j])) for j in range(F)]
                             for r in range(rows)], np.float32)
        assert np.array_equal(h.view(np.uint32), expect_h.view(np.uint32))
        q2, s2, _, _ = oracle.mx_quantize_f32(h, rule, colwise=False)
        assert np.array_equal(q, q2) and np.array_equal(s, s2)
