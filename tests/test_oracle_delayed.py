"""Pins of the oracle's delayed per-tensor scaling ("3.8 Mixed Precision, bf16 & FP8 Training", the DelayedScale
sketch of the delayed-scaling recipe; "FP8-LM" Section 3.4, delayed scaling): this call's scale comes from the
maximum of the amax history of earlier calls (clamped at 1e-12), FMAX over it times the margin; the call's own amax
is then written at the ring position, which advances cyclically.

The expected scale sequence and ring contents below were worked out by hand from that definition; the remaining
checks reduce the delayed functions to the current-scaling ones, which carry their own pins."""
import numpy as np
import pytest

import oracle

F32 = np.float32


def bf16_const_matrix(rows, cols, amax, seed):
    """bf16 matrix whose largest magnitude is exactly `amax` (a bf16 value), the rest drawn well below it."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * amax * 0.1).astype(np.float32)
    x = np.clip(x, -0.5 * amax, 0.5 * amax)
    x[rows // 2, cols // 3] = -amax
    return oracle.bf16_from_f32(x)


def test_ring_window_and_order_of_scale_and_push():
    H = 3
    history = np.zeros(H, F32)
    pos = np.zeros(1, np.int32)
    amaxes = [1.0, 4.0, 2.0, 8.0, 3.0]
    # scale uses the history BEFORE this call's push; empty history -> 448 / 1e-12
    expected_scales = [F32(448.0) / F32(1e-12), 448.0, 112.0, 112.0, 56.0]
    for i, (a, s_exp) in enumerate(zip(amaxes, expected_scales)):
        x = bf16_const_matrix(64, 96, a, seed=i)
        amax, s, q, qt = oracle.pertensor_quantize_delayed(x, history, pos, oracle.E4M3)
        assert amax == a
        assert s == F32(s_exp), (i, s, s_exp)
    assert history.tolist() == [8.0, 3.0, 2.0]
    assert int(pos[0]) == 2


def test_empty_history_saturates_every_nonzero_value():
    history = np.zeros(16, F32)
    pos = np.zeros(1, np.int32)
    x = bf16_const_matrix(32, 64, 2.0, seed=7)
    amax, s, q, qt = oracle.pertensor_quantize_delayed(x, history, pos, oracle.E4M3)
    xf = oracle.bf16_to_f32(x)
    nz = xf != 0
    assert np.all(q[nz & (xf > 0)] == 0x7E) and np.all(q[nz & (xf < 0)] == 0xFE)
    assert history[0] == 2.0 and int(pos[0]) == 1


def test_margin_and_e5m2():
    history = np.array([0.5, 3.0, 1.5, 0.0], F32)
    assert oracle.delayed_scale(history, oracle.E5M2, 0.5) == F32(F32(57344.0) / F32(3.0)) * F32(0.5)
    assert oracle.delayed_scale(np.array([np.nan, 1.0], F32), oracle.E4M3, 1.0) != oracle.delayed_scale(
        np.array([1.0], F32), oracle.E4M3, 1.0)   # a NaN entry propagates


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_history_holding_this_amax_equals_current_scaling(fmt):
    rng = np.random.default_rng(3)
    x = oracle.bf16_from_f32((rng.standard_normal((96, 160)) * 3).astype(np.float32))
    amax_c, s_c, q_c, qt_c = oracle.pertensor_quantize(x, fmt)
    history = np.array([amax_c], F32)
    pos = np.zeros(1, np.int32)
    amax_d, s_d, q_d, qt_d = oracle.pertensor_quantize_delayed(x, history, pos, fmt)
    assert amax_d == amax_c and s_d == s_c
    assert np.array_equal(q_d, q_c) and np.array_equal(qt_d, qt_c)
    assert history[0] == amax_c and int(pos[0]) == 0        # H = 1: the position wraps to 0


def _adam_state(n, seed):
    rng = np.random.default_rng(seed)
    theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = oracle.bf16_from_f32((rng.standard_normal(n) * 1e-3).astype(np.float32))
    m_q = oracle.fp8_encode((rng.standard_normal(n) * 50).astype(np.float64), oracle.E4M3)
    v16 = oracle.f16_from_f32((rng.random(n) * 1e-6).astype(np.float32))
    return theta, g, m_q, v16


def test_adam_delayed_with_history_of_this_amax_equals_current_scaling():
    n = 5000
    hp = oracle.AdamHP(3e-4, 0.9, 0.95, 1e-8, 0.0, 3)
    theta, g, m_q, v16 = _adam_state(n, 11)
    a = [theta.copy(), m_q.copy(), np.array([2.5e4], np.float32), v16.copy()]
    amax_c, w_c = oracle.adam_step(a[0], g, a[1], a[2], a[3], hp)
    b = [theta.copy(), m_q.copy(), np.array([2.5e4], np.float32), v16.copy()]
    history = np.array([0.0, amax_c, 0.5 * amax_c], np.float32)
    pos = np.array([2], np.int32)
    amax_d, w_d = oracle.adam_step_delayed(b[0], g, b[1], b[2], b[3], hp, history, pos)
    assert amax_d == amax_c
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
    assert np.array_equal(w_c, w_d)
    assert history.tolist() == [0.0, amax_c, amax_c] and int(pos[0]) == 0


def test_adam_delayed_empty_history_saturates_first_moment():
    n = 2000
    hp = oracle.AdamHP(3e-4, 0.9, 0.95, 1e-8, 0.0, 1)
    theta, g, _, v16 = _adam_state(n, 12)
    m_q = np.zeros(n, np.uint8)
    m_scale = np.ones(1, np.float32)
    history = np.zeros(4, np.float32)
    pos = np.zeros(1, np.int32)
    amax, _ = oracle.adam_step_delayed(theta, g, m_q, m_scale, np.zeros(n, np.uint16), hp, history, pos)
    gf = oracle.bf16_to_f32(g)
    assert m_scale[0] == np.float32(448.0) / np.float32(1e-12)
    assert np.all(m_q[gf > 0] == 0x7E) and np.all(m_q[gf < 0] == 0xFE)
    assert history[0] == amax and int(pos[0]) == 1
