"""Pins for the oracle's precision-decoupled FP8 AdamW step (FP8-LM: AdamW update rule, Eq. 7-8).

The pages fix the formula, not the fp32 rounding sequence, so bit-level agreement between oracle and GPU is
pinned by the operation order stated in the oracle. Here the oracle is tied to an fp64 evaluation of the update
rule from the same decoded stored states, to closed forms at t = 1, and to library casts for the stored bytes.
"""
import numpy as np
import torch

import oracle
from mxfp8_precision_numerics_amd import workloads


def _state(n, t0=1):
    theta = workloads.workload5_params(n).numpy().copy()
    m_q = np.zeros(n, np.uint8)
    m_scale = np.ones(1, np.float32)
    v16 = np.zeros(n, np.uint16)
    return theta, m_q, m_scale, v16


def _hp(t, wd=0.0):
    return oracle.AdamHP(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=wd, step=t)


def test_adam_matches_fp64_update_rule_over_three_steps():
    n = 200_000
    theta, m_q, m_scale, v16 = _state(n)
    for t in (1, 2, 3):
        g = workloads.as_u16(workloads.workload5_grad(n, t))
        hp = _hp(t, wd=0.1 if t == 3 else 0.0)
        # fp64 evaluation of the update rule from the same decoded stored states
        gf = oracle.bf16_to_f32(g).astype(np.float64)
        m_old = oracle.fp8_value(m_q, oracle.E4M3) / float(m_scale[0])
        v_old = np.array([oracle.f16_value(b) for b in v16[:2000]])
        v_old_full = np.frombuffer(v16.tobytes(), np.float16).astype(np.float64)
        m = 0.9 * m_old + 0.1 * gf
        v = 0.95 * v_old_full + 0.05 * gf * gf
        mh = m / (1 - 0.9 ** t); vh = v / (1 - 0.95 ** t)
        den = np.sqrt(vh) + 1e-8
        u64 = mh / den + hp.weight_decay * theta.astype(np.float64)
        theta64 = theta.astype(np.float64) - 3e-4 * u64
        # first-order bound on fp32 rounding, from each intermediate's magnitude (cancellation in m is allowed for)
        r = 2.0 ** -22
        err_m = r * (0.9 * np.abs(m_old) + 0.1 * np.abs(gf)) + r * np.abs(m)
        err_v = r * (0.95 * v_old_full + 0.05 * gf * gf)
        ch = 1 / (1 - 0.9 ** t)
        err_u = ch * err_m / den + np.abs(mh / den) * (0.5 * err_v / np.maximum(v, 1e-300) * np.sqrt(vh) / den + 4 * r)
        err_u += hp.weight_decay * np.abs(theta) * 2 * r
        bound = r * np.abs(theta.astype(np.float64)) + 3e-4 * (err_u + 2 * r * np.abs(u64)) + r * np.abs(theta64)
        assert np.array_equal(v_old, v_old_full[:2000])
        amax, w = oracle.adam_step(theta, g, m_q, m_scale, v16, hp)
        assert np.all(np.abs(theta.astype(np.float64) - theta64) <= bound)
        # the bound is far below the step itself, so a dropped term or a wrong sign would fall outside it
        assert np.median(bound / (3e-4 * np.abs(u64))) < 1e-3
        assert amax == np.float32(np.abs(m).max()) or abs(amax - np.abs(m).max()) < 1e-6 * amax
        assert m_scale[0] == np.float32(448.0) / np.float32(amax)
        # stored bytes: bf16 copy and fp16 second moment are RNE casts of the fp32 values
        assert np.array_equal(w, torch.from_numpy(theta).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        i = np.argmax(np.abs(oracle.fp8_value(m_q, oracle.E4M3)))
        assert (m_q[i] & 0x7F) == 0x7E                           # the max-|m| element stores as +-448


def test_first_step_from_zero_state_moves_by_lr():
    n = 50_000
    theta, m_q, m_scale, v16 = _state(n)
    theta0 = theta.copy()
    g = workloads.as_u16(workloads.workload5_grad(n, 1))
    gf = oracle.bf16_to_f32(g).astype(np.float64)
    oracle.adam_step(theta, g, m_q, m_scale, v16, _hp(1))
    big = np.abs(gf) > 1e-5                                       # |g| >> eps: u = sign(g) (1 - O(eps/|g|))
    step = theta0.astype(np.float64) - theta.astype(np.float64)
    assert np.allclose(step[big], 3e-4 * np.sign(gf[big]), rtol=2e-3)


def test_fp16_second_moment_and_e4m3_first_moment_bytes():
    n = 4096
    theta, m_q, m_scale, v16 = _state(n)
    g = workloads.as_u16(workloads.workload5_grad(n, 1))
    gf = oracle.bf16_to_f32(g)
    oracle.adam_step(theta, g, m_q, m_scale, v16, _hp(1))
    v32 = (np.float32(0.95) * np.float32(0.0) + np.float32(1.0 - 0.95) * (gf * gf)).astype(np.float32)
    assert np.array_equal(v16, v32.astype(np.float16).view(np.uint16))
    m32 = (np.float32(0.9) * np.float32(0.0) + np.float32(1.0 - 0.9) * gf).astype(np.float32)
    assert np.array_equal(m_q, oracle.fp8_encode((m32 * m_scale[0]).astype(np.float32).astype(np.float64), oracle.E4M3))


def test_sampled_elements_match_full_step():
    n = 30_000
    theta, m_q, m_scale, v16 = _state(n)
    g1 = workloads.as_u16(workloads.workload5_grad(n, 1))
    oracle.adam_step(theta, g1, m_q, m_scale, v16, _hp(1))
    g2 = workloads.as_u16(workloads.workload5_grad(n, 2))
    before = (theta.copy(), m_q.copy(), float(m_scale[0]), v16.copy())
    amax = oracle.adam_amax(g2, m_q, v16, float(m_scale[0]), _hp(2))
    s_new = np.float32(448.0) / np.float32(max(amax, 1e-12))
    idx = np.array([0, 7, 12345, n - 1])
    om, oq, ov, ow = oracle.adam_elements(before[0], g2, before[1], before[3], before[2], s_new, idx, _hp(2))
    amax_full, w = oracle.adam_step(theta, g2, m_q, m_scale, v16, _hp(2))
    assert amax_full == amax and m_scale[0] == s_new
    assert np.array_equal(om, theta[idx]) and np.array_equal(oq, m_q[idx])
    assert np.array_equal(ov, v16[idx]) and np.array_equal(ow, w[idx])
