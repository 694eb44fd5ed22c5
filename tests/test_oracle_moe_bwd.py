"""Pins of the oracle's routed-expert backward ("OLMo-core MoE, Section 11: MXFP8 Training", Section 11.4.1, backward
of the routed experts, and Section 11.4.4, Table 25):

- the SwiGLU backward against the calculus: its analytic form against a finite difference of the float64 forward,
  the fp32 values against that float64 form, and the values at zero and in both saturated limits;
- the fused SwiGLU-backward quantize and the route-weighted gradient quantize against the fp32-input and bf16-input MX
  quantizers (pinned on their own), with power-of-two route weights that only move scale bytes;
- the per-expert contraction over token ranges (routed Wgrad) against numpy matrix products of the dequantized slices,
  the full-range GEMM reference, the sum over experts, empty experts and a pure-Python brute force."""
import math

import numpy as np
import pytest

import oracle
from mxfp8_precision_numerics_amd import workloads


def _silu64(g):
    return g / (1.0 + math.exp(-g))


def _dgate64(g, u, dh):
    s = 1.0 / (1.0 + math.exp(-g))
    return dh * u * s * (1.0 + g * (1.0 - s))


def test_swiglu_bwd_formula_is_the_derivative():
    """The analytic d_gate / d_up are the partial derivatives of h = silu(g) u (central differences in float64)."""
    rng = np.random.default_rng(21)
    for g, u, dh in rng.standard_normal((400, 3)) * np.array([4.0, 2.0, 1.5]):
        step = 1e-6 * max(1.0, abs(g))
        num_g = dh * (_silu64(g + step) * u - _silu64(g - step) * u) / (2 * step)
        num_u = dh * (_silu64(g) * (u + 1e-6) - _silu64(g) * (u - 1e-6)) / 2e-6
        assert abs(_dgate64(g, u, dh) - num_g) <= 1e-6 * (1 + abs(num_g))
        assert abs(dh * _silu64(g) - num_u) <= 1e-6 * (1 + abs(num_u))


def test_swiglu_bwd_f32_against_float64():
    rng = np.random.default_rng(22)
    vals = (rng.standard_normal((3000, 3)) * np.array([5.0, 2.0, 1e-2])).astype(np.float32)
    vals[:200, 0] = np.linspace(-1.5, -1.1, 200, dtype=np.float32)      # around the zero of silu'(g) (g ~ -1.278)
    vals[200:260, 0] = np.linspace(15.0, 40.0, 60, dtype=np.float32)    # sigma(g) rounds to 1
    vals[260:320, 0] = np.linspace(-40.0, -15.0, 60, dtype=np.float32)  # sigma(g) tiny
    for g, u, dh in vals:
        dg, du = oracle.swiglu_bwd_f32(float(g), float(u), float(dh))
        g64, u64, dh64 = float(g), float(u), float(dh)
        s = 1.0 / (1.0 + math.exp(-g64))
        ref_g = _dgate64(g64, u64, dh64)
        ref_u = dh64 * _silu64(g64)
        tol_g = 2.0 ** -19 * abs(dh64 * u64) * s * (1.0 + abs(g64)) + 1e-44
        tol_u = 2.0 ** -20 * abs(ref_u) + 1e-44
        assert abs(float(dg) - ref_g) <= tol_g, (g, u, dh, dg, ref_g)
        assert abs(float(du) - ref_u) <= tol_u, (g, u, dh, du, ref_u)


def test_swiglu_bwd_special_values():
    dg, du = oracle.swiglu_bwd_f32(0.0, 3.0, 0.25)        # sigma(0) = 1/2, silu'(0) = 1/2, silu(0) = 0
    assert dg == np.float32(0.375) and du == 0.0
    dg, du = oracle.swiglu_bwd_f32(100.0, 1.5, -2.0)      # sigma -> 1: silu' -> 1, silu -> g
    assert dg == np.float32(-3.0) and du == np.float32(-200.0)
    dg, du = oracle.swiglu_bwd_f32(-100.0, 1.5, 2.0)      # sigma -> 0: both vanish
    assert dg == 0.0 and du == 0.0
    dg, du = oracle.swiglu_bwd_f32(float("nan"), 1.0, 1.0)
    assert np.isnan(dg) and np.isnan(du)


@pytest.mark.parametrize("rule", [oracle.RCEIL, oracle.FLOOR])
def test_swiglu_bwd_quantize_is_mx_quantize_of_the_gradients(rule):
    rng = np.random.default_rng(23)
    rows, F = 64, 96
    c = oracle.bf16_from_f32((rng.standard_normal((rows, 2 * F)) * 2).astype(np.float32))
    dh = oracle.bf16_from_f32((rng.standard_normal((rows, F)) * 1e-3).astype(np.float32))
    qr, sr, qc, sc, dc = oracle.swiglu_bwd_mx_quantize(c, dh, rule, want_dc=True)
    cf = oracle.bf16_to_f32(c).reshape(rows, 2 * F)
    hf = oracle.bf16_to_f32(dh).reshape(rows, F)
    for r in range(0, rows, 7):
        for j in range(F):
            dg, du = oracle.swiglu_bwd_f32(float(cf[r, j]), float(cf[r, F + j]), float(hf[r, j]))
            assert dc[r, j].view(np.uint32) == np.float32(dg).view(np.uint32)
            assert dc[r, F + j].view(np.uint32) == np.float32(du).view(np.uint32)
    q2r, s2r, q2c, s2c = oracle.mx_quantize_f32(dc, rule)
    assert np.array_equal(qr, q2r) and np.array_equal(sr, s2r)
    assert np.array_equal(qc, q2c) and np.array_equal(sc, s2c)


@pytest.mark.parametrize("rule", [oracle.RCEIL, oracle.FLOOR])
def test_route_weighted_quantize_unit_and_power_of_two_weights(rule):
    rows, cols = 96, 160
    dy = workloads.as_u16(workloads.normal_bf16((rows, cols), 1e-3, 4, 9))
    ones = np.ones(rows, np.float32)
    qr, sr, qc, sc, x = oracle.route_weighted_mx_quantize(dy, ones, rule, want_x=True)
    br, bsr, bc, bsc = oracle.mx_quantize(dy, rule)
    assert np.array_equal(qr, br) and np.array_equal(sr, bsr) and np.array_equal(qc, bc) and np.array_equal(sc, bsc)
    # per-row powers of two: row codes unchanged, each row's scale bytes move by its exponent
    ex = np.arange(rows) % 7 - 3
    p = np.ldexp(np.ones(rows, np.float32), ex).astype(np.float32)
    qr2, sr2, _, _, x2 = oracle.route_weighted_mx_quantize(dy, p, rule, colwise=False, want_x=True)
    assert np.array_equal(qr2, qr)
    assert np.array_equal(sr2.astype(np.int64), sr.astype(np.int64) + ex[:, None])
    assert np.array_equal(x2, (p[:, None] * oracle.bf16_to_f32(dy).reshape(rows, cols)).astype(np.float32))
    # one power of two for all rows: the column orientation moves the same way
    _, _, qc3, sc3, _ = oracle.route_weighted_mx_quantize(dy, np.full(rows, 0.25, np.float32), rule, rowwise=False)
    assert np.array_equal(qc3, qc) and np.array_equal(sc3.astype(np.int64), sc.astype(np.int64) - 2)


def test_route_weighted_quantize_general_weights_and_zero_rows():
    rows, cols = 64, 128
    rng = np.random.default_rng(24)
    dy = workloads.as_u16(workloads.normal_bf16((rows, cols), 1e-3, 4, 10))
    p = rng.uniform(0.01, 1.0, rows).astype(np.float32)
    p[5] = 0.0
    p[40:64] = 0.0                                        # padding rows of an expert group carry weight 0
    qr, sr, qc, sc, x = oracle.route_weighted_mx_quantize(dy, p, oracle.RCEIL, want_x=True)
    assert np.array_equal(x, (p[:, None] * oracle.bf16_to_f32(dy).reshape(rows, cols)).astype(np.float32))
    f = oracle.mx_quantize_f32(x, oracle.RCEIL)
    assert np.array_equal(qr, f[0]) and np.array_equal(sr, f[1]) and np.array_equal(qc, f[2]) and np.array_equal(sc, f[3])
    assert not np.any(qr[5] & 0x7F) and not np.any(qr[40:] & 0x7F) and not np.any(sr[40:])
    assert not np.any(qc[:, 40:] & 0x7F)


# ---------------------------------------------------------------- routed Wgrad
def _mx_operand(rows, kt, seed, std=1.0):
    """Column-orientation MX operand [rows][kt] from an fp32 matrix [kt][rows] (blocks of 32 along kt)."""
    x = workloads.normal_bf16((kt, rows), std, 4, seed)
    _, _, q, s = oracle.mx_quantize(workloads.as_u16(x), oracle.RCEIL, rowwise=False)
    return q, s


def _dequant(q, s):
    v = oracle.fp8_value(q.reshape(-1), oracle.E4M3).reshape(q.shape)
    return v * np.ldexp(1.0, np.repeat(s.astype(np.int64) - 127, 32, axis=1))


def test_wgrad_ref_matches_numpy_slices():
    M, N = 48, 40
    off = np.array([0, 96, 96, 160, 416, 448], np.int64)       # an empty expert, odd block counts
    kt = int(off[-1])
    aq, as_ = _mx_operand(M, kt, 11)
    bq, bs = _mx_operand(N, kt, 12, 0.3)
    y, S = oracle.grouped_wgrad_ref(aq, as_, bq, bs, off)
    A = _dequant(aq, as_)
    B = _dequant(bq, bs)
    for g in range(off.size - 1):
        lo, hi = off[g], off[g + 1]
        ref = A[:, lo:hi] @ B[:, lo:hi].T
        sabs = np.abs(A[:, lo:hi]) @ np.abs(B[:, lo:hi]).T
        assert np.all(np.abs(y[g] - ref) <= 1e-12 * sabs + 1e-300)
        assert np.allclose(S[g], sabs, rtol=1e-12, atol=0)
    assert np.all(y[1] == 0.0) and np.all(S[1] == 0.0)
    full_y, full_S = oracle.gemm_ref(aq, as_, oracle.E4M3, bq, bs, oracle.E4M3, oracle.MX_BLOCK32)
    assert np.all(np.abs(y.sum(axis=0) - full_y) <= 1e-12 * full_S + 1e-300)


def test_wgrad_ref_single_group_is_the_gemm_reference():
    M, N, kt = 32, 24, 256
    aq, as_ = _mx_operand(M, kt, 13)
    bq, bs = _mx_operand(N, kt, 14)
    y, S = oracle.grouped_wgrad_ref(aq, as_, bq, bs, np.array([0, kt], np.int64))
    fy, fS = oracle.gemm_ref(aq, as_, oracle.E4M3, bq, bs, oracle.E4M3, oracle.MX_BLOCK32)
    assert np.array_equal(y[0], fy) and np.array_equal(S[0], fS)


def test_wgrad_ref_brute_force_tiny():
    off = [0, 32, 32, 96]
    rng = np.random.default_rng(25)
    aq = rng.integers(0, 256, (2, 96)).astype(np.uint8)
    bq = rng.integers(0, 256, (3, 96)).astype(np.uint8)
    aq[(aq & 0x7F) == 0x7F] = 0x3C                          # no NaN codes
    bq[(bq & 0x7F) == 0x7F] = 0xB8
    as_ = rng.integers(118, 136, (2, 3)).astype(np.uint8)
    bs = rng.integers(118, 136, (3, 3)).astype(np.uint8)
    y, S = oracle.grouped_wgrad_ref(aq, as_, bq, bs, np.array(off, np.int64), groups=[2, 1, 0], rows=[1, 0],
                                    cols=[2, 0])
    for gi, g in enumerate([2, 1, 0]):
        for i, m in enumerate([1, 0]):
            for j, n in enumerate([2, 0]):
                acc = 0.0
                for k in range(off[g], off[g + 1]):
                    a = float(oracle.fp8_value(aq[m, k:k + 1], oracle.E4M3)[0]) * 2.0 ** (int(as_[m, k // 32]) - 127)
                    b = float(oracle.fp8_value(bq[n, k:k + 1], oracle.E4M3)[0]) * 2.0 ** (int(bs[n, k // 32]) - 127)
                    acc += a * b
                assert y[gi, i, j] == acc
