"""Pins of the oracle's MXFP8 quantize of fp32 input (the weight-cache refresh from the fp32 master weight,
"OLMo-core MoE, Section 11: MXFP8 Training", Section 11.3.2 and Figure 55; block rule of Eq. 58 and Section 11.3.5).

1. On fp32 values that bf16 holds exactly it must equal the bf16 quantizer (pinned elsewhere), both rules and both
   orientations.
2. On fp32 values with full 23-bit mantissas (which the bf16 path never sees) every scale byte must be the smallest
   byte whose power of two keeps the block maximum within 448 (rceil; brute force over all 255 bytes), and every
   code the nearest E4M3 value to x / s with ties to the even code and saturation (brute force over all codes, in
   float64, from the pinned code table)."""
import numpy as np
import pytest

import oracle


def _table():
    codes = np.arange(0x7F, dtype=np.uint8)                      # non-negative finite E4M3 codes 0x00 .. 0x7E
    return codes, oracle.fp8_value(codes, oracle.E4M3)


def _nearest(v: float, codes, vals) -> int:
    a = abs(v)
    if a >= 448.0:
        c = 0x7E
    else:
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        c = int(codes[best[0]]) if len(best) == 1 else int(codes[best[codes[best] % 2 == 0][0]])
    return c | (0x80 if np.signbit(v) else 0)


@pytest.mark.parametrize("rule", [oracle.RCEIL, oracle.FLOOR])
def test_equals_bf16_path_on_bf16_values(rule):
    rng = np.random.default_rng(5)
    xb = oracle.bf16_from_f32((rng.standard_normal((96, 160)) * 3).astype(np.float32))
    xf = oracle.bf16_to_f32(xb)
    a = oracle.mx_quantize(xb, rule)
    b = oracle.mx_quantize_f32(xf, rule)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_full_mantissa_blocks_brute_force():
    rng = np.random.default_rng(6)
    codes, vals = _table()
    rows, cols = 8, 64
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 20, size=(rows, 1)))).astype(np.float32)
    x[0, :32] = np.float32(17.0) + np.float32(1.5e-6) * np.arange(32, dtype=np.float32)   # near a tie, not bf16
    x[0, 5] = np.float32(448.0)                                                       # that block's max: s = 1
    q, s, _, _ = oracle.mx_quantize_f32(x, oracle.RCEIL, colwise=False)
    for r in range(rows):
        for b in range(cols // 32):
            blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.max(np.abs(blk))
            byte = min(k for k in range(255) if amax <= 448.0 * 2.0 ** (k - 127))
            assert s[r, b] == byte, (r, b)
            scale = 2.0 ** (byte - 127)
            for i in range(32):
                assert q[r, 32 * b + i] == _nearest(blk[i] / scale, codes, vals), (r, b, i)


def test_column_orientation_is_row_of_transpose():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 96)) * 0.02).astype(np.float32)
    _, _, qc, sc = oracle.mx_quantize_f32(x, oracle.RCEIL, rowwise=False)
    qr, sr, _, _ = oracle.mx_quantize_f32(np.ascontiguousarray(x.T), oracle.RCEIL, colwise=False)
    assert np.array_equal(qc, qr) and np.array_equal(sc, sr)
