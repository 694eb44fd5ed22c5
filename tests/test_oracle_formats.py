"""Pins for the oracle's number formats (E4M3, E5M2, E8M0, BF16, FP16).

Each check ties the oracle to something other than itself: values printed on the pages (tests/golden), a
library routine (torch's float8 / bfloat16 casts, numpy's float16 cast), or an independent arithmetic encoder
written here with frexp/rint instead of the oracle's table search.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _p2(v):
    return float(v[0]) ** v[1] if isinstance(v, list) else float(v)


ALL = np.arange(256, dtype=np.uint8)


# ----------------------------------------------------------------- page-printed format constants
def test_figure49_format_table():
    g = _load("olmo11_figure49_formats.json")
    e4 = oracle.fp8_value(ALL, oracle.E4M3)
    e5 = oracle.fp8_value(ALL, oracle.E5M2)
    fin4 = e4[np.isfinite(e4)]
    fin5 = e5[np.isfinite(e5)]
    assert fin4.max() == g["E4M3"]["largest_finite"]
    assert fin5.max() == g["E5M2"]["largest_finite"]
    for vals, key in ((fin4, "E4M3"), (fin5, "E5M2")):
        pos = np.sort(vals[vals > 0])
        mbits = 3 if key == "E4M3" else 2
        sub = pos[pos < _p2(g[key]["smallest_normal"])]
        assert pos[0] == _p2(g[key]["smallest_subnormal"])
        assert np.min(pos[pos >= _p2(g[key]["smallest_normal"])]) == _p2(g[key]["smallest_normal"])
        assert len(sub) == 2 ** mbits - 1                   # subnormal ladder below the smallest normal
        above1 = pos[pos > 1.0][0]
        assert above1 - 1.0 == _p2(g[key]["spacing_above_1"])
    # E4M3 codes named on the pages' example and the format maxima
    assert oracle.fp8_value(np.array([0x7E, 0x08, 0x01, 0x39], np.uint8), oracle.E4M3).tolist() == [448, 2 ** -6, 2 ** -9, 1.125]
    assert oracle.fp8_value(np.array([0x7B, 0x04, 0x01], np.uint8), oracle.E5M2).tolist() == [57344, 2 ** -14, 2 ** -16]
    # E8M0: byte = e + 127; largest 2^127 (byte 254), smallest 2^-127 (byte 0)
    assert oracle.mx_scale_exp([1e300])[0] == 127 and oracle.mx_scale_exp([0.0])[0] == -127
    # BF16 row: largest finite ~3.39e38, smallest normal 2^-126, smallest subnormal 2^-133, spacing 2^-7
    assert abs(float(oracle.bf16_to_f32(np.array([0x7F7F], np.uint16))[0]) - g["BF16"]["largest_finite_approx"]) < 0.01e38
    assert float(oracle.bf16_to_f32(np.array([0x0080], np.uint16))[0]) == _p2(g["BF16"]["smallest_normal"])
    assert float(oracle.bf16_to_f32(np.array([0x0001], np.uint16))[0]) == _p2(g["BF16"]["smallest_subnormal"])
    assert float(oracle.bf16_to_f32(np.array([0x3F81], np.uint16))[0]) - 1.0 == _p2(g["BF16"]["spacing_above_1"])


def test_text_format_ranges():
    """Maxima and minima printed in the FP8-LM summary and the textbook chapter (3 significant digits)."""
    g = _load("format_ranges_text.json")
    for key, fmt in (("E4M3", oracle.E4M3), ("E5M2", oracle.E5M2)):
        v = oracle.fp8_value(ALL, fmt)
        v = v[np.isfinite(v) & (v > 0)]
        assert v.max() == g[key]["max_normal"]
        mbits = 3 if key == "E4M3" else 2
        min_normal = np.sort(v)[2 ** mbits - 1]
        assert f"{min_normal:.2e}" == f"{g[key]['min_normal']:.2e}"
        assert f"{v.min():.2e}" == f"{g[key]['min_subnormal']:.2e}"
    assert oracle.f16_value(0x7BFF) == g["FP16"]["max_normal"]


def test_bf16_pi_example():
    g = _load("llmsb_bf16_pi.json")
    bits = int(oracle.bf16_from_f32(np.array([g["fp32"]], np.float32))[0])
    assert bits == int(g["bf16_bits"], 16)
    assert float(oracle.bf16_to_f32(np.array([bits], np.uint16))[0]) == g["bf16_value"]


# ----------------------------------------------------------------- decode vs library, exhaustive round trips
@pytest.mark.parametrize("fmt,tdtype", [(oracle.E4M3, torch.float8_e4m3fn), (oracle.E5M2, torch.float8_e5m2)])
def test_decode_matches_torch_float8(fmt, tdtype):
    ours = oracle.fp8_value(ALL, fmt)
    lib = torch.from_numpy(ALL.copy()).view(tdtype).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], lib[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(lib[fin]))


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_exhaustive_256_code_round_trip(fmt):
    v = oracle.fp8_value(ALL, fmt)
    back = oracle.fp8_encode(v, fmt)
    maxc = 0x7E if fmt == oracle.E4M3 else 0x7B
    for c in range(256):
        val = v[c]
        if np.isnan(val):
            b = back[c]
            assert np.isnan(oracle.fp8_value(np.array([b], np.uint8), fmt)[0]), (fmt, c)
        elif np.isinf(val):                       # E5M2 +-inf saturates to +-max
            assert back[c] == (maxc | (c & 0x80))
        else:
            assert back[c] == c, (fmt, hex(c), val, hex(back[c]))
    # non-negative finite codes are ordered by value (the table search relies on it)
    pos = v[: maxc + 1]
    assert np.all(np.diff(pos) > 0)


# ----------------------------------------------------------------- encode: independent arithmetic encoder
def _encode_arith(v, fmt):
    """Round-to-nearest-even by exponent arithmetic (frexp + rint), then pack the bit fields."""
    mbits, emin, bias, maxv = (3, -6, 7, 448.0) if fmt == oracle.E4M3 else (2, -14, 15, 57344.0)
    v = np.asarray(v, np.float64)
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        _, ex = np.frexp(a)
        E = np.maximum(ex - 1, emin)                     # subnormals share the smallest exponent's quantum
        quantum = np.ldexp(1.0, (E - mbits).astype(np.int32))
        r = np.rint(a / quantum) * quantum               # np.rint: ties to even integer (= even mantissa)
        r = np.minimum(r, maxv)                          # saturate
        _, ex2 = np.frexp(np.where(r > 0, r, 1.0))
        E2 = ex2 - 1
        normal = r >= 2.0 ** emin
        mant_n = np.where(normal, r / np.ldexp(1.0, E2.astype(np.int32)) - 1.0, 0) * (1 << mbits)
        mant_s = r / 2.0 ** (emin - mbits)
        code = np.where(normal, ((E2 + bias) << mbits) + np.rint(mant_n).astype(np.int64), np.rint(mant_s).astype(np.int64))
    code = np.where(a >= maxv, int(maxv == 448.0) * 0x7E + int(maxv != 448.0) * 0x7B, code)
    return (code | sign).astype(np.uint8)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_all_bf16_times_all_scales_vs_arithmetic_encoder(fmt):
    """All 65,536 bf16 patterns (finite) divided by every E8M0 scale 2^e, e in [-127, 127]: two encoders agree."""
    bits = np.arange(65536, dtype=np.uint32)
    f32 = (bits << 16).view(np.float32)
    x = f32[np.isfinite(f32)].astype(np.float64)
    for e0 in range(-127, 128, 17):
        es = np.arange(e0, min(e0 + 17, 128))
        v = (x[None, :] * np.ldexp(1.0, -es)[:, None]).reshape(-1)   # exact in double
        assert np.array_equal(oracle.fp8_encode(v, fmt), _encode_arith(v, fmt))


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_random_f32_vs_arithmetic_encoder(fmt):
    rng = np.random.default_rng(7)
    b = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = b.view(np.float32)
    f = f[np.isfinite(f)].astype(np.float64)
    assert np.array_equal(oracle.fp8_encode(f, fmt), _encode_arith(f, fmt))


@pytest.mark.parametrize("fmt,tdtype,maxv", [(oracle.E4M3, torch.float8_e4m3fn, 448.0), (oracle.E5M2, torch.float8_e5m2, 57344.0)])
def test_encode_matches_torch_cast_in_range(fmt, tdtype, maxv):
    """torch's CPU cast rounds to nearest even; its overflow handling differs, so compare in-range values only."""
    rng = np.random.default_rng(3)
    f = (rng.standard_normal(1_000_000) * np.exp(rng.uniform(-12, 7, 1_000_000))).astype(np.float32)
    f = f[np.abs(f) < maxv * (1 + (2 ** -4 if fmt == oracle.E4M3 else 2 ** -3) / 2)]   # below the overflow midpoint
    lib = torch.from_numpy(f).to(tdtype).view(torch.uint8).numpy()
    assert np.array_equal(oracle.fp8_encode(f.astype(np.float64), fmt), lib)


def test_encode_ties_saturation_and_sign():
    E = oracle.E4M3
    # exact midpoints go to the even code
    assert oracle.fp8_encode([2.0 ** -10], E)[0] == 0x00          # between 0 and 2^-9
    assert oracle.fp8_encode([17.0], E)[0] == 0x58                # 16 (0x58) vs 18 (0x59)
    assert oracle.fp8_encode([19.0], E)[0] == 0x5A                # 18 vs 20 (0x5A)
    # saturation at the largest finite value (OLMo Section 11.2 Figure 49 caption), infinities included
    assert oracle.fp8_encode([464.0, 1e9, np.inf, -np.inf], E).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert oracle.fp8_encode([61440.0, np.inf], oracle.E5M2).tolist() == [0x7B, 0x7B]
    # sign of zero is kept
    assert oracle.fp8_encode([-0.0, -2.0 ** -11, 0.0], E).tolist() == [0x80, 0x80, 0x00]
    # NaN stays NaN
    assert np.isnan(oracle.fp8_value(oracle.fp8_encode([np.nan], E), E)[0])


# ----------------------------------------------------------------- bf16 and fp16 conversions vs library routines
def test_bf16_from_f32_matches_torch():
    rng = np.random.default_rng(11)
    b = rng.integers(0, 2 ** 32, size=3_000_000, dtype=np.uint64).astype(np.uint32)
    f = b.view(np.float32)
    f = f[np.isfinite(f)]
    # add exact ties on the 16 dropped bits
    ties = ((rng.integers(0, 2 ** 16, 100_000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    f = np.concatenate([f, ties[np.isfinite(ties)]])
    lib = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_from_f32(f), lib)


def test_f16_from_f32_matches_numpy():
    rng = np.random.default_rng(12)
    b = rng.integers(0, 2 ** 32, size=3_000_000, dtype=np.uint64).astype(np.uint32)
    f = b.view(np.float32)
    f = f[np.isfinite(f)]
    small = (rng.standard_normal(1_000_000) * np.exp(rng.uniform(-25, 12, 1_000_000))).astype(np.float32)
    f = np.concatenate([f, small, np.array([65504, 65519.99, 65520, 2 ** -24, 2 ** -25, 3 * 2 ** -26], np.float32)])
    with np.errstate(over="ignore"):
        lib = f.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_from_f32(f), lib)
    assert oracle.f16_value(0x0001) == 2.0 ** -24 and f"{2.0 ** -24:.3g}" == "5.96e-08"
