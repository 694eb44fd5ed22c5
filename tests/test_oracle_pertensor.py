"""Pins for the oracle's per-tensor current scaling (FP8-LM tensor scaling; llm-stack-book 3.8 per-tensor scaling
and Exercise 6): s = (FMAX / max(amax, 1e-12)) * margin in fp32, q = FP8(fp32(x * s)), x ~ q / s."""
import numpy as np
import pytest

import oracle
from mxfp8_precision_numerics_amd import workloads


@pytest.mark.parametrize("fmt,fmax", [(oracle.E4M3, 448.0), (oracle.E5M2, 57344.0)])
def test_scale_matches_numpy_float32_and_amax_maps_to_fmax(fmt, fmax):
    x = workloads.as_u16(workloads.normal_bf16((64, 96), 0.02, 95, 0))
    amax, s, q, qt = oracle.pertensor_quantize(x, fmt)
    xf = oracle.bf16_to_f32(x)
    assert amax == float(np.abs(xf).max())
    assert s == np.float32(fmax) / np.float32(amax)                    # one IEEE fp32 division
    i = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
    maxc = 0x7E if fmt == oracle.E4M3 else 0x7B
    assert q[i] & 0x7F == maxc                                        # the amax element lands on +-FMAX
    assert np.array_equal(qt, q.T)
    # every element: fp32 product then FP8 (a library-free restatement: numpy float32 multiply, exact encode)
    p = (xf * np.float32(s)).astype(np.float32).astype(np.float64)
    assert np.array_equal(q, oracle.fp8_encode(p, fmt))


def test_dequantized_error_within_unit_roundoff():
    x = workloads.as_u16(workloads.normal_bf16((128, 128), 1.0, 94, 0))
    amax, s, q, _ = oracle.pertensor_quantize(x, oracle.E4M3)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    xh = oracle.fp8_value(q, oracle.E4M3) / float(s)
    normal = np.abs(xf) * float(s) >= 2.0 ** -6
    assert np.all(np.abs(xh - xf)[normal] <= 2.0 ** -4 * np.abs(xf)[normal] * (1 + 2 ** -20))


def test_zero_tensor_margin_and_delayed_scale():
    z = np.zeros((32, 32), np.uint16)
    amax, s, q, _ = oracle.pertensor_quantize(z, oracle.E4M3)
    assert amax == 0.0 and s == np.float32(448.0) / np.float32(1e-12) and np.all(q == 0)
    x = workloads.as_u16(workloads.normal_bf16((32, 64), 1.0, 93, 0))
    _, s1, _, _ = oracle.pertensor_quantize(x, oracle.E4M3, margin=0.5)
    _, s0, _, _ = oracle.pertensor_quantize(x, oracle.E4M3)
    assert s1 == np.float32(s0) * np.float32(0.5)
    # delayed mode: the given scale is used, amax still reported, values above FMAX saturate
    amax, s, q, _ = oracle.pertensor_quantize(x, oracle.E4M3, scale_in=1000.0)
    assert s == np.float32(1000.0) and amax == float(np.abs(oracle.bf16_to_f32(x)).max())
    assert np.any(q & 0x7F == 0x7E)
    assert not np.any(q & 0x7F == 0x7F)
