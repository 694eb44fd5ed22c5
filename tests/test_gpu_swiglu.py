"""GPU parity of swiglu_mx_quantize against the oracle: codes and scale bytes of silu(gate) * up, byte for byte,
from small and ragged shapes up to the routed experts' hidden size of the grouped workload (132,160 rows, F = 1024)."""
import numpy as np
import pytest
import torch

import mxfp8_precision_numerics_amd as mxq
import oracle
from gpu_util import DEV, need_gpu, say, u16, u8
from mxfp8_precision_numerics_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,F,std,rule", [(1, 32, 1.0, mxq.RCEIL), (37, 96, 10.0, mxq.RCEIL),
                                             (256, 512, 45.0, mxq.FLOOR), (132_160, 1024, 45.0, mxq.RCEIL)])
def test_swiglu_quantize(rows, F, std, rule):
    need_gpu()
    say("swiglu", rows, F, std, rule)
    c = workloads.normal_bf16((rows, 2 * F), std, 4, 40, DEV)
    out = mxq.swiglu_mx_quantize(c, rule)
    torch.cuda.synchronize()
    q, s, _ = oracle.swiglu_mx_quantize(u16(c), rule)
    assert np.array_equal(u8(out.s_row), s)
    assert np.array_equal(u8(out.q_row), q)


def test_swiglu_extremes():
    need_gpu()
    vals = np.array([0.0, -0.0, 1e-30, -1e-30, 88.0, 89.0, -88.0, -104.5, 200.0, -200.0, 3.0e38, -3.0e38,
                     np.inf, -np.inf, 1.0, -1.0], np.float32)
    rows, F = 16, 64
    g = np.resize(vals, (rows, F)).astype(np.float32)
    u = np.resize(vals[::-1], (rows, F)).astype(np.float32)
    c = oracle.bf16_from_f32(np.concatenate([g, u], axis=1))
    ct = torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).to(DEV)
    out = mxq.swiglu_mx_quantize(ct)
    torch.cuda.synchronize()
    q, s, _ = oracle.swiglu_mx_quantize(c)
    assert np.array_equal(u8(out.s_row), s) and np.array_equal(u8(out.q_row), q)
