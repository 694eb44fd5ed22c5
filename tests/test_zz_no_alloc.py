"""fp8_quantize_pertensor_noalloc (the allocation-free entry point, scratch in the library's own device array)
against fp8_quantize_pertensor (caller workspace), through the C ABI: amax, scale, q and q_t bit for bit, on two
calls in a row, the second with a smaller input (the array keeps the first call's partials), in both formats, plus a
delayed-mode call (scale_in given), a check of the second call against the oracle, and a tensor of more than 2^31
elements checked against the oracle on its last rows."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, need_gpu, say, u16, u8
from mxfp8_precision_numerics_amd import _lib, workloads

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _run(fn_name, x, fmt, scale_in=None):
    rows, cols = x.shape
    q = torch.full((rows, cols), 0xEE, dtype=torch.uint8, device=DEV)
    qt = torch.full((cols, rows), 0xEE, dtype=torch.uint8, device=DEV)
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    scale = torch.zeros(1, dtype=torch.float32, device=DEV)
    lib = _lib.load()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if fn_name == "fp8_quantize_pertensor":
        ws = torch.empty(lib.mxq_workspace_bytes(b"pertensor", rows * cols), dtype=torch.uint8, device=DEV)
        st = lib.fp8_quantize_pertensor(_p(x), rows, cols, fmt, C.c_float(1.0), _p(scale_in), _p(amax), _p(scale),
                                        _p(q), _p(qt), _p(ws), ws.numel(), stream)
    else:
        st = lib.fp8_quantize_pertensor_noalloc(_p(x), rows, cols, fmt, C.c_float(1.0), _p(scale_in), _p(amax),
                                                _p(scale), _p(q), _p(qt), stream)
    assert st == 0, (fn_name, st)
    return amax, scale, q, qt


@pytest.mark.parametrize("fmt", [0, 1])
def test_noalloc_matches_workspace_entry_on_two_calls(fmt):
    need_gpu()
    big = workloads.normal_bf16((4096, 12288), 1.0, 40, 1 + fmt, DEV)        # 2048 partial maxima
    small = workloads.normal_bf16((96, 200), 1e-3, 40, 3 + fmt, DEV)        # one partial
    for x in (big, small):
        say("noalloc per-tensor", fmt, tuple(x.shape))
        ref = _run("fp8_quantize_pertensor", x, fmt)
        got = _run("fp8_quantize_pertensor_noalloc", x, fmt)
        torch.cuda.synchronize()
        for r, g in zip(ref, got):
            assert torch.equal(r.view(torch.uint8), g.view(torch.uint8))
    oa, osc, oq, oqt = oracle.pertensor_quantize(u16(small), oracle.E4M3 if fmt == 0 else oracle.E5M2)
    assert got[0].item() == oa and got[1].item() == osc
    assert np.array_equal(u8(got[2]), oq) and np.array_equal(u8(got[3]), oqt)


def test_noalloc_delayed_scale_and_repeat():
    need_gpu()
    x = workloads.normal_bf16((512, 1024), 1.0, 40, 7, DEV)
    s_in = torch.tensor([3.0], dtype=torch.float32, device=DEV)
    ref = _run("fp8_quantize_pertensor", x, 0, s_in)
    got1 = _run("fp8_quantize_pertensor_noalloc", x, 0, s_in)
    got2 = _run("fp8_quantize_pertensor_noalloc", x[:64], 0, s_in)
    torch.cuda.synchronize()
    for r, g in zip(ref, got1):
        assert torch.equal(r.view(torch.uint8), g.view(torch.uint8))
    assert got1[1].item() == 3.0
    assert torch.equal(got2[2], ref[2][:64])


def test_noalloc_past_2_31_elements():
    """A 66048 x 32768 tensor (2.16e9 elements, its largest magnitude planted at the last element): amax and scale
    equal the oracle's on the last rows (which hold the tensor's amax), and q and q_t of those rows bit for bit."""
    need_gpu()
    rows, cols = 66048, 32768
    say("noalloc per-tensor past 2^31 elements", rows, cols)
    x = workloads.normal_bf16((rows, cols), 1.0, 40, 9, DEV)
    x[-1, -1] = 100.0
    amax, scale, q, qt = _run("fp8_quantize_pertensor_noalloc", x, 0)
    torch.cuda.synchronize()
    r0 = rows - 64
    oa, osc, oq, oqt = oracle.pertensor_quantize(u16(x[r0:]), oracle.E4M3)
    assert oa == 100.0 and amax.item() == oa and np.float32(scale.item()) == osc
    assert np.array_equal(u8(q[r0:]), oq) and np.array_equal(u8(qt[:, r0:]), oqt)
    del x, q, qt
    torch.cuda.empty_cache()
