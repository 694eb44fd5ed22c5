"""Host-side checks of the Python binding (no GPU needed): the wrappers refuse host tensors, wrong dtypes and
non-contiguous views before any library call, and a missing library raises instead of falling back to anything.
Nothing here launches a kernel."""
import os

import pytest
import torch

import mxfp8_precision_numerics_amd as mxq
from mxfp8_precision_numerics_amd import _lib


def test_wrappers_refuse_host_tensors():
    x = torch.zeros((64, 64), dtype=torch.bfloat16)
    u = torch.zeros((64, 64), dtype=torch.uint8)
    calls = [
        lambda: mxq.mx_quantize(x),
        lambda: mxq.pertensor_quantize(x),
        lambda: mxq.swiglu_mx_quantize(x),
        lambda: mxq.swiglu_mx_quantize_oriented(x),
        lambda: mxq.route_weighted_mx_quantize(x, torch.ones(64)),
        lambda: mxq.swiglu_backward_mx_quantize(x, x[:, :32].contiguous()),
        lambda: mxq.scaled_gemm(u, torch.ones(1), u, torch.ones(1), mxq.PER_TENSOR),
        lambda: mxq.grouped_scaled_gemm(u, u, torch.zeros(2, dtype=torch.int64), u.view(1, 64, 64), u),
        lambda: mxq.grouped_wgrad_mx(u, u[:, :2].contiguous(), u, u[:, :2].contiguous(),
                                     torch.zeros(2, dtype=torch.int64)),
        lambda: mxq.fp8_adam_step(torch.zeros(8), torch.zeros(8, dtype=torch.bfloat16),
                                  torch.zeros(8, dtype=torch.uint8), torch.ones(1), torch.zeros(8, dtype=torch.float16),
                                  None, mxq.AdamHParams(3e-4, 0.9, 0.95, 1e-8, 0.0, 1)),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="device tensor"):
            call()


def test_missing_library_raises(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "LIB_PATH", os.path.join(str(tmp_path), "absent.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


def test_status_errors_carry_names():
    err = _lib.MXQError("scaled_gemm", 2)
    assert "MXQ_ERR_SHAPE" in str(err) and err.status == 2
    with pytest.raises(_lib.MXQError):
        _lib.check("mxq_quantize", 3)
    _lib.check("mxq_quantize", 0)
