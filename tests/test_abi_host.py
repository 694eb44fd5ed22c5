"""Host-side checks of the C ABI (no GPU needed): libmxq.so loads, exports every function include/mxq.h declares,
and argument validation returns the documented status codes before anything is enqueued. Only inputs that fail
validation are passed here (fake, aligned pointer values are never dereferenced)."""
import ctypes as C
import os
import re

import pytest

from conftest import ROOT
from mxfp8_precision_numerics_amd import _lib

HEADER = os.path.join(ROOT, "include", "mxq.h")
PROBE_HEADER = os.path.join(ROOT, "include", "mxq_probe.h")
P = 0x10000          # a fake 16-byte-aligned address: validation rejects before any use
MIS = 0x10001        # misaligned


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)) - {"defined"})


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_measurement_library_is_apart_from_the_method_library():
    """The measurement kernels live in libmxq_probe.so (include/mxq_probe.h), not in the method's library."""
    from mxfp8_precision_numerics_amd import _probe
    lib, probe = _lib.load(), _probe.load()
    names = declared_functions(PROBE_HEADER)
    assert set(names) == set(_probe.SIGNATURES), names
    for n in names:
        assert hasattr(probe, n), n
        assert not hasattr(lib, n), n
        assert n not in declared_functions()


def test_status_strings_and_version():
    lib = _lib.load()
    assert lib.mxq_abi_version() == 1
    for s in range(7):
        assert lib.mxq_status_string(s)
    assert lib.mxq_status_string(99) == b"unknown status"


def test_workspace_sizes():
    lib = _lib.load()
    assert lib.mxq_workspace_bytes(b"pertensor", 16384 * 8192) >= 4
    assert lib.mxq_workspace_bytes(b"adam", 1_300_000_000) >= 4 * 16
    assert lib.mxq_workspace_bytes(b"nope", 10) == 0
    assert lib.mxq_workspace_bytes(b"adam", -1) == 0


def test_mx_quantize_validation():
    f = _lib.load().mxq_quantize
    ok = 0
    assert f(None, 64, 64, P, P, P, P, 0, None) == 1                  # NULL x
    assert f(P, 64, 64, None, None, None, None, 0, None) == 1         # no orientation requested
    assert f(P, 64, 64, P, None, None, None, 0, None) == 1            # q_row without s_row
    assert f(P, 64, 48, P, P, None, None, 0, None) == 2               # row orientation needs cols % 32
    assert f(P, 48, 64, None, None, P, P, 0, None) == 2               # col orientation needs rows % 32
    assert f(P, 64, 36, None, None, P, P, 0, None) == 2               # cols % 8
    assert f(P, -32, 64, P, P, None, None, 0, None) == 2
    assert f(P, 64, 64, P, P, None, None, 7, None) == 4               # unknown rule
    assert f(MIS, 64, 64, P, P, None, None, 0, None) == 3
    assert f(P, 64, 64, MIS, P, None, None, 0, None) == 3
    assert f(P, 0, 64, P, P, P, P, 0, None) == ok                      # empty: nothing enqueued


def test_pertensor_validation():
    f = _lib.load().fp8_quantize_pertensor
    ws = _lib.load().mxq_workspace_bytes(b"pertensor", 64 * 64)
    assert f(P, 64, 64, 0, C.c_float(1.0), None, None, P, P, P, P, ws, None) == 1
    assert f(P, 64, 64, 2, C.c_float(1.0), None, P, P, P, P, P, ws, None) == 4
    assert f(P, 48, 64, 0, C.c_float(1.0), None, P, P, P, P, P, ws, None) == 2    # q_t needs rows % 32
    assert f(P, 64, 64, 0, C.c_float(1.0), None, P, P, P, P, None, ws, None) == 5
    assert f(P, 64, 64, 0, C.c_float(1.0), None, P, P, P, P, P, ws - 1, None) == 5
    assert f(MIS, 64, 64, 0, C.c_float(1.0), None, P, P, P, P, P, ws, None) == 3


@pytest.mark.parametrize("name", ["scaled_gemm", "scaled_gemm_exact", "scaled_gemm_fp8"])
def test_gemm_validation(name):
    f = getattr(_lib.load(), name)
    assert f(None, P, 0, P, P, 0, 64, 64, 64, 1, P, 64, None) == 1
    assert f(P, P, 0, P, P, 0, 64, 64, 48, 1, P, 64, None) == 2        # K % 32
    assert f(P, P, 0, P, P, 0, 64, 64, 0, 1, P, 64, None) == 2         # K > 0
    assert f(P, P, 0, P, P, 0, 64, 64, 64, 1, P, 32, None) == 2        # ldc < N
    assert f(P, P, 0, P, P, 0, 64, 64, 64, 1, P + 1, 64, None) == 3    # C must be 2-byte aligned
    assert f(P, P, 1, P, P, 0, 64, 64, 64, 1, P, 64, None) == 4        # MX needs E4M3
    assert f(P, P, 0, P, P, 0, 64, 64, 64, 5, P, 64, None) == 4
    assert f(P, P, 0, MIS, P, 0, 64, 64, 64, 1, P, 64, None) == 3
    assert f(P, P, 0, P, P, 0, 0, 64, 64, 1, P, 64, None) == 0         # empty


def test_grouped_and_adam_validation():
    lib = _lib.load()
    g = lib.grouped_scaled_gemm
    assert g(P, P, None, 4, 128, P, P, 64, 64, P, None) == 1
    assert g(P, P, P, 0, 128, P, P, 64, 64, P, None) == 2
    assert g(P, P, P, 4, 128, P, P, 64, 40, P, None) == 2
    assert g(P, P, P + 4, 4, 128, P, P, 64, 64, P, None) == 3
    hp = _lib.AdamHParams(3e-4, 0.9, 0.95, 1e-8, 0.0, 0)
    ws = lib.mxq_workspace_bytes(b"adam", 1024)
    a = lib.fp8_adam_step
    assert a(P, P, P, P, P, None, 1024, C.byref(hp), P, ws, None) == 2          # step must be >= 1
    hp.step = 1
    assert a(P, P, P, P, P, None, 1024, None, P, ws, None) == 1
    assert a(P, P, P, P, P, None, 1024, C.byref(hp), P, ws - 1, None) == 5
    assert a(P, MIS, P, P, P, None, 1024, C.byref(hp), P, ws, None) == 3


def test_delayed_validation():
    lib = _lib.load()
    f = lib.fp8_quantize_pertensor_delayed
    ws = lib.mxq_workspace_bytes(b"pertensor_delayed", 64 * 64)
    assert ws >= 4
    assert f(P, 64, 64, 0, C.c_float(1.0), None, P, 4, P, P, P, P, P, ws, None) == 1     # no history
    assert f(P, 64, 64, 0, C.c_float(1.0), P, P, 0, P, P, P, P, P, ws, None) == 2        # history_len >= 1
    assert f(P, 64, 64, 3, C.c_float(1.0), P, P, 4, P, P, P, P, P, ws, None) == 4
    assert f(P, 64, 64, 0, C.c_float(1.0), P, P, 4, P, P, P, P, None, ws, None) == 5
    assert f(P, 64, 64, 0, C.c_float(1.0), P + 2, P, 4, P, P, P, P, P, ws, None) == 3    # history 4-aligned
    g = lib.fp8_adam_step_delayed
    hp = _lib.AdamHParams(3e-4, 0.9, 0.95, 1e-8, 0.0, 1)
    wsa = lib.mxq_workspace_bytes(b"adam_delayed", 1024)
    assert g(P, P, P, P, P, None, 1024, C.byref(hp), None, P, 4, P, wsa, None) == 1
    assert g(P, P, P, P, P, None, 1024, C.byref(hp), P, P, 0, P, wsa, None) == 2
    assert g(P, P, P, P, P, None, 1024, C.byref(hp), P, P, 4, P, wsa - 1, None) == 5
    assert g(P, P, P, P, P, None, 0, C.byref(hp), None, None, 4, None, 0, None) == 0     # empty


def test_weight_cache_validation():
    lib = _lib.load()
    f = lib.fp8_adam_step_mx_cache
    hp = _lib.AdamHParams(3e-4, 0.9, 0.95, 1e-8, 0.0, 1)
    ws = lib.mxq_workspace_bytes(b"adam", 64 * 64)
    assert f(P, P, P, P, P, None, 64, 64, None, None, None, None, 0, C.byref(hp), P, ws, None) == 1   # no cache
    assert f(P, P, P, P, P, None, 64, 64, P, None, None, None, 0, C.byref(hp), P, ws, None) == 1      # q without s
    assert f(P, P, P, P, P, None, 64, 48, P, P, None, None, 0, C.byref(hp), P, ws, None) == 2         # cols % 32
    assert f(P, P, P, P, P, None, 48, 64, None, None, P, P, 0, C.byref(hp), P, ws, None) == 2         # rows % 32
    assert f(P, P, P, P, P, None, 64, 64, P, P, P, P, 9, C.byref(hp), P, ws, None) == 4
    assert f(P, P, P, P, P, None, 64, 64, P, P, P, P, 0, C.byref(hp), P, ws - 1, None) == 5
    assert f(P, P, P, P, P, None, 64, 64, MIS, P, P, P, 0, C.byref(hp), P, ws, None) == 3
    assert f(P, P, P, P, P, None, 0, 64, P, P, P, P, 0, C.byref(hp), None, 0, None) == 0              # empty


def test_swiglu_validation():
    f = _lib.load().swiglu_mx_quantize
    assert f(P, 64, 48, P, P, 0, None) == 2          # F % 32
    assert f(P, 64, 64, P, P, 3, None) == 4
    assert f(None, 64, 64, P, P, 0, None) == 1
    assert f(MIS, 64, 64, P, P, 0, None) == 3
    assert f(None, 0, 64, None, None, 0, None) == 0   # empty


def test_gradcomm_validation():
    lib = _lib.load()
    f = lib.fp8_autoscale_cast
    assert f(P, 64, 2, P, P, P, P, P, 256, None) == 4           # unsupported format
    assert f(P, -1, 0, P, P, P, P, P, 256, None) == 2
    assert f(P, 64, 0, None, P, P, P, P, 256, None) == 1        # mu
    assert f(None, 64, 0, P, P, P, P, P, 256, None) == 1
    assert f(P, 64, 0, P, P, P, P, P, 8, None) == 5             # workspace too small
    assert f(P, 64, 0, P, P, P, P + 4, P, 256, None) == 3       # overflow counter not 8-byte aligned
    assert f(MIS, 64, 0, P, P, P, P, P, 256, None) == 3
    assert lib.mxq_workspace_bytes(b"autoscale", 1 << 20) >= 8
    r = lib.fp8_requantize_shared
    assert r(P, 64, 0, P, P, 0, 0, P, P, P, None) == 2          # no ranks
    assert r(P, 64, 0, P, P, 8, 5, P, P, P, None) == 4
    assert r(P, 64, 0, None, P, 8, 0, P, P, P, None) == 1
    assert r(None, 64, 0, P, P, 8, 0, P, P, P, None) == 1
    assert r(P, 64, 0, P, P, 8, 0, MIS, P, P, None) == 3


def test_probe_validation():
    from mxfp8_precision_numerics_amd import _probe
    f = _probe.load().mxq_probe_mfma_fp8
    assert f(None, 10, 4, P, None) == 1
    assert f(P, 10, 4, None, None) == 1
    assert f(P, 0, 4, P, None) == 2
    assert f(P, 10, 0, P, None) == 2
    assert f(P, 10, 70000, P, None) == 2
    assert f(MIS, 10, 4, P, None) == 3
    c = _probe.load().mxq_probe_copy
    assert c(P, P, 24, 4, 4, None) == 2                 # bytes % 16
    assert c(P, P, 32, -1, 4, None) == 2
    assert c(P, P, 32, 4, 5, None) == 2                 # unroll 4, 8 or 16
    assert c(None, P, 32, 4, 4, None) == 1
    assert c(MIS, P, 32, 4, 8, None) == 3
    assert c(None, None, 0, 4, 16, None) == 0           # empty
    r = _probe.load().mxq_probe_read
    assert r(P, 24, 0, 8, P, None) == 2
    assert r(P, 32, 0, 3, P, None) == 2
    assert r(P, 32, 0, 8, None, None) == 1
    assert r(None, 32, 0, 8, P, None) == 1
    assert r(MIS, 32, 0, 8, P, None) == 3
    assert r(None, 0, 0, 8, P, None) == 0
    d = _probe.load().mxq_probe_read_lds
    assert d(P, 65536 + 16, 4, P, None) == 2             # whole 64 KiB pieces only
    assert d(P, -65536, 4, P, None) == 2
    assert d(P, 65536, 0, P, None) == 2                  # 1 <= blocks <= 65536
    assert d(P, 65536, 70000, P, None) == 2
    assert d(P, 65536, 4, None, None) == 1
    assert d(None, 65536, 4, P, None) == 1
    assert d(MIS, 65536, 4, P, None) == 3


def test_routed_backward_validation():
    lib = _lib.load()
    for f in (lib.route_weighted_mx_quantize, lib.swiglu_backward_mx_quantize):
        assert f(P, P, 64, 64, None, None, None, None, 0, None) == 1          # no orientation
        assert f(P, P, 64, 64, P, None, None, None, 0, None) == 1             # q_row without s_row
        assert f(P, P, 64, 48, P, P, None, None, 0, None) == 2                # cols / F % 32
        assert f(P, P, 48, 64, P, P, None, None, 0, None) == 2                # rows % 32, also for the row orientation
        assert f(P, P, 64, 64, P, P, P, P, 5, None) == 4
        assert f(P, None, 64, 64, P, P, P, P, 0, None) == 1
        assert f(MIS, P, 64, 64, P, P, P, P, 0, None) == 3
        assert f(P, P, 64, 64, P, P, MIS, P, 0, None) == 3
        assert f(None, None, 0, 64, P, P, P, P, 0, None) == 0                 # empty: nothing enqueued
    assert lib.route_weighted_mx_quantize(P, P + 2, 64, 64, P, P, P, P, 0, None) == 3   # weights 4-byte aligned
    s = lib.swiglu_mx_quantize_oriented
    assert s(P, 64, 64, None, None, None, None, 0, None) == 1
    assert s(P, 64, 48, P, P, P, P, 0, None) == 2
    assert s(P, 48, 64, P, P, P, P, 0, None) == 2
    assert s(P, 64, 64, P, P, P, P, 2, None) == 4
    assert s(None, 64, 64, P, P, P, P, 0, None) == 1
    assert s(MIS, 64, 64, P, P, P, P, 0, None) == 3
    assert s(None, 0, 64, P, P, P, P, 0, None) == 0


def test_grouped_strided_and_wgrad_validation():
    lib = _lib.load()
    g = lib.grouped_scaled_gemm_strided
    #        a_q a_s off G  rows b_q b_s ldb  bgs  ldbs bsgs N   K   c  ldc
    assert g(P, P, None, 4, 128, P, P, 256, 64, 8, 2, 64, 64, P, 64, None) == 1
    assert g(P, P, P, 4, 128, P, P, 32, 64, 8, 2, 64, 64, P, 64, None) == 2             # ldb < K
    assert g(P, P, P, 4, 128, P, P, 256, 64, 1, 2, 64, 64, P, 64, None) == 2            # ldbs < K/32
    assert g(P, P, P, 4, 128, P, P, 256, 64, 8, 2, 64, 64, P, 32, None) == 2            # ldc < N
    assert g(P, P, P, 4, 128, P, P, 256, -64, 8, 2, 64, 64, P, 64, None) == 2           # negative group stride
    assert g(P, P, P, 4, 128, P, P, 264, 64, 8, 2, 64, 64, P, 64, None) == 3            # ldb % 16
    assert g(P, P, P, 4, 128, P, P, 256, 72, 8, 2, 64, 64, P, 64, None) == 3            # group stride % 16
    assert g(P, P, P, 4, 128, P, P, 256, 64, 8, 2, 64, 40, P, 64, None) == 2            # K % 32
    assert g(P, P, P + 4, 4, 128, P, P, 256, 64, 8, 2, 64, 64, P, 64, None) == 3
    assert g(P, P, P, 4, 0, P, P, 256, 64, 8, 2, 64, 64, P, 64, None) == 0              # no rows: nothing enqueued
    w = lib.grouped_wgrad_mx
    #        a_q a_s b_q b_s off G  M   N   Kt   c     cf
    assert w(P, P, P, P, P, 4, 64, 64, 128, None, None, None) == 1                      # no output
    assert w(P, P, P, P, P, 4, 64, 64, 128, P, P, None) == 1                            # two outputs
    assert w(P, P, P, P, None, 4, 64, 64, 128, P, None, None) == 1
    assert w(P, P, P, P, P, 0, 64, 64, 128, P, None, None) == 2
    assert w(P, P, P, P, P, 4, 0, 64, 128, P, None, None) == 2
    assert w(P, P, P, P, P, 4, 64, 64, 48, P, None, None) == 2                          # Kt % 32
    assert w(None, P, P, P, P, 4, 64, 64, 128, P, None, None) == 1
    assert w(MIS, P, P, P, P, 4, 64, 64, 128, P, None, None) == 3
    assert w(P, P, P, P, P + 4, 4, 64, 64, 128, P, None, None) == 3


@pytest.mark.parametrize("b1,b2", [(1.0, 0.95), (0.9, 1.0), (-0.1, 0.95), (0.9, -1e-30), (float("nan"), 0.95),
                                   (0.9, float("inf"))])
def test_adam_betas_outside_unit_interval_rejected(b1, b2):
    """Adam's bias corrections divide by 1 - beta^t, so each beta must lie in [0, 1). The check precedes the early
    return for an empty tensor, so it is exercised here with n == 0 and no device call."""
    lib = _lib.load()
    hp = _lib.AdamHParams(3e-4, b1, b2, 1e-8, 0.0, 5)
    assert lib.fp8_adam_step(None, None, None, None, None, None, 0, C.byref(hp), None, 0, None) == 4
    assert lib.fp8_adam_step_delayed(None, None, None, None, None, None, 0, C.byref(hp), None, None, 4, None, 0,
                                     None) == 4
    assert lib.fp8_adam_step_mx_cache(None, None, None, None, None, None, 0, 64, P, P, None, None, 0, C.byref(hp),
                                      None, 0, None) == 4
    ok = _lib.AdamHParams(3e-4, 0.0, 0.999, 1e-8, 0.0, 5)                  # 0 is allowed
    assert lib.fp8_adam_step(None, None, None, None, None, None, 0, C.byref(ok), None, 0, None) == 0
    assert lib.mxq_status_string(4).decode().endswith("optimizer setting")
