"""ctypes binding of libmxq.so (the C ABI of include/mxq.h). Argument marshalling only: every step of the path
runs in the gfx950 kernels. If the library is missing this module raises; there is no CPU fallback."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmxq.so")

MXQ_OK = 0
STATUS_NAMES = {0: "MXQ_OK", 1: "MXQ_ERR_NULL", 2: "MXQ_ERR_SHAPE", 3: "MXQ_ERR_ALIGN", 4: "MXQ_ERR_UNSUPPORTED",
                5: "MXQ_ERR_WORKSPACE", 6: "MXQ_ERR_HIP"}

E4M3, E5M2 = 0, 1
RCEIL, FLOOR = 0, 1
PER_TENSOR, MX_BLOCK32 = 0, 1


class AdamHParams(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("step", C.c_int64)]


_P, _I64, _I, _F, _SZ = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_size_t

# name -> (restype, argtypes); the names and order are those of include/mxq.h
SIGNATURES = {
    "mxq_status_string": (C.c_char_p, [_I]),
    "mxq_abi_version": (_I, []),
    "mxq_workspace_bytes": (_SZ, [C.c_char_p, _I64]),
    "mxq_quantize": (_I, [_P, _I64, _I64, _P, _P, _P, _P, _I, _P]),
    "mxq_quantize_ranged": (_I, [_P, _I64, _I64, _P, _P, _P, _P, _I, _P, _P, _P]),
    "scaled_gemm_ranged": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P]),
    "fp8_quantize_pertensor": (_I, [_P, _I64, _I64, _I, _F, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fp8_quantize_pertensor_noalloc": (_I, [_P, _I64, _I64, _I, _F, _P, _P, _P, _P, _P, _P]),
    "scaled_gemm": (_I, [_P, _P, _I, _P, _P, _I, _I64, _I64, _I64, _I, _P, _I64, _P]),
    "scaled_gemm_exact": (_I, [_P, _P, _I, _P, _P, _I, _I64, _I64, _I64, _I, _P, _I64, _P]),
    "scaled_gemm_fp8": (_I, [_P, _P, _I, _P, _P, _I, _I64, _I64, _I64, _I, _P, _I64, _P]),
    "grouped_scaled_gemm": (_I, [_P, _P, _P, _I64, _I64, _P, _P, _I64, _I64, _P, _P]),
    "fp8_adam_step": (_I, [_P, _P, _P, _P, _P, _P, _I64, C.POINTER(AdamHParams), _P, _SZ, _P]),
    "fp8_quantize_pertensor_delayed": (_I, [_P, _I64, _I64, _I, _F, _P, _P, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "fp8_autoscale_cast": (_I, [_P, _I64, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "fp8_requantize_shared": (_I, [_P, _I64, _I, _P, _P, _I64, _I, _P, _P, _P, _P]),
    "swiglu_mx_quantize": (_I, [_P, _I64, _I64, _P, _P, _I, _P]),
    "fp8_adam_step_mx_cache": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _I, C.POINTER(AdamHParams),
                                    _P, _SZ, _P]),
    "fp8_adam_step_delayed": (_I, [_P, _P, _P, _P, _P, _P, _I64, C.POINTER(AdamHParams), _P, _P, _I64, _P, _SZ, _P]),
    "swiglu_mx_quantize_oriented": (_I, [_P, _I64, _I64, _P, _P, _P, _P, _I, _P]),
    "route_weighted_mx_quantize": (_I, [_P, _P, _I64, _I64, _P, _P, _P, _P, _I, _P]),
    "swiglu_backward_mx_quantize": (_I, [_P, _P, _I64, _I64, _P, _P, _P, _P, _I, _P]),
    "grouped_scaled_gemm_strided": (_I, [_P, _P, _P, _I64, _I64, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P,
                                         _I64, _P]),
    "grouped_wgrad_mx": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P]),
}

_lib = None


def load():
    """Load libmxq.so (built in-tree by __graft_entry__.build() or mxfp8_precision_numerics_amd._build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class MXQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().mxq_status_string(status).decode()
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != MXQ_OK:
        raise MXQError(fn, status)
