"""ctypes binding of libmxq_probe.so (include/mxq_probe.h): the measurement kernels that give the ceilings this part
sustains (a streaming copy, a streaming read, an MFMA-only loop). Not a step of the method; only the benchmark and
its tests use it. Raises if the library is missing."""
from __future__ import annotations

import ctypes as C
import os

import torch

from . import _lib

LIB_PATH = os.path.join(_lib.PKG, "libmxq_probe.so")

_P, _I64, _I = C.c_void_p, C.c_int64, C.c_int
SIGNATURES = {
    "mxq_probe_mfma_fp8": (_I, [_P, _I64, _I64, _P, _P]),
    "mxq_probe_copy": (_I, [_P, _P, _I64, _I64, _I64, _P]),
    "mxq_probe_read": (_I, [_P, _I64, _I64, _I64, _P, _P]),
    "mxq_probe_read_lds": (_I, [_P, _I64, _I64, _P, _P]),
}

_lib_probe = None


def load():
    global _lib_probe
    if _lib_probe is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
        _lib.load()                       # status strings come from libmxq.so
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib_probe = lib
    return _lib_probe


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def mfma_fp8(operand_bytes: torch.Tensor, iters: int, blocks: int, sink: torch.Tensor = None) -> int:
    """Enqueue the MFMA-only loop; returns the FLOP it performs (time it with events on the stream)."""
    if not (operand_bytes.is_cuda and operand_bytes.dtype == torch.uint8 and operand_bytes.is_contiguous()):
        raise ValueError("operand_bytes must be a contiguous uint8 device tensor")
    if operand_bytes.numel() < 131072:
        raise ValueError("operand_bytes must hold at least 131072 bytes")
    dev = operand_bytes.device
    if sink is None:
        sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    _lib.check("mxq_probe_mfma_fp8", load().mxq_probe_mfma_fp8(_ptr(operand_bytes), iters, blocks, _ptr(sink),
                                                               _stream(dev)))
    return blocks * 4 * iters * 16 * 131072


def _bytes(t: torch.Tensor) -> int:
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError("probe buffers must be contiguous device tensors")
    return t.numel() * t.element_size()


def copy(src: torch.Tensor, dst: torch.Tensor, blocks: int = 4096, unroll: int = 4) -> int:
    """Enqueue dst = src (same byte size); blocks = 0 is one workgroup per piece. Returns the bytes moved (read +
    written)."""
    nbytes = _bytes(src)
    if _bytes(dst) != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    _lib.check("mxq_probe_copy", load().mxq_probe_copy(_ptr(src), _ptr(dst), nbytes, blocks, unroll,
                                                       _stream(src.device)))
    return 2 * nbytes


def read(src: torch.Tensor, sink: torch.Tensor, blocks: int = 0, unroll: int = 8) -> int:
    """Enqueue a streaming read of src (one xor word per workgroup into sink, uint32). Returns the bytes read."""
    nbytes = _bytes(src)
    if not (sink.is_cuda and sink.dtype == torch.int32):
        raise ValueError("sink must be an int32 device tensor")
    groups = blocks if blocks > 0 else nbytes // (4096 * unroll) + 1
    if sink.numel() < groups:
        raise ValueError(f"sink needs {groups} entries")
    _lib.check("mxq_probe_read", load().mxq_probe_read(_ptr(src), nbytes, blocks, unroll, _ptr(sink),
                                                       _stream(src.device)))
    return nbytes


def read_lds(src: torch.Tensor, sink: torch.Tensor, blocks: int = 256) -> int:
    """Enqueue a streaming read of src into LDS through the GEMM's global-to-LDS copy instruction (one xor word per
    workgroup into sink, int32[blocks]). src holds a whole number of 64 KiB pieces. Returns the bytes read."""
    nbytes = _bytes(src)
    if not (sink.is_cuda and sink.dtype == torch.int32) or sink.numel() < blocks:
        raise ValueError(f"sink must be an int32 device tensor of at least {blocks} entries")
    _lib.check("mxq_probe_read_lds", load().mxq_probe_read_lds(_ptr(src), nbytes, blocks, _ptr(sink),
                                                               _stream(src.device)))
    return nbytes
