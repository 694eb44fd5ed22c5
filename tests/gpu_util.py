"""Helpers for the GPU parity tests: device selection, host copies and a per-step progress print."""
import sys

import numpy as np
import pytest
import torch

DEV = "cuda:0"


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def say(*a):
    print("[gpu-test]", *a, file=sys.stderr, flush=True)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def from_u16(a: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dtype).to(DEV)


def any_wide_window(q, s, fmt_e4m3=True):
    """The FP8 range definition shared by scaled_gemm's check and the quantizers' range words, evaluated plainly on
    the host: q [rows][K] codes, s [rows][K/32] E8M0 bytes (MX) or None (per-tensor). A 64-value window of K is wide
    if it holds a nonzero code and at least 24 of its codes (binade = exponent field + scale byte) lie more than 6
    binades below its largest."""
    q = q.astype(np.int64)
    rows, K = q.shape
    e = (q >> 3) & 15 if fmt_e4m3 else (q >> 2) & 31
    if s is not None:
        e = e + np.repeat(s.astype(np.int64), 32, axis=1)
    w = e.reshape(rows, K // 64, 64)
    nonzero = ((q & 0x7F) != 0).reshape(rows, K // 64, 64).any(axis=2)
    top = w.max(axis=2, keepdims=True)
    small = (w < top - 6).sum(axis=2)
    return bool(((small >= 24) & nonzero).any())
