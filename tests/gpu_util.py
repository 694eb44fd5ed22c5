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
