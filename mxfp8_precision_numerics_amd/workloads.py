"""Seeded synthetic inputs shaped like the workloads on the pages.

This module holds none of the method's arithmetic (no scaling, quantization, GEMM or optimizer math). It only
draws random tensors, so that the GPU path and the CPU oracle can be fed the same bytes. Every tensor is drawn
from its own torch.Generator seeded by (workload id, tensor index), in fp32, scaled by the stated standard
deviation, then rounded to bf16 by torch's cast. Streams differ between CPU and GPU generators, so a test that
compares both sides draws once (usually on the GPU) and hands the same bytes to each.

Workloads (sizes are those of the five configurations; the tests also use smaller shapes with the same recipe):
  1  MX quantize + block-scaled GEMM: A [256][256], B [K=256][N=256], both N(0, 1).
  2  GPT-175B QKV linear (d_model 12288, N = 3 * 12288): X [4096][12288] N(0,1), W [36864][12288] N(0,0.02),
     dY [4096][36864] N(0,1e-3).
  3  MX quantize of an activation [16384][8192] N(0,1) with round(0.001 n) positions, drawn without replacement,
     multiplied by 100 before the bf16 cast.
  4  Grouped expert GEMM: 16384 tokens routed to 8 distinct experts of 64, expert weights proportional to
     rank^-1.1 (Gumbel top-k), each group padded to a multiple of 32 rows (zero rows at the group's end);
     A_up [rows][2048], A_down [rows][1024], W_up [64][1024][2048], W_down [64][2048][1024], all N(0,1); route
     weights (backward of the routed MLP) uniform in [0.01, 1), 0 on padding rows.
  5  Adam step over n parameters: theta fp32 N(0,0.02), gradient bf16 N(0,1e-3) for step t drawn with index t.
  6  FP8 gradient all-reduce pieces: per rank r of 8, the weight gradient of workload 2's W (36864 x 12288 values),
     N(0, 1e-3 * 2^(r/4)) with round(2e-5 n) positions multiplied by 1000 before the bf16 cast (step t: index
     16 t + 2 r, positions 16 t + 2 r + 1).
Wide-range operands (GEMM accuracy tests beyond the normal data of the configurations): N(0,1) values with
  "outliers"    workload 3's recipe (0.1 % of positions x 100),
  "loguniform"  random signs and magnitudes 2^u, u uniform in [-12, 12),
  "colscale"    every column scaled by 2^u, u uniform in [-8, 8),
  "sparse"      90 % of the values zeroed (uniform mask).
"""
from __future__ import annotations

import numpy as np
import torch


def seed_for(workload: int, k: int) -> int:
    return (0x5EED0000 + 1_000_003 * int(workload) + 7919 * int(k)) & 0x7FFFFFFFFFFF


def _gen(workload: int, k: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(workload, k))
    return g


def normal_f32(shape, std: float, workload: int, k: int, device="cpu") -> torch.Tensor:
    g = _gen(workload, k, device)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def uniform_f32(shape, lo: float, hi: float, workload: int, k: int, device="cpu") -> torch.Tensor:
    g = _gen(workload, k, device)
    return torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def normal_bf16(shape, std: float, workload: int, k: int, device="cpu") -> torch.Tensor:
    return normal_f32(shape, std, workload, k, device).to(torch.bfloat16)


WIDE_RANGE_KINDS = ("outliers", "loguniform", "colscale", "sparse")


def wide_range_bf16(shape, kind: str, workload: int, k: int, device="cpu") -> torch.Tensor:
    """A [rows][cols] operand whose 32-value blocks span a wide range of magnitudes (kinds in the module notes)."""
    rows, cols = shape
    if kind == "outliers":
        return normal_bf16_with_outliers(shape, 1.0, 0.001, 100.0, workload, k, k + 1, device)
    x = normal_f32(shape, 1.0, workload, k, device)
    u = _gen(workload, k + 1, device)
    if kind == "loguniform":
        x = torch.sign(x) * torch.exp2(torch.rand(tuple(shape), generator=u, device=device) * 24.0 - 12.0)
    elif kind == "colscale":
        x = x * torch.exp2(torch.rand((1, cols), generator=u, device=device) * 16.0 - 8.0)
    elif kind == "sparse":
        x = x * (torch.rand(tuple(shape), generator=u, device=device) < 0.1)
    else:
        raise ValueError(kind)
    return x.to(torch.bfloat16)


def normal_bf16_with_outliers(shape, std: float, frac: float, factor: float, workload: int, k: int,
                              k_pos: int, device="cpu") -> torch.Tensor:
    x = normal_f32(shape, std, workload, k, device)
    n = x.numel()
    count = int(round(frac * n))
    gp = _gen(workload, k_pos, device)
    pos = torch.randperm(n, generator=gp, device=device)[:count]
    flat = x.view(-1)
    flat[pos] = flat[pos] * factor
    return x.to(torch.bfloat16)


def as_u16(x: torch.Tensor) -> np.ndarray:
    """bf16 / fp16 tensor -> numpy uint16 bit patterns (host copy)."""
    return x.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# ------------------------------------------------------------------ workload 4: routing
def zipf_routing(tokens: int = 16384, experts: int = 64, topk: int = 8, alpha: float = 1.1, pad: int = 32,
                 seed: int | None = None):
    """Per-expert token counts for top-k routing with Zipf(alpha) expert popularity.

    Each token picks `topk` distinct experts without replacement with probability proportional to
    rank^-alpha (Gumbel top-k). Returns (counts[experts], padded_counts[experts], offsets[experts + 1]) with
    every group padded up to a multiple of `pad` rows; expert id = popularity rank.
    """
    rng = np.random.default_rng(seed_for(4, 0) if seed is None else seed)
    logw = -alpha * np.log(np.arange(1, experts + 1, dtype=np.float64))
    keys = logw[None, :] + rng.gumbel(size=(tokens, experts))
    chosen = np.argpartition(-keys, topk - 1, axis=1)[:, :topk]
    counts = np.bincount(chosen.reshape(-1), minlength=experts).astype(np.int64)
    padded = ((counts + pad - 1) // pad) * pad
    offsets = np.zeros(experts + 1, np.int64)
    offsets[1:] = np.cumsum(padded)
    return counts, padded, offsets


def route_weights(counts, padded, offsets, workload: int = 4, k: int = 5, device="cpu") -> torch.Tensor:
    """One fp32 route weight per routed row (expert order), uniform in [0.01, 1); padding rows get 0."""
    p = uniform_f32((int(offsets[-1]),), 0.01, 1.0, workload, k, device)
    return zero_padding_rows(p, counts, padded, offsets)


def zero_padding_rows(a: torch.Tensor, counts, padded, offsets) -> torch.Tensor:
    """Zero the padding rows at the end of each group (in place)."""
    for g in range(len(counts)):
        lo = int(offsets[g]) + int(counts[g])
        hi = int(offsets[g]) + int(padded[g])
        if hi > lo:
            a[lo:hi].zero_()
    return a


# ------------------------------------------------------------------ the five workloads
def workload1(device="cpu", M=256, N=256, K=256):
    A = normal_bf16((M, K), 1.0, 1, 0, device)
    B = normal_bf16((K, N), 1.0, 1, 1, device)       # K x N; column blocks run along K
    return A, B


def workload2(device="cpu", M=4096, N=36864, K=12288):
    X = normal_bf16((M, K), 1.0, 2, 0, device)
    W = normal_bf16((N, K), 0.02, 2, 1, device)
    dY = normal_bf16((M, N), 1e-3, 2, 2, device)
    return X, W, dY


def workload3(device="cpu", rows=16384, cols=8192):
    return normal_bf16_with_outliers((rows, cols), 1.0, 0.001, 100.0, 3, 0, 1, device)


def workload4(device="cpu", tokens=16384, experts=64, topk=8, d_model=2048, d_ff=1024):
    counts, padded, offsets = zipf_routing(tokens, experts, topk)
    rows = int(offsets[-1])
    a_up = zero_padding_rows(normal_bf16((rows, d_model), 1.0, 4, 1, device), counts, padded, offsets)
    a_down = zero_padding_rows(normal_bf16((rows, d_ff), 1.0, 4, 2, device), counts, padded, offsets)
    w_up = normal_bf16((experts, d_ff, d_model), 1.0, 4, 3, device)
    w_down = normal_bf16((experts, d_model, d_ff), 1.0, 4, 4, device)
    return dict(counts=counts, padded=padded, offsets=offsets, a_up=a_up, a_down=a_down, w_up=w_up, w_down=w_down)


def workload5_params(n: int, device="cpu") -> torch.Tensor:
    return normal_f32((n,), 0.02, 5, 0, device)


def workload5_grad(n: int, t: int, device="cpu") -> torch.Tensor:
    return normal_bf16((n,), 1e-3, 5, t, device)


def workload6_grad(n: int, rank: int, t: int = 0, device="cpu") -> torch.Tensor:
    k = 16 * int(t) + 2 * int(rank)
    return normal_bf16_with_outliers((n,), 1e-3 * 2.0 ** (rank / 4), 2e-5, 1000.0, 6, k, k + 1, device)
