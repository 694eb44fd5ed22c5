"""FP8 / MXFP8 training numerics on MI355X (gfx950).

The functions below take torch tensors (PyTorch supplies device memory and the current HIP stream), allocate the
outputs, and call the C ABI of libmxq.so with raw pointers. All arithmetic happens in the library's gfx950 kernels.

  mx_quantize            MXFP8 row/column quantization (E4M3 payload, E8M0 scale per 32 values)
  pertensor_quantize     per-tensor current/delayed scaling to E4M3 or E5M2 (+ transposed copy)
  scaled_gemm            C = A B^T with FP8 operands (per-tensor or MX block scales), fp32 accumulate, bf16 out
  grouped_scaled_gemm    the MX GEMM over ragged expert row groups (and a strided-B form for the routed dgrad)
  grouped_wgrad_mx       the routed Wgrad: one MX contraction per expert over its token rows
  fp8_adam_step          precision-decoupled FP8 AdamW step (fp32 master, E4M3 m + scale, fp16 v, bf16 copy)
  swiglu_mx_quantize(_oriented), swiglu_backward_mx_quantize, route_weighted_mx_quantize
                         the routed MLP's fused elementwise + MX quantize steps (forward and backward)
"""
from __future__ import annotations

import ctypes as C
from typing import NamedTuple, Optional

import torch

from . import _lib
from ._lib import E4M3, E5M2, FLOOR, MX_BLOCK32, PER_TENSOR, RCEIL, AdamHParams, MXQError  # noqa: F401

__all__ = ["mx_quantize", "mx_quantize_ranged", "pertensor_quantize", "scaled_gemm", "scaled_gemm_ranged", "grouped_scaled_gemm", "fp8_adam_step",
           "swiglu_mx_quantize", "swiglu_mx_quantize_oriented", "swiglu_backward_mx_quantize", "route_weighted_mx_quantize",
           "grouped_scaled_gemm_strided", "grouped_wgrad_mx",
           "workspace_bytes", "MXTensor", "AdamHParams", "MXQError", "E4M3", "E5M2", "RCEIL", "FLOOR",
           "PER_TENSOR", "MX_BLOCK32"]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class MXTensor(NamedTuple):
    """One MXFP8 tensor in both orientations: qdata and E8M0 scales travel together (either pair may be None)."""
    q_row: Optional[torch.Tensor]   # [rows][cols] uint8, blocks of 32 along each row
    s_row: Optional[torch.Tensor]   # [rows][cols/32] uint8
    q_col: Optional[torch.Tensor]   # [cols][rows] uint8, blocks of 32 down each column, stored transposed
    s_col: Optional[torch.Tensor]   # [cols][rows/32] uint8


def workspace_bytes(op: str, n: int) -> int:
    return int(_lib.load().mxq_workspace_bytes(op.encode(), int(n)))


def mx_quantize(x: torch.Tensor, rowwise: bool = True, colwise: bool = True, rule: int = RCEIL,
                out: Optional[MXTensor] = None) -> MXTensor:
    _dev(x, torch.bfloat16, "x")
    rows, cols = x.shape
    if out is None:
        dev = x.device
        e = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
        out = MXTensor(e(rows, cols) if rowwise else None, e(rows, cols // 32) if rowwise else None,
                       e(cols, rows) if colwise else None, e(cols, rows // 32) if colwise else None)
    st = _lib.load().mxq_quantize(_ptr(x), rows, cols, _ptr(out.q_row), _ptr(out.s_row), _ptr(out.q_col),
                                  _ptr(out.s_col), rule, _stream(x.device))
    _lib.check("mxq_quantize", st)
    return out


def mx_quantize_ranged(x: torch.Tensor, rowwise: bool = True, colwise: bool = True, rule: int = RCEIL,
                       out: Optional[MXTensor] = None, words: Optional[torch.Tensor] = None):
    """mx_quantize plus each orientation's range word (int32 device scalars: 1 if a 64-value window is wide).
    Returns (MXTensor, words) with words = int32[2]: [row orientation, column orientation]."""
    _dev(x, torch.bfloat16, "x")
    rows, cols = x.shape
    dev = x.device
    if out is None:
        e = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
        out = MXTensor(e(rows, cols) if rowwise else None, e(rows, cols // 32) if rowwise else None,
                       e(cols, rows) if colwise else None, e(cols, rows // 32) if colwise else None)
    if words is None:
        words = torch.zeros(2, dtype=torch.int32, device=dev)
    st = _lib.load().mxq_quantize_ranged(_ptr(x), rows, cols, _ptr(out.q_row), _ptr(out.s_row), _ptr(out.q_col),
                                         _ptr(out.s_col), rule,
                                         C.c_void_p(words.data_ptr()) if out.q_row is not None else None,
                                         C.c_void_p(words.data_ptr() + 4) if out.q_col is not None else None,
                                         _stream(dev))
    _lib.check("mxq_quantize_ranged", st)
    return out, words


def scaled_gemm_ranged(a_q: torch.Tensor, a_s: torch.Tensor, a_wide: torch.Tensor, b_q: torch.Tensor,
                       b_s: torch.Tensor, b_wide: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MX C = A B^T (bf16) with the instruction picked on the device from the operands' range words (int32 device
    scalars, e.g. words[0:1] / words[1:2] of mx_quantize_ranged)."""
    _dev(a_q, torch.uint8, "a_q"); _dev(b_q, torch.uint8, "b_q")
    M, K = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != K:
        raise ValueError("a_q and b_q must share K")
    if not (a_wide.is_cuda and b_wide.is_cuda and a_wide.dtype == torch.int32 and b_wide.dtype == torch.int32):
        raise ValueError("range words must be int32 device tensors")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    st = _lib.load().scaled_gemm_ranged(_ptr(a_q), _ptr(a_s), C.c_void_p(a_wide.data_ptr()), _ptr(b_q), _ptr(b_s),
                                        C.c_void_p(b_wide.data_ptr()), M, N, K, _ptr(out), out.stride(0),
                                        _stream(a_q.device))
    _lib.check("scaled_gemm_ranged", st)
    return out


def swiglu_mx_quantize(c: torch.Tensor, rule: int = RCEIL, out: Optional[MXTensor] = None) -> MXTensor:
    """c: bf16 [rows][2F] (gate | up) -> MXFP8 row orientation of silu(gate) * up: MXTensor(q_row, s_row, None, None)."""
    _dev(c, torch.bfloat16, "c")
    rows, f2 = c.shape
    F = f2 // 2
    if out is None:
        out = MXTensor(torch.empty((rows, F), dtype=torch.uint8, device=c.device),
                       torch.empty((rows, F // 32), dtype=torch.uint8, device=c.device), None, None)
    st = _lib.load().swiglu_mx_quantize(_ptr(c), rows, F, _ptr(out.q_row), _ptr(out.s_row), rule, _stream(c.device))
    _lib.check("swiglu_mx_quantize", st)
    return out


def _mx_out(rows: int, cols: int, rowwise: bool, colwise: bool, dev) -> MXTensor:
    e = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
    return MXTensor(e(rows, cols) if rowwise else None, e(rows, cols // 32) if rowwise else None,
                    e(cols, rows) if colwise else None, e(cols, rows // 32) if colwise else None)


def swiglu_mx_quantize_oriented(c: torch.Tensor, rowwise: bool = True, colwise: bool = True, rule: int = RCEIL,
                                out: Optional[MXTensor] = None) -> MXTensor:
    """c: bf16 [rows][2F] (gate | up) -> MXFP8 of silu(gate) * up [rows][F] in the requested orientations (the
    column one is the down projection's Wgrad operand)."""
    _dev(c, torch.bfloat16, "c")
    rows, f2 = c.shape
    F = f2 // 2
    if out is None:
        out = _mx_out(rows, F, rowwise, colwise, c.device)
    st = _lib.load().swiglu_mx_quantize_oriented(_ptr(c), rows, F, _ptr(out.q_row), _ptr(out.s_row), _ptr(out.q_col),
                                                 _ptr(out.s_col), rule, _stream(c.device))
    _lib.check("swiglu_mx_quantize_oriented", st)
    return out


def route_weighted_mx_quantize(dy: torch.Tensor, route_w: torch.Tensor, rowwise: bool = True, colwise: bool = True,
                               rule: int = RCEIL, out: Optional[MXTensor] = None) -> MXTensor:
    """dy: bf16 [rows][cols] (routed rows in expert order), route_w: float32[rows] -> MXFP8 of route_w[r] * dy[r][c]
    in the requested orientations (the down projection's dgrad and Wgrad operands)."""
    _dev(dy, torch.bfloat16, "dy"); _dev(route_w, torch.float32, "route_w")
    rows, cols = dy.shape
    if route_w.numel() != rows:
        raise ValueError("route_w must hold one weight per row of dy")
    if out is None:
        out = _mx_out(rows, cols, rowwise, colwise, dy.device)
    st = _lib.load().route_weighted_mx_quantize(_ptr(dy), _ptr(route_w), rows, cols, _ptr(out.q_row),
                                                _ptr(out.s_row), _ptr(out.q_col), _ptr(out.s_col), rule,
                                                _stream(dy.device))
    _lib.check("route_weighted_mx_quantize", st)
    return out


def swiglu_backward_mx_quantize(c: torch.Tensor, dh: torch.Tensor, rowwise: bool = True, colwise: bool = True,
                                rule: int = RCEIL, out: Optional[MXTensor] = None) -> MXTensor:
    """c: bf16 [rows][2F] (gate | up, the forward up/gate GEMM output), dh: bf16 [rows][F] (gradient of
    silu(gate) * up) -> MXFP8 of (d_gate | d_up) [rows][2F] in the requested orientations."""
    _dev(c, torch.bfloat16, "c"); _dev(dh, torch.bfloat16, "dh")
    rows, f2 = c.shape
    F = f2 // 2
    if tuple(dh.shape) != (rows, F) or f2 != 2 * F:
        raise ValueError("dh must be [rows][F] for c of shape [rows][2F]")
    if out is None:
        out = _mx_out(rows, f2, rowwise, colwise, c.device)
    st = _lib.load().swiglu_backward_mx_quantize(_ptr(c), _ptr(dh), rows, F, _ptr(out.q_row), _ptr(out.s_row),
                                                 _ptr(out.q_col), _ptr(out.s_col), rule, _stream(c.device))
    _lib.check("swiglu_backward_mx_quantize", st)
    return out


class PerTensorFP8(NamedTuple):
    q: Optional[torch.Tensor]       # [rows][cols] uint8
    q_t: Optional[torch.Tensor]     # [cols][rows] uint8
    amax: torch.Tensor              # float32[1] on the device
    scale: torch.Tensor             # float32[1] on the device (q ~ x * scale)


def _pt_out(x: torch.Tensor, want_q: bool, want_qt: bool, out: Optional[PerTensorFP8]):
    """Output buffers of a per-tensor cast: `out` checked against x's shape (its q / q_t, either may be None, decide
    which orientations are written), else new ones."""
    rows, cols = x.shape
    dev = x.device
    if out is None:
        return (torch.empty((rows, cols), dtype=torch.uint8, device=dev) if want_q else None,
                torch.empty((cols, rows), dtype=torch.uint8, device=dev) if want_qt else None,
                torch.empty(1, dtype=torch.float32, device=dev), torch.empty(1, dtype=torch.float32, device=dev))
    for t, shape, dt, name in ((out.q, (rows, cols), torch.uint8, "out.q"), (out.q_t, (cols, rows), torch.uint8, "out.q_t"),
                               (out.amax, (1,), torch.float32, "out.amax"), (out.scale, (1,), torch.float32, "out.scale")):
        if t is None and name in ("out.q", "out.q_t"):
            continue
        if t is None or tuple(t.shape) != shape or t.dtype != dt or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {shape} on {dev}")
    return out.q, out.q_t, out.amax, out.scale


def pertensor_quantize(x: torch.Tensor, fmt: int = E4M3, margin: float = 1.0, scale_in: Optional[torch.Tensor] = None,
                       want_q: bool = True, want_qt: bool = True, workspace: Optional[torch.Tensor] = None,
                       out: Optional[PerTensorFP8] = None) -> PerTensorFP8:
    """Per-tensor FP8 cast of x (bf16 [rows][cols]) to q and its transpose q_t. `out` reuses caller buffers."""
    _dev(x, torch.bfloat16, "x")
    rows, cols = x.shape
    dev = x.device
    q, qt, amax, scale = _pt_out(x, want_q, want_qt, out)
    nbytes = workspace_bytes("pertensor", rows * cols)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if scale_in is not None:
        _dev(scale_in, torch.float32, "scale_in")
    st = _lib.load().fp8_quantize_pertensor(_ptr(x), rows, cols, fmt, C.c_float(margin), _ptr(scale_in), _ptr(amax),
                                            _ptr(scale), _ptr(q), _ptr(qt), _ptr(workspace), workspace.numel(),
                                            _stream(dev))
    _lib.check("fp8_quantize_pertensor", st)
    return PerTensorFP8(q, qt, amax, scale)


def pertensor_quantize_delayed(x: torch.Tensor, amax_history: torch.Tensor, hist_pos: torch.Tensor, fmt: int = E4M3,
                               margin: float = 1.0, want_q: bool = True, want_qt: bool = True,
                               workspace: Optional[torch.Tensor] = None,
                               out: Optional[PerTensorFP8] = None) -> PerTensorFP8:
    """Delayed-scaling cast: scale from the amax history (float32[H], updated in place with this call's amax at
    hist_pos, an int32[1] that advances). `out` reuses caller buffers."""
    _dev(x, torch.bfloat16, "x"); _dev(amax_history, torch.float32, "amax_history"); _dev(hist_pos, torch.int32, "hist_pos")
    rows, cols = x.shape
    dev = x.device
    q, qt, amax, scale = _pt_out(x, want_q, want_qt, out)
    if workspace is None:
        workspace = torch.empty(workspace_bytes("pertensor_delayed", rows * cols), dtype=torch.uint8, device=dev)
    st = _lib.load().fp8_quantize_pertensor_delayed(_ptr(x), rows, cols, fmt, C.c_float(margin), _ptr(amax_history),
                                                    _ptr(hist_pos), amax_history.numel(), _ptr(amax), _ptr(scale),
                                                    _ptr(q), _ptr(qt), _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check("fp8_quantize_pertensor_delayed", st)
    return PerTensorFP8(q, qt, amax, scale)


def scaled_gemm(a_q: torch.Tensor, a_scale: torch.Tensor, b_q: torch.Tensor, b_scale: torch.Tensor,
                scaling: int = MX_BLOCK32, a_fmt: int = E4M3, b_fmt: int = E4M3,
                out: Optional[torch.Tensor] = None, exact: bool = False, path: str = "checked") -> torch.Tensor:
    """C[M][N] = A[M][K] B[N][K]^T in bf16. MX: scales are E8M0 grids [M][K/32], [N][K/32]; per-tensor: float32[1].
    path "checked" calls scaled_gemm (the FP8 instruction where a device-side range check allows it, else the exact
    path), "exact" (or exact=True) scaled_gemm_exact, "fp8" scaled_gemm_fp8 (FP8 instruction at every K, bound not
    guaranteed)."""
    _dev(a_q, torch.uint8, "a_q"); _dev(b_q, torch.uint8, "b_q")
    M, K = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != K:
        raise ValueError("a_q and b_q must share K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    ldc = out.stride(0)
    if exact:
        path = "exact"
    name = {"checked": "scaled_gemm", "exact": "scaled_gemm_exact", "fp8": "scaled_gemm_fp8"}[path]
    st = getattr(_lib.load(), name)(_ptr(a_q), _ptr(a_scale), a_fmt, _ptr(b_q), _ptr(b_scale), b_fmt, M, N, K,
                                    scaling, _ptr(out), ldc, _stream(a_q.device))
    _lib.check(name, st)
    return out


def grouped_scaled_gemm(a_q: torch.Tensor, a_s: torch.Tensor, offsets: torch.Tensor, b_q: torch.Tensor,
                        b_s: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _dev(a_q, torch.uint8, "a_q"); _dev(b_q, torch.uint8, "b_q"); _dev(offsets, torch.int64, "offsets")
    total, K = a_q.shape
    G, N, Kb = b_q.shape
    if Kb != K or offsets.numel() != G + 1:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((total, N), dtype=torch.bfloat16, device=a_q.device)
    st = _lib.load().grouped_scaled_gemm(_ptr(a_q), _ptr(a_s), _ptr(offsets), G, total, _ptr(b_q), _ptr(b_s), N, K,
                                         _ptr(out), _stream(a_q.device))
    _lib.check("grouped_scaled_gemm", st)
    return out


def grouped_scaled_gemm_strided(a_q: torch.Tensor, a_s: torch.Tensor, offsets: torch.Tensor, b_q: torch.Tensor,
                                b_s: torch.Tensor, G: int, N: int, K: int, ldb: int, b_group_stride: int, ldbs: int,
                                bs_group_stride: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The grouped MX GEMM with expert g's B row n at b_q[g * b_group_stride + n * ldb] (K bytes) and its scales at
    b_s[g * bs_group_stride + n * ldbs] (K/32 bytes): e.g. a column-orientation weight cache read in place."""
    _dev(a_q, torch.uint8, "a_q"); _dev(b_q, torch.uint8, "b_q"); _dev(offsets, torch.int64, "offsets")
    _dev(a_s, torch.uint8, "a_s"); _dev(b_s, torch.uint8, "b_s")
    total, Ka = a_q.shape
    if Ka != K or offsets.numel() != G + 1:
        raise ValueError("shape mismatch")
    last = (G - 1) * b_group_stride + (N - 1) * ldb + K
    last_s = (G - 1) * bs_group_stride + (N - 1) * ldbs + K // 32
    if b_q.numel() < last or b_s.numel() < last_s:
        raise ValueError("b_q / b_s do not hold every expert's rows at the given strides")
    if out is None:
        out = torch.empty((total, N), dtype=torch.bfloat16, device=a_q.device)
    elif out.dtype != torch.bfloat16 or out.shape[0] != total or out.shape[1] < N or out.stride(1) != 1:
        raise ValueError("out must be bf16 [total_rows][>= N] with unit column stride")
    st = _lib.load().grouped_scaled_gemm_strided(_ptr(a_q), _ptr(a_s), _ptr(offsets), G, total, _ptr(b_q), _ptr(b_s),
                                                 ldb, b_group_stride, ldbs, bs_group_stride, N, K, _ptr(out),
                                                 out.stride(0), _stream(a_q.device))
    _lib.check("grouped_scaled_gemm_strided", st)
    return out


def grouped_wgrad_mx(a_q: torch.Tensor, a_s: torch.Tensor, b_q: torch.Tensor, b_s: torch.Tensor,
                     offsets: torch.Tensor, out: Optional[torch.Tensor] = None,
                     accumulate: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-expert contraction over token ranges: C_g = A[:, off_g:off_g+1] B[:, off_g:off_g+1]^T for column-
    orientation operands a_q [M][Kt], b_q [N][Kt]. Returns bf16 [G][M][N], or adds into `accumulate` (float32
    [G][M][N]) and returns it."""
    _dev(a_q, torch.uint8, "a_q"); _dev(b_q, torch.uint8, "b_q"); _dev(offsets, torch.int64, "offsets")
    _dev(a_s, torch.uint8, "a_s"); _dev(b_s, torch.uint8, "b_s")
    M, Kt = a_q.shape
    N = b_q.shape[0]
    G = offsets.numel() - 1
    if b_q.shape[1] != Kt or tuple(a_s.shape) != (M, Kt // 32) or tuple(b_s.shape) != (N, Kt // 32):
        raise ValueError("shape mismatch")
    if accumulate is not None:
        _dev(accumulate, torch.float32, "accumulate")
        if tuple(accumulate.shape) != (G, M, N):
            raise ValueError("accumulate must be float32 [G][M][N]")
        c_bf16, c_f32, res = None, accumulate, accumulate
    else:
        if out is None:
            out = torch.empty((G, M, N), dtype=torch.bfloat16, device=a_q.device)
        _dev(out, torch.bfloat16, "out")
        if tuple(out.shape) != (G, M, N):
            raise ValueError("out must be bf16 [G][M][N]")
        c_bf16, c_f32, res = out, None, out
    st = _lib.load().grouped_wgrad_mx(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), _ptr(offsets), G, M, N, Kt,
                                      _ptr(c_bf16), _ptr(c_f32), _stream(a_q.device))
    _lib.check("grouped_wgrad_mx", st)
    return res


def fp8_adam_step(master: torch.Tensor, grad: torch.Tensor, m_q: torch.Tensor, m_scale: torch.Tensor,
                  v: torch.Tensor, w: Optional[torch.Tensor], hp: AdamHParams,
                  workspace: Optional[torch.Tensor] = None) -> None:
    """In place on master, m_q, m_scale, v; writes w (bf16 copy) when given."""
    _dev(master, torch.float32, "master"); _dev(grad, torch.bfloat16, "grad"); _dev(m_q, torch.uint8, "m_q")
    _dev(m_scale, torch.float32, "m_scale"); _dev(v, torch.float16, "v")
    n = master.numel()
    if workspace is None:
        workspace = torch.empty(workspace_bytes("adam", n), dtype=torch.uint8, device=master.device)
    st = _lib.load().fp8_adam_step(_ptr(master), _ptr(grad), _ptr(m_q), _ptr(m_scale), _ptr(v), _ptr(w), n,
                                   C.byref(hp), _ptr(workspace), workspace.numel(), _stream(master.device))
    _lib.check("fp8_adam_step", st)


def fp8_adam_step_delayed(master: torch.Tensor, grad: torch.Tensor, m_q: torch.Tensor, m_scale: torch.Tensor,
                          v: torch.Tensor, w: Optional[torch.Tensor], hp: AdamHParams, m_history: torch.Tensor,
                          hist_pos: torch.Tensor, workspace: Optional[torch.Tensor] = None) -> None:
    """fp8_adam_step with the first-moment scale from the amax history (one pass over the state)."""
    _dev(master, torch.float32, "master"); _dev(grad, torch.bfloat16, "grad"); _dev(m_q, torch.uint8, "m_q")
    _dev(m_scale, torch.float32, "m_scale"); _dev(v, torch.float16, "v")
    _dev(m_history, torch.float32, "m_history"); _dev(hist_pos, torch.int32, "hist_pos")
    n = master.numel()
    if workspace is None:
        workspace = torch.empty(workspace_bytes("adam_delayed", n), dtype=torch.uint8, device=master.device)
    st = _lib.load().fp8_adam_step_delayed(_ptr(master), _ptr(grad), _ptr(m_q), _ptr(m_scale), _ptr(v), _ptr(w), n,
                                           C.byref(hp), _ptr(m_history), _ptr(hist_pos), m_history.numel(),
                                           _ptr(workspace), workspace.numel(), _stream(master.device))
    _lib.check("fp8_adam_step_delayed", st)


def fp8_adam_step_mx_cache(master: torch.Tensor, grad: torch.Tensor, m_q: torch.Tensor, m_scale: torch.Tensor,
                           v: torch.Tensor, w: Optional[torch.Tensor], hp: AdamHParams, rows: int, cols: int,
                           rowwise: bool = True, colwise: bool = True, rule: int = RCEIL,
                           out: Optional[MXTensor] = None, workspace: Optional[torch.Tensor] = None) -> MXTensor:
    """fp8_adam_step on a [rows][cols] weight that also rebuilds its MXFP8 caches from the updated fp32 master."""
    _dev(master, torch.float32, "master"); _dev(grad, torch.bfloat16, "grad"); _dev(m_q, torch.uint8, "m_q")
    _dev(m_scale, torch.float32, "m_scale"); _dev(v, torch.float16, "v")
    dev = master.device
    if out is None:
        e = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
        out = MXTensor(e(rows, cols) if rowwise else None, e(rows, cols // 32) if rowwise else None,
                       e(cols, rows) if colwise else None, e(cols, rows // 32) if colwise else None)
    if workspace is None:
        workspace = torch.empty(workspace_bytes("adam", rows * cols), dtype=torch.uint8, device=dev)
    st = _lib.load().fp8_adam_step_mx_cache(_ptr(master), _ptr(grad), _ptr(m_q), _ptr(m_scale), _ptr(v), _ptr(w),
                                            rows, cols, _ptr(out.q_row), _ptr(out.s_row), _ptr(out.q_col),
                                            _ptr(out.s_col), rule, C.byref(hp), _ptr(workspace), workspace.numel(),
                                            _stream(dev))
    _lib.check("fp8_adam_step_mx_cache", st)
    return out


class AutoScaled(NamedTuple):
    q: torch.Tensor                 # uint8 codes
    scale: torch.Tensor             # float32[1]: the mu these codes carry
    overflow: torch.Tensor          # int64[1]: codes at the maximum magnitude


def fp8_autoscale_cast(g: torch.Tensor, mu: torch.Tensor, fmt: int = E4M3,
                       workspace: Optional[torch.Tensor] = None, out: Optional[AutoScaled] = None) -> AutoScaled:
    """q = FP8(mu * g); mu (float32[1], device) is updated in place for the next step. `out` reuses caller buffers
    (q uint8 of g's shape, scale float32[1], overflow int64[1])."""
    _dev(g, torch.bfloat16, "g"); _dev(mu, torch.float32, "mu")
    dev = g.device
    n = g.numel()
    if out is None:
        q = torch.empty(g.shape, dtype=torch.uint8, device=dev)
        scale = torch.empty(1, dtype=torch.float32, device=dev)
        overflow = torch.empty(1, dtype=torch.int64, device=dev)
    else:
        q, scale, overflow = out.q, out.scale, out.overflow
        for t, shape, dt, name in ((q, tuple(g.shape), torch.uint8, "out.q"), (scale, (1,), torch.float32, "out.scale"),
                                   (overflow, (1,), torch.int64, "out.overflow")):
            if tuple(t.shape) != shape or t.dtype != dt or t.device != dev or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {shape} on {dev}")
    if workspace is None:
        workspace = torch.empty(workspace_bytes("autoscale", n), dtype=torch.uint8, device=dev)
    st = _lib.load().fp8_autoscale_cast(_ptr(g), n, fmt, _ptr(mu), _ptr(q), _ptr(scale), _ptr(overflow),
                                        _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check("fp8_autoscale_cast", st)
    return AutoScaled(q, scale, overflow)


def fp8_requantize_shared(q: torch.Tensor, fmt_in: int, scale_in: torch.Tensor, gathered_scales: torch.Tensor,
                          fmt_out: int = E4M3, out: Optional[torch.Tensor] = None):
    """Returns (q_out, shared scale s_g, sum scale N * s_g), all on the device."""
    _dev(q, torch.uint8, "q"); _dev(scale_in, torch.float32, "scale_in")
    _dev(gathered_scales, torch.float32, "gathered_scales")
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, torch.uint8, "out")
        if out.numel() != q.numel():
            raise ValueError("out must hold as many codes as q")
    sg = torch.empty(1, dtype=torch.float32, device=dev)
    ssum = torch.empty(1, dtype=torch.float32, device=dev)
    st = _lib.load().fp8_requantize_shared(_ptr(q), q.numel(), fmt_in, _ptr(scale_in), _ptr(gathered_scales),
                                           gathered_scales.numel(), fmt_out, _ptr(out), _ptr(sg), _ptr(ssum),
                                           _stream(dev))
    _lib.check("fp8_requantize_shared", st)
    return out, sg, ssum
