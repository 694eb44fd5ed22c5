"""mxq oracle: a plain, slow CPU reference of the FP8 / MXFP8 training numerics.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package. The GPU library never imports, links or calls it, and the two share no code: the seeded input
generators are the only thing both sides see, and they live in a module of their own.

The arithmetic lives in ``mxq_oracle.c`` (plain C, gcc -O2 -ffp-contract=off, no fast-math); this module only
builds it, loads it with ctypes and marshals numpy arrays. Function-level citations of the pages are in the C file.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

E4M3, E5M2 = 0, 1
RCEIL, FLOOR = 0, 1
PER_TENSOR, MX_BLOCK32 = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host gcc. Returns the path of the shared library."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
               "-fPIC", "-shared", "-pthread", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = C.CDLL(_LIB)
        P, I64, I, D, F = C.c_void_p, C.c_int64, C.c_int, C.c_double, C.c_float
        L.orc_e4m3_value.restype = D; L.orc_e4m3_value.argtypes = [C.c_uint8]
        L.orc_e5m2_value.restype = D; L.orc_e5m2_value.argtypes = [C.c_uint8]
        L.orc_f16_value.restype = D; L.orc_f16_value.argtypes = [C.c_uint16]
        L.orc_fp8_encode.restype = C.c_uint8; L.orc_fp8_encode.argtypes = [D, I]
        L.orc_bf16_from_f32.restype = C.c_uint16; L.orc_bf16_from_f32.argtypes = [F]
        L.orc_f16_from_f32.restype = C.c_uint16; L.orc_f16_from_f32.argtypes = [F]
        L.orc_mx_scale_exp.restype = I; L.orc_mx_scale_exp.argtypes = [D, I]
        L.orc_fp8_encode_array.argtypes = [P, I64, I, P]
        L.orc_fp8_value_array.argtypes = [P, I64, I, P]
        L.orc_bf16_from_f32_array.argtypes = [P, I64, P]
        L.orc_f16_from_f32_array.argtypes = [P, I64, P]
        L.orc_mx_scale_exp_array.argtypes = [P, I64, I, P]
        L.orc_mx_quantize.argtypes = [P, I64, I64, I, P, P, P, P, I]
        L.orc_pertensor_quantize.argtypes = [P, I64, I64, I, F, P, P, P, P, P, I]
        L.orc_gemm_ref.argtypes = [P, P, I, P, P, I, I64, I64, I64, I, P, I64, P, I64, P, P, I]
        L.orc_grouped_gemm_ref.argtypes = [P, P, P, I64, P, P, I64, I64, P, I64, P, I64, P, P, I]
        L.orc_adam_step.restype = F
        L.orc_adam_step.argtypes = [P, P, P, P, P, P, I64, P, I]
        L.orc_adam_amax.restype = F
        L.orc_adam_amax.argtypes = [P, P, P, F, I64, P, I]
        L.orc_mx_quantize_f32.argtypes = [P, I64, I64, I, P, P, P, P, I]
        L.orc_exp_f32.restype = F; L.orc_exp_f32.argtypes = [F]
        L.orc_swiglu_f32.restype = F; L.orc_swiglu_f32.argtypes = [F, F]
        L.orc_swiglu_mx_quantize.argtypes = [P, I64, I64, I, P, P, P]
        L.orc_autoscale_cast.argtypes = [P, I64, I, P, P, P, P]
        L.orc_min_scale.restype = F; L.orc_min_scale.argtypes = [P, I64]
        L.orc_requantize_shared.argtypes = [P, I64, I, F, F, I, P]
        L.orc_delayed_scale.restype = F
        L.orc_delayed_scale.argtypes = [P, I64, I, F]
        L.orc_history_push.argtypes = [P, I64, P, F]
        L.orc_pertensor_quantize_delayed.argtypes = [P, I64, I64, I, F, P, I64, P, P, P, P, P, I]
        L.orc_adam_step_delayed.restype = F
        L.orc_adam_step_delayed.argtypes = [P, P, P, P, P, P, I64, P, P, I64, P, I]
        L.orc_adam_elements.argtypes = [P, P, P, P, F, F, P, I64, P, P, P, P, P]
        L.orc_route_weighted_mx_quantize.argtypes = [P, P, I64, I64, I, P, P, P, P, P, I]
        L.orc_swiglu_bwd_f32.argtypes = [F, F, F, P, P]
        L.orc_swiglu_bwd_mx_quantize.argtypes = [P, P, I64, I64, I, P, P, P, P, P, I]
        L.orc_grouped_wgrad_ref.argtypes = [P, P, P, P, P, I64, P, I64, P, I64, P, I64, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    """Threads for the oracle's independent outputs: MXQ_ORACLE_THREADS if set, else the CPUs available (max 16)."""
    env = os.environ.get("MXQ_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, len(os.sched_getaffinity(0))))


# ---------------------------------------------------------------- codecs
def fp8_value(codes, fmt: int) -> np.ndarray:
    c = _c(codes, np.uint8).reshape(-1)
    out = np.empty(c.size, np.float64)
    lib().orc_fp8_value_array(_p(c), c.size, fmt, _p(out))
    return out.reshape(np.shape(codes))


def fp8_encode(values, fmt: int) -> np.ndarray:
    v = _c(values, np.float64).reshape(-1)
    out = np.empty(v.size, np.uint8)
    lib().orc_fp8_encode_array(_p(v), v.size, fmt, _p(out))
    return out.reshape(np.shape(values))


def bf16_from_f32(values) -> np.ndarray:
    v = _c(values, np.float32).reshape(-1)
    out = np.empty(v.size, np.uint16)
    lib().orc_bf16_from_f32_array(_p(v), v.size, _p(out))
    return out.reshape(np.shape(values))


def bf16_to_f32(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f16_from_f32(values) -> np.ndarray:
    v = _c(values, np.float32).reshape(-1)
    out = np.empty(v.size, np.uint16)
    lib().orc_f16_from_f32_array(_p(v), v.size, _p(out))
    return out.reshape(np.shape(values))


def f16_value(bits) -> float:
    return lib().orc_f16_value(int(bits))


def mx_scale_exp(amax, rule: int = RCEIL) -> np.ndarray:
    a = _c(amax, np.float64).reshape(-1)
    out = np.empty(a.size, np.int32)
    lib().orc_mx_scale_exp_array(_p(a), a.size, rule, _p(out))
    return out.reshape(np.shape(amax))


# ---------------------------------------------------------------- quantizers
def mx_quantize(x_bf16, rule: int = RCEIL, rowwise: bool = True, colwise: bool = True, nthreads: int | None = None):
    """Returns (q_row, s_row, q_col, s_col); skipped orientations are None."""
    x = _c(x_bf16, np.uint16)
    R, Ccols = x.shape
    q_row = np.empty((R, Ccols), np.uint8) if rowwise else None
    s_row = np.empty((R, Ccols // 32), np.uint8) if rowwise else None
    q_col = np.empty((Ccols, R), np.uint8) if colwise else None
    s_col = np.empty((Ccols, R // 32), np.uint8) if colwise else None
    lib().orc_mx_quantize(_p(x), R, Ccols, rule, _p(q_row), _p(s_row), _p(q_col), _p(s_col),
                          nthreads or default_threads())
    return q_row, s_row, q_col, s_col


def mx_quantize_f32(x_f32, rule: int = RCEIL, rowwise: bool = True, colwise: bool = True, nthreads=None):
    """MXFP8 quantize of an fp32 [rows][cols] matrix. Returns (q_row, s_row, q_col, s_col) (None where not asked)."""
    x = _c(x_f32, np.float32)
    R, Ccols = x.shape
    q_row = np.empty((R, Ccols), np.uint8) if rowwise else None
    s_row = np.empty((R, Ccols // 32), np.uint8) if rowwise else None
    q_col = np.empty((Ccols, R), np.uint8) if colwise else None
    s_col = np.empty((Ccols, R // 32), np.uint8) if colwise else None
    lib().orc_mx_quantize_f32(_p(x), R, Ccols, rule, _p(q_row), _p(s_row), _p(q_col), _p(s_col),
                              nthreads or default_threads())
    return q_row, s_row, q_col, s_col


def exp_f32(x: float) -> np.float32:
    return np.float32(lib().orc_exp_f32(C.c_float(x)))


def swiglu_f32(g: float, u: float) -> np.float32:
    return np.float32(lib().orc_swiglu_f32(C.c_float(g), C.c_float(u)))


def swiglu_mx_quantize(c_bf16, rule: int = RCEIL, want_h: bool = False):
    """c_bf16: [rows][2F] (gate | up). Returns (q[rows][F], s[rows][F/32], h fp32 or None)."""
    c = _c(c_bf16, np.uint16)
    R, F2 = c.shape
    F = F2 // 2
    q = np.empty((R, F), np.uint8)
    s = np.empty((R, F // 32), np.uint8)
    h = np.empty((R, F), np.float32) if want_h else None
    lib().orc_swiglu_mx_quantize(_p(c), R, F, rule, _p(q), _p(s), _p(h))
    return q, s, h


# ---------------------------------------------------------------- routed-expert backward
def route_weighted_mx_quantize(dy_bf16, p_f32, rule: int = RCEIL, rowwise: bool = True, colwise: bool = True,
                               want_x: bool = False, nthreads=None):
    """x = fp32(p[r] * dy[r][c]) quantized to MXFP8. Returns (q_row, s_row, q_col, s_col, x or None)."""
    dy = _c(dy_bf16, np.uint16)
    p = _c(p_f32, np.float32)
    R, Ccols = dy.shape
    q_row = np.empty((R, Ccols), np.uint8) if rowwise else None
    s_row = np.empty((R, Ccols // 32), np.uint8) if rowwise else None
    q_col = np.empty((Ccols, R), np.uint8) if colwise else None
    s_col = np.empty((Ccols, R // 32), np.uint8) if colwise else None
    x = np.empty((R, Ccols), np.float32) if want_x else None
    lib().orc_route_weighted_mx_quantize(_p(dy), _p(p), R, Ccols, rule, _p(q_row), _p(s_row), _p(q_col), _p(s_col),
                                         _p(x), nthreads or default_threads())
    return q_row, s_row, q_col, s_col, x


def swiglu_bwd_f32(g: float, u: float, dh: float):
    """(d_gate, d_up) of h = silu(g) u for the incoming gradient dh, in the oracle's fp32 operation order."""
    dg = C.c_float(); du = C.c_float()
    lib().orc_swiglu_bwd_f32(C.c_float(g), C.c_float(u), C.c_float(dh), C.byref(dg), C.byref(du))
    return np.float32(dg.value), np.float32(du.value)


def swiglu_bwd_mx_quantize(c_bf16, dh_bf16, rule: int = RCEIL, rowwise: bool = True, colwise: bool = True,
                           want_dc: bool = False, nthreads=None):
    """c_bf16 [rows][2F] (gate | up), dh_bf16 [rows][F]. dc = (d_gate | d_up) [rows][2F] quantized to MXFP8.
    Returns (q_row, s_row, q_col, s_col, dc fp32 or None)."""
    c = _c(c_bf16, np.uint16)
    dh = _c(dh_bf16, np.uint16)
    R, F2 = c.shape
    F = F2 // 2
    assert dh.shape == (R, F)
    q_row = np.empty((R, F2), np.uint8) if rowwise else None
    s_row = np.empty((R, F2 // 32), np.uint8) if rowwise else None
    q_col = np.empty((F2, R), np.uint8) if colwise else None
    s_col = np.empty((F2, R // 32), np.uint8) if colwise else None
    dc = np.empty((R, F2), np.float32) if want_dc else None
    lib().orc_swiglu_bwd_mx_quantize(_p(c), _p(dh), R, F, rule, _p(q_row), _p(s_row), _p(q_col), _p(s_col), _p(dc),
                                     nthreads or default_threads())
    return q_row, s_row, q_col, s_col, dc


def grouped_wgrad_ref(a_q, a_s, b_q, b_s, offsets, groups=None, rows=None, cols=None):
    """Per-expert contraction over token ranges: y[g][m][n] = sum_{k in group g} a_hat[m][k] b_hat[n][k] (fp64),
    with a_q [M][Kt], b_q [N][Kt] and scales [.][Kt/32]. Returns (y, S) of shape [groups][rows][cols]."""
    aq = _c(a_q, np.uint8); as_ = _c(a_s, np.uint8)
    bq = _c(b_q, np.uint8); bs = _c(b_s, np.uint8)
    off = _c(offsets, np.int64)
    M, Kt = aq.shape
    N = bq.shape[0]
    assert bq.shape[1] == Kt and as_.shape == (M, Kt // 32) and bs.shape == (N, Kt // 32)
    G = off.size - 1
    groups = np.arange(G, dtype=np.int64) if groups is None else _c(groups, np.int64)
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    cols = np.arange(N, dtype=np.int64) if cols is None else _c(cols, np.int64)
    y = np.empty((groups.size, rows.size, cols.size), np.float64)
    S = np.empty((groups.size, rows.size, cols.size), np.float64)
    lib().orc_grouped_wgrad_ref(_p(aq), _p(as_), _p(bq), _p(bs), _p(off), Kt, _p(groups), groups.size, _p(rows),
                                rows.size, _p(cols), cols.size, _p(y), _p(S))
    return y, S


def autoscale_cast(g_bf16, mu: float, fmt: int = E4M3):
    """Returns (q, overflow_count, scale used (= mu), mu for the next step)."""
    g = _c(g_bf16, np.uint16).reshape(-1)
    m = np.array([mu], np.float32)
    q = np.empty(g.size, np.uint8)
    cnt = np.zeros(1, np.uint64)
    sc = np.zeros(1, np.float32)
    lib().orc_autoscale_cast(_p(g), g.size, fmt, _p(m), _p(q), _p(cnt), _p(sc))
    return q, int(cnt[0]), np.float32(sc[0]), np.float32(m[0])


def min_scale(scales) -> np.float32:
    s = _c(scales, np.float32)
    return np.float32(lib().orc_min_scale(_p(s), s.size))


def requantize_shared(q_in, fmt_in: int, s_in: float, s_g: float, fmt_out: int):
    q = _c(q_in, np.uint8).reshape(-1)
    out = np.empty(q.size, np.uint8)
    lib().orc_requantize_shared(_p(q), q.size, fmt_in, C.c_float(s_in), C.c_float(s_g), fmt_out, _p(out))
    return out


def pertensor_quantize(x_bf16, fmt: int = E4M3, margin: float = 1.0, scale_in: float | None = None,
                       want_q: bool = True, want_qt: bool = True, nthreads: int | None = None):
    """Returns (amax, scale, q, q_t)."""
    x = _c(x_bf16, np.uint16)
    R, Ccols = x.shape
    amax = np.zeros(1, np.float32)
    scale = np.zeros(1, np.float32)
    sin = None if scale_in is None else np.array([scale_in], np.float32)
    q = np.empty((R, Ccols), np.uint8) if want_q else None
    qt = np.empty((Ccols, R), np.uint8) if want_qt else None
    lib().orc_pertensor_quantize(_p(x), R, Ccols, fmt, C.c_float(margin), _p(sin), _p(amax), _p(scale), _p(q), _p(qt),
                                 nthreads or default_threads())
    return float(amax[0]), np.float32(scale[0]), q, qt


def delayed_scale(history, fmt: int = E4M3, margin: float = 1.0) -> np.float32:
    """Scale of a delayed-scaling cast: FMAX / max(max(history), 1e-12) * margin (fp32)."""
    h = _c(history, np.float32)
    return np.float32(lib().orc_delayed_scale(_p(h), h.size, fmt, C.c_float(margin)))


def history_push(history, pos, amax: float) -> None:
    """Write amax at the ring position and advance it (history float32[H], pos int32[1], in place)."""
    assert history.dtype == np.float32 and pos.dtype == np.int32
    lib().orc_history_push(_p(history), history.size, _p(pos), C.c_float(amax))


def pertensor_quantize_delayed(x_bf16, history, pos, fmt: int = E4M3, margin: float = 1.0, want_q: bool = True,
                               want_qt: bool = True, nthreads: int | None = None):
    """One delayed-scaling cast. history (float32[H]) and pos (int32[1]) are updated in place.
    Returns (amax, scale, q, q_t)."""
    assert history.dtype == np.float32 and history.flags.c_contiguous
    assert pos.dtype == np.int32 and pos.size == 1
    x = _c(x_bf16, np.uint16)
    R, Ccols = x.shape
    amax = np.zeros(1, np.float32)
    scale = np.zeros(1, np.float32)
    q = np.empty((R, Ccols), np.uint8) if want_q else None
    qt = np.empty((Ccols, R), np.uint8) if want_qt else None
    lib().orc_pertensor_quantize_delayed(_p(x), R, Ccols, fmt, C.c_float(margin), _p(history), history.size, _p(pos),
                                         _p(amax), _p(scale), _p(q), _p(qt), nthreads or default_threads())
    return float(amax[0]), np.float32(scale[0]), q, qt


# ---------------------------------------------------------------- GEMM references
def gemm_ref(a_q, a_scale, a_fmt, b_q, b_scale, b_fmt, scaling, rows=None, cols=None, nthreads=None):
    """y, S over rows x cols of C = A B^T (fp64). a_q [M][K], b_q [N][K]; scales are E8M0 grids (MX) or fp32 scalars."""
    aq = _c(a_q, np.uint8); bq = _c(b_q, np.uint8)
    M, K = aq.shape
    N = bq.shape[0]
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    cols = np.arange(N, dtype=np.int64) if cols is None else _c(cols, np.int64)
    if scaling == MX_BLOCK32:
        sa = _c(a_scale, np.uint8); sb = _c(b_scale, np.uint8)
    else:
        sa = np.array([a_scale], np.float32); sb = np.array([b_scale], np.float32)
    y = np.empty((rows.size, cols.size), np.float64)
    S = np.empty((rows.size, cols.size), np.float64)
    lib().orc_gemm_ref(_p(aq), _p(sa), a_fmt, _p(bq), _p(sb), b_fmt, M, N, K, scaling, _p(rows), rows.size, _p(cols),
                       cols.size, _p(y), _p(S), nthreads or default_threads())
    return y, S


def grouped_gemm_ref(a_q, a_s, offsets, b_q, b_s, rows=None, cols=None, nthreads=None):
    aq = _c(a_q, np.uint8); as_ = _c(a_s, np.uint8)
    bq = _c(b_q, np.uint8); bs = _c(b_s, np.uint8)
    off = _c(offsets, np.int64)
    G, N, K = bq.shape
    total = aq.shape[0]
    rows = np.arange(total, dtype=np.int64) if rows is None else _c(rows, np.int64)
    cols = np.arange(N, dtype=np.int64) if cols is None else _c(cols, np.int64)
    y = np.empty((rows.size, cols.size), np.float64)
    S = np.empty((rows.size, cols.size), np.float64)
    lib().orc_grouped_gemm_ref(_p(aq), _p(as_), _p(off), G, _p(bq), _p(bs), N, K, _p(rows), rows.size, _p(cols),
                               cols.size, _p(y), _p(S), nthreads or default_threads())
    return y, S


# ---------------------------------------------------------------- Adam
class AdamHP(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("step", C.c_int64)]


def adam_step(master, grad_bf16, m_q, m_scale, v16, hp: AdamHP, want_w=True, nthreads=None):
    """In place on master (f32), m_q (u8), m_scale (f32[1]), v16 (u16). Returns (amax_m, w_bf16)."""
    for a, dt in ((master, np.float32), (m_q, np.uint8), (m_scale, np.float32), (v16, np.uint16)):
        assert a.dtype == dt and a.flags.c_contiguous
    g = _c(grad_bf16, np.uint16)
    n = master.size
    w = np.empty(n, np.uint16) if want_w else None
    amax = lib().orc_adam_step(_p(master), _p(g), _p(m_q), _p(m_scale), _p(v16), _p(w), n, C.byref(hp),
                               nthreads or default_threads())
    return float(amax), w


def adam_step_delayed(master, grad_bf16, m_q, m_scale, v16, hp: AdamHP, history, pos, want_w=True, nthreads=None):
    """Adam step whose m scale comes from the amax history (float32[H], int32[1] position; both updated in place).
    In place on master, m_q, m_scale, v16 as adam_step. Returns (amax_m, w_bf16)."""
    for a, dt in ((master, np.float32), (m_q, np.uint8), (m_scale, np.float32), (v16, np.uint16),
                  (history, np.float32), (pos, np.int32)):
        assert a.dtype == dt and a.flags.c_contiguous
    g = _c(grad_bf16, np.uint16)
    n = master.size
    w = np.empty(n, np.uint16) if want_w else None
    amax = lib().orc_adam_step_delayed(_p(master), _p(g), _p(m_q), _p(m_scale), _p(v16), _p(w), n, C.byref(hp),
                                       _p(history), history.size, _p(pos), nthreads or default_threads())
    return float(amax), w


def adam_amax(grad_bf16, m_q, v16, m_scale_old, hp: AdamHP, nthreads=None) -> float:
    g = _c(grad_bf16, np.uint16); mq = _c(m_q, np.uint8); v = _c(v16, np.uint16)
    return float(lib().orc_adam_amax(_p(g), _p(mq), _p(v), C.c_float(m_scale_old), g.size, C.byref(hp),
                                     nthreads or default_threads()))


def adam_elements(master, grad_bf16, m_q, v16, m_scale_old, s_new, idx, hp: AdamHP):
    """Pass-2 outputs for the listed element indices (inputs are full arrays): (master', m_q', v16', w_bf16)."""
    th = _c(master, np.float32); g = _c(grad_bf16, np.uint16); mq = _c(m_q, np.uint8); v = _c(v16, np.uint16)
    ix = _c(idx, np.int64)
    om = np.empty(ix.size, np.float32); oq = np.empty(ix.size, np.uint8)
    ov = np.empty(ix.size, np.uint16); ow = np.empty(ix.size, np.uint16)
    lib().orc_adam_elements(_p(th), _p(g), _p(mq), _p(v), C.c_float(m_scale_old), C.c_float(s_new), _p(ix), ix.size,
                            C.byref(hp), _p(om), _p(oq), _p(ov), _p(ow))
    return om, oq, ov, ow
