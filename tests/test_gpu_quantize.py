"""GPU parity of the quantize kernels against the oracle: qdata, scale bytes, amax and scale must match bit for bit.

Inputs are seeded synthetic tensors drawn on the GPU and copied to the host for the oracle. Non-finite inputs are
outside the numeric contract; their bytes are still defined (NaN codes compared as NaN, scale byte 0xFF)."""
import numpy as np
import pytest
import torch

import mxfp8_precision_numerics_amd as mxq
import oracle
from gpu_util import DEV, from_u16, need_gpu, say, u16, u8
from mxfp8_precision_numerics_amd import workloads

pytestmark = pytest.mark.gpu

RULES = [(mxq.RCEIL, oracle.RCEIL), (mxq.FLOOR, oracle.FLOOR)]


def _check_mx(x: torch.Tensor, rule, orule, rowwise=True, colwise=True):
    out = mxq.mx_quantize(x, rowwise=rowwise, colwise=colwise, rule=rule)
    torch.cuda.synchronize()
    qr, sr, qc, sc = oracle.mx_quantize(u16(x), orule, rowwise, colwise)
    if rowwise:
        assert np.array_equal(u8(out.s_row), sr), "row scales"
        assert np.array_equal(u8(out.q_row), qr), "row qdata"
    if colwise:
        assert np.array_equal(u8(out.s_col), sc), "col scales"
        assert np.array_equal(u8(out.q_col), qc), "col qdata"
    return out


@pytest.mark.parametrize("shape", [(32, 32), (128, 128), (96, 160), (160, 96), (256, 320), (416, 288), (32, 1024)])
@pytest.mark.parametrize("rule,orule", RULES)
def test_mx_quantize_small_shapes(shape, rule, orule):
    need_gpu()
    say("mx quantize", shape, rule)
    x = workloads.normal_bf16_with_outliers(shape, 1.0, 0.01, 100.0, 11, shape[0], shape[1], DEV)
    _check_mx(x, rule, orule)
    _check_mx(x, rule, orule, rowwise=True, colwise=False)
    _check_mx(x, rule, orule, rowwise=False, colwise=True)


@pytest.mark.parametrize("rule,orule", RULES)
def test_mx_quantize_every_block_maximum(rule, orule):
    """One 32-value block per positive finite bf16 maximum (all 32,640), plus zero and subnormal blocks; the other
    31 values are random fractions of the maximum with random signs (RNE ties and subnormal results included)."""
    need_gpu()
    rng = np.random.default_rng(5)
    amax_bits = np.arange(0, 0x7F80, dtype=np.uint32)
    nb = amax_bits.size
    frac_bits = rng.integers(0, 0x3F80, size=(nb, 31), dtype=np.uint32)   # |value| < 1.0 as bf16
    amax_f = (amax_bits << 16).view(np.float32)
    vals = (frac_bits << 16).view(np.float32) * amax_f[:, None]
    vals = oracle.bf16_from_f32(vals.astype(np.float32))
    vals = np.minimum(vals & 0x7FFF, amax_bits[:, None].astype(np.uint16)) | (rng.integers(0, 2, (nb, 31)) << 15).astype(np.uint16)
    blocks = np.concatenate([amax_bits[:, None].astype(np.uint16) | (rng.integers(0, 2, (nb, 1)) << 15).astype(np.uint16), vals], axis=1)
    pos = rng.permuted(np.tile(np.arange(32), (nb, 1)), axis=1)
    blocks = np.take_along_axis(blocks, pos, axis=1)
    x = blocks.reshape(-1, 32 * 32)                 # 1020 rows x 1024 cols: 32 blocks per row
    x = np.concatenate([x, np.zeros((1024 - x.shape[0], 1024), np.uint16)])   # zero blocks pad to 1024 rows
    say("exhaustive block maxima", x.shape, rule)
    _check_mx(from_u16(x), rule, orule, rowwise=True, colwise=False)
    # the same blocks laid down columns
    _check_mx(from_u16(np.ascontiguousarray(x.T)), rule, orule, rowwise=False, colwise=True)


@pytest.mark.parametrize("rule,orule", RULES)
def test_mx_quantize_non_finite_and_special_blocks(rule, orule):
    need_gpu()
    x = np.full((64, 64), 0x3F80, np.uint16)
    x[0, :32] = 0                                   # all zero
    x[1, :32] = 0x8000                              # all negative zero
    x[2, 5] = 0x7F80                                # +inf in a block
    x[3, 40] = 0xFF80                               # -inf
    x[4, 7] = 0x7FC0                                # NaN
    x[5, 33] = 0xFFC1                               # -NaN
    x[6, :32] = 0x0001                              # bf16 subnormals
    x[7, 3] = 0x43E0                                # 448 exactly
    x[8, 3] = 0x43E8                                # 464: a tie that saturates under floor
    x[9, 0:32] = 0x7F7F                             # bf16 max
    x[:, 63] = 0xC3F0                               # -480 in every row's last block (floor saturates)
    x[40, :] = 0x7FC0                               # a NaN row: every column block below sees a NaN
    xt = from_u16(x)
    out = mxq.mx_quantize(xt, rule=rule)
    torch.cuda.synchronize()
    qr, sr, qc, sc = oracle.mx_quantize(x, orule)
    assert np.array_equal(u8(out.s_row), sr) and np.array_equal(u8(out.s_col), sc)
    for got, want in ((u8(out.q_row), qr), (u8(out.q_col), qc)):
        nan_w = (want & 0x7F) == 0x7F
        assert np.array_equal(nan_w, (got & 0x7F) == 0x7F)
        assert np.array_equal(got[~nan_w], want[~nan_w])


def test_mx_quantize_workload1_operands():
    need_gpu()
    A, B = workloads.workload1(DEV)
    _check_mx(A, mxq.RCEIL, oracle.RCEIL, rowwise=True, colwise=False)
    _check_mx(B, mxq.RCEIL, oracle.RCEIL, rowwise=False, colwise=True)


def test_mx_quantize_workload3_full_size_and_storage():
    """The 16384 x 8192 activation with 0.1% x100 outliers, both orientations, bit-exact; 33/32 bytes per value."""
    need_gpu()
    x = workloads.workload3(DEV)
    say("workload3 full size", tuple(x.shape))
    out = _check_mx(x, mxq.RCEIL, oracle.RCEIL)
    n = x.numel()
    assert (out.q_row.numel() + out.s_row.numel()) * 32 == 33 * n
    assert (out.q_col.numel() + out.s_col.numel()) * 32 == 33 * n
    again = mxq.mx_quantize(x)
    torch.cuda.synchronize()
    for a, b in zip(out, again):
        assert torch.equal(a, b)                    # deterministic: same bytes on a second run


# ------------------------------------------------------------------------------------------- per-tensor
def _check_pt(x, fmt, ofmt, margin=1.0, scale_in=None, want_q=True, want_qt=True):
    sin_t = None if scale_in is None else torch.tensor([scale_in], dtype=torch.float32, device=DEV)
    r = mxq.pertensor_quantize(x, fmt, margin, sin_t, want_q, want_qt)
    torch.cuda.synchronize()
    amax, s, q, qt = oracle.pertensor_quantize(u16(x), ofmt, margin, scale_in, want_q, want_qt)
    assert r.amax.item() == amax
    assert np.float32(r.scale.item()) == s
    for got, want in ((r.q, q), (r.q_t, qt)):
        if got is None:
            continue
        g = u8(got)
        assert np.array_equal(g, want)
    return r


@pytest.mark.parametrize("shape", [(32, 32), (128, 256), (96, 200), (352, 136)])
@pytest.mark.parametrize("fmt,ofmt,std", [(mxq.E4M3, oracle.E4M3, 1.0), (mxq.E5M2, oracle.E5M2, 1e-3)])
def test_pertensor_small_shapes(shape, fmt, ofmt, std):
    need_gpu()
    say("per-tensor", shape, fmt)
    x = workloads.normal_bf16(shape, std, 12, shape[0] * 7 + shape[1], DEV)
    _check_pt(x, fmt, ofmt)
    _check_pt(x, fmt, ofmt, want_qt=False)
    _check_pt(x, fmt, ofmt, want_q=False)
    _check_pt(x, fmt, ofmt, margin=0.5)


@pytest.mark.parametrize("fmt,ofmt", [(mxq.E4M3, oracle.E4M3), (mxq.E5M2, oracle.E5M2)])
def test_pertensor_delayed_scale_saturates_and_zero_tensor(fmt, ofmt):
    need_gpu()
    x = workloads.normal_bf16((64, 64), 1.0, 13, 0, DEV)
    _check_pt(x, fmt, ofmt, scale_in=4096.0)       # a stale (delayed) scale far too large: saturation
    z = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    _check_pt(z, fmt, ofmt)


def test_pertensor_workload2_tensors_full_size():
    need_gpu()
    X, W, dY = workloads.workload2(DEV)
    for name, t, fmt, ofmt in (("X", X, mxq.E4M3, oracle.E4M3), ("W", W, mxq.E4M3, oracle.E4M3),
                               ("dY", dY, mxq.E5M2, oracle.E5M2)):
        say("workload2 per-tensor", name, tuple(t.shape))
        _check_pt(t, fmt, ofmt)


@pytest.mark.parametrize("rows,cols", [(0, 64), (64, 0), (0, 0)])
@pytest.mark.parametrize("fmt,fmax", [(mxq.E4M3, 448.0), (mxq.E5M2, 57344.0)])
def test_pertensor_empty_tensor_with_outputs(rows, cols, fmt, fmax):
    """An empty x with both code outputs given: MXQ_OK, amax 0 and the scale of the 1e-12 clamp, and nothing written
    to q or q_t (guard bytes stay as they were)."""
    import ctypes as C

    from mxfp8_precision_numerics_amd import _lib
    need_gpu()
    x = torch.empty(16, dtype=torch.bfloat16, device=DEV)
    q = torch.full((64,), 0x5A, dtype=torch.uint8, device=DEV)
    qt = torch.full((64,), 0x5A, dtype=torch.uint8, device=DEV)
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    scale = torch.zeros(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(mxq.workspace_bytes("pertensor", 0), dtype=torch.uint8, device=DEV)
    ptr = lambda t: C.c_void_p(t.data_ptr())  # noqa: E731
    st = _lib.load().fp8_quantize_pertensor(ptr(x), rows, cols, fmt, C.c_float(1.0), None, ptr(amax), ptr(scale),
                                            ptr(q), ptr(qt), ptr(ws), ws.numel(),
                                            C.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert amax.item() == 0.0
    assert scale.item() == np.float32(fmax) / np.float32(1e-12)
    assert torch.all(q == 0x5A) and torch.all(qt == 0x5A)
