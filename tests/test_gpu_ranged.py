"""GPU checks of the range words (mxq_quantize_ranged) and the ranged GEMM (scaled_gemm_ranged).

- mxq_quantize_ranged writes the same codes and scale bytes as mxq_quantize, and each orientation's word equals the
  range definition evaluated on the host over that orientation's codes (normal and wide-range operands, ragged
  tiles, windows planted at either side of the 23 / 24 boundary along a row and down a column, zero tensors).
- scaled_gemm_ranged, given the words of its operands, returns scaled_gemm's bytes (the checked path) on normal and
  wide-range operands, and on the workload-2 forward shape the words of X and W are 0, so the FP8 instruction runs.
"""
import numpy as np
import pytest
import torch

import mxfp8_precision_numerics_amd as mxq
import oracle
from gpu_util import DEV, any_wide_window, from_u16, need_gpu, say, u16, u8
from mxfp8_precision_numerics_amd import workloads

pytestmark = pytest.mark.gpu


def _check_words(x, rule=mxq.RCEIL):
    got, words = mxq.mx_quantize_ranged(x, rule=rule)
    ref = mxq.mx_quantize(x, rule=rule)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
    w = words.cpu().numpy()
    want = (any_wide_window(u8(got.q_row), u8(got.s_row)), any_wide_window(u8(got.q_col), u8(got.s_col)))
    assert (bool(w[0]), bool(w[1])) == want, (w, want)
    return want


@pytest.mark.parametrize("shape", [(64, 64), (192, 320), (256, 512), (320, 192), (1024, 768)])
@pytest.mark.parametrize("kind", ["normal"] + list(workloads.WIDE_RANGE_KINDS))
def test_range_words_match_the_definition(shape, kind):
    need_gpu()
    say("range words", shape, kind)
    if kind == "normal":
        x = workloads.normal_bf16(shape, 1.0, 45, shape[0] + shape[1], DEV)
    else:
        x = workloads.wide_range_bf16(shape, kind, 45, shape[0] + 7 * shape[1], DEV)
    want = _check_words(x)
    if kind == "normal":
        assert want == (False, False)
    elif shape[0] * shape[1] >= 65536 and kind in ("loguniform", "sparse"):
        assert want == (True, True)
    elif shape[0] * shape[1] >= 65536 and kind == "colscale":     # scaled columns spread along rows only
        assert want[0]


@pytest.mark.parametrize("n_small", [23, 24])
@pytest.mark.parametrize("orient", ["row", "col"])
def test_range_words_planted_window(n_small, orient):
    """A 64-value window (along a row, or down a column) of 1.0 values in which n_small values are 2^-8: with the
    block scale 2^-8 the ones are code 0x78 (exponent field 15) and the small ones 0x38 (field 7), 8 binades down."""
    need_gpu()
    say("range words planted", orient, n_small)
    rows, cols = 256, 384
    x = u16(workloads.normal_bf16((rows, cols), 1.0, 46, 1, DEV))
    one, tiny = 0x3F80, 0x3B80                    # bf16 1.0 and 2^-8
    if orient == "row":
        x[37, 128:192] = one
        x[37, 128:128 + n_small] = tiny
    else:
        x[64:128, 201] = one
        x[64:64 + n_small, 201] = tiny
    want = _check_words(from_u16(x))
    assert want == ((orient == "row" and n_small == 24), (orient == "col" and n_small == 24))


def test_range_words_zero_and_empty():
    """An all-zero tensor has no wide window; an empty x (rows = 0) still clears both words (through the C ABI, with
    output buffers that are never written)."""
    import ctypes as C

    from mxfp8_precision_numerics_amd import _lib
    need_gpu()
    _check_words(torch.zeros((128, 256), dtype=torch.bfloat16, device=DEV))
    buf = torch.full((256,), 0x5A, dtype=torch.uint8, device=DEV)
    words = torch.full((2,), 7, dtype=torch.int32, device=DEV)
    p = lambda t, off=0: C.c_void_p(t.data_ptr() + off)  # noqa: E731
    st = _lib.load().mxq_quantize_ranged(p(buf), 0, 64, p(buf), p(buf, 64), p(buf, 128), p(buf, 192), 0,
                                         p(words), p(words, 4), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert words.tolist() == [0, 0]
    assert torch.all(buf == 0x5A)


@pytest.mark.parametrize("kind", ["normal"] + list(workloads.WIDE_RANGE_KINDS))
@pytest.mark.parametrize("M,N,K", [(512, 576, 12288), (256, 320, 12288), (640, 512, 4096)])
def test_ranged_gemm_equals_checked_gemm(kind, M, N, K):
    need_gpu()
    say("ranged gemm", kind, M, N, K)
    if kind == "normal":
        A = workloads.normal_bf16((M, K), 1.0, 47, 1, DEV)
        B = workloads.normal_bf16((N, K), 1.0, 47, 2, DEV)
    else:
        A = workloads.wide_range_bf16((M, K), kind, 47, 3, DEV)
        B = workloads.wide_range_bf16((N, K), kind, 47, 4, DEV)
    qa, wa = mxq.mx_quantize_ranged(A, colwise=False)
    qb, wb = mxq.mx_quantize_ranged(B, colwise=False)
    c_r = mxq.scaled_gemm_ranged(qa.q_row, qa.s_row, wa[0:1], qb.q_row, qb.s_row, wb[0:1])
    c_c = mxq.scaled_gemm(qa.q_row, qa.s_row, qb.q_row, qb.s_row, mxq.MX_BLOCK32)
    torch.cuda.synchronize()
    assert torch.equal(c_r.view(torch.int16), c_c.view(torch.int16))
    y, S = oracle.gemm_ref(u8(qa.q_row), u8(qa.s_row), oracle.E4M3, u8(qb.q_row), u8(qb.s_row), oracle.E4M3,
                           oracle.MX_BLOCK32)
    err = np.abs(c_r.float().cpu().numpy().astype(np.float64) - y)
    assert np.all(err <= 2.0 ** -7 * np.abs(y) + 2.0 ** -20 * S)


def test_workload2_words_take_fp8():
    """The linear layer's operands (X, W, dY in both orientations) are normal: every word is 0, and the ranged forward
    and dgrad GEMMs at full size return the FP8 instruction's bytes."""
    need_gpu()
    X, W, dY = workloads.workload2(DEV)
    (qx, wx), (qw, ww), (qd, wd) = (mxq.mx_quantize_ranged(t) for t in (X, W, dY))
    del X, W, dY
    torch.cuda.synchronize()
    assert wx.tolist() == [0, 0] and ww.tolist() == [0, 0] and wd.tolist() == [0, 0]
    for a, aw, b, bw in ((qx.q_row, qx.s_row, qw.q_row, qw.s_row), (qd.q_row, qd.s_row, qw.q_col, qw.s_col)):
        c_r = mxq.scaled_gemm_ranged(a, aw, wx[0:1], b, bw, ww[0:1])
        c_f = mxq.scaled_gemm(a, aw, b, bw, mxq.MX_BLOCK32, path="fp8")
        torch.cuda.synchronize()
        assert torch.equal(c_r.view(torch.int16), c_f.view(torch.int16))
        del c_r, c_f
