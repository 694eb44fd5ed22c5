"""GPU parity of the routed-expert backward pieces ("OLMo-core MoE, Section 11: MXFP8 Training", Section 11.4.1 and
Section 11.4.4 / Table 25) against the oracle:

- route_weighted_mx_quantize, swiglu_backward_mx_quantize and swiglu_mx_quantize_oriented: codes and scale bytes
  byte for byte in both orientations, from small and ragged shapes to the grouped workload's full size;
- grouped_scaled_gemm_strided (dgrad reading the column-orientation weight cache in place) and grouped_wgrad_mx (one
  contraction per expert over its token rows, bf16 output or fp32 accumulation) within the GEMM error bound
  |C_gpu - y_ref| <= 2^-7 |y_ref| + 2^-20 S, all elements at small sizes and sampled ones at full size."""
import numpy as np
import pytest
import torch

import mxfp8_precision_numerics_amd as mxq
import oracle
from gpu_util import DEV, need_gpu, say, u16, u8
from mxfp8_precision_numerics_amd import workloads

pytestmark = pytest.mark.gpu

REL, ABS_S = 2.0 ** -7, 2.0 ** -20


def _bound_check(got, y, S, what, extra=None):
    got = np.asarray(got, np.float64)
    err = np.abs(got - y)
    lim = REL * np.abs(y) + ABS_S * S
    if extra is not None:
        lim = lim + extra
    bad = err > lim
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside the bound; first at {i}: gpu={got[i]!r} "
                             f"ref={y[i]!r} S={S[i]!r}")


def _eq_mx(out, ref, what):
    qr, sr, qc, sc = ref[:4]
    if out.q_row is not None:
        assert np.array_equal(u8(out.s_row), sr), what + " s_row"
        assert np.array_equal(u8(out.q_row), qr), what + " q_row"
    if out.q_col is not None:
        assert np.array_equal(u8(out.s_col), sc), what + " s_col"
        assert np.array_equal(u8(out.q_col), qc), what + " q_col"


# ----------------------------------------------------------------------------------------------- route weighting
@pytest.mark.parametrize("rows,cols,rule", [(32, 32, mxq.RCEIL), (96, 160, mxq.FLOOR), (320, 1056, mxq.RCEIL),
                                            (64, 4096, mxq.FLOOR), (256, 384, mxq.RCEIL)])
def test_route_weighted_quantize(rows, cols, rule):
    need_gpu()
    say("route weighted", rows, cols, rule)
    dy = workloads.normal_bf16((rows, cols), 1e-3, 4, 30 + rows, DEV)
    p = workloads.uniform_f32((rows,), 0.01, 1.0, 4, 31 + rows, DEV)
    p[rows // 3] = 0.0
    out = mxq.route_weighted_mx_quantize(dy, p, rule=rule)
    torch.cuda.synchronize()
    ref = oracle.route_weighted_mx_quantize(u16(dy), p.cpu().numpy(), rule)
    _eq_mx(out, ref, "route weighted")


def test_route_weighted_quantize_single_orientations():
    need_gpu()
    rows, cols = 128, 256
    dy = workloads.normal_bf16((rows, cols), 1.0, 4, 32, DEV)
    p = workloads.uniform_f32((rows,), 0.01, 1.0, 4, 33, DEV)
    ref = oracle.route_weighted_mx_quantize(u16(dy), p.cpu().numpy())
    _eq_mx(mxq.route_weighted_mx_quantize(dy, p, rowwise=True, colwise=False), ref, "row only")
    _eq_mx(mxq.route_weighted_mx_quantize(dy, p, rowwise=False, colwise=True), ref, "col only")


def test_route_weighted_quantize_workload4():
    """The combine backward at the grouped workload's size: 132,160 routed rows x d_model 2048, Zipf routing."""
    need_gpu()
    counts, padded, offsets = workloads.zipf_routing()
    rows = int(offsets[-1])
    say("route weighted workload4", rows, 2048)
    dy = workloads.zero_padding_rows(workloads.normal_bf16((rows, 2048), 1e-3, 4, 6, DEV), counts, padded, offsets)
    p = workloads.route_weights(counts, padded, offsets, device=DEV)
    out = mxq.route_weighted_mx_quantize(dy, p)
    torch.cuda.synchronize()
    ref = oracle.route_weighted_mx_quantize(u16(dy), p.cpu().numpy())
    _eq_mx(out, ref, "route weighted workload4")


def test_route_weighted_quantize_extremes():
    """Zero, subnormal, large and infinite gradients with zero, tiny and large weights. Where the fp32 product is a
    NaN made by the arithmetic (0 x inf) its sign is not fixed by IEEE 754, so there both sides must give a NaN code
    and the E8M0 NaN scale byte; every other byte must match."""
    need_gpu()
    vals = np.array([0.0, -0.0, 1e-40, -3e-39, 1.0, -1.5, 3.0e38, -3.3e38, np.inf, -np.inf, 448.0, 449.0, 65504.0,
                     -1e-3, 2.5e-5, 7.0], np.float32)
    rows, cols = 64, 128
    dy = oracle.bf16_from_f32(np.resize(vals, (rows, cols)))
    p = np.resize(np.array([1.0, 0.0, 2.0 ** -30, 3.0, 0.5, 1e30, 2.0 ** 20, 0.75], np.float32), rows)
    out = mxq.route_weighted_mx_quantize(torch.from_numpy(dy.view(np.int16)).view(torch.bfloat16).to(DEV),
                                         torch.from_numpy(p).to(DEV))
    torch.cuda.synchronize()
    qr, sr, qc, sc, x = oracle.route_weighted_mx_quantize(dy, p, want_x=True)
    _compare_nan_tolerant(out, (qr, sr, qc, sc), x)


def _compare_nan_tolerant(out, ref, x):
    qr, sr, qc, sc = ref
    nan = np.isnan(x)
    gr, gc = u8(out.q_row), u8(out.q_col)
    assert np.array_equal(u8(out.s_row), sr) and np.array_equal(u8(out.s_col), sc)
    assert np.array_equal(gr[~nan], qr[~nan]) and np.array_equal(gc[~nan.T], qc[~nan.T])
    assert np.all(gr[nan] & 0x7F == 0x7F) and np.all(qr[nan] & 0x7F == 0x7F)
    assert np.all(gc[nan.T] & 0x7F == 0x7F) and np.all(qc[nan.T] & 0x7F == 0x7F)


# ----------------------------------------------------------------------------------------------- SwiGLU
@pytest.mark.parametrize("rows,F,rule", [(32, 32, mxq.RCEIL), (96, 96, mxq.FLOOR), (320, 544, mxq.RCEIL),
                                         (64, 1024, mxq.RCEIL), (256, 256, mxq.FLOOR)])
def test_swiglu_backward_quantize(rows, F, rule):
    need_gpu()
    say("swiglu backward", rows, F, rule)
    c = workloads.normal_bf16((rows, 2 * F), 2.0, 4, 40 + rows, DEV)
    dh = workloads.normal_bf16((rows, F), 1e-3, 4, 41 + rows, DEV)
    out = mxq.swiglu_backward_mx_quantize(c, dh, rule=rule)
    torch.cuda.synchronize()
    _eq_mx(out, oracle.swiglu_bwd_mx_quantize(u16(c), u16(dh), rule), "swiglu backward")


def test_swiglu_backward_quantize_workload4():
    """The routed MLP's SwiGLU backward at full size: c [132,160][2 x 1024], dh [132,160][1024]."""
    need_gpu()
    counts, padded, offsets = workloads.zipf_routing()
    rows, F = int(offsets[-1]), 1024
    say("swiglu backward workload4", rows, F)
    c = workloads.zero_padding_rows(workloads.normal_bf16((rows, 2 * F), 2.0, 4, 7, DEV), counts, padded, offsets)
    dh = workloads.zero_padding_rows(workloads.normal_bf16((rows, F), 1e-3, 4, 8, DEV), counts, padded, offsets)
    out = mxq.swiglu_backward_mx_quantize(c, dh)
    torch.cuda.synchronize()
    _eq_mx(out, oracle.swiglu_bwd_mx_quantize(u16(c), u16(dh)), "swiglu backward workload4")


def test_swiglu_backward_quantize_single_orientations():
    need_gpu()
    rows, F = 64, 160
    c = workloads.normal_bf16((rows, 2 * F), 3.0, 4, 42, DEV)
    dh = workloads.normal_bf16((rows, F), 1.0, 4, 43, DEV)
    ref = oracle.swiglu_bwd_mx_quantize(u16(c), u16(dh))
    _eq_mx(mxq.swiglu_backward_mx_quantize(c, dh, rowwise=True, colwise=False), ref, "row only")
    _eq_mx(mxq.swiglu_backward_mx_quantize(c, dh, rowwise=False, colwise=True), ref, "col only")


def test_swiglu_backward_quantize_extremes():
    need_gpu()
    vals = np.array([0.0, -0.0, 1e-30, -1e-30, 88.0, 89.0, -88.0, -104.5, 200.0, -200.0, 3.0e38, -3.0e38,
                     np.inf, -np.inf, 1.0, -1.278], np.float32)
    rows, F = 32, 64
    g = np.resize(vals, (rows, F)).astype(np.float32)
    u = np.resize(vals[::-1], (rows, F)).astype(np.float32)
    dhv = np.resize(np.array([1.0, -2.0, 0.0, 1e-3, 3e38, -1e-38, 0.5], np.float32), (rows, F))
    c = oracle.bf16_from_f32(np.concatenate([g, u], axis=1))
    dh = oracle.bf16_from_f32(dhv)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)  # noqa: E731
    out = mxq.swiglu_backward_mx_quantize(to_dev(c), to_dev(dh))
    torch.cuda.synchronize()
    qr, sr, qc, sc, dc = oracle.swiglu_bwd_mx_quantize(c, dh, want_dc=True)
    _compare_nan_tolerant(out, (qr, sr, qc, sc), dc)


@pytest.mark.parametrize("rows,F,rule", [(32, 32, mxq.RCEIL), (96, 160, mxq.FLOOR), (384, 256, mxq.RCEIL),
                                         (132_160, 1024, mxq.RCEIL)])
def test_swiglu_forward_oriented(rows, F, rule):
    """Row orientation equals swiglu_mx_quantize; the column one is the fp32 MX quantize of the same h."""
    need_gpu()
    say("swiglu forward oriented", rows, F, rule)
    c = workloads.normal_bf16((rows, 2 * F), 4.0, 4, 44 + rows, DEV)
    out = mxq.swiglu_mx_quantize_oriented(c, rule=rule)
    row_only = mxq.swiglu_mx_quantize(c, rule)
    torch.cuda.synchronize()
    q, s, h = oracle.swiglu_mx_quantize(u16(c), rule, want_h=True)
    _, _, qc, sc = oracle.mx_quantize_f32(h, rule, rowwise=False)
    _eq_mx(out, (q, s, qc, sc), "swiglu oriented")
    assert torch.equal(out.q_row, row_only.q_row) and torch.equal(out.s_row, row_only.s_row)


# ----------------------------------------------------------------------------------------------- dgrad, strided B
def _col_cache(W):
    """Column-orientation MX cache of expert weights W[G][D][F] refreshed as one [G*D][F] matrix."""
    G, D, F = W.shape
    return mxq.mx_quantize(W.reshape(G * D, F), rowwise=False, colwise=True)


def _experts_from_cache(cache, G, D, F):
    """Host copy of each expert's B operand [G][F][D] and its scales [G][F][D/32] (slicing, no arithmetic)."""
    q = u8(cache.q_col).reshape(F, G, D).transpose(1, 0, 2).copy()
    s = u8(cache.s_col).reshape(F, G, D // 32).transpose(1, 0, 2).copy()
    return q, s


@pytest.mark.parametrize("G,D,F,tokens,extra_cols", [(8, 256, 192, 512, 24), (4, 512, 512, 1024, 0),
                                                     (3, 96, 40, 100, 8)])
def test_grouped_dgrad_strided(G, D, F, tokens, extra_cols):
    need_gpu()
    counts, padded, offsets = workloads.zipf_routing(tokens=tokens, experts=G, topk=2, seed=50 + G)
    if G > 3:
        counts[1] = 0; padded[1] = 0                                   # an empty expert
        offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    total = int(offsets[-1])
    say("grouped dgrad strided", G, D, F, total, extra_cols)
    dY = workloads.zero_padding_rows(workloads.normal_bf16((total, D), 1.0, 4, 51, DEV), counts, padded, offsets)
    W = workloads.normal_bf16((G, D, F), 1.0, 4, 52, DEV)
    qa = mxq.mx_quantize(dY, colwise=False)
    cache = _col_cache(W)
    off_t = torch.from_numpy(offsets).to(DEV)
    out = torch.full((total, F + extra_cols), 7.0, dtype=torch.bfloat16, device=DEV)
    mxq.grouped_scaled_gemm_strided(qa.q_row, qa.s_row, off_t, cache.q_col, cache.s_col, G, F, D, ldb=G * D,
                                    b_group_stride=D, ldbs=G * D // 32, bs_group_stride=D // 32, out=out)
    torch.cuda.synchronize()
    bq, bs = _experts_from_cache(cache, G, D, F)
    y, S = oracle.grouped_gemm_ref(u8(qa.q_row), u8(qa.s_row), offsets, bq, bs)
    got = out.float().cpu().numpy()
    _bound_check(got[:, :F], y, S, "grouped dgrad strided")
    assert np.all(got[:, F:] == 7.0)                                   # past N: untouched
    for g in range(G):
        assert np.all(got[offsets[g] + counts[g]:offsets[g + 1], :F] == 0)


def test_grouped_dgrad_strided_workload4_sampled():
    """The routed down projection's dgrad at full size: dY [132,160][2048] against W_down [64][2048][1024] read from
    its column cache in place (N = 1024, K = 2048)."""
    need_gpu()
    wl_counts, wl_padded, offsets = workloads.zipf_routing()
    total, G, D, F = int(offsets[-1]), 64, 2048, 1024
    say("grouped dgrad strided workload4", total, D, F)
    dY = workloads.zero_padding_rows(workloads.normal_bf16((total, D), 1.0, 4, 9, DEV), wl_counts, wl_padded, offsets)
    W = workloads.normal_bf16((G, D, F), 1.0, 4, 4, DEV)
    qa = mxq.mx_quantize(dY, colwise=False)
    cache = _col_cache(W)
    off_t = torch.from_numpy(offsets).to(DEV)
    C = mxq.grouped_scaled_gemm_strided(qa.q_row, qa.s_row, off_t, cache.q_col, cache.s_col, G, F, D, ldb=G * D,
                                        b_group_stride=D, ldbs=G * D // 32, bs_group_stride=D // 32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(53)
    big, small = int(np.argmax(wl_counts)), int(np.argmin(wl_counts))
    rows = np.concatenate([rng.choice(np.arange(offsets[big], offsets[big] + wl_counts[big]), 6, replace=False),
                           rng.choice(np.arange(offsets[small], offsets[small] + wl_counts[small]), 6, replace=False),
                           rng.choice(total, 12, replace=False)])
    bq, bs = _experts_from_cache(cache, G, D, F)
    y, S = oracle.grouped_gemm_ref(u8(qa.q_row), u8(qa.s_row), offsets, bq, bs, rows=rows)
    _bound_check(C.float().cpu().numpy()[rows], y, S, "grouped dgrad strided workload4")


# ----------------------------------------------------------------------------------------------- Wgrad over tokens
def _token_operand(kt, m, k, std=1.0, counts=None, padded=None, offsets=None):
    """Column-orientation MX operand [m][kt] of a token-major bf16 matrix [kt][m] (blocks of 32 tokens)."""
    x = workloads.normal_bf16((kt, m), std, 4, k, DEV)
    if counts is not None:
        workloads.zero_padding_rows(x, counts, padded, offsets)
    q = mxq.mx_quantize(x, rowwise=False, colwise=True)
    return q.q_col, q.s_col


@pytest.mark.parametrize("M,N,off", [(48, 40, [0, 96, 96, 160, 416, 448]), (200, 136, [0, 64, 64, 64, 352, 544]),
                                     (136, 264, [0, 32]), (64, 64, [0, 0, 0])])
def test_grouped_wgrad_all_elements(M, N, off):
    need_gpu()
    offsets = np.array(off, np.int64)
    G, kt = offsets.size - 1, int(offsets[-1])
    say("grouped wgrad", M, N, offsets.tolist())
    if kt == 0:
        aq = torch.empty((M, 0), dtype=torch.uint8, device=DEV); as_ = torch.empty((M, 0), dtype=torch.uint8, device=DEV)
        bq = torch.empty((N, 0), dtype=torch.uint8, device=DEV); bs = torch.empty((N, 0), dtype=torch.uint8, device=DEV)
    else:
        aq, as_ = _token_operand(kt, M, 60 + M)
        bq, bs = _token_operand(kt, N, 61 + N, 0.3)
    off_t = torch.from_numpy(offsets).to(DEV)
    C = mxq.grouped_wgrad_mx(aq, as_, bq, bs, off_t)
    acc0 = torch.zeros((G, M, N), dtype=torch.float32, device=DEV)
    mxq.grouped_wgrad_mx(aq, as_, bq, bs, off_t, accumulate=acc0)
    torch.cuda.synchronize()
    if kt == 0:
        assert torch.all(C == 0) and torch.all(acc0 == 0)
        return
    y, S = oracle.grouped_wgrad_ref(u8(aq), u8(as_), u8(bq), u8(bs), offsets)
    got = C.float().cpu().numpy()
    _bound_check(got, y, S, "grouped wgrad bf16")
    f32 = acc0.cpu().numpy()
    _bound_check(f32, y, S, "grouped wgrad fp32")
    # the bf16 output is the RNE of the same fp32 sum
    assert np.array_equal(u16(C), oracle.bf16_from_f32(f32))
    for g in range(G):
        if offsets[g] == offsets[g + 1]:
            assert np.all(got[g] == 0) and np.all(f32[g] == 0)


# Large-tile path (M, N >= 256): K ranges of 32 mod 64 end in a half stage, odd Kt/32 leaves scale rows unaligned,
# the last expert ends at the operands' last byte, ranges span several 16-block scale groups.
@pytest.mark.parametrize("M,N,off", [
    (512, 320, [0, 32, 32, 96, 160, 1216, 1248, 1760, 1792]),
    (296, 264, [0, 0, 64, 608, 640, 2784]),
    (256, 256, [0, 32]),
    (264, 512, [0, 544, 544, 1088, 1120, 1632, 1696, 2208]),
])
def test_grouped_wgrad_large_tiles_all_elements(M, N, off):
    need_gpu()
    offsets = np.array(off, np.int64)
    G, kt = offsets.size - 1, int(offsets[-1])
    say("grouped wgrad large tiles", M, N, offsets.tolist())
    aq, as_ = _token_operand(kt, M, 80 + M)
    bq, bs = _token_operand(kt, N, 81 + N, 0.3)
    off_t = torch.from_numpy(offsets).to(DEV)
    C = mxq.grouped_wgrad_mx(aq, as_, bq, bs, off_t)
    acc0 = torch.zeros((G, M, N), dtype=torch.float32, device=DEV)
    mxq.grouped_wgrad_mx(aq, as_, bq, bs, off_t, accumulate=acc0)
    torch.cuda.synchronize()
    y, S = oracle.grouped_wgrad_ref(u8(aq), u8(as_), u8(bq), u8(bs), offsets)
    got = C.float().cpu().numpy()
    f32 = acc0.cpu().numpy()
    _bound_check(got, y, S, "grouped wgrad large tiles bf16")
    _bound_check(f32, y, S, "grouped wgrad large tiles fp32")
    assert np.array_equal(u16(C), oracle.bf16_from_f32(f32))
    for g in range(G):
        if offsets[g] == offsets[g + 1]:
            assert np.all(got[g] == 0) and np.all(f32[g] == 0)


def test_grouped_wgrad_large_tiles_accumulate():
    need_gpu()
    M, N = 256, 384
    offsets = np.array([0, 96, 96, 672], np.int64)
    kt = int(offsets[-1])
    aq, as_ = _token_operand(kt, M, 90)
    bq, bs = _token_operand(kt, N, 91)
    off_t = torch.from_numpy(offsets).to(DEV)
    base = workloads.normal_f32((3, M, N), 5.0, 4, 92, DEV)
    sink = base.clone()
    mxq.grouped_wgrad_mx(aq, as_, bq, bs, off_t, accumulate=sink)
    fresh = torch.zeros_like(base)
    mxq.grouped_wgrad_mx(aq, as_, bq, bs, off_t, accumulate=fresh)
    torch.cuda.synchronize()
    assert np.array_equal(sink.cpu().numpy(), (base.cpu().numpy() + fresh.cpu().numpy()).astype(np.float32))


def test_grouped_wgrad_accumulates_into_fp32():
    """Two calls into one fp32 sink: each adds its sum with one rounding (the high-precision gradient sink)."""
    need_gpu()
    M, N = 96, 80
    offsets = np.array([0, 128, 160, 416], np.int64)
    kt = int(offsets[-1])
    aq, as_ = _token_operand(kt, M, 70)
    bq, bs = _token_operand(kt, N, 71)
    off_t = torch.from_numpy(offsets).to(DEV)
    base = workloads.normal_f32((3, M, N), 5.0, 4, 72, DEV)
    sink = base.clone()
    mxq.grouped_wgrad_mx(aq, as_, bq, bs, off_t, accumulate=sink)
    once = sink.clone()
    mxq.grouped_wgrad_mx(aq, as_, bq, bs, off_t, accumulate=sink)
    fresh = torch.zeros_like(base)
    mxq.grouped_wgrad_mx(aq, as_, bq, bs, off_t, accumulate=fresh)
    torch.cuda.synchronize()
    s = fresh.cpu().numpy()
    b = base.cpu().numpy()
    assert np.array_equal(once.cpu().numpy(), (b + s).astype(np.float32))
    assert np.array_equal(sink.cpu().numpy(), ((b + s).astype(np.float32) + s).astype(np.float32))
    y, S = oracle.grouped_wgrad_ref(u8(aq), u8(as_), u8(bq), u8(bs), offsets)
    _bound_check(s, y, S, "fresh sink")


def test_grouped_wgrad_workload4_sampled():
    """The routed down projection's Wgrad at full size: dW_g [2048][1024] = dY_g^T h_g over each expert's token
    rows (132,160 routed rows), operands in the column orientation; sampled experts, rows and columns."""
    need_gpu()
    counts, padded, offsets = workloads.zipf_routing()
    kt, G, D, F = int(offsets[-1]), 64, 2048, 1024
    say("grouped wgrad workload4", kt, D, F)
    aq, as_ = _token_operand(kt, D, 10, 1e-3, counts, padded, offsets)
    bq, bs = _token_operand(kt, F, 11, 1.0, counts, padded, offsets)
    off_t = torch.from_numpy(offsets).to(DEV)
    C = mxq.grouped_wgrad_mx(aq, as_, bq, bs, off_t)
    torch.cuda.synchronize()
    rng = np.random.default_rng(73)
    groups = np.array([int(np.argmax(counts)), int(np.argmin(counts)), 17], np.int64)
    rows = rng.choice(D, 24, replace=False)
    cols = rng.choice(F, 24, replace=False)
    y, S = oracle.grouped_wgrad_ref(u8(aq), u8(as_), u8(bq), u8(bs), offsets, groups=groups, rows=rows, cols=cols)
    got = C.float().cpu().numpy()[groups][:, rows][:, :, cols]
    _bound_check(got, y, S, "grouped wgrad workload4")
