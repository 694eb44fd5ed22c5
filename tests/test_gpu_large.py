"""GPU checks past 32-bit offsets: every entry point here is driven with tensors of more than 2^31 elements (or
operands of more than 2^31 bytes), and slabs at the far end (and around the 2^31 boundary) are compared with the
oracle, so that an index or byte offset computed in 32 bits anywhere on the path would show.

- mx_quantize, both orientations, x of 66048 x 32768 bf16 (2.16e9 elements): the row-orientation codes and scales of
  three 32-row slabs (the first rows, across element 2^31, the last rows) and the column-orientation codes and scales
  of the same rows (those land past byte 2^31 of q_col for the high columns), bit for bit.
- fp8_quantize_pertensor on the same x with its largest magnitude planted at the last element: amax and scale equal
  the oracle's (the slab holding the planted value has the tensor's amax), q and q^T of the last rows bit for bit.
- scaled_gemm (checked, FP8 instruction and exact path; large and small tiles) and grouped_scaled_gemm with an MX
  operand of 196608 x 12288 codes (2.4 GB): rows past byte 2^31 and around it within the bound of the oracle's fp64
  GEMM.
- fp8_adam_step over 2^31 + 4099 parameters (a ragged tail): the m scale equals the oracle's over every element and
  sampled elements past 2^31 (and the tail) match bit for bit.
- On the same 2.16e9-element x: the delayed-scaling cast (amax, history, q and q^T of the last rows), the auto-scaled
  gradient cast and the requantize to a shared scale (only the planted value saturates, so the overflow count and
  the next mu follow from the last rows), and the fused SwiGLU quantize with x as [gate | up]; and the Adam step fused
  with the weight-cache refresh on a 66048 x 32768 weight, both cache orientations of three row slabs.
- The rest of the boundary: mxq_quantize_ranged (codes of both orientations), scaled_gemm_ranged on the large operand
  with its range words, swiglu_mx_quantize_oriented, route_weighted_mx_quantize and swiglu_backward_mx_quantize on x
  (both orientations), grouped_scaled_gemm_strided with B at padded row and expert strides, grouped_wgrad_mx over
  4.2e6 tokens (a 2.1 GB operand, so the token-range kernel runs past byte 2^31), and fp8_adam_step_delayed over
  2^31 + 4099 parameters.
"""
import numpy as np
import pytest
import torch

import mxfp8_precision_numerics_amd as mxq
import oracle
from gpu_util import DEV, need_gpu, say, u8, u16
from mxfp8_precision_numerics_amd import workloads

pytestmark = pytest.mark.gpu

REL, ABS_S = 2.0 ** -7, 2.0 ** -20
QR, QC = 66048, 32768                      # 2,164,260,864 elements
GM, GK = 196608, 12288                     # 2,415,919,104 code bytes
PLANT = 100.0                              # far above any N(0, 1) sample, exact in bf16


@pytest.fixture(scope="module")
def big_x():
    need_gpu()
    say("large x", QR, QC)
    x = workloads.normal_bf16((QR, QC), 1.0, 61, 1, DEV)
    x[-1, -1] = PLANT
    yield x
    del x
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def big_a():
    """The MX row orientation of a 196608 x 12288 operand and its range words (from mx_quantize_ranged)."""
    need_gpu()
    say("large A", GM, GK)
    qa, wa = mxq.mx_quantize_ranged(workloads.normal_bf16((GM, GK), 1.0, 62, 1, DEV), colwise=False)
    torch.cuda.empty_cache()
    yield qa, wa
    del qa, wa
    torch.cuda.empty_cache()


def _slabs(rows, cols, block):
    """Row slabs (start, stop): the first rows, the rows holding element (or byte) 2^31, the last rows."""
    cross = (2 ** 31 // cols) // block * block
    return [(0, block), (cross, cross + 2 * block), (rows - 3 * block, rows)]


def test_mx_quantize_past_2_31_elements(big_x):
    say("mx_quantize past 2^31 elements")
    out = mxq.mx_quantize(big_x)
    torch.cuda.synchronize()
    for r0, r1 in _slabs(QR, QC, 32):
        xs = u16(big_x[r0:r1])
        q_row, s_row, q_col, s_col = oracle.mx_quantize(xs)
        assert np.array_equal(u8(out.q_row[r0:r1]), q_row), (r0, r1)
        assert np.array_equal(u8(out.s_row[r0:r1]), s_row), (r0, r1)
        assert np.array_equal(u8(out.q_col[:, r0:r1]), q_col), (r0, r1)
        assert np.array_equal(u8(out.s_col[:, r0 // 32:r1 // 32]), s_col), (r0, r1)
    del out
    torch.cuda.empty_cache()


def test_pertensor_quantize_past_2_31_elements(big_x):
    say("fp8_quantize_pertensor past 2^31 elements")
    pt = mxq.pertensor_quantize(big_x, mxq.E4M3)
    torch.cuda.synchronize()
    r0 = QR - 64
    amax, scale, q, qt = oracle.pertensor_quantize(u16(big_x[r0:]), oracle.E4M3)
    assert amax == PLANT
    assert np.float32(pt.amax.item()) == np.float32(amax) and np.float32(pt.scale.item()) == scale
    assert np.array_equal(u8(pt.q[r0:]), q)
    assert np.array_equal(u8(pt.q_t[:, r0:]), qt)
    del pt
    torch.cuda.empty_cache()


def _ratio(C, y, S):
    err = np.abs(C.float().cpu().numpy().astype(np.float64) - y)
    return float(np.max(err / (REL * np.abs(y) + ABS_S * S)))


@pytest.mark.parametrize("N,path", [(512, "checked"), (512, "exact"), (256, "fp8"), (256, "exact")],
                         ids=["large tiles checked", "large tiles exact", "small tiles fp8", "small tiles exact"])
def test_scaled_gemm_past_2_31_bytes(big_a, N, path):
    say("scaled_gemm past 2^31 bytes", N, path)
    big_a = big_a[0]
    qb = mxq.mx_quantize(workloads.normal_bf16((N, GK), 1.0, 62, 2, DEV), colwise=False)
    C = mxq.scaled_gemm(big_a.q_row, big_a.s_row, qb.q_row, qb.s_row, mxq.MX_BLOCK32, path=path)
    torch.cuda.synchronize()
    bq, bs = u8(qb.q_row), u8(qb.s_row)
    for r0, r1 in _slabs(GM, GK, 64)[1:]:
        y, S = oracle.gemm_ref(u8(big_a.q_row[r0:r1]), u8(big_a.s_row[r0:r1]), oracle.E4M3, bq, bs, oracle.E4M3,
                               oracle.MX_BLOCK32)
        r = _ratio(C[r0:r1], y, S)
        say(f"  rows {r0}..{r1}: worst |err| / bound {r:.3f}")
        assert r <= 1.0


def test_grouped_gemm_past_2_31_bytes(big_a):
    say("grouped_scaled_gemm past 2^31 bytes")
    big_a = big_a[0]
    G, N = 4, 512
    offsets = np.array([0, 32768, 65536 + 96, 131072 + 32, GM], np.int64)
    W = workloads.normal_bf16((G * N, GK), 1.0, 62, 3, DEV)
    qw = mxq.mx_quantize(W, colwise=False)
    del W
    bq, bs = qw.q_row.view(G, N, GK), qw.s_row.view(G, N, GK // 32)
    C = mxq.grouped_scaled_gemm(big_a.q_row, big_a.s_row, torch.from_numpy(offsets).to(DEV), bq, bs)
    torch.cuda.synchronize()
    hq, hs = u8(bq), u8(bs)
    for r0, r1 in _slabs(GM, GK, 64)[1:]:
        # the slab lies in the last group, whose rows start at offsets[3]
        sub_off = np.array([0, 0, 0, 0, r1 - r0], np.int64)
        y, S = oracle.grouped_gemm_ref(u8(big_a.q_row[r0:r1]), u8(big_a.s_row[r0:r1]), sub_off, hq, hs)
        r = _ratio(C[r0:r1], y, S)
        say(f"  rows {r0}..{r1}: worst |err| / bound {r:.3f}")
        assert r <= 1.0


def test_adam_past_2_31_elements():
    need_gpu()
    n = 2 ** 31 + 4099
    say("adam past 2^31 elements", n)
    theta = workloads.workload5_params(n, DEV)
    m_q = torch.zeros(n, dtype=torch.uint8, device=DEV)
    m_scale = torch.ones(1, dtype=torch.float32, device=DEV)
    v = torch.zeros(n, dtype=torch.float16, device=DEV)
    w = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    g = workloads.workload5_grad(n, 1, DEV)
    hp = mxq.AdamHParams(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
    ohp = oracle.AdamHP(1e-4, 0.9, 0.95, 1e-8, 0.1, 1)
    rng = np.random.default_rng(63)
    idx = np.unique(np.concatenate([rng.choice(n, 200_000, replace=False), np.arange(2 ** 31 - 64, 2 ** 31 + 64),
                                    np.arange(n - 4099 - 8, n)])).astype(np.int64)
    gh, mh, vh = u16(g), u8(m_q), u16(v)
    idx_t = torch.from_numpy(idx).to(DEV)
    th_s = theta[idx_t].cpu().numpy()
    amax = oracle.adam_amax(gh, mh, vh, np.float32(1.0), ohp)
    s_new = np.float32(448.0) / np.float32(max(amax, 1e-12))
    full_th = np.zeros(n, np.float32)
    full_th[idx] = th_s
    om, oq, ov, ow = oracle.adam_elements(full_th, gh, mh, vh, np.float32(1.0), s_new, idx, ohp)
    del gh, mh, vh, full_th
    mxq.fp8_adam_step(theta, g, m_q, m_scale, v, w, hp)
    torch.cuda.synchronize()
    assert np.float32(m_scale.item()) == s_new
    assert np.array_equal(theta[idx_t].cpu().numpy().view(np.uint32), om.view(np.uint32))
    assert np.array_equal(m_q[idx_t].cpu().numpy(), oq)
    assert np.array_equal(v[idx_t].cpu().numpy().view(np.uint16), ov)
    assert np.array_equal(w[idx_t].view(torch.int16).cpu().numpy().view(np.uint16), ow)
    del theta, m_q, v, w, g
    torch.cuda.empty_cache()


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


def test_pertensor_delayed_past_2_31_elements(big_x):
    say("fp8_quantize_pertensor_delayed past 2^31 elements")
    hist = torch.tensor([3.0, 5.0], dtype=torch.float32, device=DEV)
    pos = torch.zeros(1, dtype=torch.int32, device=DEV)
    r = mxq.pertensor_quantize_delayed(big_x, hist, pos, mxq.E4M3)
    torch.cuda.synchronize()
    r0 = QR - 64
    o_hist, o_pos = np.array([3.0, 5.0], np.float32), np.zeros(1, np.int32)
    a, s, q, qt = oracle.pertensor_quantize_delayed(u16(big_x[r0:]), o_hist, o_pos, oracle.E4M3)
    assert a == PLANT and np.float32(r.amax.item()) == np.float32(a)
    assert _bits(r.scale)[0] == np.float32(s).view(np.uint32)
    assert np.array_equal(u8(r.q[r0:]), q) and np.array_equal(u8(r.q_t[:, r0:]), qt)
    assert np.array_equal(_bits(hist), o_hist.view(np.uint32)) and int(pos.item()) == int(o_pos[0])
    del r
    torch.cuda.empty_cache()


def test_autoscale_and_requantize_past_2_31_elements(big_x):
    say("fp8_autoscale_cast + fp8_requantize_shared past 2^31 elements")
    g = big_x.view(-1)
    mu = torch.tensor([5.0], dtype=torch.float32, device=DEV)
    r = mxq.fp8_autoscale_cast(g, mu, mxq.E4M3)
    torch.cuda.synchronize()
    tail = 64 * QC                      # the last 64 rows; 5 x PLANT is the only value past 448
    q, cnt, s, o_mu = oracle.autoscale_cast(u16(g[-tail:]), 5.0, oracle.E4M3)
    assert cnt == 1 and int(r.overflow.item()) == 1
    assert _bits(r.scale)[0] == s.view(np.uint32) and _bits(mu)[0] == o_mu.view(np.uint32)
    assert np.array_equal(u8(r.q[-tail:]), q)
    gathered = torch.cat([r.scale, 2.0 ** torch.arange(-3, 4, dtype=torch.float32, device=DEV)])
    rq, sg, _ = mxq.fp8_requantize_shared(r.q, mxq.E4M3, r.scale, gathered, mxq.E4M3)
    torch.cuda.synchronize()
    o_sg = oracle.min_scale(gathered.cpu().numpy())
    assert _bits(sg)[0] == o_sg.view(np.uint32)
    assert np.array_equal(u8(rq[-tail:]), oracle.requantize_shared(q, oracle.E4M3, float(s), float(o_sg), oracle.E4M3))
    del r, rq
    torch.cuda.empty_cache()


def test_swiglu_quantize_past_2_31_elements(big_x):
    say("swiglu_mx_quantize past 2^31 input elements")
    out = mxq.swiglu_mx_quantize(big_x)
    torch.cuda.synchronize()
    for r0, r1 in _slabs(QR, QC, 32):
        q, s, _ = oracle.swiglu_mx_quantize(u16(big_x[r0:r1]))
        assert np.array_equal(u8(out.q_row[r0:r1]), q), (r0, r1)
        assert np.array_equal(u8(out.s_row[r0:r1]), s), (r0, r1)
    del out
    torch.cuda.empty_cache()


def test_adam_weight_cache_past_2_31_elements():
    need_gpu()
    rows, cols = QR, QC
    n = rows * cols
    say("fp8_adam_step_mx_cache past 2^31 elements", rows, cols)
    theta = workloads.workload5_params(n, DEV)
    m_q = torch.zeros(n, dtype=torch.uint8, device=DEV)
    m_scale = torch.ones(1, dtype=torch.float32, device=DEV)
    v = torch.zeros(n, dtype=torch.float16, device=DEV)
    g = workloads.workload5_grad(n, 1, DEV)
    hp = mxq.AdamHParams(3e-4, 0.9, 0.95, 1e-8, 0.1, 1)
    ohp = oracle.AdamHP(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
    slabs = _slabs(rows, cols, 32)
    idx = np.concatenate([np.arange(r0 * cols, r1 * cols, dtype=np.int64) for r0, r1 in slabs])
    gh, mh, vh = u16(g), u8(m_q), u16(v)
    idx_t = torch.from_numpy(idx).to(DEV)
    th_s = theta[idx_t].cpu().numpy()
    amax = oracle.adam_amax(gh, mh, vh, np.float32(1.0), ohp)
    s_new = np.float32(448.0) / np.float32(max(amax, 1e-12))
    full_th = np.zeros(n, np.float32)
    full_th[idx] = th_s
    om, oq, ov, _ = oracle.adam_elements(full_th, gh, mh, vh, np.float32(1.0), s_new, idx, ohp)
    del gh, mh, vh, full_th
    cache = mxq.fp8_adam_step_mx_cache(theta, g, m_q, m_scale, v, None, hp, rows, cols)
    torch.cuda.synchronize()
    assert np.float32(m_scale.item()) == s_new
    assert np.array_equal(theta[idx_t].cpu().numpy().view(np.uint32), om.view(np.uint32))
    assert np.array_equal(m_q[idx_t].cpu().numpy(), oq)
    assert np.array_equal(v[idx_t].cpu().numpy().view(np.uint16), ov)
    at = 0
    for r0, r1 in slabs:
        k = (r1 - r0) * cols
        qr, sr, qc, sc = oracle.mx_quantize_f32(om[at:at + k].reshape(r1 - r0, cols))
        at += k
        assert np.array_equal(u8(cache.q_row[r0:r1]), qr) and np.array_equal(u8(cache.s_row[r0:r1]), sr), (r0, r1)
        assert np.array_equal(u8(cache.q_col[:, r0:r1]), qc), (r0, r1)
        assert np.array_equal(u8(cache.s_col[:, r0 // 32:r1 // 32]), sc), (r0, r1)
    del theta, m_q, v, g, cache
    torch.cuda.empty_cache()


def _check_mx_slabs(out, ref_fn, rows, block=32):
    """Both orientations of `out` on the three row slabs, against ref_fn(r0, r1) -> (q_row, s_row, q_col, s_col)."""
    for r0, r1 in _slabs(rows, QC, block):
        q_row, s_row, q_col, s_col = ref_fn(r0, r1)[:4]
        assert np.array_equal(u8(out.q_row[r0:r1]), q_row), (r0, r1)
        assert np.array_equal(u8(out.s_row[r0:r1]), s_row), (r0, r1)
        assert np.array_equal(u8(out.q_col[:, r0:r1]), q_col), (r0, r1)
        assert np.array_equal(u8(out.s_col[:, r0 // 32:r1 // 32]), s_col), (r0, r1)


def test_ranged_quantize_past_2_31_elements(big_x):
    say("mxq_quantize_ranged past 2^31 elements")
    out, words = mxq.mx_quantize_ranged(big_x)
    torch.cuda.synchronize()
    _check_mx_slabs(out, lambda r0, r1: oracle.mx_quantize(u16(big_x[r0:r1])), QR)
    assert set(words.cpu().tolist()) <= {0, 1}
    del out
    torch.cuda.empty_cache()


def test_scaled_gemm_ranged_past_2_31_bytes(big_a):
    say("scaled_gemm_ranged past 2^31 bytes")
    qa, wa = big_a
    qb, wb = mxq.mx_quantize_ranged(workloads.normal_bf16((512, GK), 1.0, 62, 2, DEV), colwise=False)
    C = mxq.scaled_gemm_ranged(qa.q_row, qa.s_row, wa[0:1], qb.q_row, qb.s_row, wb[0:1])
    torch.cuda.synchronize()
    bq, bs = u8(qb.q_row), u8(qb.s_row)
    for r0, r1 in _slabs(GM, GK, 64)[1:]:
        y, S = oracle.gemm_ref(u8(qa.q_row[r0:r1]), u8(qa.s_row[r0:r1]), oracle.E4M3, bq, bs, oracle.E4M3,
                               oracle.MX_BLOCK32)
        r = _ratio(C[r0:r1], y, S)
        say(f"  rows {r0}..{r1}: worst |err| / bound {r:.3f}")
        assert r <= 1.0


def test_swiglu_oriented_past_2_31_elements(big_x):
    say("swiglu_mx_quantize_oriented past 2^31 input elements")
    out = mxq.swiglu_mx_quantize_oriented(big_x)
    torch.cuda.synchronize()

    def ref(r0, r1):
        q, s, h = oracle.swiglu_mx_quantize(u16(big_x[r0:r1]), want_h=True)
        _, _, qc, sc = oracle.mx_quantize_f32(h, rowwise=False)
        return q, s, qc, sc
    _check_mx_slabs(out, ref, QR)
    del out
    torch.cuda.empty_cache()


def test_route_weighted_quantize_past_2_31_elements(big_x):
    say("route_weighted_mx_quantize past 2^31 elements")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(64)
    p = torch.rand(QR, generator=gen, device=DEV) * 0.99 + 0.01
    out = mxq.route_weighted_mx_quantize(big_x, p)
    torch.cuda.synchronize()
    ph = p.cpu().numpy()
    _check_mx_slabs(out, lambda r0, r1: oracle.route_weighted_mx_quantize(u16(big_x[r0:r1]), ph[r0:r1]), QR)
    del out
    torch.cuda.empty_cache()


def test_swiglu_backward_quantize_past_2_31_elements(big_x):
    say("swiglu_backward_mx_quantize past 2^31 elements")
    dh = workloads.normal_bf16((QR, QC // 2), 1.0, 61, 2, DEV)
    out = mxq.swiglu_backward_mx_quantize(big_x, dh)
    torch.cuda.synchronize()
    _check_mx_slabs(out, lambda r0, r1: oracle.swiglu_bwd_mx_quantize(u16(big_x[r0:r1]), u16(dh[r0:r1])), QR)
    del out, dh
    torch.cuda.empty_cache()


def test_grouped_gemm_strided_past_2_31_bytes(big_a):
    say("grouped_scaled_gemm_strided past 2^31 bytes")
    qa = big_a[0]
    G, N = 4, 512
    ldb, ldbs = GK + 256, GK // 32 + 16                      # padded rows (16-byte multiples)
    bgs, bsgs = N * ldb + 4096, N * ldbs + 64                 # padded experts
    offsets = np.array([0, 32768, 65536 + 96, 131072 + 32, GM], np.int64)
    qw = mxq.mx_quantize(workloads.normal_bf16((G * N, GK), 1.0, 62, 4, DEV), colwise=False)
    bq_store = torch.zeros(G * bgs, dtype=torch.uint8, device=DEV)
    bs_store = torch.zeros(G * bsgs, dtype=torch.uint8, device=DEV)
    bq_store.as_strided((G, N, GK), (bgs, ldb, 1)).copy_(qw.q_row.view(G, N, GK))
    bs_store.as_strided((G, N, GK // 32), (bsgs, ldbs, 1)).copy_(qw.s_row.view(G, N, GK // 32))
    C = mxq.grouped_scaled_gemm_strided(qa.q_row, qa.s_row, torch.from_numpy(offsets).to(DEV), bq_store, bs_store,
                                        G, N, GK, ldb, bgs, ldbs, bsgs)
    torch.cuda.synchronize()
    hq, hs = u8(qw.q_row).reshape(G, N, GK), u8(qw.s_row).reshape(G, N, GK // 32)
    for r0, r1 in _slabs(GM, GK, 64)[1:]:
        sub_off = np.array([0, 0, 0, 0, r1 - r0], np.int64)      # the slab lies in the last group
        y, S = oracle.grouped_gemm_ref(u8(qa.q_row[r0:r1]), u8(qa.s_row[r0:r1]), sub_off, hq, hs)
        r = _ratio(C[r0:r1], y, S)
        say(f"  rows {r0}..{r1}: worst |err| / bound {r:.3f}")
        assert r <= 1.0


def test_grouped_wgrad_past_2_31_bytes():
    need_gpu()
    M, N, Kt = 512, 256, 4_194_304 + 1024                      # a_q: 2,148,007,936 bytes
    say("grouped_wgrad_mx past 2^31 bytes", M, N, Kt)
    qa = mxq.mx_quantize(workloads.normal_bf16((M, Kt), 1.0, 65, 1, DEV), colwise=False)
    qb = mxq.mx_quantize(workloads.normal_bf16((N, Kt), 1.0, 65, 2, DEV), colwise=False)
    torch.cuda.empty_cache()
    offsets = np.array([0, 1_048_576 + 32, 2_097_152 + 64, 3_145_728 + 96, Kt], np.int64)
    C = mxq.grouped_wgrad_mx(qa.q_row, qa.s_row, qb.q_row, qb.s_row, torch.from_numpy(offsets).to(DEV))
    torch.cuda.synchronize()
    rows = np.arange(M - 8, M, dtype=np.int64)
    cols = np.array([0, 1, 77, 128, 200, 253, 254, 255], np.int64)
    y, S = oracle.grouped_wgrad_ref(u8(qa.q_row[M - 8:]), u8(qa.s_row[M - 8:]), u8(qb.q_row[cols]),
                                    u8(qb.s_row[cols]), offsets)
    got = C[:, M - 8:][:, :, torch.from_numpy(cols).to(DEV)]
    r = _ratio(got, y, S)
    say(f"  worst |err| / bound {r:.3f}")
    assert r <= 1.0
    del qa, qb, C
    torch.cuda.empty_cache()


def test_adam_delayed_past_2_31_elements():
    need_gpu()
    n = 2 ** 31 + 4099
    say("fp8_adam_step_delayed past 2^31 elements", n)
    theta = workloads.workload5_params(n, DEV)
    m_q = torch.zeros(n, dtype=torch.uint8, device=DEV)
    m_scale = torch.ones(1, dtype=torch.float32, device=DEV)
    v = torch.zeros(n, dtype=torch.float16, device=DEV)
    w = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    g = workloads.workload5_grad(n, 1, DEV)
    hist = torch.tensor([2e-4, 1e-4], dtype=torch.float32, device=DEV)
    pos = torch.ones(1, dtype=torch.int32, device=DEV)
    o_hist, o_pos = np.array([2e-4, 1e-4], np.float32), np.ones(1, np.int32)
    hp = mxq.AdamHParams(3e-4, 0.9, 0.95, 1e-8, 0.1, 1)
    ohp = oracle.AdamHP(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
    rng = np.random.default_rng(66)
    idx = np.unique(np.concatenate([rng.choice(n, 200_000, replace=False), np.arange(2 ** 31 - 64, 2 ** 31 + 64),
                                    np.arange(n - 4099 - 8, n)])).astype(np.int64)
    gh, mh, vh = u16(g), u8(m_q), u16(v)
    idx_t = torch.from_numpy(idx).to(DEV)
    th_s = theta[idx_t].cpu().numpy()
    s_new = oracle.delayed_scale(o_hist, oracle.E4M3)           # from the history as it was before the step
    amax = oracle.adam_amax(gh, mh, vh, np.float32(1.0), ohp)
    full_th = np.zeros(n, np.float32)
    full_th[idx] = th_s
    om, oq, ov, ow = oracle.adam_elements(full_th, gh, mh, vh, np.float32(1.0), s_new, idx, ohp)
    del gh, mh, vh, full_th
    oracle.history_push(o_hist, o_pos, amax)
    mxq.fp8_adam_step_delayed(theta, g, m_q, m_scale, v, w, hp, hist, pos)
    torch.cuda.synchronize()
    assert _bits(m_scale)[0] == s_new.view(np.uint32)
    assert np.array_equal(_bits(hist), o_hist.view(np.uint32)) and int(pos.item()) == int(o_pos[0])
    assert np.array_equal(theta[idx_t].cpu().numpy().view(np.uint32), om.view(np.uint32))
    assert np.array_equal(m_q[idx_t].cpu().numpy(), oq)
    assert np.array_equal(v[idx_t].cpu().numpy().view(np.uint16), ov)
    assert np.array_equal(w[idx_t].view(torch.int16).cpu().numpy().view(np.uint16), ow)
    del theta, m_q, v, w, g
    torch.cuda.empty_cache()
