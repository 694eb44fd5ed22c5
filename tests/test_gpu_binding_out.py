"""The binding's caller-buffer forms (out=) of the per-tensor casts and the auto-scaled cast: the same bytes as the
forms that allocate their outputs, buffers reused across calls, and mis-shaped buffers refused before any launch."""
import pytest
import torch

from gpu_util import DEV, need_gpu
import mxfp8_precision_numerics_amd as mxq

pytestmark = pytest.mark.gpu


def _x(rows, cols, seed, sigma=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(rows, cols, generator=g) * sigma).to(torch.bfloat16).to(DEV)


def _buffers(rows, cols):
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=DEV)  # noqa: E731
    f = lambda: torch.empty(1, dtype=torch.float32, device=DEV)  # noqa: E731
    return mxq.PerTensorFP8(u8(rows, cols), u8(cols, rows), f(), f())


@pytest.mark.parametrize("fmt", [mxq.E4M3, mxq.E5M2])
def test_pertensor_out_matches_allocating_form(fmt):
    need_gpu()
    out = _buffers(96, 160)
    for seed in (1, 2):                                    # the second call overwrites the first one's buffers
        x = _x(96, 160, seed, 0.5 * seed)
        ref = mxq.pertensor_quantize(x, fmt)
        got = mxq.pertensor_quantize(x, fmt, out=out)
        torch.cuda.synchronize()
        assert got.q.data_ptr() == out.q.data_ptr() and got.q_t.data_ptr() == out.q_t.data_ptr()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)


def test_pertensor_out_single_orientation_and_delayed():
    need_gpu()
    x = _x(64, 128, 3)
    out = _buffers(64, 128)
    only_t = mxq.PerTensorFP8(None, out.q_t, out.amax, out.scale)
    got = mxq.pertensor_quantize(x, mxq.E4M3, out=only_t)
    ref = mxq.pertensor_quantize(x, mxq.E4M3)
    torch.cuda.synchronize()
    assert got.q is None and torch.equal(got.q_t, ref.q_t) and torch.equal(got.scale, ref.scale)
    hist_a = torch.full((4,), 3.0, dtype=torch.float32, device=DEV)
    hist_b = hist_a.clone()
    pos_a = torch.zeros(1, dtype=torch.int32, device=DEV)
    pos_b = pos_a.clone()
    ref = mxq.pertensor_quantize_delayed(x, hist_a, pos_a, mxq.E4M3)
    got = mxq.pertensor_quantize_delayed(x, hist_b, pos_b, mxq.E4M3, out=out)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    assert torch.equal(hist_a, hist_b) and torch.equal(pos_a, pos_b)


def test_autoscale_out_matches_allocating_form():
    need_gpu()
    g = _x(128, 256, 4, 1e-3)
    mu_a = torch.full((1,), 4096.0, dtype=torch.float32, device=DEV)
    mu_b = mu_a.clone()
    out = mxq.AutoScaled(torch.empty((128, 256), dtype=torch.uint8, device=DEV),
                         torch.empty(1, dtype=torch.float32, device=DEV), torch.empty(1, dtype=torch.int64, device=DEV))
    for _ in range(2):
        ref = mxq.fp8_autoscale_cast(g, mu_a, mxq.E4M3)
        got = mxq.fp8_autoscale_cast(g, mu_b, mxq.E4M3, out=out)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        assert torch.equal(mu_a, mu_b)


def test_out_shapes_refused():
    need_gpu()
    x = _x(64, 128, 5)
    bad = _buffers(128, 64)                                # transposed shapes
    with pytest.raises(ValueError):
        mxq.pertensor_quantize(x, mxq.E4M3, out=bad)
    good = _buffers(64, 128)
    with pytest.raises(ValueError):
        mxq.pertensor_quantize(x, mxq.E4M3, out=good._replace(amax=torch.empty(2, dtype=torch.float32, device=DEV)))
    with pytest.raises(ValueError):
        mxq.fp8_autoscale_cast(x, torch.ones(1, dtype=torch.float32, device=DEV), mxq.E4M3,
                               out=mxq.AutoScaled(torch.empty((64, 64), dtype=torch.uint8, device=DEV),
                                                  torch.empty(1, dtype=torch.float32, device=DEV),
                                                  torch.empty(1, dtype=torch.int64, device=DEV)))
