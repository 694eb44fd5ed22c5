"""GPU checks of the measurement kernels bench.py uses for the attainable ceilings: the streaming copy reproduces its
source byte for byte (several grid sizes, a size that ends inside a grid-stride trip), and the MFMA-only loop over
operands of E4M3 1.0 (0x38) with unit scales leaves every lane the closed-form sum 16 accumulators x 16 values x
(64 products of 1) x iters."""
import numpy as np
import pytest
import torch

import mxfp8_precision_numerics_amd as mxq
from gpu_util import DEV, need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (1 << 20, 4), (3 * (1 << 20) + 48, 7), (64 << 20, 4096)])
def test_copy_probe_is_a_copy(nbytes, blocks):
    need_gpu()
    g = torch.Generator(device=DEV)
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    dst = torch.zeros_like(src)
    moved = mxq.probe_copy(src, dst, blocks)
    torch.cuda.synchronize()
    assert moved == 2 * nbytes
    assert torch.equal(src, dst)


@pytest.mark.parametrize("iters", [1, 2, 7])
def test_mfma_probe_closed_form(iters):
    need_gpu()
    ops = torch.full((131072,), 0x38, dtype=torch.uint8, device=DEV)
    sink = torch.empty(3 * 256, dtype=torch.float32, device=DEV)
    flop = mxq.probe_mfma_fp8(ops, iters, 3, sink)
    torch.cuda.synchronize()
    assert flop == 3 * 4 * iters * 16 * 131072
    assert np.all(sink.cpu().numpy() == np.float32(16 * 16 * 64 * iters))
