"""GPU checks of the measurement kernels (libmxq_probe.so) the benchmark uses for the sustained ceilings: the streaming
copy reproduces its source byte for byte (looping and full grids, 4, 8 and 16 loads in flight, sizes that end inside a
trip), the streaming read leaves the xor of the words read (as does the read into LDS through the GEMM's copy
instruction, per workgroup over its 64 KiB pieces), and the MFMA-only loop over operands of E4M3 1.0 (0x38)
with unit scales leaves every lane the closed-form sum 16 accumulators x 16 values x (64 products of 1) x iters."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, need_gpu
from mxfp8_precision_numerics_amd import _probe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks,unroll", [(16, 1, 4), (1 << 20, 4, 8), (3 * (1 << 20) + 48, 7, 16),
                                                  (64 << 20, 4096, 4), (3 * (1 << 20) + 48, 0, 4),
                                                  (64 << 20, 0, 8), (5 * 4096 * 16 + 16, 0, 16)])
def test_copy_probe_is_a_copy(nbytes, blocks, unroll):
    need_gpu()
    g = torch.Generator(device=DEV)
    g.manual_seed(nbytes + blocks)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    dst = torch.zeros_like(src)
    moved = _probe.copy(src, dst, blocks, unroll)
    torch.cuda.synchronize()
    assert moved == 2 * nbytes
    assert torch.equal(src, dst)


@pytest.mark.parametrize("nbytes,blocks,unroll", [(16, 0, 8), (3 * (1 << 20) + 48, 0, 8), (1 << 20, 5, 16),
                                                  (7 << 20, 0, 4)])
def test_read_probe_xor(nbytes, blocks, unroll):
    need_gpu()
    g = torch.Generator(device=DEV)
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    groups = blocks if blocks > 0 else nbytes // (4096 * unroll) + 1
    sink = torch.zeros(groups, dtype=torch.int32, device=DEV)
    assert _probe.read(src, sink, blocks, unroll) == nbytes
    torch.cuda.synchronize()
    words = src.cpu().numpy().view(np.uint32)
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("iters", [1, 2, 7])
def test_mfma_probe_closed_form(iters):
    need_gpu()
    ops = torch.full((131072,), 0x38, dtype=torch.uint8, device=DEV)
    sink = torch.empty(3 * 256, dtype=torch.float32, device=DEV)
    flop = _probe.mfma_fp8(ops, iters, 3, sink)
    torch.cuda.synchronize()
    assert flop == 3 * 4 * iters * 16 * 131072
    assert np.all(sink.cpu().numpy() == np.float32(16 * 16 * 64 * iters))


@pytest.mark.parametrize("pieces,blocks", [(0, 1), (1, 1), (37, 16), (256, 256), (1000, 300)])
def test_read_lds_probe_xor(pieces, blocks):
    need_gpu()
    nbytes = pieces * 65536
    g = torch.Generator(device=DEV)
    g.manual_seed(pieces * 7 + blocks)
    src = torch.randint(0, 256, (max(nbytes, 16),), dtype=torch.uint8, device=DEV, generator=g)[:nbytes]
    sink = torch.full((blocks,), -1, dtype=torch.int32, device=DEV)
    assert _probe.read_lds(src, sink, blocks) == nbytes
    torch.cuda.synchronize()
    words = src.cpu().numpy().view(np.uint32).reshape(pieces, 16384) if pieces else np.zeros((0, 16384), np.uint32)
    per_piece = np.bitwise_xor.reduce(words, axis=1) if pieces else np.zeros(0, np.uint32)
    want = np.zeros(blocks, dtype=np.uint32)
    for w in range(blocks):
        if w < pieces:
            want[w] = np.bitwise_xor.reduce(per_piece[w::blocks])
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)
