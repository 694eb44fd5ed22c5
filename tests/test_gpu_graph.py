"""The first workload's three launches (MX quantize of A, of B, the 256^3 block-scaled GEMM) captured in a HIP graph
and replayed: every replay must equal the eager launches bit for bit, on new inputs written between replays by the
program's own eager work, and meet the GEMM bound against the oracle. Nothing in the captured calls allocates or
clears memory; the outputs are preallocated."""
import numpy as np
import pytest
import torch

import mxfp8_precision_numerics_amd as mxq
import oracle
from gpu_util import DEV, need_gpu, say, u16, u8
from mxfp8_precision_numerics_amd import workloads

pytestmark = pytest.mark.gpu


def _buffers():
    e = lambda *s: torch.empty(s, dtype=torch.uint8, device=DEV)  # noqa: E731
    qa = mxq.MXTensor(e(256, 256), e(256, 8), None, None)
    qb = mxq.MXTensor(None, None, e(256, 256), e(256, 8))
    C = torch.empty((256, 256), dtype=torch.bfloat16, device=DEV)
    return qa, qb, C


def _path(A, B, qa, qb, C):
    mxq.mx_quantize(A, colwise=False, out=qa)
    mxq.mx_quantize(B, rowwise=False, out=qb)
    mxq.scaled_gemm(qa.q_row, qa.s_row, qb.q_col, qb.s_col, mxq.MX_BLOCK32, out=C)


def test_workload1_graph_replays():
    need_gpu()
    A, B = workloads.workload1(DEV)
    A_static, B_static = A.clone(), B.clone()
    qa, qb, C = _buffers()
    _path(A_static, B_static, qa, qb, C)                     # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _path(A_static, B_static, qa, qb, C)
    torch.cuda.synchronize()
    eq, eb, eC = _buffers()
    for rep in range(4):
        say("graph replay", rep)
        if rep:
            # the program's own eager work between replays: new inputs written into the captured buffers
            A_static.copy_(workloads.normal_bf16((256, 256), 1.0, 40, rep, DEV))
            B_static.copy_(workloads.normal_bf16((256, 256), 0.5, 41, rep, DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _path(A_static, B_static, eq, eb, eC)                # the same launches, eager
        torch.cuda.synchronize()
        assert torch.equal(qa.q_row, eq.q_row) and torch.equal(qa.s_row, eq.s_row), f"replay {rep}: A codes"
        assert torch.equal(qb.q_col, eb.q_col) and torch.equal(qb.s_col, eb.s_col), f"replay {rep}: B codes"
        assert torch.equal(C, eC), f"replay {rep}: C"
        r = oracle.mx_quantize(u16(A_static), oracle.RCEIL, colwise=False)
        assert np.array_equal(u8(qa.q_row), r[0]) and np.array_equal(u8(qa.s_row), r[1])
        y, S = oracle.gemm_ref(u8(qa.q_row), u8(qa.s_row), oracle.E4M3, u8(qb.q_col), u8(qb.s_col), oracle.E4M3,
                               oracle.MX_BLOCK32)
        err = np.abs(C.float().cpu().numpy().astype(np.float64) - y)
        assert np.all(err <= 2.0 ** -7 * np.abs(y) + 2.0 ** -20 * S), f"replay {rep}: GEMM bound"
