"""Benchmark of the FP8 / MXFP8 hot path on one MI355X.

One step is one pass over every row of the hot path, on seeded synthetic inputs already resident in HBM:
  mx_linear     GPT-175B QKV linear (X 4096x12288, W 36864x12288, dY 4096x36864) in MXFP8: quantize X, W and dY in
                both orientations, then Y = X W^T, dX = dY W, dW = dY^T X (block-scaled GEMMs, bf16 out)
  pt_linear     the same layer with per-tensor current scaling (E4M3 X and W, E5M2 dY; q and q^T) and three GEMMs
  mx_quant      MX quantize of a 16384x8192 activation with 0.1% x100 outliers, row and column orientation (and,
                timed as mx_quant_act_row, the row orientation alone: 406.8 MB)
  grouped       64-expert grouped MX GEMM (Zipf(1.1) top-8 routing of 16384 tokens, up 2048->1024 and down
                1024->2048), including the row quantize of both activations (expert weights quantized once); the
                activation quantizes and the two grouped GEMMs are timed separately as well
  adam          precision-decoupled FP8 Adam step over 1.3e9 parameters (2 passes)
  small         MX quantize + 256^3 block-scaled GEMM (three launches), and small_graph: the same three launches
                captured once in a HIP graph and replayed
  pt_quant_delayed  the per-tensor casts of X, W, dY with delayed scaling (16-slot amax histories): one pass each
  adam_delayed  the Adam step with a delayed first-moment scale: one pass over the state (18 B/param)
  wcache_fused  Adam on W's 36864 x 12288 state fused with the refresh of W's two MXFP8 caches from the fp32 master
  wcache_unfused  the same as two calls: Adam writing a bf16 copy, then MX quantize of that copy
  moe_swiglu_mlp  the routed MLP of the grouped workload with SwiGLU: activation quantize, up/gate grouped GEMM
                (2048 -> 2 x 1024), fused SwiGLU + MX quantize, down grouped GEMM (1024 -> 2048)
  swiglu_quant  the fused SwiGLU + MX quantize alone (132,160 x 2048 bf16 in, 132,160 x 1024 MXFP8 out)
  grad_cast     the auto-scaled FP8 cast of the weight gradient dW (36864 x 12288 bf16 -> E4M3, overflow count, mu
                update): the part of the FP8 all-reduce that runs before the scales are gathered
  grad_requant  the re-quantize of those codes to the shared scale (the min over 8 gathered scales)
  moe_fwd_train the routed MLP's forward as training runs it: the activation quantized in both orientations, the
                up/gate grouped GEMM, SwiGLU + MX quantize saving h in both orientations, the down grouped GEMM
  moe_bwd       its backward (seeded output gradient N(0,1e-3), route weights uniform): route weighting fused with
                the gradient's MX quantize (both orientations), down dgrad over W_down's column cache, SwiGLU
                backward fused with the MX quantize of (d_gate | d_up), up/gate dgrad over W_gu's column cache, and
                the two routed Wgrad contractions over each expert's tokens into fp32 gradient sinks
The headline value is the MXFP8 linear layer's GEMM FLOPs (11.13 TFLOP) divided by the device time of its quantize
and GEMM launches ("MXFP8 GEMM TFLOP/s incl. quantize"). Device times come from events on the stream the kernels
run on; the JSON line also carries every part's rate, the MX GEMM's roofline, the ceilings this part attains
(a 1 GiB device copy, an MFMA-only loop), measured after the timed steps, and the CPU oracle baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP8 GEMM TFLOP/s incl. quantize (% FP8 MFMA peak); quantize GB/s (% HBM)"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 (no sparsity)
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=512)
    ap.add_argument("--profile-kernel", choices=PROFILE_KERNELS, default=None,
                    help="run only this kernel (10 launches) for hardware-counter passes, print its timing, exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1 (sharding across GPUs is not "
                                   "implemented)", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp8_precision_numerics_amd as mxq
    from mxfp8_precision_numerics_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.profile_kernel:
        profile_kernel(args.profile_kernel, dev)
        return

    # ------------------------------------------------------------------ inputs (resident before timing)
    log("generating inputs")
    X, W, dY = workloads.workload2(dev)
    M, N, K = X.shape[0], W.shape[0], X.shape[1]
    act3 = workloads.workload3(dev)
    wl4 = workloads.workload4(dev)
    off4 = torch.from_numpy(wl4["offsets"]).to(dev)
    n_adam = 1_300_000_000
    theta = workloads.workload5_params(n_adam, dev)
    grad = workloads.workload5_grad(n_adam, 2, dev)
    m_q = torch.zeros(n_adam, dtype=torch.uint8, device=dev)
    m_scale = torch.ones(1, dtype=torch.float32, device=dev)
    v16 = torch.zeros(n_adam, dtype=torch.float16, device=dev)
    w16 = torch.empty(n_adam, dtype=torch.bfloat16, device=dev)
    adam_ws = torch.empty(mxq.workspace_bytes("adam", n_adam), dtype=torch.uint8, device=dev)
    A1, B1 = workloads.workload1(dev)
    # workload 1 is launch-bound: its three launches are also captured in a HIP graph (outputs preallocated)
    qa1 = mxq.MXTensor(torch.empty((256, 256), dtype=torch.uint8, device=dev),
                       torch.empty((256, 8), dtype=torch.uint8, device=dev), None, None)
    qb1 = mxq.MXTensor(None, None, torch.empty((256, 256), dtype=torch.uint8, device=dev),
                       torch.empty((256, 8), dtype=torch.uint8, device=dev))
    C1 = torch.empty((256, 256), dtype=torch.bfloat16, device=dev)

    def small_path():
        mxq.mx_quantize(A1, colwise=False, out=qa1)
        mxq.mx_quantize(B1, rowwise=False, out=qb1)
        mxq.scaled_gemm(qa1.q_row, qa1.s_row, qb1.q_col, qb1.s_col, mxq.MX_BLOCK32, out=C1)

    small_path()
    torch.cuda.synchronize()
    small_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(small_graph):
        small_path()
    torch.cuda.synchronize()

    # preallocated outputs (the library never allocates)
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
    words = torch.zeros((3, 2), dtype=torch.int32, device=dev)     # range words of X, W, dY: [row, col]
    mxX = mxq.MXTensor(u8(M, K), u8(M, K // 32), u8(K, M), u8(K, M // 32))
    mxW = mxq.MXTensor(u8(N, K), u8(N, K // 32), u8(K, N), u8(K, N // 32))
    mxD = mxq.MXTensor(u8(M, N), u8(M, N // 32), u8(N, M), u8(N, M // 32))
    mx3 = mxq.MXTensor(u8(*act3.shape), u8(act3.shape[0], act3.shape[1] // 32), u8(act3.shape[1], act3.shape[0]),
                       u8(act3.shape[1], act3.shape[0] // 32))
    mx3_row = mxq.MXTensor(mx3.q_row, mx3.s_row, None, None)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    ws_pt = torch.empty(mxq.workspace_bytes("pertensor", N * K), dtype=torch.uint8, device=dev)
    f32 = lambda: torch.empty(1, dtype=torch.float32, device=dev)  # noqa: E731
    # per-tensor casts' codes (q, q^T) and scalars; the delayed casts reuse them once the per-tensor GEMMs have run
    pt_out = {"X": mxq.PerTensorFP8(u8(M, K), u8(K, M), f32(), f32()),
              "W": mxq.PerTensorFP8(u8(N, K), u8(K, N), f32(), f32()),
              "dY": mxq.PerTensorFP8(u8(M, N), u8(N, M), f32(), f32())}
    # grouped: weights quantized once (cache), activations each step
    G, d_ff, d_model = wl4["w_up"].shape
    qwu = mxq.mx_quantize(wl4["w_up"].reshape(G * d_ff, d_model), colwise=False)
    qwd = mxq.mx_quantize(wl4["w_down"].reshape(G * d_model, d_ff), colwise=False)
    rows4 = wl4["a_up"].shape[0]
    mx_up = mxq.MXTensor(u8(rows4, d_model), u8(rows4, d_model // 32), None, None)
    mx_dn = mxq.MXTensor(u8(rows4, d_ff), u8(rows4, d_ff // 32), None, None)
    C_up = torch.empty((rows4, d_ff), dtype=torch.bfloat16, device=dev)
    C_dn = torch.empty((rows4, d_model), dtype=torch.bfloat16, device=dev)
    # routed MLP with SwiGLU: gate|up expert weights [G][2 d_ff][d_model] (seeded N(0,1), quantized once), the fused
    # SwiGLU + MX quantize between the up/gate and down grouped GEMMs
    w_gu = workloads.normal_bf16((G * 2 * d_ff, d_model), 1.0, 4, 5, dev)
    qwgu = mxq.mx_quantize(w_gu, colwise=True)             # row cache (forward) and column cache (dgrad)
    del w_gu
    qwd_c = mxq.mx_quantize(wl4["w_down"].reshape(G * d_model, d_ff), rowwise=False, colwise=True)
    C_gu = torch.empty((rows4, 2 * d_ff), dtype=torch.bfloat16, device=dev)
    mx_h = mxq.MXTensor(u8(rows4, d_ff), u8(rows4, d_ff // 32), None, None)
    # routed MLP training forward (saved operands in both orientations) and backward
    mx_x2 = mxq.MXTensor(u8(rows4, d_model), u8(rows4, d_model // 32), u8(d_model, rows4), u8(d_model, rows4 // 32))
    mx_h2 = mxq.MXTensor(u8(rows4, d_ff), u8(rows4, d_ff // 32), u8(d_ff, rows4), u8(d_ff, rows4 // 32))
    dy4 = workloads.zero_padding_rows(workloads.normal_bf16((rows4, d_model), 1e-3, 4, 6, dev), wl4["counts"],
                                      wl4["padded"], wl4["offsets"])
    p4 = workloads.route_weights(wl4["counts"], wl4["padded"], wl4["offsets"], device=dev)
    mx_dyw = mxq.MXTensor(u8(rows4, d_model), u8(rows4, d_model // 32), u8(d_model, rows4), u8(d_model, rows4 // 32))
    mx_dc = mxq.MXTensor(u8(rows4, 2 * d_ff), u8(rows4, 2 * d_ff // 32), u8(2 * d_ff, rows4),
                         u8(2 * d_ff, rows4 // 32))
    dh4 = torch.empty((rows4, d_ff), dtype=torch.bfloat16, device=dev)
    dx4 = torch.empty((rows4, d_model), dtype=torch.bfloat16, device=dev)
    sink_wd = torch.zeros((G, d_model, d_ff), dtype=torch.float32, device=dev)
    sink_wgu = torch.zeros((G, 2 * d_ff, d_model), dtype=torch.float32, device=dev)
    hp = mxq.AdamHParams(3e-4, 0.9, 0.95, 1e-8, 0.0, 2)
    # delayed scaling: amax histories (16 slots) seeded with one current-scaling call each
    hists, hpos = {}, {}
    for name, t, fmt in (("X", X, mxq.E4M3), ("W", W, mxq.E4M3), ("dY", dY, mxq.E5M2)):
        r = mxq.pertensor_quantize(t, fmt, want_q=False, want_qt=False, workspace=ws_pt)
        hists[name] = torch.zeros(16, dtype=torch.float32, device=dev)
        hists[name][0] = r.amax[0]
        hpos[name] = torch.ones(1, dtype=torch.int32, device=dev)
    m_hist = torch.zeros(16, dtype=torch.float32, device=dev)
    m_pos = torch.zeros(1, dtype=torch.int32, device=dev)
    ws_del = torch.empty(mxq.workspace_bytes("pertensor_delayed", N * K), dtype=torch.uint8, device=dev)
    ws_adel = torch.empty(mxq.workspace_bytes("adam_delayed", n_adam), dtype=torch.uint8, device=dev)
    mxq.fp8_adam_step(theta, grad, m_q, m_scale, v16, w16, hp, workspace=adam_ws)
    m_hist[0] = 448.0 / m_scale[0]           # the amax that step's scale came from
    m_pos[0] = 1
    # weight-cache refresh on W's shape: Adam state of a 36864 x 12288 weight and its two MX caches
    nw = N * K
    th_w = W.float().reshape(-1).clone()
    g_w = workloads.normal_bf16((nw,), 1e-3, 5, 7, dev)
    mq_w = torch.zeros(nw, dtype=torch.uint8, device=dev)
    ms_w = torch.ones(1, dtype=torch.float32, device=dev)
    v_w = torch.zeros(nw, dtype=torch.float16, device=dev)
    wb_w = torch.empty(nw, dtype=torch.bfloat16, device=dev)
    cache_w = mxq.MXTensor(u8(N, K), u8(N, K // 32), u8(K, N), u8(K, N // 32))
    ws_w = torch.empty(mxq.workspace_bytes("adam", nw), dtype=torch.uint8, device=dev)
    # FP8 all-reduce pieces on dW: mu, the codes, and 8 gathered scales (this rank's and 7 seeded others)
    mu_g = torch.ones(1, dtype=torch.float32, device=dev)
    ws_g = torch.empty(mxq.workspace_bytes("autoscale", nw), dtype=torch.uint8, device=dev)
    others = 2.0 ** torch.arange(-3, 4, dtype=torch.float32, device=dev)
    gathered = torch.empty(8, dtype=torch.float32, device=dev)
    q_req = torch.empty(nw, dtype=torch.uint8, device=dev)
    gc_out = mxq.AutoScaled(torch.empty((N, K), dtype=torch.uint8, device=dev), f32(),
                            torch.empty(1, dtype=torch.int64, device=dev))
    torch.cuda.synchronize()

    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    # Parts bound by HBM bandwidth start with the last-level cache scrubbed (outside their timed window): a 512 MiB
    # write evicts the 256 MB Infinity Cache, so no part reads its input from a cache a previous part filled.
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    HBM_PARTS = {"mx_quant_XWdY", "pt_quant", "mx_quant_act", "grouped_q_up", "grouped_q_down", "adam",
                 "pt_quant_delayed", "adam_delayed", "wcache_fused", "wcache_unfused", "swiglu_quant", "grad_cast",
                 "grad_requant", "bwd_rw_quant", "bwd_swiglu_quant", "mx_quant_act_row"}
    parts = []
    cur = {}

    def part(name, rec):
        """Context for one timed part: scrub first if it is HBM-bound, then events around its launches."""
        class _P:
            def __enter__(self_):
                if name in HBM_PARTS:
                    scrub.zero_()
                if name not in parts:
                    parts.append(name)
                e0, e1 = Ev(), Ev()
                rec[name] = (e0, e1)
                e0.record(stream)

            def __exit__(self_, *exc):
                rec[name][1].record(stream)
                return False
        return _P()

    def step(rec):
        # the MX linear layer: each quantize also emits its orientations' range words, and each GEMM picks the FP8
        # instruction or the exact path from its operands' words on the device
        with part("mx_quant_XWdY", rec):
            mxq.mx_quantize_ranged(X, out=mxX, words=words[0])
            mxq.mx_quantize_ranged(W, out=mxW, words=words[1])
            mxq.mx_quantize_ranged(dY, out=mxD, words=words[2])
        with part("mx_gemm_fwd", rec):                                                             # Y = X W^T
            mxq.scaled_gemm_ranged(mxX.q_row, mxX.s_row, words[0, 0:1], mxW.q_row, mxW.s_row, words[1, 0:1], out=Y)
        with part("mx_gemm_dgrad", rec):                                                           # dX = dY W
            mxq.scaled_gemm_ranged(mxD.q_row, mxD.s_row, words[2, 0:1], mxW.q_col, mxW.s_col, words[1, 1:2], out=dX)
        with part("mx_gemm_wgrad", rec):                                                           # dW = dY^T X
            mxq.scaled_gemm_ranged(mxD.q_col, mxD.s_col, words[2, 1:2], mxX.q_col, mxX.s_col, words[0, 1:2], out=dW)
        # the same fwd and dgrad through the default entry point, which checks the codes itself
        with part("mx_gemm_fwd_checked", rec):
            mxq.scaled_gemm(mxX.q_row, mxX.s_row, mxW.q_row, mxW.s_row, mxq.MX_BLOCK32, out=Y)
        with part("mx_gemm_dgrad_checked", rec):
            mxq.scaled_gemm(mxD.q_row, mxD.s_row, mxW.q_col, mxW.s_col, mxq.MX_BLOCK32, out=dX)
        with part("pt_quant", rec):
            px = mxq.pertensor_quantize(X, mxq.E4M3, workspace=ws_pt, out=pt_out["X"])
            pw = mxq.pertensor_quantize(W, mxq.E4M3, workspace=ws_pt, out=pt_out["W"])
            pd = mxq.pertensor_quantize(dY, mxq.E5M2, workspace=ws_pt, out=pt_out["dY"])
        with part("pt_gemm_fwd", rec):
            mxq.scaled_gemm(px.q, px.scale, pw.q, pw.scale, mxq.PER_TENSOR, mxq.E4M3, mxq.E4M3, out=Y)
        with part("pt_gemm_dgrad", rec):
            mxq.scaled_gemm(pd.q, pd.scale, pw.q_t, pw.scale, mxq.PER_TENSOR, mxq.E5M2, mxq.E4M3, out=dX)
        with part("pt_gemm_wgrad", rec):
            mxq.scaled_gemm(pd.q_t, pd.scale, px.q_t, px.scale, mxq.PER_TENSOR, mxq.E5M2, mxq.E4M3, out=dW)
        with part("mx_quant_act", rec):
            mxq.mx_quantize(act3, out=mx3)
        with part("mx_quant_act_row", rec):
            mxq.mx_quantize(act3, colwise=False, out=mx3_row)
        with part("grouped_q_up", rec):
            mxq.mx_quantize(wl4["a_up"], colwise=False, out=mx_up)
        with part("grouped_gemm_up", rec):
            mxq.grouped_scaled_gemm(mx_up.q_row, mx_up.s_row, off4, qwu.q_row.view(G, d_ff, d_model),
                                    qwu.s_row.view(G, d_ff, d_model // 32), out=C_up)
        with part("grouped_q_down", rec):
            mxq.mx_quantize(wl4["a_down"], colwise=False, out=mx_dn)
        with part("grouped_gemm_down", rec):
            mxq.grouped_scaled_gemm(mx_dn.q_row, mx_dn.s_row, off4, qwd.q_row.view(G, d_model, d_ff),
                                    qwd.s_row.view(G, d_model, d_ff // 32), out=C_dn)
        with part("adam", rec):
            mxq.fp8_adam_step(theta, grad, m_q, m_scale, v16, w16, hp, workspace=adam_ws)
        with part("small", rec):
            small_path()
        with part("small_graph", rec):
            small_graph.replay()
        # the same two with the stream kept busy (a ~0.1 ms spin) while the host submits, so the window holds device
        # time only and not the host's submission latency
        torch.cuda._sleep(200_000)
        with part("small_queued", rec):
            small_path()
        torch.cuda._sleep(200_000)
        with part("small_graph_queued", rec):
            small_graph.replay()
        with part("pt_quant_delayed", rec):
            mxq.pertensor_quantize_delayed(X, hists["X"], hpos["X"], mxq.E4M3, workspace=ws_del, out=pt_out["X"])
            mxq.pertensor_quantize_delayed(W, hists["W"], hpos["W"], mxq.E4M3, workspace=ws_del, out=pt_out["W"])
            mxq.pertensor_quantize_delayed(dY, hists["dY"], hpos["dY"], mxq.E5M2, workspace=ws_del, out=pt_out["dY"])
        with part("adam_delayed", rec):
            mxq.fp8_adam_step_delayed(theta, grad, m_q, m_scale, v16, w16, hp, m_hist, m_pos, workspace=ws_adel)
        with part("wcache_fused", rec):
            mxq.fp8_adam_step_mx_cache(th_w, g_w, mq_w, ms_w, v_w, None, hp, N, K, out=cache_w, workspace=ws_w)
        with part("wcache_unfused", rec):
            mxq.fp8_adam_step(th_w, g_w, mq_w, ms_w, v_w, wb_w, hp, workspace=ws_w)
            mxq.mx_quantize(wb_w.view(N, K), out=cache_w)
        with part("moe_swiglu_mlp", rec):
            mxq.mx_quantize(wl4["a_up"], colwise=False, out=mx_up)
            mxq.grouped_scaled_gemm(mx_up.q_row, mx_up.s_row, off4, qwgu.q_row.view(G, 2 * d_ff, d_model),
                                    qwgu.s_row.view(G, 2 * d_ff, d_model // 32), out=C_gu)
            mxq.swiglu_mx_quantize(C_gu, out=mx_h)
            mxq.grouped_scaled_gemm(mx_h.q_row, mx_h.s_row, off4, qwd.q_row.view(G, d_model, d_ff),
                                    qwd.s_row.view(G, d_model, d_ff // 32), out=C_dn)
        with part("swiglu_quant", rec):
            mxq.swiglu_mx_quantize(C_gu, out=mx_h)
        with part("grad_cast", rec):
            gc = mxq.fp8_autoscale_cast(dW, mu_g, mxq.E4M3, workspace=ws_g, out=gc_out)
        gathered[:1] = gc.scale
        gathered[1:] = others
        with part("grad_requant", rec):
            mxq.fp8_requantize_shared(gc.q, mxq.E4M3, gc.scale, gathered, mxq.E4M3, out=q_req)
        with part("moe_fwd_train", rec):
            mxq.mx_quantize(wl4["a_up"], out=mx_x2)
            mxq.grouped_scaled_gemm(mx_x2.q_row, mx_x2.s_row, off4, qwgu.q_row.view(G, 2 * d_ff, d_model),
                                    qwgu.s_row.view(G, 2 * d_ff, d_model // 32), out=C_gu)
            mxq.swiglu_mx_quantize_oriented(C_gu, out=mx_h2)
            mxq.grouped_scaled_gemm(mx_h2.q_row, mx_h2.s_row, off4, qwd.q_row.view(G, d_model, d_ff),
                                    qwd.s_row.view(G, d_model, d_ff // 32), out=C_dn)
        with part("bwd_rw_quant", rec):
            mxq.route_weighted_mx_quantize(dy4, p4, out=mx_dyw)
        with part("bwd_dgrad_down", rec):
            mxq.grouped_scaled_gemm_strided(mx_dyw.q_row, mx_dyw.s_row, off4, qwd_c.q_col, qwd_c.s_col, G, d_ff,
                                            d_model, ldb=G * d_model, b_group_stride=d_model,
                                            ldbs=G * d_model // 32, bs_group_stride=d_model // 32, out=dh4)
        with part("bwd_swiglu_quant", rec):
            mxq.swiglu_backward_mx_quantize(C_gu, dh4, out=mx_dc)
        with part("bwd_dgrad_up", rec):
            mxq.grouped_scaled_gemm_strided(mx_dc.q_row, mx_dc.s_row, off4, qwgu.q_col, qwgu.s_col, G, d_model,
                                            2 * d_ff, ldb=G * 2 * d_ff, b_group_stride=2 * d_ff,
                                            ldbs=G * 2 * d_ff // 32, bs_group_stride=2 * d_ff // 32, out=dx4)
        with part("bwd_wgrad_down", rec):
            mxq.grouped_wgrad_mx(mx_dyw.q_col, mx_dyw.s_col, mx_h2.q_col, mx_h2.s_col, off4, accumulate=sink_wd)
        with part("bwd_wgrad_up", rec):
            mxq.grouped_wgrad_mx(mx_dc.q_col, mx_dc.s_col, mx_x2.q_col, mx_x2.s_col, off4, accumulate=sink_wgu)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step({})
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    recs = [{} for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(recs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # each part: the median over the timed steps of its event-timed device duration
    ms = {p: float(np.median([recs[s][p][0].elapsed_time(recs[s][p][1]) for s in range(args.steps)])) for p in parts}
    spread = {p: [round(float(np.min([recs[s][p][0].elapsed_time(recs[s][p][1]) for s in range(args.steps)])), 4),
                  round(float(np.max([recs[s][p][0].elapsed_time(recs[s][p][1]) for s in range(args.steps)])), 4)]
              for p in parts}
    step_ms = float(np.median([recs[s][parts[0]][0].elapsed_time(recs[s][parts[-1]][1]) for s in range(args.steps)]))
    ms["pt_gemms"] = ms["pt_gemm_fwd"] + ms["pt_gemm_dgrad"] + ms["pt_gemm_wgrad"]
    ms["grouped"] = sum(ms[p] for p in ("grouped_q_up", "grouped_gemm_up", "grouped_q_down", "grouped_gemm_down"))
    grouped_gemm_ms = ms["grouped_gemm_up"] + ms["grouped_gemm_down"]
    bwd_parts = ("bwd_rw_quant", "bwd_dgrad_down", "bwd_swiglu_quant", "bwd_dgrad_up", "bwd_wgrad_down",
                 "bwd_wgrad_up")
    ms["moe_bwd"] = sum(ms[p] for p in bwd_parts)
    log("per-part ms (median):", json.dumps({k: round(v, 4) for k, v in ms.items()}))

    # ------------------------------------------------------------------ rates
    flop_gemm = 2.0 * M * N * K                              # each of fwd, dgrad, wgrad
    mx_linear_ms = ms["mx_quant_XWdY"] + ms["mx_gemm_fwd"] + ms["mx_gemm_dgrad"] + ms["mx_gemm_wgrad"]
    value = 3 * flop_gemm / (mx_linear_ms * 1e-3) / 1e12
    q_bytes = lambda r, c: 2 * r * c + 2 * (r * c + r * c // 32)   # read bf16, write both orientations  # noqa: E731
    mxq_XWdY_bytes = q_bytes(M, K) + q_bytes(N, K) + q_bytes(M, N)
    act_bytes = q_bytes(*act3.shape)
    pt_bytes = sum(6 * r * c for r, c in ((M, K), (N, K), (M, N)))
    rows_valid = int(wl4["counts"].sum())
    grouped_flop = 2.0 * rows_valid * d_ff * d_model * 2
    adam_bytes = 21 * n_adam
    rate = {
        "mx_linear_tflops_incl_quant": value,
        "mx_linear_tflops_cached_weight": 3 * flop_gemm / ((mx_linear_ms - ms["mx_quant_XWdY"]
                                                            + (q_bytes(M, K) + q_bytes(M, N)) / mxq_XWdY_bytes
                                                            * ms["mx_quant_XWdY"]) * 1e-3) / 1e12,
        "mx_gemm_fwd_tflops": flop_gemm / (ms["mx_gemm_fwd"] * 1e-3) / 1e12,
        "mx_gemm_dgrad_tflops": flop_gemm / (ms["mx_gemm_dgrad"] * 1e-3) / 1e12,
        "mx_gemm_wgrad_tflops": flop_gemm / (ms["mx_gemm_wgrad"] * 1e-3) / 1e12,
        "mx_gemm_fwd_checked_tflops": flop_gemm / (ms["mx_gemm_fwd_checked"] * 1e-3) / 1e12,
        "mx_gemm_dgrad_checked_tflops": flop_gemm / (ms["mx_gemm_dgrad_checked"] * 1e-3) / 1e12,
        "mx_linear_tflops_incl_quant_checked_gemms": 3 * flop_gemm / ((mx_linear_ms - ms["mx_gemm_fwd"]
                                                                        - ms["mx_gemm_dgrad"] + ms["mx_gemm_fwd_checked"]
                                                                        + ms["mx_gemm_dgrad_checked"]) * 1e-3) / 1e12,
        "mx_quant_XWdY_gbs": mxq_XWdY_bytes / (ms["mx_quant_XWdY"] * 1e-3) / 1e9,
        "pt_linear_tflops_incl_quant": 3 * flop_gemm / ((ms["pt_quant"] + ms["pt_gemms"]) * 1e-3) / 1e12,
        "pt_gemms_tflops": 3 * flop_gemm / (ms["pt_gemms"] * 1e-3) / 1e12,
        "pt_gemm_fwd_tflops": flop_gemm / (ms["pt_gemm_fwd"] * 1e-3) / 1e12,
        "pt_gemm_dgrad_tflops": flop_gemm / (ms["pt_gemm_dgrad"] * 1e-3) / 1e12,
        "pt_gemm_wgrad_tflops": flop_gemm / (ms["pt_gemm_wgrad"] * 1e-3) / 1e12,
        "pt_quant_gbs": pt_bytes / (ms["pt_quant"] * 1e-3) / 1e9,
        "mx_quant_act_gbs": act_bytes / (ms["mx_quant_act"] * 1e-3) / 1e9,
        "mx_quant_act_row_gbs": (2 + 33 / 32) * act3.numel() / (ms["mx_quant_act_row"] * 1e-3) / 1e9,
        "grouped_tflops_incl_act_quant": grouped_flop / (ms["grouped"] * 1e-3) / 1e12,
        "grouped_gemm_only_tflops": grouped_flop / (grouped_gemm_ms * 1e-3) / 1e12,
        "adam_gbs": adam_bytes / (ms["adam"] * 1e-3) / 1e9,
        "adam_gbs_vs_18B_ideal": 18 * n_adam / (ms["adam"] * 1e-3) / 1e9,
        "small_us": ms["small"] * 1e3,
        "small_graph_us": ms["small_graph"] * 1e3,
        "small_queued_us": ms["small_queued"] * 1e3,
        "small_graph_queued_us": ms["small_graph_queued"] * 1e3,
        "pt_quant_delayed_gbs": sum(4 * r * c for r, c in ((M, K), (N, K), (M, N))) / (ms["pt_quant_delayed"] * 1e-3) / 1e9,
        "adam_delayed_gbs": 18 * n_adam / (ms["adam_delayed"] * 1e-3) / 1e9,
        "wcache_fused_gbs": (21 + 2 / 32) * N * K / (ms["wcache_fused"] * 1e-3) / 1e9,
        "wcache_fused_speedup_vs_unfused": ms["wcache_unfused"] / ms["wcache_fused"],
        "moe_swiglu_mlp_tflops_incl_quant": 2.0 * rows_valid * (2 * d_ff * d_model + d_ff * d_model)
                                            / (ms["moe_swiglu_mlp"] * 1e-3) / 1e12,
        "swiglu_quant_gbs": rows4 * (4 * d_ff + d_ff + d_ff // 32) / (ms["swiglu_quant"] * 1e-3) / 1e9,
        "grad_cast_gbs": 3 * nw / (ms["grad_cast"] * 1e-3) / 1e9,
        "grad_requant_gbs": 2 * nw / (ms["grad_requant"] * 1e-3) / 1e9,
        "moe_fwd_train_tflops_incl_quant": 2.0 * rows_valid * 3 * d_ff * d_model / (ms["moe_fwd_train"] * 1e-3) / 1e12,
        "moe_bwd_tflops_incl_quant": 2.0 * rows_valid * 6 * d_ff * d_model / (ms["moe_bwd"] * 1e-3) / 1e12,
        "bwd_rw_quant_gbs": rows4 * (d_model * (2 + 2 * 33 / 32) + 4) / (ms["bwd_rw_quant"] * 1e-3) / 1e9,
        "bwd_swiglu_quant_gbs": rows4 * d_ff * (4 + 2 + 2 * 2 * 33 / 32) / (ms["bwd_swiglu_quant"] * 1e-3) / 1e9,
        "bwd_dgrad_down_tflops": 2.0 * rows_valid * d_ff * d_model / (ms["bwd_dgrad_down"] * 1e-3) / 1e12,
        "bwd_dgrad_up_tflops": 2.0 * rows_valid * 2 * d_ff * d_model / (ms["bwd_dgrad_up"] * 1e-3) / 1e12,
        "bwd_wgrad_down_tflops": 2.0 * rows_valid * d_ff * d_model / (ms["bwd_wgrad_down"] * 1e-3) / 1e12,
        "bwd_wgrad_up_tflops": 2.0 * rows_valid * 2 * d_ff * d_model / (ms["bwd_wgrad_up"] * 1e-3) / 1e12,
    }
    for k, v in rate.items():
        rate[k] = round(v, 3)
    log("rates:", json.dumps(rate))

    attainable = measure_attainable(mxX.q_row, dev, stream)
    log("attainable:", json.dumps(attainable))

    # Every MX GEMM is priced against the dense FP8 peak (its operands are FP8, whichever matrix instruction the
    # library picks); the bf16-peak fraction of the exact-path GEMMs is kept as a secondary field. The headline
    # roofline is the layer's dominant kernel, the GEMM that takes longest.
    gemm_kernels = {
        "mx_gemm_fwd": ("scaled_gemm_ranged fwd Y = X W^T, 4096x36864x12288", "mx_gemm_fwd_tflops"),
        "mx_gemm_dgrad": ("scaled_gemm_ranged dgrad dX = dY W, 4096x12288x36864", "mx_gemm_dgrad_tflops"),
        "mx_gemm_wgrad": ("scaled_gemm_ranged wgrad dW = dY^T X, 36864x12288x4096", "mx_gemm_wgrad_tflops"),
    }

    def gemm_roof(part_name):
        label, key = gemm_kernels[part_name]
        t = rate[key]
        return {"kernel": label + " (" + path_of[part_name] + ")", "bound": "mfma", "achieved": t,
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(t / PEAK_FP8_TFLOPS, 4),
                "traffic": measured_traffic(part_name),
                "frac_of_attainable": round(t / attainable["mfma_fp8_tflops"], 4),
                "frac_of_bf16_peak": round(t / PEAK_BF16_TFLOPS, 4),
                "algorithmic_flop_per_launch": flop_gemm, "avg_launch_ms": round(ms[part_name], 4),
                "share_of_layer": round(ms[part_name] / mx_linear_ms, 4)}

    path_of = {"mx_gemm_fwd": "K = 12288, range words 0: block-scaled FP8 MFMA",
               "mx_gemm_dgrad": "K = 36864, range words 0: block-scaled FP8 MFMA",
               "mx_gemm_wgrad": "K = 4096: exact path, bf16 MFMA on exactly dequantized operands"}
    dominant = max(gemm_kernels, key=lambda p: ms[p])
    roofline = gemm_roof(dominant)

    # The other large kernels of the step against their own bounds: the remaining MX GEMMs (FP8 peak) and the
    # quantize and Adam streams (HBM).
    def hbm(name, gbs, part=None):
        return {"kernel": name, "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4),
                "frac_of_attainable": round(gbs / attainable["hbm_copy_gbs"], 4),
                "traffic": measured_traffic(part) if part else None}
    rooflines_other = [gemm_roof(p) for p in gemm_kernels if p != dominant] + [
        hbm("mxq_quantize of X, W, dY, both orientations", rate["mx_quant_XWdY_gbs"]),
        hbm("mxq_quantize 16384x8192 with outliers, both orientations", rate["mx_quant_act_gbs"], "mx_quant_act"),
        hbm("fp8_adam_step, 1.3e9 params, 21 B/param (amax pass + update pass)", rate["adam_gbs"], "adam"),
        hbm("fp8_adam_step_delayed, 1.3e9 params, 18 B/param (one pass)", rate["adam_delayed_gbs"]),
    ]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(X, W, args.cpu_sample_rows)

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "GPT-175B QKV linear fwd+dgrad+wgrad in MXFP8 (X 4096x12288, W 36864x12288, "
                               "dY 4096x36864): mxq_quantize_ranged of X, W, dY (both orientations, range words) "
                               "and three scaled_gemm_ranged GEMMs, quantize included; plus per-tensor layer, MX "
                               "quantize 16384x8192, grouped 64-expert GEMM and FP8 Adam over 1.3e9 params in the "
                               "same step",
                   "gemm_flop_per_step": 3 * flop_gemm},
        "frac_of_fp8_peak": round(value / PEAK_FP8_TFLOPS, 4),
        "device_ms_per_step": round(step_ms, 3),
        "parts_ms": {k: round(v, 4) for k, v in ms.items()},
        "parts_ms_min_max": spread,
        "timing": f"median of {args.steps} steps per part (events on the launch stream); HBM-bound parts start with "
                  "the last-level cache scrubbed by a 512 MiB write outside their timed window",
        "rates": rate,
        "roofline": roofline,
        "rooflines_other": rooflines_other,
        "attainable": attainable,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mxfp8_precision_numerics_amd", "csrc")


def measured_traffic(part):
    """HBM bytes per launch of one kernel from its committed hardware-counter summary (profiles/*_pmc.md): the line
    'bench-traffic: kernel=<part> fetch_kib=F write_kib=W copy_fetch_per_byte=a copy_write_per_byte=b source=<file>
    source_sha256=<hash>' gives FETCH_SIZE and WRITE_SIZE (KiB per dispatch) and what the same counters read per byte
    of a plain copy of known size; each counter is divided by its copy factor. None when no summary names the kernel,
    or when the kernel's source has changed since the counters were taken."""
    import glob
    import hashlib
    import re

    pat = re.compile(r"bench-traffic: kernel=(\S+) fetch_kib=([\d.e+]+) write_kib=([\d.e+]+) "
                     r"copy_fetch_per_byte=([\d.e+-]+) copy_write_per_byte=([\d.e+-]+) source=(\S+) "
                     r"source_sha256=([0-9a-f]{64})")
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_pmc.md"))):
        for m in pat.finditer(open(path).read()):
            if m.group(1) != part:
                continue
            src = os.path.join(CSRC, m.group(6))
            try:
                if hashlib.sha256(open(src, "rb").read()).hexdigest() != m.group(7):
                    return None
            except OSError:
                return None
            fetch = float(m.group(2)) * 1024 / float(m.group(4))
            write = float(m.group(3)) * 1024 / float(m.group(5))
            return round(fetch + write)
    return None


PROFILE_KERNELS = ["mx_gemm_fwd", "mx_gemm_dgrad", "mx_gemm_wgrad", "grouped_gemm_up", "grouped_gemm_down",
                   "mx_quant_act", "adam", "copy", "read_lds"]


def profile_kernel(name, dev):
    """Ten launches of one kernel (or one call) on the benchmark's seeded inputs, for rocprofv3 counter passes (one
    pass per counter set). Prints the average event-timed duration of the call."""
    import torch

    import mxfp8_precision_numerics_amd as mxq
    from mxfp8_precision_numerics_amd import _probe, workloads

    if name == "copy":
        n = 1 << 30                                            # 1 GiB read + 1 GiB written per launch
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        run = lambda: _probe.copy(src, dst, 0, 8)  # noqa: E731
    elif name == "read_lds":
        n = 1 << 30                                            # 1 GiB read into LDS by the GEMM's copy instruction
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        sink = torch.empty(256, dtype=torch.int32, device=dev)
        run = lambda: _probe.read_lds(src, sink, 256)  # noqa: E731
    elif name in ("mx_gemm_fwd", "mx_gemm_dgrad", "mx_gemm_wgrad"):
        X, W, dY = workloads.workload2(dev)
        (qx, wx), (qw, ww), (qd, wd) = (mxq.mx_quantize_ranged(t) for t in (X, W, dY))
        del X, W, dY
        a, b = {"mx_gemm_fwd": ((qx.q_row, qx.s_row, wx[0:1]), (qw.q_row, qw.s_row, ww[0:1])),
                "mx_gemm_dgrad": ((qd.q_row, qd.s_row, wd[0:1]), (qw.q_col, qw.s_col, ww[1:2])),
                "mx_gemm_wgrad": ((qd.q_col, qd.s_col, wd[1:2]), (qx.q_col, qx.s_col, wx[1:2]))}[name]
        out = torch.empty((a[0].shape[0], b[0].shape[0]), dtype=torch.bfloat16, device=dev)
        run = lambda: mxq.scaled_gemm_ranged(a[0], a[1], a[2], b[0], b[1], b[2], out=out)  # noqa: E731
    elif name in ("grouped_gemm_up", "grouped_gemm_down"):
        wl4 = workloads.workload4(dev)
        off4 = torch.from_numpy(wl4["offsets"]).to(dev)
        A, Wt = (wl4["a_up"], wl4["w_up"]) if name == "grouped_gemm_up" else (wl4["a_down"], wl4["w_down"])
        G, Nn, Kk = Wt.shape
        qa = mxq.mx_quantize(A, colwise=False)
        qw = mxq.mx_quantize(Wt.reshape(G * Nn, Kk), colwise=False)
        out = torch.empty((A.shape[0], Nn), dtype=torch.bfloat16, device=dev)
        run = lambda: mxq.grouped_scaled_gemm(qa.q_row, qa.s_row, off4, qw.q_row.view(G, Nn, Kk),  # noqa: E731
                                              qw.s_row.view(G, Nn, Kk // 32), out=out)
    elif name == "mx_quant_act":
        act3 = workloads.workload3(dev)
        out = mxq.mx_quantize(act3)
        run = lambda: mxq.mx_quantize(act3, out=out)  # noqa: E731
    else:                                                      # adam: the two-pass step over 1.3e9 parameters
        n = 1_300_000_000
        theta = workloads.workload5_params(n, dev)
        grad = workloads.workload5_grad(n, 2, dev)
        m_q = torch.zeros(n, dtype=torch.uint8, device=dev)
        m_scale = torch.ones(1, dtype=torch.float32, device=dev)
        v16 = torch.zeros(n, dtype=torch.float16, device=dev)
        w16 = torch.empty(n, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(mxq.workspace_bytes("adam", n), dtype=torch.uint8, device=dev)
        hp = mxq.AdamHParams(3e-4, 0.9, 0.95, 1e-8, 0.0, 2)
        run = lambda: mxq.fp8_adam_step(theta, grad, m_q, m_scale, v16, w16, hp, workspace=ws)  # noqa: E731
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        run()
    e1.record()
    torch.cuda.synchronize()
    print(json.dumps({"profile_kernel": name, "avg_ms": round(e0.elapsed_time(e1) / 10, 4)}), flush=True)


def measure_attainable(operand_bytes, dev, stream):
    """What this part sustains, measured in the same run beside the spec peaks (libmxq_probe.so): the best of a 1 GiB
    streaming copy (HBM read + write) over looping and full grids with 4, 8 or 16 loads in flight per thread, the
    best streaming read of the same 1 GiB, and the MFMA-only loop of the block-scaled FP8 instruction on real
    quantized operand bytes."""
    import torch

    from mxfp8_precision_numerics_amd import _probe

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    rsink = torch.empty(65536 * 16, dtype=torch.int32, device=dev)
    sink = torch.empty(256 * 256, dtype=torch.float32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    _probe.mfma_fp8(operand_bytes, 200, 256, sink)
    torch.cuda.synchronize()

    def best(fn):
        fn()
        ev[0].record(stream)
        for _ in range(10):
            moved = fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return 10 * moved / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9

    copy_gbs, copy_cfg, read_gbs, read_cfg = 0.0, None, 0.0, None
    for blocks in (0, 1024, 2048, 4096, 8192):
        for unroll in (4, 8, 16):
            g = best(lambda: _probe.copy(src, dst, blocks, unroll))
            if g > copy_gbs:
                copy_gbs, copy_cfg = g, (blocks, unroll)
            g = best(lambda: _probe.read(src, rsink, blocks, unroll))
            if g > read_gbs:
                read_gbs, read_cfg = g, (blocks, unroll)
    ev[2].record(stream)
    flop = _probe.mfma_fp8(operand_bytes, 8000, 256, sink)
    ev[3].record(stream)
    torch.cuda.synchronize()
    mfma_tflops = flop / (ev[2].elapsed_time(ev[3]) * 1e-3) / 1e12
    del src, dst
    grid = lambda c: ("full grid" if c[0] == 0 else f"{c[0]} looping workgroups") + f", {c[1]} loads in flight"  # noqa: E731
    return {"hbm_copy_gbs": round(copy_gbs, 1), "hbm_copy_frac_of_peak": round(copy_gbs / PEAK_HBM_GBS, 4),
            "hbm_copy_config": grid(copy_cfg),
            "hbm_read_gbs": round(read_gbs, 1), "hbm_read_frac_of_peak": round(read_gbs / PEAK_HBM_GBS, 4),
            "hbm_read_config": grid(read_cfg),
            "mfma_fp8_tflops": round(mfma_tflops, 1), "mfma_fp8_frac_of_peak": round(mfma_tflops / PEAK_FP8_TFLOPS, 4)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(X, W, rows):
    """The oracle (unchanged) on the host cores: MX quantize of `rows` rows of X and all of W, then the fp64 GEMM
    of those rows against W (the forward GEMM of the MX linear layer), as TFLOP/s of the sample."""
    import numpy as np

    import oracle
    from mxfp8_precision_numerics_amd import workloads

    threads = oracle.default_threads()
    xs = workloads.as_u16(X[:rows])
    wh = workloads.as_u16(W)
    t0 = time.perf_counter()
    qx, sx, _, _ = oracle.mx_quantize(xs, oracle.RCEIL, colwise=False, nthreads=threads)
    qw, sw, _, _ = oracle.mx_quantize(wh, oracle.RCEIL, colwise=False, nthreads=threads)
    t1 = time.perf_counter()
    oracle.gemm_ref(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3, oracle.MX_BLOCK32, nthreads=threads)
    t2 = time.perf_counter()
    flop = 2.0 * rows * W.shape[0] * W.shape[1]
    log(f"cpu oracle: quantize {t1 - t0:.2f}s, gemm {t2 - t1:.2f}s on {threads} threads")
    # the same computation on one thread, on a smaller sample with the GEMM still dominant: 128 rows of X against
    # the first 1024 rows of W
    r1, n1 = 128, 1024
    t3 = time.perf_counter()
    q1, s1, _, _ = oracle.mx_quantize(xs[:r1], oracle.RCEIL, colwise=False, nthreads=1)
    q2, s2, _, _ = oracle.mx_quantize(wh[:n1], oracle.RCEIL, colwise=False, nthreads=1)
    oracle.gemm_ref(q1, s1, oracle.E4M3, q2, s2, oracle.E4M3, oracle.MX_BLOCK32, nthreads=1)
    t4 = time.perf_counter()
    flop1 = 2.0 * r1 * n1 * W.shape[1]
    log(f"cpu oracle, one thread: {t4 - t3:.2f}s")
    return {"value": round(flop / (t2 - t0) / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"forward GEMM of the MX linear layer for {rows} of 4096 rows of X (2*{rows}*36864*12288 FLOP) "
                      f"in fp64, including MX quantize of those rows and of all of W ({t2 - t0:.1f} s)",
            "single_thread": {"value": round(flop1 / (t4 - t3) / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                              "sample": f"{r1} rows of X against the first {n1} rows of W (2*{r1}*{n1}*12288 FLOP), "
                                        f"including MX quantize of both ({t4 - t3:.1f} s)"}}


if __name__ == "__main__":
    main()
