#!/usr/bin/env python3
"""Benchmark of the NVFP4 hot path on one MI355X (gfx950).

Headline workload (one "step"): qqmm prefill, x bf16 [2048, 4096] Normal(0, 1)
against w NVFP4 [14336, 4096] (quantized once, untimed, from bf16 Normal(0,
0.02) with g_w = amax(w), then packed once into the matrix-core order,
untimed, nvfp4_mfma_pack).  A step is the whole path for one batch: the
activation amax g_x (tensor_amax), then nvfp4_qqmm_packed (the x round trip
into bf16 x_hat, then the MFMA contraction with w decoded in the kernel).
`value` is the step's algorithmic TFLOP/s, 2*M*N*K / step time.

Beside it, on the same run:
  row_major_weight_step  the same step on the row-major weight (nvfp4_qqmm);
  roofline    the contraction kernel alone (nvfp4_qmm_packed on x_hat), per-launch
              time from HIP events on the launch stream, vs 2.5 PFLOP/s bf16;
  qmv         decode x bf16 [1, 4096] @ the same w: algorithmic bytes per
              launch / kernel time, vs 8 TB/s, with the weight rotated over
              copies totalling > 512 MB so the Infinity Cache cannot serve it;
  small_batch_qqmm  qqmm with x bf16 [m, 4096], m = 2, 4, 8, 16, @ the same w,
              row-major and packed (cold weights as for qmv), GB/s of
              algorithmic bytes;
  qqmm_backward  the vjp of the prefill qqmm (dx and dw, 2 x 2 M N K flop) and
              its columnwise passes alone;
  mx_qqmm     the prefill shape in the mxfp4 / mxfp8 modes on the block-scaled
              matrix cores: the whole qqmm, the product alone (vs the dense
              fp4 10.1 / fp8 5.0 PFLOP/s peaks) and the x pre-pass;
  quantize    amax / quantize / dequantize of w bf16 [4096, 4096] with 0.1 %
              outliers (also rotated), GB/s each;
  gather_qmm  MoE: 4096 tokens, 8 experts of [14336, 4096] (packed once,
              untimed; the row-major weight beside it), top-2, TFLOP/s;
  gather_qmm_indexed  the same MoE shape through the indexed form: weights
              stored [k, n] (transpose = False), and the routed and
              sorted_indices paths of transpose = True;
  cpu_baseline  the oracle (plain C, double accumulation) on a bounded row
              sample of the headline workload, on this host's cores.
Inputs are synthetic and already resident in device memory when timing starts.
Each timed section first runs its own work untimed for 50-150 ms (the clocks
ramp for about 40 ms once sustained load starts), then the warm-up calls, then
the timed calls.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "nvfp4 qmv HBM GB/s + qqmm TFLOP/s on 1 MI355X; % of HBM/MFMA roofline"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0

M, N, K = 2048, 14336, 4096

# HBM bytes per launch from two rocprofv3 counter runs (FETCH_SIZE, then
# WRITE_SIZE), each scaled by what the same counter reads for a 512 MiB device
# copy (fetch x 1.9999, write x 1.0000).  A figure holds only for the kernel
# source it was measured on (sha256 prefix of the file and the two headers it
# includes, source_hash), else it is reported
# as null.  Summary and commands: profiles/hbm_traffic_qqmm_gemm_and_qmv.txt.
MEASURED_TRAFFIC = {
    "gemm": ("gemm.hip", "5234486403a77559", 360639669),
    "qmv": ("qmv.hip", "d60a195df5353e3e", 33206718),
    "qmv_packed": ("qmv_packed.hip", "3e6aa809d46492b5", 33226101),
}


def source_hash(src):
    """sha256[:16] of a kernel source together with the two headers it includes."""
    import hashlib
    h = hashlib.sha256()
    for f in (src, "nvfp4_device.h", "nvfp4_internal.h"):
        with open(os.path.join(ROOT, "nvfp4_block_scaled_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    src, sha, nbytes = MEASURED_TRAFFIC[kernel]
    try:
        cur = source_hash(src)
    except OSError:
        return None
    return nbytes if cur == sha else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def settle(fn, seconds=0.15):
    """Run fn untimed for `seconds` of continuous GPU work.  The MI355X's clocks
    ramp for about 40 ms after sustained matrix-core load starts (the qqmm
    contraction runs ~20 % slower in its first milliseconds); the steady state
    is what a serving loop sees, so every timed section starts after this."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def timed(fn, iters, warmup, graph=False):
    """Average milliseconds per call of fn() over `iters` calls, from HIP events
    recorded on the current stream (the stream the library launches on).  With
    graph=True the calls are captured once into a HIP graph and replayed."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(iters):
                    fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        g.replay()
        end.record()
        end.synchronize()
        return start.elapsed_time(end) / iters
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(iters):
        fn()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) / iters


def _pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]


def timed_stats(fn, iters, warmup, graph=False, reps=9):
    """Per-call milliseconds: `mean`, and the median, p10 and p90 of per-call
    means.  Eager: `mean` is that of `iters` calls run back to back between
    two HIP events on the launch stream, as in timed(); the spread comes from
    `reps` further passes of `iters` calls, each pass between two events (an
    event recorded between single calls leaves the GPU idle for about 6 us on
    this runtime, so per-call events would inflate every call).  Graph:
    `reps` replays of one captured graph of `iters` calls, each replay timed;
    `mean` over all replays, the spread over the replays' per-call means."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(iters):
                    fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for r in range(reps):
            g.replay()
            ev[r + 1].record()
        ev[-1].synchronize()
        per = [ev[r].elapsed_time(ev[r + 1]) / iters for r in range(reps)]
        mean = ev[0].elapsed_time(ev[-1]) / (iters * reps)
    else:
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(iters):
            fn()
        end.record()
        end.synchronize()
        mean = start.elapsed_time(end) / iters
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for r in range(reps):
            for _ in range(iters):
                fn()
            ev[r + 1].record()
        ev[-1].synchronize()
        per = [ev[r].elapsed_time(ev[r + 1]) / iters for r in range(reps)]
    return dict(mean=mean, median=_pct(per, 0.5), p10=_pct(per, 0.1), p90=_pct(per, 0.9), n=len(per))


def bench_qqmm(args, nv, torch, W):
    x, w = W.qqmm_inputs(device="cuda")
    gw = nv.nvfp4_tensor_amax(w)
    wc, ws = nv.nvfp4_quantize(w, gw)
    w_host = w.cpu()  # for the oracle's own quantization in the CPU baseline
    del w
    out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    gx = torch.empty(1, dtype=torch.float32, device="cuda")
    wsp, nbytes = nv.qqmm_workspace(M, N, K, torch.bfloat16, "cuda")
    # the weight's packed copy for the matrix-core kernel, made once (untimed,
    # like the quantization itself)
    wp = nv.nvfp4_mfma_pack(wc, ws)

    def step():
        nv.nvfp4_tensor_amax(x, out=gx)
        nv.nvfp4_qqmm_packed(x, wp, gx, gw, out=out, workspace=wsp)

    def step_row_major():
        nv.nvfp4_tensor_amax(x, out=gx)
        nv.nvfp4_qqmm(x, wc, ws, gx, gw, out=out, workspace=wsp)

    settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st_step = timed_stats(step, args.steps, 0)
    wall = time.perf_counter() - t0
    ms_step = st_step["mean"]
    flop = 2.0 * M * N * K
    # the same step on the row-major weight
    ms_step_rm = timed(step_row_major, args.steps, 2)
    # the contraction kernel alone, on x_hat
    xhat = nv.nvfp4_quant_dequant(x, gx)
    gemm = lambda: nv.nvfp4_qmm_packed(xhat, wp, gw, out=out)
    settle(gemm, 0.05)
    st_gemm = timed_stats(gemm, args.steps, 2)
    ms_gemm = st_gemm["mean"]
    ms_prepass = timed(lambda: nv.nvfp4_quant_dequant(x, gx, out=xhat), args.steps, 2, graph=True)
    ms_amax = timed(lambda: nv.nvfp4_tensor_amax(x, out=gx), args.steps, 2, graph=True)
    torch.cuda.synchronize()
    return dict(ms_step=ms_step, wall=wall, tflops=flop / ms_step / 1e9, ms_gemm=ms_gemm,
                gemm_tflops=flop / ms_gemm / 1e9, ms_prepass=ms_prepass, ms_amax=ms_amax, flop=flop,
                ms_step_rm=ms_step_rm, data=(x, w_host), st_step=st_step, st_gemm=st_gemm)


def bench_qmv(args, nv, torch, W):
    x, w = W.qmv_inputs(device="cuda")
    gx, gw = nv.nvfp4_tensor_amax(x), nv.nvfp4_tensor_amax(w)
    wc, ws = nv.nvfp4_quantize(w, gw)
    del w
    per = wc.numel() + ws.numel()
    copies = max(2, -(-600_000_000 // per))  # > 512 MB of weights in rotation
    wcs = [wc.clone() for _ in range(copies)]
    wss = [ws.clone() for _ in range(copies)]
    out = torch.empty(1, N, dtype=torch.bfloat16, device="cuda")
    state = {"i": 0}

    def call():
        i = state["i"] % copies
        state["i"] += 1
        nv.nvfp4_qmv(x, wcs[i], wss[i], gx, gw, out=out)

    # the same weights packed for the matrix cores (the copy the prefill step
    # reads): one row of x through nvfp4_qqmm_packed, the fp4 matrix-core qmv
    wps = [nv.nvfp4_mfma_pack(wcs[i], wss[i]) for i in range(copies)]
    wsp, _ = nv.qqmm_workspace(2, N, K, torch.bfloat16, "cuda")

    def call_packed():
        i = state["i"] % copies
        state["i"] += 1
        nv.nvfp4_qqmm_packed(x, wps[i], gx, gw, out=out, workspace=wsp)

    iters = copies * 4
    settle(call, 0.05)
    st = timed_stats(call, iters, copies, graph=True)
    ms = st["mean"]
    settle(call_packed, 0.05)
    st_packed = timed_stats(call_packed, iters, copies, graph=True)
    ms_packed = st_packed["mean"]
    nbytes = per + x.numel() * 2 + N * 2
    # warm (cache-resident) numbers for context: always the same copy
    ms_warm = timed(lambda: nv.nvfp4_qmv(x, wc, ws, gx, gw, out=out), 64, 8, graph=True)
    ms_packed_warm = timed(lambda: nv.nvfp4_qqmm_packed(x, wps[0], gx, gw, out=out, workspace=wsp),
                           64, 8, graph=True)
    return dict(ms=ms, gbs=nbytes / ms / 1e6, bytes=nbytes, copies=copies, ms_warm=ms_warm,
                gbs_warm=nbytes / ms_warm / 1e6, ms_packed=ms_packed,
                gbs_packed=nbytes / ms_packed / 1e6, gbs_packed_warm=nbytes / ms_packed_warm / 1e6,
                st=st, st_packed=st_packed)


def bench_small(args, nv, torch, W):
    """qqmm with a few rows of x (the decode shape batched): x bf16 [m, 4096]
    Normal(0, 1) with its round trip inside the kernel, cold weights rotated
    as for qmv, row-major and packed; bytes = weight codes + scales + x + out."""
    _, w = W.qmv_inputs(device="cuda")
    gw = nv.nvfp4_tensor_amax(w)
    wc, ws = nv.nvfp4_quantize(w, gw)
    del w
    per = wc.numel() + ws.numel()
    copies = max(2, -(-600_000_000 // per))
    wcs = [wc.clone() for _ in range(copies)]
    wss = [ws.clone() for _ in range(copies)]
    wps = [nv.nvfp4_mfma_pack(wc, ws) for _ in range(copies)]
    r = {}
    for m in (2, 4, 8, 16):
        x = W.normal((m, K), 1.0, 100 + m, "bf16", device="cuda")
        gx = nv.nvfp4_tensor_amax(x)
        out = torch.empty(m, N, dtype=torch.bfloat16, device="cuda")
        wsp, _ = nv.qqmm_workspace(m, N, K, torch.bfloat16, "cuda")
        state = {"i": 0}

        def row_major():
            i = state["i"] % copies
            state["i"] += 1
            nv.nvfp4_qqmm(x, wcs[i], wss[i], gx, gw, out=out, workspace=wsp)

        def packed():
            i = state["i"] % copies
            state["i"] += 1
            nv.nvfp4_qqmm_packed(x, wps[i], gx, gw, out=out, workspace=wsp)

        nbytes = per + m * K * 2 + m * N * 2
        r[m] = {}
        for name, fn in (("row_major", row_major), ("packed", packed)):
            settle(fn, 0.05)
            ms = timed(fn, copies * 4, copies, graph=True)
            r[m][name] = dict(ms=ms, gbs=nbytes / ms / 1e6, bytes=nbytes)
    return r


def bench_backward(args, nv, torch, W):
    """The vjp of the prefill qqmm: x bf16 [2048, 4096], w bf16 [14336, 4096],
    dy bf16 [2048, 14336] Normal(0, 0.01); g_x = amax(x), g_w = amax(w);
    dx and dw, 2 x 2 M N K flop, and the columnwise passes alone."""
    x, w = W.qqmm_inputs(device="cuda")
    dy = W.normal((M, N), 0.01, 7, "bf16", device="cuda")
    gx, gw = nv.nvfp4_tensor_amax(x), nv.nvfp4_tensor_amax(w)
    ws = torch.empty(nv.load_library().nvfp4_qqmm_vjp_workspace_size(M, N, K, 2), dtype=torch.uint8,
                     device="cuda")
    vjp = lambda: nv.nvfp4_qqmm_vjp(x, w, dy, gx, gw, workspace=ws)
    settle(vjp, 0.1)
    ms = timed(vjp, max(args.steps // 2, 5), 2)
    wc = torch.empty(K, N // 2, dtype=torch.uint8, device="cuda")
    wsc = torch.empty(K, N // 16, dtype=torch.uint8, device="cuda")
    dyt = torch.empty(N, M, dtype=torch.bfloat16, device="cuda")
    ms_wcol = timed(lambda: nv.nvfp4_quantize_columnwise(w, gw, codes=wc, scales=wsc), 20, 3, graph=True)
    ms_dycol = timed(lambda: nv.nvfp4_quant_dequant_columnwise(dy, gx, out=dyt), 20, 3, graph=True)
    flop = 2 * 2.0 * M * N * K
    return dict(ms=ms, tflops=flop / ms / 1e9, flop=flop, ms_wcol=ms_wcol,
                wcol_gbs=(N * K * 2 + N * K // 2 + N * K // 16) / ms_wcol / 1e6,
                ms_dycol=ms_dycol, dycol_gbs=(M * N * 4) / ms_dycol / 1e6)


PEAK_MX_TFLOPS = {"mxfp4": 10100.0, "mxfp8": 5000.0}  # dense fp4 / fp8 matrix-core peaks


def bench_mx(args, nv, torch, W):
    """The prefill shape in the mx modes: x bf16 [2048, 4096] quantized in the
    mode (x pre-pass straight into the packed layout), w [14336, 4096]
    quantized and packed once (untimed), the block-scaled product; the whole
    qqmm, the product alone and the pre-pass alone."""
    x, w = W.qqmm_inputs(device="cuda")
    out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    flop = 2.0 * M * N * K
    r = {}
    for mode in ("mxfp4", "mxfp8"):
        wc, ws = nv.nvfp4_mx_quantize(w, mode)
        wp = nv.nvfp4_mx_pack(wc, ws, mode)
        del wc, ws
        wsp, _ = nv.mx_qqmm_workspace(mode, M, N, K, True, "cuda")
        step = lambda: nv.nvfp4_mx_qqmm_packed(x, wp, out=out, workspace=wsp)
        settle(step, 0.1)
        ms = timed(step, args.steps, 2)
        xp = nv.nvfp4_mx_quantize_packed(x, mode)
        gemm = lambda: nv.nvfp4_mx_mm_packed(xp, wp, out=out)
        settle(gemm, 0.05)
        ms_gemm = timed(gemm, args.steps, 2)
        ms_pre = timed(lambda: nv.nvfp4_mx_quantize_packed(x, mode, out=xp), args.steps, 2, graph=True)
        peak = PEAK_MX_TFLOPS[mode]
        r[mode] = dict(ms=ms, tflops=flop / ms / 1e9, ms_gemm=ms_gemm, gemm_tflops=flop / ms_gemm / 1e9,
                       frac=flop / ms_gemm / 1e9 / peak, peak=peak, ms_prepass=ms_pre, flop=flop)
        del wp, wsp, xp
        torch.cuda.synchronize()
        # the decode shape in the mode: one row of x (the streaming kernel),
        # cold weights rotated as for qmv
        x1 = W.normal((1, K), 1.0, 3, "bf16", device="cuda")
        wc, ws = nv.nvfp4_mx_quantize(w, mode)
        per = wc.numel() + ws.numel()
        copies = max(2, -(-600_000_000 // per))
        wcs = [wc.clone() for _ in range(copies)]
        wss = [ws.clone() for _ in range(copies)]
        del wc, ws
        o1 = torch.empty(1, N, dtype=torch.bfloat16, device="cuda")
        wsp1, _ = nv.mx_qqmm_workspace(mode, 1, N, K, False, "cuda")
        state = {"i": 0}

        def call():
            i = state["i"] % copies
            state["i"] += 1
            nv.nvfp4_mx_qqmm(x1, wcs[i], wss[i], mode, out=o1, workspace=wsp1)

        settle(call, 0.05)
        ms_qmv = timed(call, copies * 4, copies, graph=True)
        nbytes = per + K * 2 + N * 2
        r[mode]["qmv"] = dict(ms=ms_qmv, gbs=nbytes / ms_qmv / 1e6, bytes=nbytes, copies=copies)
        del wcs, wss, wsp1
        torch.cuda.synchronize()
    return r


def bench_gather_ex(args, nv, torch, W):
    """The MoE shape (4096 tokens, top-2 of 8 experts, n 14336, k 4096) in the
    indexed form: transpose = False (each expert's [k, n] weight quantized
    along n) and the sorted_indices path of transpose = True (pairs already
    grouped by expert) beside the routed one."""
    T, E, Nn, Kk, top_k = 4096, 8, N, K, 2
    x = W.normal((T, Kk), 1.0, 5, "bf16", device="cuda")
    idx = W.expert_indices(T, E, top_k, 205, device="cuda")
    g = torch.empty(E, dtype=torch.float32, device="cuda")
    flop = 2.0 * T * top_k * Nn * Kk
    r = {}
    # transpose = False
    wc = torch.empty(E, Kk, Nn // 2, dtype=torch.uint8, device="cuda")
    wsc = torch.empty(E, Kk, Nn // 16, dtype=torch.uint8, device="cuda")
    for e in range(E):
        wt = W.normal((Kk, Nn), 0.02, 300 + e, "bf16", device="cuda")
        nv.nvfp4_tensor_amax(wt, out=g[e:e + 1])
        nv.nvfp4_quantize(wt, g[e:e + 1], codes=wc[e], scales=wsc[e])
        del wt
    lhs = (torch.arange(T * top_k, device="cuda", dtype=torch.int32) // top_k).to(torch.int32)
    rhs = idx.reshape(-1).contiguous()
    out = torch.empty(T * top_k, Nn, dtype=torch.bfloat16, device="cuda")
    wsp = torch.empty(nv.load_library().nvfp4_gather_qmm_indexed_workspace_size(T * top_k, 1, E, 1),
                      dtype=torch.uint8, device="cuda")
    f = lambda: nv.nvfp4_gather_qmm_indexed(x, wc, wsc, rhs, lhs, g, transpose=False, out=out, workspace=wsp)
    settle(f, 0.1)
    ms = timed(f, max(3, args.steps // 4), 2)
    r["transpose_false"] = dict(ms=ms, tflops=flop / ms / 1e9)
    del wc, wsc
    torch.cuda.synchronize()
    # transpose = True, routed vs sorted_indices (the same pairs sorted by expert)
    wc = torch.empty(E, Nn, Kk // 2, dtype=torch.uint8, device="cuda")
    wsc = torch.empty(E, Nn, Kk // 16, dtype=torch.uint8, device="cuda")
    for e in range(E):
        w = W.normal((Nn, Kk), 0.02, 400 + e, "bf16", device="cuda")
        nv.nvfp4_tensor_amax(w, out=g[e:e + 1])
        nv.nvfp4_quantize(w, g[e:e + 1], codes=wc[e], scales=wsc[e])
        del w
    order = torch.argsort(rhs.to(torch.int64), stable=True)
    rhs_s = rhs[order].contiguous()
    lhs_s = lhs[order].contiguous()
    for name, srt, rr, ll in (("routed", False, rhs, lhs), ("sorted_indices", True, rhs_s, lhs_s)):
        f = lambda: nv.nvfp4_gather_qmm_indexed(x, wc, wsc, rr, ll, g, transpose=True,
                                                sorted_indices=srt, out=out, workspace=wsp)
        settle(f, 0.1)
        ms = timed(f, max(3, args.steps // 4), 2)
        r[name] = dict(ms=ms, tflops=flop / ms / 1e9)
    torch.cuda.synchronize()
    return r


def bench_quantize(args, nv, torch, W):
    w = W.quantize_weight(device="cuda")
    rows, k = w.shape
    copies = 16
    ws_ = [w.clone() for _ in range(copies)]
    g = nv.nvfp4_tensor_amax(w)
    codes = [torch.empty(rows, k // 2, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    scales = [torch.empty(rows, k // 16, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    deq = [torch.empty(rows, k, dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    for i in range(copies):
        nv.nvfp4_quantize(ws_[i], g, codes=codes[i], scales=scales[i])
    st = {"a": 0, "q": 0, "d": 0}

    def amax():
        i = st["a"] % copies
        st["a"] += 1
        nv.nvfp4_tensor_amax(ws_[i], out=g)

    def quant():
        i = st["q"] % copies
        st["q"] += 1
        nv.nvfp4_quantize(ws_[i], g, codes=codes[i], scales=scales[i])

    def dequant():
        i = st["d"] % copies
        st["d"] += 1
        nv.nvfp4_dequantize(codes[i], scales[i], g, out=deq[i])

    n = rows * k
    b_amax = n * 2
    b_q = n * 2 + n // 2 + n // 16
    b_d = n // 2 + n // 16 + n * 2
    r = {}
    for name, fn, b in (("amax", amax, b_amax), ("quantize", quant, b_q), ("dequantize", dequant, b_d)):
        ms = timed(fn, copies * 2, copies, graph=True)
        r[name] = dict(ms=ms, gbs=b / ms / 1e6, bytes=b, frac=b / ms / 1e6 / PEAK_HBM_GBS)
    return r


def bench_gather(args, nv, torch, W):
    T, E, Nn, Kk, top_k = 4096, 8, N, K, 2
    x, w, idx = W.gather_inputs(device="cuda")
    g = torch.empty(E, dtype=torch.float32, device="cuda")
    wc = torch.empty(E, Nn, Kk // 2, dtype=torch.uint8, device="cuda")
    wsc = torch.empty(E, Nn, Kk // 16, dtype=torch.uint8, device="cuda")
    for e in range(E):
        nv.nvfp4_tensor_amax(w[e], out=g[e:e + 1])
        nv.nvfp4_quantize(w[e], g[e:e + 1], codes=wc[e], scales=wsc[e])
    # the same experts in the mx modes (row-major, as nvfp4_mx_gather_qmm takes them)
    mxw = {}
    for mode, cb in (("mxfp4", Kk // 2), ("mxfp8", Kk)):
        c = torch.empty(E, Nn, cb, dtype=torch.uint8, device="cuda")
        sc = torch.empty(E, Nn, Kk // 32, dtype=torch.uint8, device="cuda")
        for e in range(E):
            nv.nvfp4_mx_quantize(w[e], mode, codes=c[e], scales=sc[e])
        mxw[mode] = (c, sc)
    del w
    # the experts' packed copy for the matrix-core kernel, made once (untimed)
    wp = nv.nvfp4_mfma_pack(wc, wsc)
    torch.cuda.synchronize()
    out = torch.empty(T, top_k, Nn, dtype=torch.bfloat16, device="cuda")
    wsp, _ = nv.gather_workspace(T, top_k, E, Nn, Kk, "cuda")
    gq = lambda: nv.nvfp4_gather_qmm_packed(x, wp, idx, g, out=out, workspace=wsp)
    settle(gq)
    ms = timed(gq, max(3, args.steps // 4), 2)
    gq_rm = lambda: nv.nvfp4_gather_qmm(x, wc, wsc, idx, g, out=out, workspace=wsp)
    settle(gq_rm, 0.05)
    ms_rm = timed(gq_rm, max(3, args.steps // 4), 2)
    flop = 2.0 * T * top_k * Nn * Kk
    mx = {}
    for mode, (c, sc) in mxw.items():
        call = lambda c=c, sc=sc, mode=mode: nv.nvfp4_mx_gather_qmm(x, c, sc, idx, mode, out=out,
                                                                    workspace=wsp)
        settle(call, 0.05)
        ms_mx = timed(call, max(3, args.steps // 4), 2)
        mx[mode] = dict(ms=ms_mx, tflops=flop / ms_mx / 1e9, frac=flop / ms_mx / 1e9 / PEAK_BF16_TFLOPS)
    return dict(ms=ms, tflops=flop / ms / 1e9, flop=flop, frac=flop / ms / 1e9 / PEAK_BF16_TFLOPS,
                ms_rm=ms_rm, tflops_rm=flop / ms_rm / 1e9, mx=mx)


def ceiling_lib():
    """libnvfp4_ceiling.so: the measurement kernels (HBM read, copy, MFMA loop)."""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "nvfp4_block_scaled_amd", "libnvfp4_ceiling.so"))
    P, U64, I64, I = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
    L.nvfp4_ceiling_read.argtypes = [P, U64, P, P]
    L.nvfp4_ceiling_copy.argtypes = [P, P, U64, P]
    L.nvfp4_ceiling_mfma.argtypes = [I64, I, P, P, P]
    for f in (L.nvfp4_ceiling_read, L.nvfp4_ceiling_copy, L.nvfp4_ceiling_mfma):
        f.restype = I
    return L


def bench_ceilings(args, torch):
    """What this GPU allows, measured beside the kernels:
      read   one pass over 33,067,008 bytes (qmv's weight codes + scales + x +
             out), rotated over copies totalling > 512 MB as for qmv;
      copy   32 MiB read + 32 MiB written, rotated the same way;
      mfma   v_mfma_f32_32x32x16_bf16 back to back (4 waves per CU x 2), and the
             shader clock it ran at."""
    L = ceiling_lib()
    stream = lambda: ctypes_stream(torch)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    rb = 33067008
    copies = max(2, -(-600_000_000 // rb))
    bufs = [torch.empty(rb, dtype=torch.uint8, device="cuda").random_(0, 256) for _ in range(copies)]
    st_i = {"i": 0}

    def rd():
        i = st_i["i"] % copies
        st_i["i"] += 1
        rc = L.nvfp4_ceiling_read(bufs[i].data_ptr(), rb, sink.data_ptr(), stream())
        assert rc == 0, rc

    settle(rd, 0.05)
    st_read = timed_stats(rd, copies * 4, copies, graph=True)
    del bufs
    cb = 32 << 20
    ccopies = max(2, -(-600_000_000 // (2 * cb)))
    srcs = [torch.empty(cb, dtype=torch.uint8, device="cuda").random_(0, 256) for _ in range(ccopies)]
    dsts = [torch.empty(cb, dtype=torch.uint8, device="cuda") for _ in range(ccopies)]

    def cp():
        i = st_i["i"] % ccopies
        st_i["i"] += 1
        rc = L.nvfp4_ceiling_copy(srcs[i].data_ptr(), dsts[i].data_ptr(), cb, stream())
        assert rc == 0, rc

    settle(cp, 0.05)
    st_copy = timed_stats(cp, ccopies * 4, ccopies, graph=True)
    assert torch.equal(srcs[0], dsts[0]), "ceiling copy is not a copy"
    del srcs, dsts
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * cus, 20000

    def mf():
        rc = L.nvfp4_ceiling_mfma(iters, blocks, sink.data_ptr(), clocks.data_ptr(), stream())
        assert rc == 0, rc

    settle(mf, 0.1)
    st_mfma = timed_stats(mf, 5, 1)
    cyc, ticks = (int(v) for v in clocks.cpu())
    sclk = cyc / (ticks / 100e6) / 1e9 if ticks > 0 else None
    flop = blocks * 4 * iters * 4 * 32768.0
    return dict(read=st_read, read_bytes=rb, read_copies=copies, copy=st_copy, copy_bytes=cb,
                mfma=st_mfma, mfma_flop=flop, sclk_ghz=sclk)


def ctypes_stream(torch):
    return torch.cuda.current_stream().cuda_stream


def stats_ms(st, scale=1.0, digits=4):
    """A timed_stats dict as {mean, median, p10, p90} in ms (or us with scale 1e3)."""
    return {k: round(st[k] * scale, digits) for k in ("mean", "median", "p10", "p90")}


def bench_copy(args, torch):
    """A plain device-to-device copy of 512 MiB: the calibration kernel for the
    HBM byte counters (FETCH_SIZE / WRITE_SIZE read against known bytes)."""
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 256)
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src), args.steps, args.warmup)
    return dict(ms=ms, bytes_read=n, bytes_written=n, gbs=2 * n / ms / 1e6)


def cpu_baseline(data, seconds_target=20.0):
    """The oracle on a sample of the headline workload, on this host's cores:
    the first `rows` rows of x against the first `cols` weight rows (the
    oracle quantizes w itself, untimed), x round trip + float32 weight decode
    + double sums.  The sample grows (rows first, then weight rows) until one
    run takes a second, then is scaled to about seconds_target."""
    import numpy as np
    import oracle as O
    x, w_host = data
    nthreads = max(1, min(16, os.cpu_count() or 1))
    xh = x.float().cpu().numpy()
    wh = w_host.float().numpy()
    gxh, gwh = O.tensor_amax(xh), O.tensor_amax(wh)
    oc, os_ = O.quantize(wh, gwh)

    def run(rows, cols):
        t0 = time.perf_counter()
        O.qqmm(xh, oc[:cols], os_[:cols], gxh, gwh, dtype="bf16", rows=np.arange(rows),
               nthreads=nthreads)
        return time.perf_counter() - t0

    rows, cols = 4, 256
    while True:
        dt = run(rows, cols)
        if dt >= 1.0 or (rows >= M and cols >= N):
            break
        if rows < M:
            rows = min(M, rows * 2)
        else:
            cols = min(N, cols * 2)
    if dt < seconds_target / 2:
        if rows < M:
            rows = min(M, max(rows, int(rows * seconds_target / dt)))
        else:
            cols = min(N, max(cols, int(cols * seconds_target / dt)))
        dt = run(rows, cols)
    flop = 2.0 * rows * cols * K
    return dict(value=round(flop / dt / 1e12, 6), unit="TFLOP/s", cores=nthreads, kind="oracle",
                sample=f"oracle qqmm on {rows} of {M} rows x {cols} of {N} weight rows, K={K} "
                       f"(x round trip, float32 weight decode, double sums): {dt:.2f} s",
                threads_used=nthreads, host_cpus=os.cpu_count(), cpu_model=cpu_model())


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="all", choices=["all", "qqmm", "qmv", "small", "backward", "mx", "quantize",
                                                      "gather", "gather_ex", "copy", "ceilings"])
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "the kernels run on one MI355X and the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_block_scaled_amd as nv
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    nv.load_library()
    torch.cuda.set_device(0)

    res = {}
    if args.only in ("all", "qqmm"):
        log("qqmm prefill ...")
        res["qqmm"] = bench_qqmm(args, nv, torch, W)
        log(f"  step {res['qqmm']['ms_step']:.3f} ms ({res['qqmm']['tflops']:.1f} TFLOP/s; row-major weight "
            f"{res['qqmm']['flop'] / res['qqmm']['ms_step_rm'] / 1e9:.1f}); "
            f"gemm {res['qqmm']['ms_gemm']:.3f} ms ({res['qqmm']['gemm_tflops']:.1f} TFLOP/s); "
            f"x pre-pass {res['qqmm']['ms_prepass'] * 1e3:.1f} us, amax of x {res['qqmm']['ms_amax'] * 1e3:.1f} us")
    if args.only in ("all", "qqmm", "qmv", "ceilings"):
        log("ceilings (HBM read / copy, bf16 MFMA loop) ...")
        res["ceil"] = bench_ceilings(args, torch)
        c = res["ceil"]
        log(f"  read {c['read']['mean'] * 1e3:.2f} us per 33 MB ({c['read_bytes'] / c['read']['mean'] / 1e6:.0f} GB/s); "
            f"copy {2 * c['copy_bytes'] / c['copy']['mean'] / 1e6:.0f} GB/s; mfma loop "
            f"{c['mfma_flop'] / c['mfma']['mean'] / 1e9:.0f} TFLOP/s at sclk {c['sclk_ghz']:.3f} GHz")
    if args.only in ("all", "qmv"):
        log("qmv decode ...")
        res["qmv"] = bench_qmv(args, nv, torch, W)
        log(f"  row-major {res['qmv']['ms'] * 1e3:.2f} us/launch, {res['qmv']['gbs']:.0f} GB/s "
            f"(warm {res['qmv']['gbs_warm']:.0f} GB/s); packed {res['qmv']['ms_packed'] * 1e3:.2f} "
            f"us/launch, {res['qmv']['gbs_packed']:.0f} GB/s (warm {res['qmv']['gbs_packed_warm']:.0f} GB/s)")
    if args.only in ("all", "small"):
        log("small-batch qqmm (m rows @ the decode weight) ...")
        res["small"] = bench_small(args, nv, torch, W)
        for m_, d in res["small"].items():
            log("  m=%d: " % m_ + ", ".join(f"{k_} {v['ms'] * 1e3:.2f} us ({v['gbs']:.0f} GB/s)"
                                            for k_, v in d.items()))
    if args.only in ("all", "backward"):
        log("qqmm backward (dx and dw of the prefill shape) ...")
        res["backward"] = bench_backward(args, nv, torch, W)
        b = res["backward"]
        log(f"  {b['ms']:.3f} ms, {b['tflops']:.1f} TFLOP/s; columnwise quantize of w "
            f"{b['ms_wcol'] * 1e3:.1f} us ({b['wcol_gbs']:.0f} GB/s), columnwise round trip of dy "
            f"{b['ms_dycol'] * 1e3:.1f} us ({b['dycol_gbs']:.0f} GB/s)")
    if args.only in ("all", "mx"):
        log("mx modes: qqmm prefill in mxfp4 / mxfp8 (block-scaled matrix cores) ...")
        res["mx"] = bench_mx(args, nv, torch, W)
        for mode, d in res["mx"].items():
            log(f"  {mode}: qqmm {d['ms'] * 1e3:.1f} us ({d['tflops']:.0f} TFLOP/s); product alone "
                f"{d['ms_gemm'] * 1e3:.1f} us ({d['gemm_tflops']:.0f} TFLOP/s, {100 * d['frac']:.1f} % of "
                f"{d['peak'] / 1000:.1f} PFLOP/s); x pre-pass {d['ms_prepass'] * 1e3:.1f} us; "
                f"qmv {d['qmv']['ms'] * 1e3:.2f} us ({d['qmv']['gbs']:.0f} GB/s)")
    if args.only in ("all", "quantize"):
        log("quantize / dequantize ...")
        res["quantize"] = bench_quantize(args, nv, torch, W)
        for k_, v in res["quantize"].items():
            log(f"  {k_}: {v['ms'] * 1e3:.2f} us, {v['gbs']:.0f} GB/s")
    if args.only in ("all", "gather"):
        log("gather_qmm MoE ...")
        res["gather"] = bench_gather(args, nv, torch, W)
        log(f"  {res['gather']['ms']:.3f} ms, {res['gather']['tflops']:.1f} TFLOP/s (row-major weight "
            f"{res['gather']['ms_rm']:.3f} ms, {res['gather']['tflops_rm']:.1f} TFLOP/s)")
        for mode, d in res["gather"]["mx"].items():
            log(f"  {mode} weights: {d['ms']:.3f} ms, {d['tflops']:.1f} TFLOP/s")

    if args.only in ("all", "gather_ex"):
        log("gather_qmm indexed forms (transpose = False; sorted_indices) ...")
        res["gather_ex"] = bench_gather_ex(args, nv, torch, W)
        for k_, v in res["gather_ex"].items():
            log(f"  {k_}: {v['ms']:.3f} ms, {v['tflops']:.1f} TFLOP/s")

    if args.only == "copy":
        c = bench_copy(args, torch)
        log(f"copy 512 MiB: {c['ms'] * 1e3:.1f} us, {c['gbs']:.0f} GB/s")
        print(json.dumps({"workload": "device copy (counter calibration)", **c}), flush=True)
        return

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded Normal activations/weights of the pages' shapes)"}
    ceil = res.get("ceil")
    if ceil is not None:
        read_gbs = ceil["read_bytes"] / ceil["read"]["mean"] / 1e6
        mfma_tf = ceil["mfma_flop"] / ceil["mfma"]["mean"] / 1e9
        line["ceilings"] = {
            "hbm_read": {"GBps": round(read_gbs, 1), "frac": round(read_gbs / PEAK_HBM_GBS, 4),
                         "us_per_launch": stats_ms(ceil["read"], 1e3, 3), "bytes": ceil["read_bytes"],
                         "copies_rotated": ceil["read_copies"],
                         "kernel": "read_kernel (nvfp4_ceiling_read: 16-byte nontemporal loads, 8 per thread)"},
            "hbm_copy": {"GBps": round(2 * ceil["copy_bytes"] / ceil["copy"]["mean"] / 1e6, 1),
                         "frac": round(2 * ceil["copy_bytes"] / ceil["copy"]["mean"] / 1e6 / PEAK_HBM_GBS, 4),
                         "us_per_launch": stats_ms(ceil["copy"], 1e3, 3),
                         "bytes_read_and_written": 2 * ceil["copy_bytes"], "kernel": "copy_kernel (nvfp4_ceiling_copy)"},
            "mfma_bf16_loop": {"TFLOPs": round(mfma_tf, 1), "frac": round(mfma_tf / PEAK_BF16_TFLOPS, 4),
                               "sclk_GHz": round(ceil["sclk_ghz"], 3) if ceil["sclk_ghz"] else None,
                               "kernel": "mfma_kernel (nvfp4_ceiling_mfma: v_mfma_f32_32x32x16_bf16, no memory)"},
            "profiles": "profiles/ceilings_read_copy_mfma.txt"}
    if "qqmm" in res:
        q = res["qqmm"]
        line.update(value=round(q["tflops"], 2), unit="TFLOP/s", ms_per_step=round(q["ms_step"], 4))
        line["ms_per_step_stats"] = stats_ms(q["st_step"])
        line["config"] = {"workload": "qqmm prefill: x bf16 [2048,4096] (amax + NVFP4 round trip) "
                                      "@ NVFP4 w [14336,4096]^T (packed once for the matrix cores), bf16 out",
                          "m": M, "n": N, "k": K, "group_size": 16}
        line["roofline"] = {"bound": "mfma",
                            "kernel": "mfma_gemm_fast_kernel<bf16, packed> (nvfp4_qmm_packed on x_hat)",
                            "achieved": round(q["gemm_tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(q["gemm_tflops"] / PEAK_BF16_TFLOPS, 4),
                            "traffic": measured_traffic("gemm"), "ms_per_launch": round(q["ms_gemm"], 4),
                            "algorithmic_flop_per_launch": q["flop"],
                            "algorithmic_bytes_per_launch": M * K * 2 + N * K // 2 + N * K // 16 + M * N * 2,
                            "ms_per_launch_stats": stats_ms(q["st_gemm"])}
        if ceil is not None and ceil["sclk_ghz"]:
            sclk = ceil["sclk_ghz"]
            peak_at = PEAK_BF16_TFLOPS * sclk / 2.4
            line["roofline"].update(
                sclk_GHz=round(sclk, 3), peak_at_sclk=round(peak_at, 1),
                frac_clock_adjusted=round(q["gemm_tflops"] / peak_at, 4),
                frac_of_mfma_loop_ceiling=round(q["gemm_tflops"] / mfma_tf, 4))
        line["x_prepass_us"] = round(q["ms_prepass"] * 1e3, 2)
        line["x_amax_us"] = round(q["ms_amax"] * 1e3, 2)
        line["row_major_weight_step"] = {"value": round(q["flop"] / q["ms_step_rm"] / 1e9, 2),
                                         "unit": "TFLOP/s", "ms_per_step": round(q["ms_step_rm"], 4)}
    if "qmv" in res:
        v = res["qmv"]
        line["qmv"] = {"value": round(v["gbs"], 1), "unit": "GB/s", "peak": PEAK_HBM_GBS,
                       "frac": round(v["gbs"] / PEAK_HBM_GBS, 4), "us_per_launch": round(v["ms"] * 1e3, 3),
                       "algorithmic_bytes_per_launch": v["bytes"], "traffic": measured_traffic("qmv"),
                       "weight_copies_rotated": v["copies"],
                       "warm_cache_GBps": round(v["gbs_warm"], 1),
                       "us_per_launch_stats": stats_ms(v["st"], 1e3, 3),
                       "kernel": "qmv_stream_kernel<bf16> (nvfp4_qmv, row-major weight)",
                       "packed_weight": {"GBps": round(v["gbs_packed"], 1),
                                         "frac": round(v["gbs_packed"] / PEAK_HBM_GBS, 4),
                                         "us_per_launch": round(v["ms_packed"] * 1e3, 3),
                                         "us_per_launch_stats": stats_ms(v["st_packed"], 1e3, 3),
                                         "warm_cache_GBps": round(v["gbs_packed_warm"], 1),
                                         "traffic": measured_traffic("qmv_packed"),
                                         "kernel": "qmv_packed_kernel<bf16> (nvfp4_qqmm_packed, m = 1)"},
                       "workload": "qmv decode: x bf16 [1,4096] @ NVFP4 w [14336,4096]^T"}
        if ceil is not None:
            line["qmv"]["frac_of_read_ceiling"] = round(v["gbs"] / read_gbs, 4)
            line["qmv"]["packed_weight"]["frac_of_read_ceiling"] = round(v["gbs_packed"] / read_gbs, 4)
    if "small" in res:
        line["small_batch_qqmm"] = {
            f"m={m_}": {k_: {"GBps": round(v["gbs"], 1), "frac": round(v["gbs"] / PEAK_HBM_GBS, 4),
                             "us": round(v["ms"] * 1e3, 3), "bytes": v["bytes"]}
                        for k_, v in d.items()}
            for m_, d in res["small"].items()}
        line["small_batch_qqmm"]["workload"] = ("qqmm x bf16 [m,4096] (round trip in the kernel) "
                                                "@ NVFP4 w [14336,4096]^T, cold weights")
    if "backward" in res:
        b = res["backward"]
        line["qqmm_backward"] = {
            "value": round(b["tflops"], 2), "unit": "TFLOP/s", "frac": round(b["tflops"] / PEAK_BF16_TFLOPS, 4),
            "ms": round(b["ms"], 4), "algorithmic_flop": b["flop"],
            "columnwise_quantize_w": {"us": round(b["ms_wcol"] * 1e3, 2), "GBps": round(b["wcol_gbs"], 1)},
            "columnwise_round_trip_dy": {"us": round(b["ms_dycol"] * 1e3, 2), "GBps": round(b["dycol_gbs"], 1)},
            "workload": "vjp of qqmm x bf16 [2048,4096] @ w [14336,4096]^T: dx and dw for dy [2048,14336]"}
    if "mx" in res:
        line["mx_qqmm"] = {mode: {"value": round(d["tflops"], 2), "unit": "TFLOP/s", "us": round(d["ms"] * 1e3, 2),
                                  "product_alone": {"TFLOPs": round(d["gemm_tflops"], 2),
                                                    "us": round(d["ms_gemm"] * 1e3, 2),
                                                    "peak": d["peak"], "frac": round(d["frac"], 4),
                                                    "kernel": f"mx_gemm_kernel<bf16, {4 if mode == 'mxfp4' else 8}>"},
                                  "x_prepass_us": round(d["ms_prepass"] * 1e3, 2),
                                  "qmv": {"GBps": round(d["qmv"]["gbs"], 1), "unit": "GB/s",
                                          "frac": round(d["qmv"]["gbs"] / PEAK_HBM_GBS, 4),
                                          "us_per_launch": round(d["qmv"]["ms"] * 1e3, 3),
                                          "algorithmic_bytes_per_launch": d["qmv"]["bytes"],
                                          "weight_copies_rotated": d["qmv"]["copies"],
                                          "kernel": f"mx_qmv_kernel<bf16, {4 if mode == 'mxfp4' else 8}>"}}
                           for mode, d in res["mx"].items()}
        line["mx_qqmm"]["workload"] = ("qqmm x bf16 [2048,4096] (quantized in the mode) @ w [14336,4096]^T "
                                       "in mxfp4 / mxfp8 (packed once), bf16 out; qmv: x bf16 [1,4096] "
                                       "@ the row-major mx weight, cold weights")
    if "quantize" in res:
        line["quantize"] = {k_: {"GBps": round(v["gbs"], 1), "frac": round(v["frac"], 4),
                                 "us": round(v["ms"] * 1e3, 3), "bytes": v["bytes"]}
                            for k_, v in res["quantize"].items()}
    if "gather" in res:
        gq = res["gather"]
        line["gather_qmm"] = {"value": round(gq["tflops"], 2), "unit": "TFLOP/s",
                              "frac": round(gq["frac"], 4), "ms": round(gq["ms"], 4),
                              "row_major_weight": {"value": round(gq["tflops_rm"], 2),
                                                   "ms": round(gq["ms_rm"], 4)},
                              "mx_weights": {mode: {"value": round(d["tflops"], 2), "frac": round(d["frac"], 4),
                                                    "ms": round(d["ms"], 4)}
                                             for mode, d in gq["mx"].items()},
                              "workload": "4096 tokens x top-2 of 8 experts, NVFP4 w [8,14336,4096] "
                                          "(packed once for the matrix cores); mx_weights: the same "
                                          "experts in mxfp4 / mxfp8, row-major (nvfp4_mx_gather_qmm)"}
    if "gather_ex" in res:
        line["gather_qmm_indexed"] = {k_: {"value": round(v["tflops"], 2), "unit": "TFLOP/s",
                                           "frac": round(v["tflops"] / PEAK_BF16_TFLOPS, 4),
                                           "ms": round(v["ms"], 4)}
                                      for k_, v in res["gather_ex"].items()}
        line["gather_qmm_indexed"]["workload"] = (
            "4096 tokens x top-2 of 8 experts, n 14336, k 4096, lhs_indices = pair // 2: transpose=False "
            "(weights [8,4096,14336] quantized along n); transpose=True routed vs sorted_indices")
    if "qqmm" in res and not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(res["qqmm"]["data"])
    if "value" not in line:
        line.update(value=None, unit=None, ms_per_step=None, config={"workload": args.only})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
