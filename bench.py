#!/usr/bin/env python3
"""Benchmark of the mixed-precision linear layer on one MI355X.

A step is one pass of the whole layer over one batch:
mixq_quantize_act_regather (amax, gate, quantize, outlier split, and the
weight's outlier-column regather, a device-side no-op unless the set
changed; two launches) and mixq_gemm_ws (INT8 x INT8 product, FP16 outlier
product, fused epilogue).
Inputs are seeded synthetic tensors already resident in HBM; several copies
of the inputs and packed weights are rotated so that the 256 MB Infinity
Cache cannot serve them from one step to the next.

Prints one JSON line.  ``value`` is the step throughput in effective TOPS
(2*M*N*K per step, outliers counted once).  ``roofline`` reports the GEMM
kernel, timed with HIP events on its stream: one event pair around each of
100 launches (median, spread) and one around the same launches back to back
(``gemm_us``, without the per-launch event overhead).
``cpu_baseline`` times the CPU oracle on a bounded row sample of the same
workload (only with --gpus 1, on rank 0).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_I8_TOPS = 5000.0       # MI355X dense INT8 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_F16_TFLOPS = 2500.0    # MI355X dense FP16 MFMA, published
PEAK_CLOCK_GHZ = 2.4        # MI355X peak engine clock (the published peaks' clock)
METRIC = "mixed-precision GEMM effective TOPS + % of INT8 MFMA peak (LLaMA shapes)"
CACHE_DEFEAT_BYTES = 768 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")
GEMM_SRC = os.path.join(ROOT, "mixed_precision_quantized_amax_amd", "csrc", "mixq_gemm.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def launch_times(stream, n: int, fn) -> dict:
    """Durations (us) of n launches of fn, each bracketed by its own HIP
    event pair on the launch stream: median, mean, min and 90th percentile.
    Then the same n launches back to back between one event pair:
    batch_us, their mean duration without the per-launch event overhead
    (the recording of an event pair adds a few microseconds to the time
    between them)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        fn(i)
        e1.record(stream)
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e3
    b0, b1 = evs[0]
    b0.record(stream)
    for i in range(n):
        fn(i)
    b1.record(stream)
    torch.cuda.synchronize()
    return {"median_us": round(float(np.median(t)), 2), "mean_us": round(float(t.mean()), 2),
            "min_us": round(float(t.min()), 2), "p90_us": round(float(np.percentile(t, 90)), 2),
            "launches": n, "batch_us": round(b0.elapsed_time(b1) * 1e3 / n, 2)}


def clock_buffer():
    """Device buffer for mixq_set_clock_record: four int64 stamps per block."""
    import torch
    return torch.zeros(4 * 4096, dtype=torch.int64, device="cuda")


def clock_summary(buf, event_us=None) -> dict:
    """Engine clock of the GEMM kernel itself: its blocks record the shader
    clock (s_memtime) and the 100 MHz real-time counter at entry and exit
    (mixq_set_clock_record); the clock of a block is the ratio of the two
    deltas.  The buffer holds the last recorded launch: median and range
    over its blocks, the block duration, and the launch's span (first entry
    to last exit), which must not exceed its event-timed duration."""
    c = buf.view(-1, 4).cpu().numpy()
    c = c[c[:, 3] > c[:, 2]]
    f = (c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 100e6) / 1e9
    span_us = (c[:, 3].max() - c[:, 2].min()) / 100.0
    out = {"ghz_median": round(float(np.median(f)), 3), "ghz_min": round(float(f.min()), 3),
           "ghz_max": round(float(f.max()), 3), "blocks": int(c.shape[0]),
           "block_us_median": round(float(np.median(c[:, 3] - c[:, 2])) / 100.0, 2),
           "kernel_span_us": round(float(span_us), 2)}
    if event_us is not None:
        out["event_us_same_launches"] = event_us
    return out


def run_mfma_probe(stream, a, b, iters: int = 128, blocks: int = 256, warmup: int = 100,
                   n: int = 100) -> dict:
    """The GEMM main loop's INT8 MFMA stream with no memory traffic
    (mixq_mfma_probe) on the given operand bytes: blocks x 4 waves, iters
    rounds of 32 MFMAs per wave.  At 256 blocks and 128 rounds it issues the
    MFMAs of the 256 x 256 GEMM at M = 2048, K = N = 8192 (2 x 2048 x 8192 x
    8192 ops), so its time is the GEMM's ceiling at the clock the board then
    sustains.  Timed like the GEMM: n launches back to back, the engine clock
    from the last one's blocks."""
    import torch
    from mixed_precision_quantized_amax_amd import mixq
    a8 = a.reshape(-1).view(torch.int8)
    b8 = b.reshape(-1).view(torch.int8)
    out = torch.empty(256 * blocks, dtype=torch.int32, device=a.device)
    clk = torch.zeros(4 * blocks, dtype=torch.int64, device=a.device)
    s = stream.cuda_stream
    for _ in range(warmup):
        mixq.mfma_probe(a8, b8, iters, blocks, out, None, s)
    t = launch_times(stream, n, lambda i: mixq.mfma_probe(a8, b8, iters, blocks, out, clk, s))
    ops = blocks * 4 * iters * 32 * 2 * 32 * 32 * 32
    tops = ops / (t["batch_us"] / 1e6) / 1e12
    return {"tops": round(tops, 1), "pct_of_published_peak": round(100.0 * tops / PEAK_I8_TOPS, 2),
            "us": t["batch_us"], "ops": ops, "blocks": blocks, "rounds": iters,
            "engine_clock": clock_summary(clk, t["batch_us"]),
            "operands": "the workload's own Xq and packed weight bytes"}


def run_vendor_int8(stream, Xqs, packs, n: int = 100, warmup: int = 50) -> dict:
    """The vendor library's plain INT8 GEMM at the same shape, for comparison
    only: torch._int_mm (hipBLASLt on ROCm) on the same operand bytes (the
    workload's Xq copies and their INT8 packed weights, rotated like the
    GEMM's), int32 output, with no quantization, outlier product, scales or
    fp32 epilogue.  Timed like the GEMM (100 launches back to back)."""
    import torch
    try:
        ops = [(x, p.wq.view(torch.int8).view(p.N, p.K).t()) for x, p in zip(Xqs, packs)]
        for i in range(warmup):
            torch._int_mm(*ops[i % len(ops)])
        t = launch_times(stream, n, lambda i: torch._int_mm(*ops[i % len(ops)]))
    except Exception as e:  # reported, never fatal for the layer's numbers
        return {"error": repr(e)}
    M, K = Xqs[0].shape
    N = packs[0].N
    return {"us": t["batch_us"], "median_us": t["median_us"],
            "tops": round(2.0 * M * N * K / (t["batch_us"] / 1e6) / 1e12, 1),
            "call": "torch._int_mm (hipBLASLt), int8 x int8 -> int32, same operand bytes"}


def gemm_source_sha() -> str:
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def gemm_traffic(workload: str):
    """HBM bytes per GEMM launch from the committed counter summary, if it was
    taken on the current GEMM source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha") != gemm_source_sha():
        return None
    w = t.get("workloads", {}).get(workload)
    return None if w is None else int(w["hbm_bytes_per_launch"])


def algorithmic_bytes(wl, k: int) -> int:
    """Bytes a GEMM launch must move at least once: Xq, the packed weight,
    the two scale vectors, the padded outlier matrices and the fp32 Y."""
    kp = (k + 31) // 32 * 32
    return (wl.M * wl.K + wl.N * wl.K * wl.bits // 8 + 4 * (wl.M + wl.N)
            + 2 * kp * (wl.M + wl.N) + 4 * wl.M * wl.N)


def run_gpu(wl, steps: int, warmup: int, group: int = 0, counters: bool = False,
            probe: bool = False):
    """group: 0, or the progressive INT4 group size (INT4 workloads).
    counters: run the warmup and timed steps only (a byte-counter pass).
    probe: also run the matrix-core rate probe on the workload's operands."""
    import torch
    from mixed_precision_quantized_amax_amd import mixq, workloads

    dev = torch.device("cuda", 0)
    log(f"[bench] workload {wl.name}: M={wl.M} K={wl.K} N={wl.N} bits={wl.bits} group={group}")
    W = torch.from_numpy(workloads.make_weight(wl)).to(dev)
    X0 = torch.from_numpy(workloads.make_activation(wl)).to(dev)
    k_cap = 256
    wq_bytes = wl.N * wl.K * wl.bits // 8
    copies = int(min(8, max(2, math.ceil(CACHE_DEFEAT_BYTES / (wq_bytes + 3 * wl.M * wl.K)))))
    state = mixq.OutlierState.create(wl.K, k_cap, dev)
    packs = [mixq.PackedWeight.create(wl.N, wl.K, wl.bits, k_cap, dev, group=group)
             for _ in range(copies)]
    for p in packs:
        mixq.pack_weight(W, state, p, mixq.PACK_FULL)
    # activation copies: the same values in different buffers
    Xs = [X0.clone() for _ in range(copies)]
    ld = mixq.outlier_ld(k_cap)
    Xq = [torch.empty(wl.M, wl.K, dtype=torch.int8, device=dev) for _ in range(copies)]
    sx = [torch.empty(wl.M, dtype=torch.float32, device=dev) for _ in range(copies)]
    Xo = [torch.zeros(wl.M * ld, dtype=torch.float16, device=dev) for _ in range(copies)]
    Y = torch.empty(wl.M, wl.N, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # split-K workspace (thin shapes, and the tail of a product a little over
    # one round of 256 x 256 tiles); N = the packed row count
    ws = mixq.gemm_workspace(wl.M, packs[0].N, wl.K, wl.bits, dev)
    steps_c = [mixq.LayerStep(Xs[c], wl.tau, state, W, packs[c], Xq[c], sx[c], Xo[c], Y, ws=ws)
               for c in range(copies)]
    # the same steps with the quantize and the column gather as separate calls
    steps_u = [mixq.LayerStep(Xs[c], wl.tau, state, W, packs[c], Xq[c], sx[c], Xo[c], Y, ws=ws,
                              fused=False) for c in range(copies)]

    def step(i, ev=None):
        s = steps_c[i % copies]
        if ev is None:
            s()
            return
        ev[0].record(stream)
        s.act()
        ev[1].record(stream)
        s.gemm()
        ev[2].record(stream)

    # first call detects the planted outlier channels
    step(0)
    torch.cuda.synchronize()
    count = int(state.count.cpu()[0])
    log(f"[bench] outlier channels detected: {count}; weight copies: {copies}")
    # one captured graph per buffer copy: a replay launches the step's four
    # kernels without a host round trip per kernel
    graphs = [] if counters else [
        mixq.LayerGraph(Xs[c], wl.tau, state, W, packs[c], Xq[c], sx[c], Xo[c], Y, ws=ws)
        for c in range(copies)]
    for i in range(warmup):
        step(i)
    if graphs:
        graphs[0].replay()
    torch.cuda.synchronize()

    # timed region: whole steps through the three library calls
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    if counters:
        return dict(ms_step=ms_step, count=count, copies=copies)

    # the same steps replayed from the captured graphs, for comparison
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        graphs[i % copies].replay()
    t1.record(stream)
    torch.cuda.synchronize()
    graph_ms_step = t0.elapsed_time(t1) / steps

    # GEMM kernel duration, one event pair around each launch on its stream:
    # clean cache (the copies rotate, as in the steps) and hot (one copy)
    nl = max(50, steps)
    # the clean-cache launches also record the engine clock (the stamps of
    # the last one remain), so that clock and duration come from the same
    # launches
    cbuf = clock_buffer()
    mixq.set_clock_record(cbuf)
    try:
        gemm_clean = launch_times(stream, nl, lambda i: steps_c[i % copies].gemm())
    finally:
        mixq.set_clock_record(None)
    clk = clock_summary(cbuf, gemm_clean["batch_us"])
    gemm_hot = launch_times(stream, nl, lambda i: steps_c[0].gemm())
    act_t = launch_times(stream, nl, lambda i: steps_c[i % copies].act())
    act_u = launch_times(stream, nl, lambda i: steps_u[i % copies].act())
    flag = int(state.flag.cpu()[0])
    mprobe = run_mfma_probe(stream, Xq[0], packs[0].wq) if probe else None
    vendor = run_vendor_int8(stream, Xq, packs) if probe and wl.bits == 8 else None
    return dict(ms_step=ms_step, graph_ms_step=graph_ms_step, gemm=gemm_clean, gemm_hot=gemm_hot,
                act=act_t, act_separate=act_u, clock=clk, count=count, flag=flag,
                copies=copies, probe=mprobe, vendor=vendor)


def run_mixed(wl, steps: int, warmup: int, salient):
    """Output-feature mixed precision on the workload's shape: the salient
    rows as an INT8 row subset, the others as progressive INT4, one
    activation pass, then both outlier-column gathers and both products into
    one Y."""
    import torch
    from mixed_precision_quantized_amax_amd import mixq, workloads

    dev = torch.device("cuda", 0)
    log(f"[bench] mixed features on {wl.name}: {int(salient.sum())} of {wl.N} rows at 8 bits")
    W = torch.from_numpy(workloads.make_weight(wl)).to(dev)
    X0 = torch.from_numpy(workloads.make_activation(wl)).to(dev)
    k_cap = 256
    copies = 4
    state = mixq.OutlierState.create(wl.K, k_cap, dev)
    mws = [mixq.MixedWeight.create(salient, wl.K, k_cap, dev) for _ in range(copies)]
    for m in mws:
        m.pack(W, state, mixq.PACK_FULL)
    Xs = [X0.clone() for _ in range(copies)]
    ld = mixq.outlier_ld(k_cap)
    Xq = [torch.empty(wl.M, wl.K, dtype=torch.int8, device=dev) for _ in range(copies)]
    sx = [torch.empty(wl.M, dtype=torch.float32, device=dev) for _ in range(copies)]
    Xo = [torch.zeros(wl.M * ld, dtype=torch.float16, device=dev) for _ in range(copies)]
    Y = torch.empty(wl.M, wl.N, dtype=torch.float32, device=dev)
    ws = mws[0].workspaces(wl.M, dev)

    def act(i):
        c = i % copies
        mixq.quantize_act(Xs[c], wl.tau, state, Xq[c], sx[c], Xo[c])
        mws[c].pack(W, state, mixq.PACK_OUTLIER_COLS)

    def gemm(i):
        c = i % copies
        mws[c].gemm(Xq[c], sx[c], Xo[c], state, Y, ws=ws)

    for i in range(warmup):
        act(i)
        gemm(i)
    stream = torch.cuda.current_stream(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fns in (("ms_step", (act, gemm)), ("gemm_ms", (gemm,)), ("act_ms", (act,))):
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(steps):
            for f in fns:
                f(i)
        t1.record(stream)
        torch.cuda.synchronize()
        res[name] = t0.elapsed_time(t1) / steps
    res["rows"] = (mws[0].w8.N if mws[0].w8 is not None else 0,
                   mws[0].w4.N if mws[0].w4 is not None else 0)
    return res


def norm_act_bytes(wl, k: int) -> int:
    """Bytes the fused RMSNorm + activation pass must move at least once:
    H in, gamma, Xq out, s_x and rstd, the padded outlier matrix."""
    kp = (k + 31) // 32 * 32
    return 3 * wl.M * wl.K + 2 * wl.K + 8 * wl.M + 2 * wl.M * kp


def run_fused_norm(wl, steps: int, warmup: int, eps: float = 1e-5):
    """The activation side with the RMSNorm before the layer fused in
    (mixq_rmsnorm_quantize_act), against the same work unfused: torch's
    rms_norm writing the normalised fp16 tokens, then mixq_quantize_act.
    Steady state: the outlier set is detected by the first call and cached."""
    import torch
    import torch.nn.functional as F
    from mixed_precision_quantized_amax_amd import mixq, workloads

    dev = torch.device("cuda", 0)
    H0 = torch.from_numpy(workloads.make_activation(wl)).to(dev)
    gamma = torch.from_numpy(workloads.make_norm_gamma(wl)).to(dev)
    k_cap = 256
    copies = int(min(16, max(2, math.ceil(CACHE_DEFEAT_BYTES / (3 * wl.M * wl.K)))))
    ld = mixq.outlier_ld(k_cap)
    Hs = [H0.clone() for _ in range(copies)]
    Xq = [torch.empty(wl.M, wl.K, dtype=torch.int8, device=dev) for _ in range(copies)]
    sx = [torch.empty(wl.M, dtype=torch.float32, device=dev) for _ in range(copies)]
    Xo = [torch.zeros(wl.M * ld, dtype=torch.float16, device=dev) for _ in range(copies)]
    rs = [torch.empty(wl.M, dtype=torch.float32, device=dev) for _ in range(copies)]
    st_f = mixq.OutlierState.create(wl.K, k_cap, dev)
    st_u = mixq.OutlierState.create(wl.K, k_cap, dev)
    st_r = mixq.OutlierState.create(wl.K, k_cap, dev)
    # residual variant: H = R + D written to its own buffer (R = the copies above)
    D0 = (torch.randn(wl.M, wl.K, generator=torch.Generator().manual_seed(7)) * 0.1).half().to(dev)
    Ho = [torch.empty_like(H0) for _ in range(copies)]
    stream = torch.cuda.current_stream(dev)

    def fused(i):
        c = i % copies
        mixq.rmsnorm_quantize_act(Hs[c], gamma, eps, wl.tau, st_f, Xq[c], sx[c], Xo[c], rs[c])

    def unfused(i):
        c = i % copies
        Xn = F.rms_norm(Hs[c], (wl.K,), gamma, eps)
        mixq.quantize_act(Xn, wl.tau, st_u, Xq[c], sx[c], Xo[c])

    def fused_add(i):
        c = i % copies
        mixq.add_rmsnorm_quantize_act(Hs[c], D0, Ho[c], gamma, eps, wl.tau, st_r, Xq[c], sx[c],
                                      Xo[c], rs[c])

    def unfused_add(i):
        c = i % copies
        torch.add(Hs[c], D0, out=Ho[c])
        Xn = F.rms_norm(Ho[c], (wl.K,), gamma, eps)
        mixq.quantize_act(Xn, wl.tau, st_u, Xq[c], sx[c], Xo[c])

    for i in range(warmup):
        fused(i)
        unfused(i)
        fused_add(i)
        unfused_add(i)
    torch.cuda.synchronize()
    count = int(st_f.count.cpu()[0])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn in (("fused", fused), ("unfused", unfused), ("fused_add", fused_add),
                     ("unfused_add", unfused_add)):
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    flag = int(st_f.flag.cpu()[0])
    us = res["fused"] * 1e3
    gbs = norm_act_bytes(wl, count) / (res["fused"] / 1e3) / 1e9
    log(f"[bench] fused rmsnorm+act {us:.2f} us ({gbs:.0f} GB/s), unfused "
        f"{res['unfused'] * 1e3:.2f} us; set {count}, last flag {flag}")
    return {"us": round(us, 2), "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": norm_act_bytes(wl, count), "outlier_channels": count,
            "last_flag": flag, "eps": eps,
            "unfused_us": round(res["unfused"] * 1e3, 2),
            "unfused": "torch rms_norm (fp16 out) + mixq_quantize_act",
            "with_residual_add_us": round(res["fused_add"] * 1e3, 2),
            "with_residual_add_gbs": round((norm_act_bytes(wl, count) + 4 * wl.M * wl.K)
                                           / (res["fused_add"] / 1e3) / 1e9, 1),
            "with_residual_add_unfused_us": round(res["unfused_add"] * 1e3, 2),
            "kernels": "gate_quant_kernel (RMSNorm prologue) + requant_kernel (no-op unless "
                       "the gate fires)"}


def run_swiglu(wl, steps: int, warmup: int):
    """The workload's weight read as a fused gate-and-up projection ([W_gate;
    W_up], I = N/2): the GEMM with the SwiGLU epilogue (fp16 silu(gate) * up,
    mixq_gemm_ex) against the same GEMM writing fp32 followed by torch's
    silu, multiply and cast to fp16."""
    import torch
    import torch.nn.functional as F
    from mixed_precision_quantized_amax_amd import mixq, workloads

    dev = torch.device("cuda", 0)
    W = torch.from_numpy(workloads.make_weight(wl)).to(dev)
    X = torch.from_numpy(workloads.make_activation(wl)).to(dev)
    k_cap = 256
    wq_bytes = wl.N * wl.K * wl.bits // 8
    copies = int(min(8, max(2, math.ceil(CACHE_DEFEAT_BYTES / wq_bytes))))
    st = mixq.OutlierState.create(wl.K, k_cap, dev)
    packs = [mixq.PackedWeight.create(wl.N, wl.K, wl.bits, k_cap, dev, gated=True)
             for _ in range(copies)]
    for p in packs:
        mixq.pack_weight(W, st, p, mixq.PACK_FULL)
    ld = mixq.outlier_ld(k_cap)
    Xq = torch.empty(wl.M, wl.K, dtype=torch.int8, device=dev)
    sx = torch.empty(wl.M, dtype=torch.float32, device=dev)
    Xo = torch.zeros(wl.M * ld, dtype=torch.float16, device=dev)
    mixq.quantize_act(X, wl.tau, st, Xq, sx, Xo)
    for p in packs:
        mixq.pack_weight(W, st, p, mixq.PACK_OUTLIER_COLS)
    I = wl.N // 2
    Yh = torch.empty(wl.M, I, dtype=torch.float16, device=dev)
    Y32 = torch.empty(wl.M, wl.N, dtype=torch.float32, device=dev)
    ws = mixq.gemm_workspace(wl.M, wl.N, wl.K, wl.bits, dev)
    stream = torch.cuda.current_stream(dev)

    def fused(i):
        mixq.gemm_ex(Xq, sx, Xo, st, packs[i % copies], Yh, mixq.OUT_SWIGLU_F16, None, ws)

    def plain(i):
        mixq.gemm_ex(Xq, sx, Xo, st, packs[i % copies], Y32, mixq.OUT_F32, None, ws)

    def unfused(i):
        plain(i)
        Yh.copy_(F.silu(Y32[:, :I]) * Y32[:, I:])

    for i in range(warmup):
        fused(i)
        unfused(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn in (("fused", fused), ("plain", plain), ("unfused", unfused)):
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps * 1e3
    tops = wl.ops / (res["fused"] * 1e-6) / 1e12
    log(f"[bench] SwiGLU GEMM {res['fused']:.1f} us ({tops:.0f} TOPS); fp32 GEMM "
        f"{res['plain']:.1f} us; fp32 GEMM + torch silu*up {res['unfused']:.1f} us")
    return {"gemm_swiglu_us": round(res["fused"], 2), "gemm_swiglu_tops": round(tops, 1),
            "gemm_f32_us": round(res["plain"], 2),
            "unfused_us": round(res["unfused"], 2),
            "unfused": "the same GEMM writing fp32, then torch silu(gate) * up cast to fp16",
            "shape": f"M={wl.M}, K={wl.K}, gate and up rows {I} each (N = {wl.N})"}


def run_decode_sequence(wl, repeats: int = 3):
    """The outlier-locality decode sequence: every step runs the whole layer on
    a new batch, the cached set carrying over; the set is re-detected only on
    steps whose uncached amax crosses the threshold.  Inputs for all steps are
    generated up front and resident on the GPU.  Returns per-step time (median
    of `repeats` timed passes, each from an empty set), the steps whose gate
    fired (read after every step of one more, untimed pass) and the GEMM and
    activation side per launch at the steady set."""
    import torch
    from mixed_precision_quantized_amax_amd import mixq, workloads

    dev = torch.device("cuda", 0)
    log(f"[bench] decode sequence: {wl.steps} steps of M={wl.M} K={wl.K} N={wl.N}")
    W = torch.from_numpy(workloads.make_weight(wl)).to(dev)
    plan = workloads.decode_plan(wl)
    Xs = [torch.from_numpy(workloads.decode_step(wl, t, plan)).to(dev) for t in range(wl.steps)]
    k_cap = 256
    ld = mixq.outlier_ld(k_cap)
    Xq = torch.empty(wl.M, wl.K, dtype=torch.int8, device=dev)
    sx = torch.empty(wl.M, dtype=torch.float32, device=dev)
    Xo = torch.zeros(wl.M * ld, dtype=torch.float16, device=dev)
    Y = torch.empty(wl.M, wl.N, dtype=torch.float32, device=dev)
    ws = mixq.gemm_workspace(wl.M, wl.N, wl.K, wl.bits, dev)  # split K
    stream = torch.cuda.current_stream(dev)

    def fresh():
        state = mixq.OutlierState.create(wl.K, k_cap, dev)   # fresh, empty set
        pw = mixq.PackedWeight.create(wl.N, wl.K, wl.bits, k_cap, dev)
        mixq.pack_weight(W, state, pw, mixq.PACK_FULL)
        return state, [mixq.LayerStep(X, wl.tau, state, W, pw, Xq, sx, Xo, Y, ws=ws) for X in Xs]

    state, steps = fresh()
    fired = []
    for t, st in enumerate(steps):
        st()
        if int(state.flag.cpu()[0]) & mixq.FLAG_FIRED:
            fired.append(t)
    times = []
    for rep in range(repeats):
        state, steps = fresh()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for st in steps:
            st()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / wl.steps)
    count = int(state.count.cpu()[0])
    gemm = launch_times(stream, 50, lambda i: steps[-1].gemm())
    act = launch_times(stream, 50, lambda i: steps[-1].act())
    return dict(ms_step=float(np.median(times)), count=count, fired=fired, gemm=gemm, act=act)


def copy_calibration(nbytes: int = 256 << 20):
    """A device-to-device copy of known size, so that the HBM byte counters
    of a profiling run can be scaled (read nbytes, write nbytes)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: {nbytes} bytes, 3 times")


# counter passes, in this order: the GEMM dispatches of the run are
# attributed to these workloads by dispatch order (equal consecutive blocks)
COUNTER_WORKLOADS = ("prefill_w8", "prefill_w4", "llama7b_up", "llama70b_up", "decode_seq")


def kernel_short_name(k: str) -> str:
    """'void ns::(anonymous namespace)::gemm_kernel<256, ...>(Args)' ->
    'gemm_kernel<256, ...>'."""
    k = k.replace("(anonymous namespace)::", "")
    if k.startswith("void "):
        k = k[5:]
    head, sep, tail = k.split("(")[0].partition("<")
    return head.split("::")[-1] + sep + tail


def read_counter_csv(path: str, counter: str, n_calib: int = 3):
    """One counter from a rocprofv3 --pmc CSV (one row per dispatch and
    counter): the mean value per dispatch of each kernel, and the GEMM
    dispatches in dispatch order as (kernel, value).  The first n_calib
    dispatches of the run are the calibration copies, under the key 'copy'."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                rows.append((int(row["Dispatch_Id"]), kernel_short_name(row["Kernel_Name"]),
                             float(row["Counter_Value"])))
    rows.sort()
    vals = {}
    gemms = []
    for i, (_, name, v) in enumerate(rows):
        if i < n_calib:
            if "copyBuffer" not in name:
                raise SystemExit(f"dispatch {i} is {name}, not the calibration copy")
            name = "copy"
        vals.setdefault(name, []).append(v)
        if name.startswith("gemm_kernel"):
            gemms.append((name, v))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}, gemms


def gemm_blocks(gemms: list, names: tuple) -> dict:
    """Split the GEMM dispatches of a counter run (in dispatch order) into one
    equal block per counter workload, in the order the workloads ran; each
    block must be one kernel (no workload here splits into two launches)."""
    n = len(gemms) // len(names)
    if n == 0 or n * len(names) != len(gemms):
        raise SystemExit(f"{len(gemms)} GEMM dispatches for {len(names)} workloads")
    out = {}
    for i, name in enumerate(names):
        blk = gemms[i * n:(i + 1) * n]
        kerns = {k for k, _ in blk}
        if len(kerns) != 1:
            raise SystemExit(f"{name}: expected one GEMM kernel, found {sorted(kerns)}")
        out[name] = (kerns.pop(), sum(v for _, v in blk) / n, n)
    return out


def traffic_summary(fetch_csv: str, write_csv: str, out_json: str, out_txt: str,
                    nbytes: int = 256 << 20):
    """HBM bytes per GEMM launch of each counter workload from a FETCH_SIZE
    pass and a WRITE_SIZE pass of ``bench.py --counters``.  Both counters
    are in KiB per dispatch; each is scaled so that the calibration copy
    (nbytes read, nbytes written) reads nbytes."""
    from mixed_precision_quantized_amax_amd import workloads
    fe, fe_g = read_counter_csv(fetch_csv, "FETCH_SIZE")
    wr, wr_g = read_counter_csv(write_csv, "WRITE_SIZE")
    rs = nbytes / 1024.0 / fe["copy"][0]
    ws_ = nbytes / 1024.0 / wr["copy"][0]
    fb = gemm_blocks(fe_g, COUNTER_WORKLOADS)
    wb = gemm_blocks(wr_g, COUNTER_WORKLOADS)
    lines = [f"calibration copy ({nbytes >> 20} MiB read + {nbytes >> 20} MiB written): "
             f"FETCH_SIZE {fe['copy'][0]:.0f} KiB, WRITE_SIZE {wr['copy'][0]:.0f} KiB",
             f"scale factors: read {rs:.4f}, write {ws_:.4f}"]
    res = {}
    for name in COUNTER_WORKLOADS:
        wl = workloads.WORKLOADS[name]
        kname, f_kib, n = fb[name]
        w_kib = wb[name][1]
        if wb[name][0] != kname or not re.match(rf"gemm_kernel<\d+, \d+, \d+, \d+, {wl.bits},",
                                                kname):
            raise SystemExit(f"{name}: kernels {kname} / {wb[name][0]} do not fit the workload")
        kern = [kname]
        hbm = int(f_kib * 1024 * rs + w_kib * 1024 * ws_)
        alg = algorithmic_bytes(wl, wl.n_outliers)
        res[name] = {"hbm_bytes_per_launch": hbm, "fetch_kib": round(f_kib, 1),
                     "write_kib": round(w_kib, 1), "read_scale": round(rs, 4),
                     "write_scale": round(ws_, 4), "dispatches": n}
        lines.append(f"{name} {kern[0]} ({n} dispatches): FETCH_SIZE {f_kib:.0f} KiB -> "
                     f"{f_kib * rs / 1024:.1f} MiB read; WRITE_SIZE {w_kib:.0f} KiB -> "
                     f"{w_kib * ws_ / 1024:.1f} MiB written; HBM bytes per launch {hbm} "
                     f"({hbm / 2**20:.1f} MiB), algorithmic {alg} ({alg / 2**20:.1f} MiB), "
                     f"ratio {hbm / alg:.2f}")
    for k in sorted(fe):
        if k.startswith(("gate_quant", "requant", "gather_cols")):
            lines.append(f"{k} ({fe[k][1]} dispatches): FETCH {fe[k][0]:.0f} KiB -> "
                         f"{fe[k][0] * rs / 1024:.1f} MiB read; WRITE {wr.get(k, (0, 0))[0]:.0f} "
                         f"KiB -> {wr.get(k, (0, 0))[0] * ws_ / 1024:.1f} MiB written")
    lines.append(f"gemm source sha256[:16]: {gemm_source_sha()}")
    with open(out_json, "w") as f:
        json.dump({"workloads": res, "gemm_source_sha": gemm_source_sha(),
                   "note": "HBM bytes per mixq_gemm launch from rocprofv3 FETCH_SIZE/WRITE_SIZE, "
                           f"scaled by a {nbytes >> 20} MiB copy"}, f, indent=1)
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace_summary(trace_csv: str, out_txt: str):
    """Per-kernel statistics of a ``rocprofv3 --kernel-trace`` CSV of a
    bench.py run (calls, mean, min, max, share of GPU time), and the
    headline GEMM's windows: the default run times the INT8 256 x 256 GEMM
    with 100 launches under per-launch events, then the same 100 back to
    back, first rotating the copies (clean cache), then on one copy (hot);
    each pair shows up as a run of at least 200 consecutive dispatches of
    that kernel, whose last 100 are the back-to-back launches.  Also the
    rate probe's back-to-back launches."""
    import csv
    rows = []
    with open(trace_csv, newline="") as f:
        for r in csv.DictReader(f):
            # blocks: grid work-items over workgroup size (one dimension here)
            blk = (int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
                   if r.get("Grid_Size_X") and r.get("Workgroup_Size_X") else 0)
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                         kernel_short_name(r["Kernel_Name"]), blk))
    rows.sort()
    total = sum(e - b for b, e, _, _ in rows)
    per = {}
    for b, e, k, g in rows:
        per.setdefault((k, g), []).append((e - b) / 1e3)
    lines = ["# kernel | blocks | calls | avg us | min us | max us | % of GPU time"]
    for (k, g), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{k:70s} | {g:6d} | {len(v):5d} | {np.mean(v):9.2f} | {min(v):9.2f} | "
                     f"{max(v):9.2f} | {100.0 * sum(v) * 1e3 / total:6.2f}")
    head = "gemm_kernel<256, 256, 2, 2, 8, 4, 6, false, false, false>"
    runs, cur = [], []
    for b, e, k, _ in rows:
        if k == head:
            cur.append((e - b) / 1e3)
        else:
            if cur:
                runs.append(cur)
            cur = []
    if cur:
        runs.append(cur)
    wins = [r[-100:] for r in runs if len(r) >= 200]
    for name, w in zip(("clean-cache", "hot-cache"), wins):
        lines.append(f"# headline GEMM, {name} window: {len(w)} back-to-back dispatches, avg "
                     f"{np.mean(w):.2f} us, median {np.median(w):.2f}, min {min(w):.2f}, "
                     f"max {max(w):.2f}")
    probe = [(e - b) / 1e3 for b, e, k, _ in rows if k.startswith("mfma_probe_kernel")]
    if len(probe) >= 100:
        w = probe[-100:]
        lines.append(f"# rate probe (mixq_mfma_probe, 256 blocks x 128 rounds): last 100 dispatches, "
                     f"avg {np.mean(w):.2f} us, median {np.median(w):.2f}")
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def run_cpu_baseline(wl, target_s: float = 12.0):
    """The CPU oracle on a row sample of the workload: gate and quantization
    of the sampled tokens, the integer product against all N weight rows, and
    the dequantize/add output.  The weight is quantized beforehand (offline,
    as on the GPU)."""
    from mixed_precision_quantized_amax_amd import workloads
    from oracle import Oracle

    o = Oracle()
    X = workloads.make_activation(wl)
    W = workloads.make_weight(wl)
    Wq, s_w = o.quantize_weight(W, wl.bits)
    in_set, cnt, _ = o.update_outlier_set(X, wl.tau, np.zeros(wl.K, np.uint8), 256)
    W_out = o.gather_weight_cols(W, in_set, 256)

    def run(rows):
        Xs = np.ascontiguousarray(X[:rows])
        t = time.perf_counter()
        s, c, _ = o.update_outlier_set(Xs, wl.tau, in_set, 256)
        Xq, s_x, X_out = o.quantize_act(Xs, s, 256)
        acc = o.int_gemm(Xq, Wq)
        o.output(acc, s_x, s_w, X_out, W_out, c)
        return time.perf_counter() - t

    rows = 2
    dt = run(rows)
    while dt < target_s / 4 and rows < wl.M:
        rows = min(wl.M, max(rows * 2, int(rows * target_s / max(dt, 1e-3) * 0.8)))
        dt = run(rows)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    tops = 2.0 * rows * wl.N * wl.K / dt / 1e12
    return {"value": tops, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {wl.M} tokens x all {wl.N} outputs x K={wl.K} "
                      f"(gate, quantize, int64-accumulated product, fp64 output) in {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the engine clock ramps up over tens of milliseconds of sustained work;
    # 200 steps (about 35 ms) reach the steady state the timed steps measure
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="prefill_w8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (for scaling byte counters)")
    ap.add_argument("--counters", action="store_true",
                    help="byte-counter pass: the calibration copy, then --steps whole steps "
                         "of each counter workload, then the fused RMSNorm passes")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_TRACE_CSV", "OUT_TXT"),
                    help="summarise a rocprofv3 --kernel-trace CSV of a bench.py run")
    ap.add_argument("--traffic-summary", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON", "OUT_TXT"),
                    help="write the GEMM's HBM bytes per launch from two --counters passes")
    ap.add_argument("--all", action="store_true",
                    help="also measure progressive INT4 and output-feature mixed precision")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the LLaMA shapes, the INT4 prefill and the decode sequence")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the layer is not sharded across GPUs; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    from mixed_precision_quantized_amax_amd import workloads
    wl = workloads.WORKLOADS[args.workload]
    if args.copy_calibration or args.counters:
        copy_calibration()
    if args.counters:
        for name in COUNTER_WORKLOADS:
            r = run_gpu(workloads.WORKLOADS[name], args.steps, args.warmup, counters=True)
            log(f"[bench] counters {name}: {args.steps} steps, {r['ms_step']:.4f} ms/step")
        # the fused RMSNorm and residual-add passes at the headline shape
        run_fused_norm(workloads.WORKLOADS[COUNTER_WORKLOADS[0]], args.steps, args.warmup)
        log("[bench] counters: fused RMSNorm passes done")
        return
    if wl.steps > 1:
        d = run_decode_sequence(wl)
        tops = wl.ops / (d["ms_step"] / 1e3) / 1e12
        print(json.dumps({"metric": METRIC, "value": round(tops, 2), "unit": "TOPS", "n_gpus": 1,
                          "steps": wl.steps, "warmup": 0, "ms_per_step": round(d["ms_step"], 5),
                          "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                          "dtype": "i8", "data": "synthetic decode sequence",
                          "config": {"workload": wl.description, "name": wl.name,
                                     "outlier_channels_final": d["count"]}}), flush=True)
        return
    r = run_gpu(wl, args.steps, args.warmup, probe=True)
    ops = wl.ops
    value = ops / (r["ms_step"] / 1e3) / 1e12
    g = r["gemm"]
    gemm_tops = ops / (g["batch_us"] / 1e6) / 1e12
    alg_bytes = algorithmic_bytes(wl, r["count"])
    traffic = gemm_traffic(wl.name)
    clk = r["clock"]
    kp = (r["count"] + 31) // 32 * 32
    # the method's own work on its own units: 2MN(K-k) INT8 ops plus 2MNk
    # FP16 flops (the kernel issues 2MN*kpad of the latter)
    t_roof_us = (2.0 * wl.M * wl.N * (wl.K - r["count"]) / (PEAK_I8_TOPS * 1e12)
                 + 2.0 * wl.M * wl.N * r["count"] / (PEAK_F16_TFLOPS * 1e12)) * 1e6
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 5),
        "graph_ms_per_step": round(r["graph_ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded N(0,1) activations with planted outlier channels, "
                "N(0,std) weights)",
        "config": {"workload": wl.description, "name": wl.name, "M": wl.M, "K": wl.K,
                   "N": wl.N, "weight_bits": wl.bits, "outlier_channels": r["count"],
                   "threshold": wl.tau, "parallelism": "single GPU"},
        "pct_int8_peak": round(100.0 * value / PEAK_I8_TOPS, 2),
        "gemm_tops": round(gemm_tops, 2),
        "gemm_us": g["batch_us"],
        "gemm_us_median": g["median_us"],
        "gemm_launches": g,
        "gemm_hot_cache": dict(r["gemm_hot"], tops=round(ops / (r["gemm_hot"]["batch_us"] / 1e6)
                                                         / 1e12, 2)),
        "act_quant_us": r["act"]["batch_us"],
        "act_quant": dict(r["act"], calls="mixq_quantize_act_regather (gate + re-quantize/regather)",
                          separate_calls_batch_us=r["act_separate"]["batch_us"]),
        "engine_clock": dict(clk, pct_of_measured_clock_peak=round(
            100.0 * gemm_tops / (PEAK_I8_TOPS * clk["ghz_median"] / PEAK_CLOCK_GHZ), 2)),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_I8_TOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / PEAK_I8_TOPS, 4),
                     "traffic": traffic, "algorithmic_bytes": alg_bytes,
                     "traffic_source": "rocprofv3 TCC FETCH_SIZE + WRITE_SIZE per GEMM launch "
                                       "(L2 to fabric: HBM plus Infinity Cache hits), scaled by "
                                       "a copy of known size",
                     "t_roof_us": round(t_roof_us, 2),
                     "frac_mixed": round(t_roof_us / g["batch_us"], 4),
                     "kernel": "mixq_gemm (int8 MFMA main loop + fp16 outlier MFMAs + epilogue)"},
    }
    if r["probe"] is not None:
        # the same MFMA stream with no memory traffic, on the same operand
        # bytes: the ceiling at the clock the board sustains for it
        out["mfma_probe"] = r["probe"]
        if r["probe"]["ops"] == ops:
            out["roofline"]["frac_of_mfma_probe"] = round(gemm_tops / r["probe"]["tops"], 4)
    if r.get("vendor") is not None:
        # the vendor library's plain INT8 GEMM on the same bytes (no outliers,
        # no dequantization, int32 out): context for the fused kernel's time
        out["vendor_int8_gemm"] = r["vendor"]
    out["fused_rmsnorm_act"] = run_fused_norm(wl, args.steps, min(args.warmup, 50))
    out["swiglu_gate_up"] = run_swiglu(wl, max(20, args.steps // 2), min(args.warmup, 50))
    others = {}
    if not args.no_workloads:
        for name in ("llama7b_up", "llama70b_up", "prefill_w4"):
            w2 = workloads.WORKLOADS[name]
            r2 = run_gpu(w2, max(20, args.steps // 2), min(args.warmup, 100))
            others[name] = {"step_tops": round(w2.ops / (r2["ms_step"] / 1e3) / 1e12, 1),
                            "gemm_tops": round(w2.ops / (r2["gemm"]["batch_us"] / 1e6) / 1e12, 1),
                            "gemm_us": r2["gemm"]["batch_us"],
                            "gemm_us_median": r2["gemm"]["median_us"],
                            "gemm_hot_us": r2["gemm_hot"]["batch_us"],
                            "act_quant_us": r2["act"]["batch_us"],
                            "engine_clock_ghz": r2["clock"]["ghz_median"],
                            "ms_per_step": round(r2["ms_step"], 4),
                            "traffic": gemm_traffic(name),
                            "algorithmic_bytes": algorithmic_bytes(w2, r2["count"])}
        dwl = workloads.WORKLOADS["decode_seq"]
        d = run_decode_sequence(dwl)
        others["decode_seq"] = {"step_tops": round(dwl.ops / (d["ms_step"] / 1e3) / 1e12, 1),
                                "ms_per_step": round(d["ms_step"], 4),
                                "gemm_us": d["gemm"]["batch_us"],
                                "gemm_us_median": d["gemm"]["median_us"],
                                "act_quant_us": d["act"]["batch_us"],
                                "fired_steps": d["fired"], "gate_firings": len(d["fired"]),
                                "outlier_channels_final": d["count"],
                                "traffic": gemm_traffic("decode_seq"),
                                "algorithmic_bytes": algorithmic_bytes(dwl, d["count"])}
    if args.all:
        w4 = workloads.WORKLOADS["prefill_w4"]
        r4 = run_gpu(w4, max(10, args.steps // 2), args.warmup, group=128)
        others["prefill_w4_progressive"] = {
            "step_tops": round(w4.ops / (r4["ms_step"] / 1e3) / 1e12, 1),
            "gemm_tops": round(w4.ops / (r4["gemm"]["batch_us"] / 1e6) / 1e12, 1),
            "gemm_us": r4["gemm"]["batch_us"],
            "act_quant_us": r4["act"]["batch_us"],
            "ms_per_step": round(r4["ms_step"], 4),
            "weights": "progressive group-wise INT4, groups of 128 (rebuilt to INT8 in the loader)"}
        sal = workloads.make_salient(w4.N)
        r5 = run_mixed(w4, max(10, args.steps // 2), args.warmup, sal)
        others["prefill_w4_mixed_features"] = {
            "step_tops": round(w4.ops / (r5["ms_step"] / 1e3) / 1e12, 1),
            "gemm_tops": round(w4.ops / (r5["gemm_ms"] / 1e3) / 1e12, 1),
            "gemm_us": round(r5["gemm_ms"] * 1e3, 1),
            "act_quant_us": round(r5["act_ms"] * 1e3, 1),
            "ms_per_step": round(r5["ms_step"], 4),
            "weights": f"{r5['rows'][0]} of {w4.N} output features 8-bit (an INT8 row subset), "
                       f"{r5['rows'][1]} progressive INT4; two products into one Y; "
                       "TOPS count 2*M*N*K"}
    if others:
        out["workloads"] = others
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = run_cpu_baseline(wl, args.cpu_seconds)
        except Exception as e:  # reported, never fatal for the GPU number
            out["cpu_baseline"] = {"value": None, "error": repr(e)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
