#!/usr/bin/env python3
"""Benchmark of the Transformer-XL relative-attention path on one MI355X.

One step = one steady segment of the hot path on the attn_w512_bf16 workload
(batch 16, d_model 512, 8 heads of 64, segment W = 512, memory M = 512 full):
the fused Q/K/V/R projections, the relative-attention kernel, the output
projection and the memory-ring update, all through the C ABI in one call
(txl_rel_attn_fwd_update: the ring copy rides along the output projection's
launch); the same steps as two calls (txl_rel_attn_fwd + txl_mem_update) are
timed beside it. Inputs are seeded synthetic tensors already resident in HBM
when the timed region starts.

Prints ONE JSON line with the whole-job throughput (tokens/s) of a timed region
that holds the steps alone, the attention kernel's roofline position (its own
launches timed with HIP event pairs in a second timed region of the same steps,
whose throughput is reported beside the first) and the CPU oracle timed on a
bounded sample of the same work. The 16-layer stacks (bf16 and fp32) and the
one-layer fp32 layer workload are timed over their segment schedules against
the MFMA peak of their own dtype.
A second timed region runs the same segments with the memory kept as projected
keys and values (txl_rel_attn_fwd_cached), reported under "kv_cache". Then
"sliding_window" compares segment-recurrent evaluation with vanilla evaluation,
which re-encodes a window of the last M + W tokens from scratch for every new
token, on the long-memory attention workload and on the 16-layer stack.
"encodings" times the same step with the encodings the pages compare against
(Shaw et al.'s clipped embeddings, absolute positions), and "backward" the
attention backward (txl_rel_attn_bwd) at the same shape.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
WORKLOAD = "attn_w512_bf16"
STACK_WORKLOADS = ("stack16_bf16", "stack16_fp32", "layer_ffn_fp32")
BF16_PEAK_TFLOPS = 2516.6        # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
FP32_PEAK_TFLOPS = 157.3         # published dense fp32 MFMA peak (256 flop/clk/CU)
HBM_PEAK_GBS = 8000.0


def attn_flops(B, H, dh, W, m):
    """Algorithmic flops of one attention launch: every causally visible
    (query, key) pair costs 2*dh for the content term, 2*dh for the distance
    term and 2*dh for P.V."""
    pairs = W * m + W * (W + 1) // 2
    return 6.0 * dh * H * B * pairs


def proj_flops(B, W, m, D):
    """Flops of the projections of one segment: q (one product serves q+u and
    q+v), k_E and v over the m + W context rows, r over the m + W distances
    (shared by the batch), and the output projection."""
    return 2.0 * B * W * D * D + 4.0 * B * (m + W) * D * D + 2.0 * (m + W) * D * D + 2.0 * B * W * D * D


def attn_bytes(B, W, m, D, es):
    """Compulsory HBM bytes of one attention launch: (q+u), (q+v), keys, values,
    distance keys in, attention output out."""
    K = m + W
    return es * (2 * B * W * D + 2 * B * K * D + K * D + B * W * D)


def kernel_digest(sources) -> str:
    """sha256 over the kernel's source files, concatenated in the given order."""
    h = hashlib.sha256()
    for src in sources:
        with open(src, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# the attention kernel's translation unit: its file and the headers it includes
ATTN_SOURCES = [os.path.join(ROOT, "transformer_xl_segment_amd", "csrc", n)
                for n in ("txl_attn.hip", "txl_attn_tile.hpp", "txl_device.hpp", "txl_internal.hpp")]


def traffic_for(sources, path: str):
    """Measured HBM bytes per launch from a committed counter summary, or None
    if the kernel's sources have changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha256") != kernel_digest(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def time_fwd_only(tb, torch, segs, ring, params, R, H, out, ws, steps):
    """txl_rel_attn_fwd alone (projections, attention kernel, output projection)
    on the full memory, without the memory update."""
    B, W = out.shape[0], out.shape[1]
    el = _timed(torch, lambda k: tb.rel_attn_fwd(segs[k % len(segs)], ring, params, R, H, out=out, workspace=ws),
                steps)
    return {"ms_per_call": el * 1e3 / steps, "tokens_per_s": B * W * steps / el,
            "call": "txl_rel_attn_fwd at m = M (fused projections + attention kernel + W_o)"}


def time_schedule(tb, torch, segs, params, R, B, M, D, H, out, ws, reps):
    """The workload's whole schedule: its S segments from an empty memory, each
    txl_rel_attn_fwd_update (attention and memory update), so the early
    segments see m < M."""
    ring = tb.MemoryRing.empty(B, M, D, out.dtype, out.device)
    W = out.shape[1]

    def sched(k):
        ring.len, ring.head = 0, 0           # an empty memory: the stale rows are never read
        for h in segs:
            tb.rel_attn_fwd_update(h, ring, params, R, H, out=out, workspace=ws)

    el = _timed(torch, sched, reps, 1)
    S = len(segs)
    return {"segments": S, "ms_per_schedule": el * 1e3 / reps, "tokens_per_s": B * W * S * reps / el,
            "memory_lengths": [min(M, k * W) for k in range(S)]}


def longmem_warm(tb, torch, syn, dev, steps):
    """The long-memory workload with its memory already full (m = 1600 for every
    segment): attention-kernel MFMA fraction and its HBM rate."""
    bf = torch.bfloat16
    wl = syn.WORKLOADS["longmem_m1600_bf16"]
    B, D, H, W, M = wl.B, wl.D, wl.H, wl.W, wl.M
    dh = D // H
    prob = syn.draw_problem(wl)
    params = tb.LayerParams.from_numpy(prob.params[0], bf, dev)
    R = tb.sinusoid_table(M + W, D, bf, dev)
    x = torch.from_numpy(prob.x).to(dev).to(bf)
    segs = [x[:, k * W:(k + 1) * W] for k in range(wl.S)]
    warm = torch.from_numpy(prob.warm_mem).to(dev).to(bf)
    ring = tb.MemoryRing.empty(B, M, D, bf, dev)
    tb.mem_update(ring, warm)
    out = torch.empty(B, W, D, dtype=bf, device=dev)
    ws = torch.empty(tb.workspace_bytes(tb.OP_REL_ATTN, bf, B, W, M, D, H), dtype=torch.uint8, device=dev)

    def step(k):
        tb.rel_attn_fwd(segs[k % wl.S], ring, params, R, H, out=out, workspace=ws)
        tb.mem_update(ring, segs[k % wl.S])

    for k in range(3):
        step(k)
    torch.cuda.synchronize()
    tb.profile_begin(steps)
    el = _timed(torch, step, steps, 0)
    attn_ms, n = tb.profile_end()
    lm = sorted(tb.profile_times(n))
    m = ring.len
    fl, by = attn_flops(B, H, dh, W, m), attn_bytes(B, W, m, D, 2)
    avg = attn_ms * 1e-3 / n
    return {"workload": wl.name, "B": B, "W": W, "m": m, "D": D, "H": H,
            "tokens_per_s": B * W * steps / el, "ms_per_step": el * 1e3 / steps,
            "attn_avg_launch_us": avg * 1e6, "attn_median_launch_us": float(np.median(lm)) * 1e3,
            "attn_min_launch_us": lm[0] * 1e3,
            "attn_tflops": fl / avg / 1e12, "attn_frac_bf16_peak": fl / avg / 1e12 / BF16_PEAK_TFLOPS,
            "attn_compulsory_gbs": by / avg / 1e9, "attn_frac_hbm_peak": by / avg / 1e9 / HBM_PEAK_GBS}


def longmem_schedule(tb, torch, syn, dev, reps):
    """The long-memory workload as scheduled: its S segments from an empty
    memory, so the memory grows W rows per segment (m = 0, W, .., (S-1) W)."""
    bf = torch.bfloat16
    wl = syn.WORKLOADS["longmem_m1600_bf16"]
    B, D, H, W, M = wl.B, wl.D, wl.H, wl.W, wl.M
    prob = syn.draw_problem(wl)
    params = tb.LayerParams.from_numpy(prob.params[0], bf, dev)
    R = tb.sinusoid_table(M + W, D, bf, dev)
    x = torch.from_numpy(prob.x).to(dev).to(bf)
    segs = [x[:, k * W:(k + 1) * W] for k in range(wl.S)]
    out = torch.empty(B, W, D, dtype=bf, device=dev)
    ws = torch.empty(tb.workspace_bytes(tb.OP_REL_ATTN, bf, B, W, M, D, H), dtype=torch.uint8, device=dev)
    r = time_schedule(tb, torch, segs, params, R, B, M, D, H, out, ws, reps)
    dh = D // H
    fl = sum(attn_flops(B, H, dh, W, m) + proj_flops(B, W, m, D) for m in r["memory_lengths"])
    r.update({"workload": wl.name, "B": B, "W": W, "M": M, "D": D, "H": H,
              "step": "txl_rel_attn_fwd_update per segment",
              "tflops_algorithmic": fl / (r["ms_per_schedule"] * 1e-3) / 1e12})
    return r


def time_mem_update(tb, torch, segs, B, M, D, dev, calls):
    """txl_mem_update alone on the headline shape (W = M rows of D moved per
    batch row: read from the segment, written into the ring), HIP events on the
    stream around the calls."""
    ring = tb.MemoryRing.empty(B, M, D, torch.bfloat16, dev)
    for k in range(3):
        tb.mem_update(ring, segs[k % len(segs)])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for k in range(calls):
        tb.mem_update(ring, segs[k % len(segs)])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    W = segs[0].shape[1]
    nbytes = 2.0 * 2 * B * min(W, M) * D
    return {"us_per_call": us, "bytes_per_call": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9,
            "frac_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def stack_flops(wl, m):
    """Algorithmic flops of one layer on one segment with m memory rows: attention,
    projections (q, k_E and v over m + W rows, r, W_o) and the FFN."""
    B, W, D, H, F = wl.B, wl.W, wl.D, wl.H, wl.F
    return attn_flops(B, H, D // H, W, m) + proj_flops(B, W, m, D) + 4.0 * B * W * D * F


def time_stack16(tb, torch, syn, dev, reps, name="stack16_bf16"):
    """A stack workload's whole segment schedule from empty memories
    (txl_stack_fwd_segments) with its algorithmic TFLOP/s against the MFMA peak
    of its own dtype (the 16-layer stacks in bf16 and fp32; the one-layer
    layer_ffn_fp32 workload runs through the same call with L = 1)."""
    wl = syn.WORKLOADS[name]
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    peak = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    B, D, H, W, M, F = wl.B, wl.D, wl.H, wl.W, wl.M, wl.F
    prob = syn.draw_problem(wl)
    x = torch.from_numpy(prob.x).to(dev).to(tdt)
    lp = [tb.LayerParams.from_numpy(p, tdt, dev) for p in prob.params]
    R = tb.sinusoid_table(M + W, D, tdt, dev)
    y = torch.empty_like(x)
    ws = torch.empty(tb.workspace_bytes(tb.OP_STACK, tdt, B, W, M, D, H, F), dtype=torch.uint8, device=dev)

    mems = [tb.MemoryRing.empty(B, M, D, tdt, dev) for _ in lp]

    def run(k):
        for r in mems:
            r.len, r.head = 0, 0            # empty memories: the stale rows are never read
        tb.stack_fwd_segments(x, mems, lp, R, H, W, F, y=y, workspace=ws)

    el = _timed(torch, run, reps, 1)
    flops = sum(stack_flops(wl, m) for m in wl.mem_schedule()) * len(lp)
    T = x.shape[1]
    tf = flops * reps / el / 1e12
    return {"workload": wl.name, "dtype": wl.dtype, "layers": len(lp), "segments": wl.S,
            "ms_per_schedule": el * 1e3 / reps, "tokens_per_s": B * T * reps / el,
            "algorithmic_tflops": tf, "peak_tflops": peak, "frac_of_peak": tf / peak,
            "memory_lengths": wl.mem_schedule()}


def time_cached(tb, torch, segs, params, R, B, M, W, D, H, out, steps, warmup):
    """The same segment stream through txl_rel_attn_fwd_cached: the memory is
    held as projected keys and values, so each segment projects W rows, not M + W."""
    bf = torch.bfloat16
    cache = tb.KVCache.empty(B, M, W, D, H, bf, out.device)
    ws = torch.empty(tb.workspace_bytes(tb.OP_REL_ATTN_CACHED, bf, B, W, M, D, H), dtype=torch.uint8,
                     device=out.device)

    def step(k):
        tb.rel_attn_fwd_cached(segs[k % len(segs)], cache, params, R, H, out=out, workspace=ws)

    for k in range(max(warmup, 1) + (M + W - 1) // W):
        step(k)
    torch.cuda.synchronize()
    assert cache.len == M
    t0 = time.perf_counter()
    for k in range(steps):
        step(k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    return {"value": B * W * steps / elapsed, "unit": "tokens/s", "ms_per_step": elapsed * 1e3 / steps,
            "step": "txl_rel_attn_fwd_cached, one steady segment (m = M)",
            "cache_bytes": 2 * B * M * D * 2}


def time_encodings(tb, torch, segs, params, B, M, W, D, H, out, steps, warmup):
    """The same steady segment step with Shaw et al.'s encoding (clip 64, tables
    N(0, 0.02)) and with absolute positions (added to each segment's rows)."""
    bf = torch.bfloat16
    dev = out.device
    dh = D // H
    g = torch.Generator().manual_seed(99)
    aK = (torch.randn(65, dh, generator=g) * 0.02).to(dev).to(bf)
    aV = (torch.randn(65, dh, generator=g) * 0.02).to(dev).to(bf)
    ws = torch.empty(tb.workspace_bytes(tb.OP_ATTN_VARIANT, bf, B, W, M, D, H), dtype=torch.uint8, device=dev)
    hp = torch.empty(B, W, D, dtype=bf, device=dev)
    res = {}
    for name, variant in (("shaw_clip64", tb.POS_SHAW), ("absolute", tb.POS_ABSOLUTE)):
        ring = tb.MemoryRing.empty(B, M, D, bf, dev)

        def step(k):
            h = segs[k % len(segs)]
            if variant == tb.POS_ABSOLUTE:
                h = tb.add_positions(h, 0, y=hp)
            tb.attn_fwd_variant(h, ring, params, variant, H, aK=aK, aV=aV, clip=64, out=out, workspace=ws)
            tb.mem_update(ring, h)

        el = _timed(torch, step, steps, warmup + (M + W - 1) // W)
        res[name] = {"value": B * W * steps / el, "unit": "tokens/s", "ms_per_step": el * 1e3 / steps}
    return res


def bwd_flops(B, H, dh, W, m):
    """Algorithmic flops of the attention backward: per causally visible pair,
    the two score terms recomputed (4 dh), dP (2 dh), dq from both terms (4 dh),
    dk, dval and dr (2 dh each)."""
    pairs = W * m + W * (W + 1) // 2
    return 16.0 * dh * H * B * pairs


def time_backward(tb, torch, B, W, M, D, H, dev, steps):
    bf = torch.bfloat16
    g = torch.Generator().manual_seed(7)
    K = M + W
    mk = lambda *shape, s=0.5: (torch.randn(*shape, generator=g) * s).to(dev).to(bf)
    q, k, val, r, u, v, dO = mk(B, W, D), mk(B, K, D), mk(B, K, D, s=1.0), mk(K, D), mk(D), mk(D), mk(B, W, D, s=1.0)
    ws = torch.empty(tb.workspace_bytes(tb.OP_REL_ATTN_BWD, bf, B, W, M, D, H), dtype=torch.uint8, device=dev)
    el = _timed(torch, lambda i: tb.rel_attn_bwd(q, k, val, r, u, v, dO, H, workspace=ws), steps)
    ms = el * 1e3 / steps
    fl = bwd_flops(B, H, D // H, W, M)
    return {"ms_per_call": ms, "tokens_per_s": B * W / (ms * 1e-3), "algorithmic_tflops": fl / (ms * 1e-3) / 1e12,
            "frac_of_bf16_peak": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, "workspace_bytes": ws.numel(),
            "call": "txl_rel_attn_bwd, B=16, W=m=512, D=512, H=8 (all gradients of the projected operands)"}


def _timed(torch, fn, calls, warm=2):
    for k in range(warm):
        fn(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(calls):
        fn(warm + k)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def sliding_window(tb, torch, syn, dev):
    """Tokens/s of segment-recurrent evaluation (memory carried, W new tokens
    per call) against vanilla evaluation (no memory; every new token re-encodes
    the window of its last M + W tokens, one token per batch row per call)."""
    bf = torch.bfloat16
    res = {}

    # one attention layer, long memory: window of M + W = 1728 keys
    wl = syn.WORKLOADS["longmem_m1600_bf16"]
    B, D, H, W, M = wl.B, wl.D, wl.H, wl.W, wl.M
    prob = syn.draw_problem(wl)
    stream = torch.from_numpy(np.concatenate([prob.warm_mem, prob.x], axis=1)).to(dev).to(bf)
    T, Lw = stream.shape[1], M + W
    params = tb.LayerParams.from_numpy(prob.params[0], bf, dev)
    R = tb.sinusoid_table(Lw, D, bf, dev)
    out = torch.empty(B, W, D, dtype=bf, device=dev)
    segs = [stream[:, M + k * W:M + (k + 1) * W] for k in range(wl.S)]
    ring = tb.MemoryRing.empty(B, M, D, bf, dev)
    tb.mem_update(ring, stream[:, :M])
    ws = torch.empty(tb.workspace_bytes(tb.OP_REL_ATTN, bf, B, W, M, D, H), dtype=torch.uint8, device=dev)

    def rec(k):
        tb.rel_attn_fwd(segs[k % wl.S], ring, params, R, H, out=out, workspace=ws)
        tb.mem_update(ring, segs[k % wl.S])

    n_rec = 60
    t_rec = _timed(torch, rec, n_rec)
    cache = tb.KVCache.empty(B, M, W, D, H, bf, dev)
    tb.kv_cache_append(cache, params, stream[:, :M], H)
    wsc = torch.empty(tb.workspace_bytes(tb.OP_REL_ATTN_CACHED, bf, B, W, M, D, H), dtype=torch.uint8,
                      device=dev)
    t_kv = _timed(torch, lambda k: tb.rel_attn_fwd_cached(segs[k % wl.S], cache, params, R, H, out=out,
                                                         workspace=wsc), n_rec)
    wout = torch.empty(B, Lw, D, dtype=bf, device=dev)
    wsv = torch.empty(tb.workspace_bytes(tb.OP_REL_ATTN, bf, B, Lw, 0, D, H), dtype=torch.uint8, device=dev)

    def van(k):
        t = Lw - 1 + (k % (T - Lw + 1))      # newest token of the window
        tb.rel_attn_fwd(stream[:, t - Lw + 1:t + 1], None, params, R, H, out=wout, workspace=wsv)

    n_van = 60
    t_van = _timed(torch, van, n_van)
    v_rec, v_kv, v_van = B * W * n_rec / t_rec, B * W * n_rec / t_kv, B * n_van / t_van
    res["attn_longmem"] = {"workload": wl.name, "window": Lw, "B": B,
                           "recurrent_tokens_per_s": v_rec, "recurrent_kv_cache_tokens_per_s": v_kv,
                           "vanilla_tokens_per_s": v_van, "vanilla_ms_per_window": t_van * 1e3 / n_van,
                           "speedup": v_rec / v_van, "speedup_kv_cache": v_kv / v_van}
    del stream, ring, cache, ws, wsc, wsv, wout

    # the 16-layer stack: window of M + W = 300 tokens, every layer re-encoded
    wl = syn.WORKLOADS["stack16_bf16"]
    B, D, H, W, M, F = wl.B, wl.D, wl.H, wl.W, wl.M, wl.F
    prob = syn.draw_problem(wl)
    x = torch.from_numpy(prob.x).to(dev).to(bf)                    # [B, 8*W, D]
    T, Lw = x.shape[1], M + W
    lp = [tb.LayerParams.from_numpy(p, bf, dev) for p in prob.params]
    R = tb.sinusoid_table(Lw, D, bf, dev)
    mems = [tb.MemoryRing.empty(B, M, D, bf, dev) for _ in lp]
    y = torch.empty_like(x)
    ws = torch.empty(tb.workspace_bytes(tb.OP_STACK, bf, B, W, M, D, H, F), dtype=torch.uint8, device=dev)
    n_rec = 3
    t_rec = _timed(torch, lambda k: tb.stack_fwd_segments(x, mems, lp, R, H, W, F, y=y, workspace=ws), n_rec, 1)
    yw = torch.empty(B, Lw, D, dtype=bf, device=dev)
    wsv = torch.empty(tb.workspace_bytes(tb.OP_STACK, bf, B, Lw, 0, D, H, F), dtype=torch.uint8, device=dev)

    def van(k):
        t = Lw - 1 + (k % (T - Lw + 1))
        tb.stack_fwd_window(x[:, t - Lw + 1:t + 1], lp, R, H, F, y=yw, workspace=wsv)

    n_van = 20
    t_van = _timed(torch, van, n_van)
    v_rec, v_van = B * T * n_rec / t_rec, B * n_van / t_van
    res["stack16"] = {"workload": wl.name, "window": Lw, "B": B, "layers": len(lp),
                      "recurrent_tokens_per_s": v_rec, "vanilla_tokens_per_s": v_van,
                      "vanilla_ms_per_window": t_van * 1e3 / n_van, "speedup": v_rec / v_van}
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(prob, R64, H):
    """The oracle on the steady segments of the workload (m = 512, all batch
    rows): segments 1 .. S-1 with the previous segment as the memory, repeated
    until about 10 s of host time have been spent. Then the oracle on one thread
    for the two small workloads (their whole schedules) and for one batch row of
    one steady segment of this workload."""
    from oracle import oracle as orc
    from transformer_xl_segment_amd import synthetic as syn
    wl = prob.wl
    W, D = wl.W, wl.D
    threads = orc.num_threads()
    t0 = time.perf_counter()
    segs = 0
    while True:
        t = 1 + segs % (wl.S - 1)
        h = prob.x[:, t * W:(t + 1) * W].astype(np.float64)
        mem = prob.x[:, (t - 1) * W:t * W].astype(np.float64)
        orc.rel_attn(h, mem, prob.params[0], R64, H)
        segs += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or segs >= 4 * (wl.S - 1):
            break
    Bx = prob.x.shape[0]
    tokens = segs * Bx * W
    seg_flops = attn_flops(Bx, H, D // H, W, W) + proj_flops(Bx, W, W, D)

    single = {}
    orc.set_num_threads(1)
    try:
        for name in ("tiny_attn_fp32", "layer_ffn_fp32"):
            w = syn.WORKLOADS[name]
            p = syn.draw_problem(w)
            Rw = orc.sinusoid_table(w.M + w.W, w.D)
            t1 = time.perf_counter()
            orc.stack_fwd(p.x, p.params, Rw, w.H, w.W, w.M, w.op == "layer")
            d1 = time.perf_counter() - t1
            single[name] = {"tokens_per_s": p.x.shape[0] * p.x.shape[1] / d1, "sample": "whole schedule",
                            "seconds": d1}
        t = 1
        h = prob.x[:1, t * W:(t + 1) * W].astype(np.float64)
        mem = prob.x[:1, (t - 1) * W:t * W].astype(np.float64)
        t1 = time.perf_counter()
        orc.rel_attn(h, mem, prob.params[0], R64, H)
        d1 = time.perf_counter() - t1
        single[WORKLOAD] = {"tokens_per_s": W / d1, "sample": "batch row 0 of one steady segment",
                            "seconds": d1,
                            "gflops": (attn_flops(1, H, D // H, W, W) + proj_flops(1, W, W, D)) / d1 / 1e9}
    finally:
        orc.set_num_threads(threads)
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{segs} steady segments of {WORKLOAD} (all {Bx} batch rows each, m={W}), "
                      f"{dt:.1f} s wall",
            "gflops": seg_flops * segs / dt / 1e9, "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)), "omp_threads": threads, "cpu_model": cpu_model(),
            "single_thread": single}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sliding-window", action="store_true",
                    help="skip the comparison with vanilla sliding-window evaluation")
    ap.add_argument("--stack16-only", action="store_true",
                    help="time only the 16-layer bf16 stack's schedule (for counter runs of its kernels)")
    ap.add_argument("--stack-only", choices=STACK_WORKLOADS, default=None,
                    help="time only this stack workload's schedule (for traces and counter runs)")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the attention backward at the headline shape (for kernel traces)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline step (for counter runs); implies the two --no-* flags")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (3 times) before the "
                         "warm-up, as the reference point for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); every run here uses a "
              f"single MI355X", file=sys.stderr)
        sys.exit(2)

    import torch
    from transformer_xl_segment_amd import binding as tb
    from transformer_xl_segment_amd import synthetic as syn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.stack16_only or args.stack_only:
        name = args.stack_only or "stack16_bf16"
        print(json.dumps({name: time_stack16(tb, torch, syn, dev, 2, name)}), flush=True)
        return
    wl = syn.WORKLOADS[WORKLOAD]
    B, D, H, W, M = wl.B, wl.D, wl.H, wl.W, wl.M
    dh = D // H
    if args.backward_only:
        print(json.dumps({"backward": time_backward(tb, torch, B, W, M, D, H, dev, 10)}), flush=True)
        return
    prob = syn.draw_problem(wl)
    bf = torch.bfloat16
    x = torch.from_numpy(prob.x).to(dev).to(bf)                 # [B, S*W, D]
    params = tb.LayerParams.from_numpy(prob.params[0], bf, dev)
    R = tb.sinusoid_table(M + W, D, bf, dev)                    # built by the library
    ring = tb.MemoryRing.empty(B, M, D, bf, dev)
    out = torch.empty(B, W, D, dtype=bf, device=dev)
    ws = torch.empty(tb.workspace_bytes(tb.OP_REL_ATTN, bf, B, W, M, D, H), dtype=torch.uint8, device=dev)
    segs = [x[:, t * W:(t + 1) * W] for t in range(wl.S)]


    def step(k):
        tb.rel_attn_fwd_update(segs[k % len(segs)], ring, params, R, H, out=out, workspace=ws)

    def step_separate(k):
        h = segs[k % len(segs)]
        tb.rel_attn_fwd(h, ring, params, R, H, out=out, workspace=ws)
        tb.mem_update(ring, h)

    # fill the memory, then warm up at the steady state m = M
    for k in range(max(args.warmup, 1) + (M + W - 1) // W):
        step(k)
    torch.cuda.synchronize()
    assert ring.len == M
    m = ring.len

    # the steps with a HIP event pair around every attention launch (stamped by
    # the kernel's own dispatch, on the stream it runs on), for the kernel's
    # launch durations
    tb.profile_begin(args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    elapsed_stamped = time.perf_counter() - t1
    attn_ms, launches = tb.profile_end()
    assert launches == args.steps
    launch_ms = sorted(tb.profile_times(launches))

    # the timed region proper: the same steps again with nothing recorded
    # between them; its throughput is the reported value
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert ring.len == m

    # the same steps as two calls, txl_rel_attn_fwd then txl_mem_update (the
    # memory update in a launch of its own)
    el_sep = _timed(torch, step_separate, args.steps, 1)

    ms_per_step = elapsed * 1e3 / args.steps
    tokens = B * W * args.steps
    a_flops = attn_flops(B, H, dh, W, m)
    a_avg_s = attn_ms * 1e-3 / launches
    a_tflops = a_flops / a_avg_s / 1e12
    traffic = traffic_for(ATTN_SOURCES,
                          os.path.join(ROOT, "profiles", "traffic_rel_attn_kernel_attn_w512_bf16.json"))
    rec = {
        "metric": "rel-attn tokens/s and TFLOP/s (% bf16 MFMA peak) at W=M=512, d_head=64, 1 GPU",
        "value": tokens / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": B, "W": W, "M": M, "m": m, "D": D, "H": H, "d_head": dh,
                   "step": "txl_rel_attn_fwd_update (attention + memory update), one steady segment"},
        "roofline": {"kernel": "rel_attn_kernel", "bound": "mfma", "achieved": a_tflops,
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": a_tflops / BF16_PEAK_TFLOPS,
                     "traffic": traffic, "avg_launch_us": a_avg_s * 1e6,
                     "median_launch_us": float(np.median(launch_ms)) * 1e3, "min_launch_us": launch_ms[0] * 1e3,
                     "frac_at_min_launch": a_flops / (launch_ms[0] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                     "algorithmic_flops_per_launch": a_flops,
                     "compulsory_bytes_per_launch": attn_bytes(B, W, m, D, 2),
                     # the peak again from this run's compute-unit count at the published
                     # 2.4 GHz (4096 dense bf16 flop per clock per CU); equal to "peak" on MI355X
                     "device": props.name, "arch": props.gcnArchName, "compute_units": props.multi_processor_count,
                     "peak_from_compute_units": props.multi_processor_count * 2.4e9 * 4096 / 1e12},
        "attn_tokens_per_s": B * W / a_avg_s,
        "event_stamped_region": {"ms_per_step": elapsed_stamped * 1e3 / args.steps,
                                 "tokens_per_s": tokens / elapsed_stamped},
        "separate_update_calls": {"ms_per_step": el_sep * 1e3 / args.steps, "tokens_per_s": tokens / el_sep,
                                  "step": "txl_rel_attn_fwd + txl_mem_update"},
        "step_tflops": (a_flops + proj_flops(B, W, m, D)) / (ms_per_step * 1e-3) / 1e12,
    }
    if args.headline_only:
        print(json.dumps(rec), flush=True)
        return
    rec["rel_attn_fwd_only"] = time_fwd_only(tb, torch, segs, ring, params, R, H, out, ws, args.steps)
    rec["schedule"] = time_schedule(tb, torch, segs, params, R, B, M, D, H, out, ws, max(3, args.steps // 8))
    rec["longmem_warm"] = longmem_warm(tb, torch, syn, dev, max(10, args.steps // 4))
    rec["longmem_schedule"] = longmem_schedule(tb, torch, syn, dev, max(3, args.steps // 8))
    rec["mem_update"] = time_mem_update(tb, torch, segs, B, M, D, dev, max(20, args.steps // 2))
    rec["stack16"] = time_stack16(tb, torch, syn, dev, 2)
    rec["stack16_fp32"] = time_stack16(tb, torch, syn, dev, 2, "stack16_fp32")
    rec["layer_ffn_fp32"] = time_stack16(tb, torch, syn, dev, 20, "layer_ffn_fp32")
    kv = time_cached(tb, torch, segs, params, R, B, M, W, D, H, out, args.steps, args.warmup)
    kv["speedup_vs_row_memory"] = kv["value"] / rec["value"]
    rec["kv_cache"] = kv
    rec["encodings"] = time_encodings(tb, torch, segs, params, B, M, W, D, H, out, args.steps, args.warmup)
    rec["backward"] = time_backward(tb, torch, B, W, M, D, H, dev, max(5, args.steps // 10))
    if not args.no_sliding_window:
        del ring, ws
        rec["sliding_window"] = sliding_window(tb, torch, syn, dev)
    if not args.no_cpu_baseline:
        from oracle import oracle as orc
        R64 = orc.sinusoid_table(M + W, D)
        rb = syn.round_to_bf16(R64.astype(np.float32)).astype(np.float64)
        rec["cpu_baseline"] = cpu_baseline(prob, rb, H)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
