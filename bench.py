#!/usr/bin/env python3
"""Throughput of causal kernelized linear attention on one MI355X.

Method: "Transformers are RNNs: Fast Autoregressive Transformers with Linear
Attention" (Katharopoulos et al., 2020) -- parallel (chunked prefill) mode and
recurrent (decode) mode, both through the C ABI of liblinattn.so.

Headline (`value`): prefill tokens/s on fp32 inputs, B=8 H=8 N=1024 D=M=64
(one token = one position across all heads), inputs resident in HBM, rotated
over enough buffer sets that the 256 MB last-level cache cannot hold them.
A step is one la_forward_chunked call over one batch.

Also reported in the same JSON line: the dominant kernel's roofline (HIP
events around each launch of it), the fp64 CPU oracle timed on a bounded
sample of the same workload, the recurrent decode workload (256 streams x 8
heads, D=M=64, 4096 steps from a zero state), the two bf16 prefill
workloads, the backward pass on the headline shape, the multi-token
decode (16 tokens per call) and the softmax-attention RNN scan.  Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
FP32_MFMA_PEAK_TFS = 157.3  # dense fp32 matrix
BF16_MFMA_PEAK_TFS = 2516.6  # dense bf16 matrix
LLC_BYTES = 256 << 20       # Infinity Cache

METRIC = "causal linear-attention tokens/sec (prefill, decode) and % of MFMA/HBM roofline"


def csrc_sha256_16() -> str:
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "efficient_transformer_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(summary: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None when the
    kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", summary)
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes_per_launch: ", "csrc_sha256_16: ")))
    if fields.get("csrc_sha256_16", "").strip() != csrc_sha256_16():
        return None
    return int(fields["traffic_bytes_per_launch"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_bytes(cfg) -> int:
    """Algorithmic bytes of one prefill call: read Q, K, V once, write out once (fp32, or
    bf16 when cfg["out"] == "bf16")."""
    s = 4 if cfg["dtype"] == "f32" else 2
    so = 2 if cfg.get("out") == "bf16" else 4
    BH, N, D, M = cfg["B"] * cfg["H"], cfg["N"], cfg["D"], cfg["M"]
    return BH * N * ((2 * D + M) * s + so * M)


def prefill_flops_min(cfg) -> int:
    """Algorithmic flops: per head-token, state update 2DM + readout 2DM + normaliser 4D + divide M."""
    BH, N, D, M = cfg["B"] * cfg["H"], cfg["N"], cfg["D"], cfg["M"]
    return BH * N * (4 * D * M + 4 * D + M)


def decode_bytes_per_step(cfg) -> int:
    """Per step: S and z read and written, q k v read, out written (all fp32)."""
    BH, D, M = cfg["B"] * cfg["H"], cfg["D"], cfg["M"]
    return BH * (2 * 4 * D * M + 2 * 4 * D + 4 * (2 * D + M) + 4 * M)


def make_prefill_sets(cfg, nsets, dev):
    import torch
    import synthetic
    sets = []
    for r in range(nsets):
        Q = synthetic.draw_torch(r, synthetic.TID_Q, (cfg["B"], cfg["H"], cfg["N"], cfg["D"]), cfg["sigma"],
                                 cfg["dtype"], dev)
        K = synthetic.draw_torch(r, synthetic.TID_K, (cfg["B"], cfg["H"], cfg["N"], cfg["D"]), cfg["sigma"],
                                 cfg["dtype"], dev)
        V = synthetic.draw_torch(r, synthetic.TID_V, (cfg["B"], cfg["H"], cfg["N"], cfg["M"]), cfg["sigma"],
                                 cfg["dtype"], dev)
        odt = torch.bfloat16 if cfg.get("out") == "bf16" else torch.float32
        out = torch.empty((cfg["B"], cfg["H"], cfg["N"], cfg["M"]), dtype=odt, device=dev)
        sets.append((Q, K, V, out))
    torch.cuda.synchronize()
    return sets


def bench_prefill(cfg, steps, warmup, dev):
    """Timings of one causal prefill workload (la_forward_chunked: one fused kernel per call)."""
    import torch
    import efficient_transformer_amd as ea
    from efficient_transformer_amd import linattn as L

    code = L.LA_F32 if cfg["dtype"] == "f32" else L.LA_BF16
    B, H, N, D, M = cfg["B"], cfg["H"], cfg["N"], cfg["D"], cfg["M"]
    C, G, wsb = ea.forward_plan(B, H, N, D, M, True, code, cfg.get("chunk", 0))
    nbytes = prefill_bytes(cfg)
    nsets = max(1, math.ceil(1.25 * LLC_BYTES / nbytes))
    sets = make_prefill_sets(cfg, nsets, dev)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)  # zeroed once; each call leaves it ready
    stream = torch.cuda.current_stream(dev)

    def step(i):
        Q, K, V, out = sets[i % nsets]
        ea.forward_chunked(Q, K, V, causal=True, chunk=C, out=out, workspace=ws, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # kernel duration: HIP events around every launch (the library enqueues one
    # kernel per causal call on `stream`)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    us_kernel = sum(per) / steps
    # the same launches on one buffer set (inputs warm in the last-level cache)
    for i in range(5):
        step(0)
    torch.cuda.synchronize()
    evw = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        evw[i][0].record(stream)
        step(0)
        evw[i][1].record(stream)
    torch.cuda.synchronize()
    warm = sorted(a.elapsed_time(b) * 1e3 for a, b in evw)
    del sets
    torch.cuda.empty_cache()
    return dict(chunk=C, segments=G, nsets=nsets, ms_per_step=ms, tokens_per_s=B * N / (ms * 1e-3),
                bytes=nbytes, flops_min=prefill_flops_min(cfg), us_kernel=us_kernel,
                us_kernel_median=per[steps // 2], us_kernel_min=per[0], us_warm_median=warm[steps // 2])


def bench_decode(cfg, reps, dev, warm_steps=64):
    import torch
    import efficient_transformer_amd as ea
    import synthetic

    B, H, D, M, T = cfg["B"], cfg["H"], cfg["D"], cfg["M"], cfg["T"]
    q = synthetic.draw_torch(0, synthetic.TID_DQ, (T, B, H, D), cfg["sigma"], cfg["dtype"], dev)
    k = synthetic.draw_torch(0, synthetic.TID_DK, (T, B, H, D), cfg["sigma"], cfg["dtype"], dev)
    v = synthetic.draw_torch(0, synthetic.TID_DV, (T, B, H, M), cfg["sigma"], cfg["dtype"], dev)
    S = torch.zeros((B, H, D, M), device=dev)
    z = torch.zeros((B, H, D), device=dev)
    out = torch.empty((B, H, M), device=dev)
    stream = torch.cuda.current_stream(dev)
    for t in range(warm_steps):
        ea.decode_step(S, z, q[t], k[t], v[t], out=out, stream=stream)
    times = []
    for _ in range(reps):
        S.zero_()
        z.zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(T):
            ea.decode_step(S, z, q[t], k[t], v[t], out=out, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    # per-launch kernel time: events around single launches
    n = 256
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for t in range(n):
        evs[t][0].record(stream)
        ea.decode_step(S, z, q[t], k[t], v[t], out=out, stream=stream)
        evs[t][1].record(stream)
    torch.cuda.synchronize()
    us_kernel = sum(a.elapsed_time(b) for a, b in evs) / n * 1e3
    best = min(times)
    per_step_bytes = decode_bytes_per_step(cfg)
    del q, k, v
    torch.cuda.empty_cache()
    return dict(ms_total_best=best, ms_total_all=times, us_per_step=best * 1e3 / T,
                tokens_per_s=B * T / (best * 1e-3), us_kernel_event=us_kernel,
                bytes_per_step=per_step_bytes,
                effective_GBs=per_step_bytes * T / (best * 1e-3) / 1e9,
                kernel_GBs=per_step_bytes / (us_kernel * 1e-6) / 1e9)


def bench_decode_hbm(dev, B=4096, H=8, D=64, M=64, T=32, reps=3):
    """Decode steps with a state larger than the last-level cache (4096 streams x H=8: 545 MB),
    so every step reads and writes the state in HBM."""
    import torch
    import efficient_transformer_amd as ea
    import synthetic

    cfg = dict(B=B, H=H, D=D, M=M, T=T, dtype="f32")
    q = synthetic.draw_torch(5, synthetic.TID_DQ, (T, B, H, D), 1.0, "f32", dev)
    k = synthetic.draw_torch(5, synthetic.TID_DK, (T, B, H, D), 1.0, "f32", dev)
    v = synthetic.draw_torch(5, synthetic.TID_DV, (T, B, H, M), 1.0, "f32", dev)
    S = torch.zeros((B, H, D, M), device=dev)
    z = torch.zeros((B, H, D), device=dev)
    out = torch.empty((B, H, M), device=dev)
    stream = torch.cuda.current_stream(dev)
    for t in range(4):
        ea.decode_step(S, z, q[t], k[t], v[t], out=out, stream=stream)
    best = None
    for _ in range(reps):
        S.zero_()
        z.zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(T):
            ea.decode_step(S, z, q[t], k[t], v[t], out=out, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    nb = decode_bytes_per_step(cfg)
    del q, k, v, S, z
    torch.cuda.empty_cache()
    us = best * 1e3 / T
    return dict(us_per_step=us, bytes_per_step=nb, GBs=nb / (us * 1e-6) / 1e9, tokens_per_s=B / (us * 1e-6))


def bench_probes(dev, nbytes=1 << 30, reps=5):
    """Attainable peaks: a plain device-to-device copy of a buffer four times the last-level
    cache (the library's copy probe, and torch's copy kernel beside it; read plus written bytes
    per second), and the library's fp32 and bf16 MFMA loops (8 independent chains per
    wavefront, 8 wavefronts per SIMD).  Best of several launches each."""
    import torch
    import efficient_transformer_amd as ea

    def best_ms(fn):
        fn()
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    n = nbytes // 4
    a = torch.ones(n, device=dev)
    b = torch.empty(n, device=dev)
    moved = 2 * n * 4
    ms_probe = best_ms(lambda: ea.probe_copy(b, a))
    ms_torch = best_ms(lambda: b.copy_(a))
    del a, b
    torch.cuda.empty_cache()
    blocks = 256 * 8  # eight 4-wavefront workgroups per CU: 8 wavefronts per SIMD
    out = torch.empty(blocks * 256, device=dev)
    mfma = {}
    for kind, iters in (("f32", 2048), ("bf16", 2048)):
        flops = ea.probe_mfma(kind, blocks, iters, out=out)[1]
        mfma[kind] = flops / (best_ms(lambda: ea.probe_mfma(kind, blocks, iters, out=out)) * 1e-3) / 1e12
    return dict(bytes=moved, us=ms_probe * 1e3, GBs=moved / (ms_probe * 1e-3) / 1e9,
                torch_GBs=moved / (ms_torch * 1e-3) / 1e9, mfma_f32_TFs=mfma["f32"], mfma_bf16_TFs=mfma["bf16"])


def backward_bytes(cfg) -> int:
    """Algorithmic bytes of one backward call: read q, k, v, out, dout; write dq, dk, dv."""
    s_in = 4 if cfg["dtype"] == "f32" else 2
    D, M = cfg["D"], cfg["M"]
    return cfg["B"] * cfg["H"] * cfg["N"] * ((2 * D + M) * s_in + 8 * M + 8 * D + 4 * M)


def bench_backward(cfg, steps, dev):
    """la_backward_chunked on a prefill workload (five kernels per call), inputs rotated over
    enough buffer sets to exceed the last-level cache."""
    import torch
    import efficient_transformer_amd as ea
    import synthetic

    B, H, N, D, M = cfg["B"], cfg["H"], cfg["N"], cfg["D"], cfg["M"]
    nbytes = backward_bytes(cfg)
    nsets = max(1, math.ceil(1.25 * LLC_BYTES / nbytes))
    sets = []
    for i in range(nsets):
        Q, K, V = [synthetic.draw_torch(10 + i, t, (B, H, N, W), cfg["sigma"], cfg["dtype"], dev)
                   for t, W in ((0, D), (1, D), (2, M))]
        dO = synthetic.draw_torch(10 + i, 7, (B, H, N, M), 1.0, "f32", dev)
        out = ea.forward_chunked(Q, K, V)
        sets.append((Q, K, V, out, dO))
    ws = torch.empty(max(16, int(ea.linattn.lib().la_backward_workspace_bytes(B, H, N, D, M, 0 if cfg["dtype"] == "f32" else 1))),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    for i in range(3):
        ea.backward(*sets[i % nsets], workspace=ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        ea.backward(*sets[i % nsets], workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del sets
    torch.cuda.empty_cache()
    return dict(ms_per_step=ms, tokens_per_s=B * N / (ms * 1e-3), bytes=nbytes, nsets=nsets,
                GBs=nbytes / (ms * 1e-3) / 1e9)


def bench_decode_steps(cfg, T, calls, dev):
    """la_decode_steps: T tokens of every head per call, the state held in registers."""
    import torch
    import efficient_transformer_amd as ea
    import synthetic

    B, H, D, M = cfg["B"], cfg["H"], cfg["D"], cfg["M"]
    q = synthetic.draw_torch(1, synthetic.TID_DQ, (B, H, T, D), cfg["sigma"], cfg["dtype"], dev)
    k = synthetic.draw_torch(1, synthetic.TID_DK, (B, H, T, D), cfg["sigma"], cfg["dtype"], dev)
    v = synthetic.draw_torch(1, synthetic.TID_DV, (B, H, T, M), cfg["sigma"], cfg["dtype"], dev)
    S = torch.zeros((B, H, D, M), device=dev)
    z = torch.zeros((B, H, D), device=dev)
    out = torch.empty((B, H, T, M), device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(5):
        ea.decode_steps(S, z, q, k, v, out=out, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        ea.decode_steps(S, z, q, k, v, out=out, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    per_call = B * H * ((8 * D * M + 8 * D) + T * (4 * (2 * D + M) + 4 * M))
    return dict(T=T, us_per_call=ms * 1e3, tokens_per_s=B * T / (ms * 1e-3), bytes_per_call=per_call,
                GBs=per_call / (ms * 1e-3) / 1e9)


def bench_softmax_scan(cfg, steps, dev):
    """la_softmax_scan (one query per head) on a prefill-shaped workload, inputs rotated past
    the last-level cache.  Algorithmic bytes: read q, k, v once, write out once."""
    import torch
    import efficient_transformer_amd as ea
    import synthetic

    B, H, N, D, M = cfg["B"], cfg["H"], cfg["N"], cfg["D"], cfg["M"]
    s_in = 4 if cfg["dtype"] == "f32" else 2
    nbytes = B * H * (D * s_in + N * (D * s_in + M * s_in + 4 * M))
    nsets = max(1, math.ceil(1.25 * LLC_BYTES / nbytes))
    sets = []
    for i in range(nsets):
        q = synthetic.draw_torch(20 + i, 9, (B, H, D), 0.125, cfg["dtype"], dev)
        K = synthetic.draw_torch(20 + i, 1, (B, H, N, D), cfg["sigma"], cfg["dtype"], dev)
        V = synthetic.draw_torch(20 + i, 2, (B, H, N, M), cfg["sigma"], cfg["dtype"], dev)
        sets.append((q, K, V, torch.empty((B, H, N, M), device=dev)))
    wsb = int(ea.linattn.lib().la_softmax_scan_workspace_bytes(B, H, N, D, M))
    ws = torch.zeros(max(16, wsb), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    for i in range(5):
        q, K, V, o = sets[i % nsets]
        ea.softmax_scan(q, K, V, out=o, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        q, K, V, o = sets[i % nsets]
        ev[i][0].record(stream)
        ea.softmax_scan(q, K, V, out=o, workspace=ws, stream=stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in ev) / steps * 1e3
    del sets
    torch.cuda.empty_cache()
    return dict(us_kernel=us, tokens_per_s=B * N / (us * 1e-6), bytes=nbytes, nsets=nsets,
                GBs=nbytes / (us * 1e-6) / 1e9)


def bench_features(cfg, steps, dev):
    """Random features (16 positive random features, orthogonal projection) then causal
    linear attention on them, on the headline shape: one la_forward_features launch per
    step (the features formed inside the attention kernel), and for comparison the two
    launches la_feature_map (Q and K) + la_forward_chunked on the features.  Inputs
    rotate past the last-level cache; each launch is bracketed by its own events."""
    import torch
    import efficient_transformer_amd as ea
    import synthetic

    B, H, N, D, M, F = (cfg[k] for k in ("B", "H", "N", "D", "M", "F"))
    map_bytes = B * H * N * (2 * D * 4 + 2 * F * 4)
    attn_bytes = B * H * N * ((2 * F + M) * 4 + 4 * M)
    fused_bytes = B * H * N * (2 * D + 2 * M) * 4  # raw q, k, v read, out written
    nsets = max(1, math.ceil(1.25 * LLC_BYTES / (map_bytes + attn_bytes)))
    W = torch.from_numpy(ea.draw_projection(F, D, "orthogonal", 0)).to(dev)
    sets = []
    for i in range(nsets):
        Xq = synthetic.draw_torch(30 + i, synthetic.TID_Q, (B, H, N, D), cfg["sigma"], "f32", dev)
        Xk = synthetic.draw_torch(30 + i, synthetic.TID_K, (B, H, N, D), cfg["sigma"], "f32", dev)
        V = synthetic.draw_torch(30 + i, synthetic.TID_V, (B, H, N, M), 1.0, "f32", dev)
        fq = torch.empty((B, H, N, F), device=dev)
        fk = torch.empty((B, H, N, F), device=dev)
        sets.append((Xq, Xk, V, fq, fk, torch.empty((B, H, N, M), device=dev)))
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        Xq, Xk, V, fq, fk, o = sets[i % nsets]
        if ev:
            ev[0].record(stream)
        ea.feature_map(Xq, W, F, cfg["feature"], out=fq, X2=Xk, out2=fk, stream=stream)
        if ev:
            ev[1].record(stream)
        ea.forward_chunked(fq, fk, V, causal=True, out=o, stream=stream, features=True)
        if ev:
            ev[2].record(stream)

    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    us_map = sum(e[0].elapsed_time(e[1]) for e in evs) / steps * 1e3
    us_attn = sum(e[1].elapsed_time(e[2]) for e in evs) / steps * 1e3
    us_two = sum(e[0].elapsed_time(e[2]) for e in evs) / steps * 1e3

    def fused(i, ev=None):
        Xq, Xk, V, _, _, o = sets[i % nsets]
        if ev:
            ev[0].record(stream)
        ea.forward_features(Xq, Xk, V, W, F, cfg["feature"], out=o, stream=stream)
        if ev:
            ev[1].record(stream)

    for i in range(5):
        fused(i)
    torch.cuda.synchronize()
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        fused(i, evf[i])
    torch.cuda.synchronize()
    us_fused = sum(e[0].elapsed_time(e[1]) for e in evf) / steps * 1e3
    del sets
    torch.cuda.empty_cache()
    return dict(us_fused=us_fused, us_two=us_two, us_map=us_map, us_attn=us_attn, map_bytes=map_bytes,
                attn_bytes=attn_bytes, fused_bytes=fused_bytes, tokens_per_s=B * N / (us_fused * 1e-6),
                two_launch_tokens_per_s=B * N / (us_two * 1e-6), nsets=nsets)


def causal_kernel_name(cfg, chunk, segments) -> str:
    n_chunks = -(-cfg["N"] // chunk)
    cps = -(-n_chunks // segments)
    kind = "onepass_causal_kernel" if cps <= 4 else "fused_causal_kernel"
    t = "float" if cfg["dtype"] == "f32" else "bf16"
    ot = "bf16" if cfg.get("out") == "bf16" else "float"
    # the one-pass kernel's raw-row width (0: no feature map) and raw-row type
    extra = f", 0, {t}" if kind == "onepass_causal_kernel" else ""
    return f"{kind}<{t}, {cfg['D']}, {cfg['M']}, {chunk}, true, {ot}{extra}>"


def cpu_baseline(cfg, target_s=12.0):
    """fp64 oracle (C, OpenMP over heads) on a bounded sample of the prefill workload."""
    import numpy as np
    import oracle
    import synthetic

    oracle.build(force=False)
    threads = len(os.sched_getaffinity(0))
    Q, K, V = synthetic.prefill_inputs(cfg, 0)
    Qf, Kf, Vf = (synthetic.as_f64(x, cfg["dtype"]) for x in (Q, K, V))
    B, N = cfg["B"], cfg["N"]
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.causal(Qf, Kf, Vf, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    # one thread on two of the 64 heads; tokens/s scaled to all H heads of a token
    Q1, K1, V1 = (x[:1, :2] for x in (Qf, Kf, Vf))
    t1 = time.perf_counter()
    reps1 = 0
    while True:
        oracle.causal(Q1, K1, V1, threads=1)
        reps1 += 1
        el1 = time.perf_counter() - t1
        if el1 >= target_s / 4 or reps1 >= 1000:
            break
    one = N * reps1 * 2 / cfg["H"] / el1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return dict(value=B * N * reps / el, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{reps} full causal passes over the B={B} H={cfg['H']} N={N} D=M={cfg['D']} "
                       f"fp32 workload ({el:.1f} s wall, fp64, {threads} threads)",
                one_thread_value=round(one, 1),
                one_thread_sample=f"{reps1} passes over 2 heads (B=1, N={N}) on one thread, {el1:.1f} s; "
                                  f"tokens/s counts a token as all {cfg['H']} heads",
                cpu_model=model)


def profile_run(dev):
    """Untimed launches for counter collection: 4 headline prefill calls, 4 decode steps,
    2 backward calls, 2 multi-token decode calls, 2 softmax scans, 2 random-feature maps and prefills
    on them, 2 calls of each bf16 prefill workload and
    4 copies of a 512 MiB fp32 buffer (known traffic: 512 MiB read + 512 MiB written each)."""
    import torch
    import efficient_transformer_amd as ea
    import synthetic
    cfg = dict(synthetic.WORKLOADS["prefill_f32_b8h8_n1024_d64"])
    sets = make_prefill_sets(cfg, 1, dev)
    Q, K, V, out = sets[0]
    for _ in range(4):
        ea.forward_chunked(Q, K, V, causal=True, out=out)
    d = dict(synthetic.WORKLOADS["decode_f32_256x8_t4096_d64"])
    B, H, D, M = d["B"], d["H"], d["D"], d["M"]
    S = torch.zeros((B, H, D, M), device=dev)
    z = torch.zeros((B, H, D), device=dev)
    q = synthetic.draw_torch(0, synthetic.TID_DQ, (B, H, D), 1.0, "f32", dev)
    k = synthetic.draw_torch(0, synthetic.TID_DK, (B, H, D), 1.0, "f32", dev)
    v = synthetic.draw_torch(0, synthetic.TID_DV, (B, H, M), 1.0, "f32", dev)
    for _ in range(4):
        ea.decode_step(S, z, q, k, v)
    # the other kernels, once each
    dO = synthetic.draw_torch(0, 7, tuple(out.shape), 1.0, "f32", dev)
    for _ in range(2):
        ea.backward(Q, K, V, out, dO)
    qs = synthetic.draw_torch(1, synthetic.TID_DQ, (B, H, 16, D), 1.0, "f32", dev)
    ks = synthetic.draw_torch(1, synthetic.TID_DK, (B, H, 16, D), 1.0, "f32", dev)
    vs = synthetic.draw_torch(1, synthetic.TID_DV, (B, H, 16, M), 1.0, "f32", dev)
    for _ in range(2):
        ea.decode_steps(S, z, qs, ks, vs)
    qs1 = synthetic.draw_torch(1, 9, (cfg["B"], cfg["H"], cfg["D"]), 0.125, "f32", dev)
    for _ in range(2):
        ea.softmax_scan(qs1, K, V)
    fc = dict(synthetic.WORKLOADS["prefill_prf16_f32_b8h8_n1024_d64"])
    Wf = torch.from_numpy(ea.draw_projection(fc["F"], fc["D"], "orthogonal", 0)).to(dev)
    for _ in range(2):
        fq, fk = ea.feature_map(Q, Wf, fc["F"], "prf", X2=K)
        ea.forward_chunked(fq, fk, V, causal=True, features=True)
        ea.forward_features(Q, K, V, Wf, fc["F"], "prf")
    for name in ("prefill_bf16_b4h8_n3072_d64", "prefill_bf16_b1h16_n65536_d128"):
        c = dict(synthetic.WORKLOADS[name])
        Qb, Kb, Vb, ob = make_prefill_sets(c, 1, dev)[0]
        for _ in range(2):
            ea.forward_chunked(Qb, Kb, Vb, causal=True, out=ob)
        del Qb, Kb, Vb, ob
    src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("profile run done")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the headline prefill workload")
    ap.add_argument("--mode", choices=["bench", "profile"], default="bench",
                    help="profile: a few untimed launches of the headline kernel, of the decode kernel and of a "
                         "plain 512 MiB device copy (for hardware-counter runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} (WORLD_SIZE={world}) is not supported; "
              "sharding over several GPUs is not part of this benchmark", file=sys.stderr)
        sys.exit(2)

    import torch
    import synthetic
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.mode == "profile":
        profile_run(dev)
        return

    cfg = dict(synthetic.WORKLOADS["prefill_f32_b8h8_n1024_d64"])
    log(f"prefill {cfg}")
    pre = bench_prefill(cfg, args.steps, args.warmup, dev)
    log(f"prefill: {pre}")
    kernel_us = pre["us_kernel"]
    achieved = pre["bytes"] / (kernel_us * 1e-6) / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=measured_traffic("prefill_f32_B8H8N1024_D64M64.md"),
                    kernel=causal_kernel_name(cfg, pre["chunk"], pre["segments"]),
                    kernel_us=round(kernel_us, 2), algorithmic_bytes=pre["bytes"],
                    mfma_fp32_frac_at_min_flops=round(pre["flops_min"] / (kernel_us * 1e-6) / 1e12
                                                      / FP32_MFMA_PEAK_TFS, 4))

    line = {
        "metric": METRIC,
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "causal linear attention prefill, fp32, B=8 H=8 N=1024 D=M=64, phi=elu+1",
                   "B": cfg["B"], "H": cfg["H"], "N": cfg["N"], "D": cfg["D"], "M": cfg["M"],
                   "chunk": pre["chunk"], "segments": pre["segments"], "buffer_sets": pre["nsets"],
                   "parallelism": "single GPU"},
        "prefill_kernel_us": {"mean": round(pre["us_kernel"], 2), "median": round(pre["us_kernel_median"], 2),
                              "min": round(pre["us_kernel_min"], 2),
                              "warm_same_buffers_median": round(pre["us_warm_median"], 2)},
        "roofline": roofline,
    }

    if not args.no_extras:
        dcfg = dict(synthetic.WORKLOADS["decode_f32_256x8_t4096_d64"])
        log("decode ...")
        dec = bench_decode(dcfg, 3, dev)
        log(f"decode: {dec}")
        line["decode"] = {
            "workload": "recurrent decode, fp32, 256 streams x H=8, D=M=64, 4096 steps from zero state",
            "tokens_per_s": round(dec["tokens_per_s"], 1), "us_per_step": round(dec["us_per_step"], 3),
            "effective_GBs": round(dec["effective_GBs"], 1),
            "frac_hbm_peak": round(dec["effective_GBs"] / HBM_PEAK_GBS, 4),
            "kernel_us_event": round(dec["us_kernel_event"], 3),
            "bytes_per_step": dec["bytes_per_step"],
            "note": "the 34 MB state stays resident in the 256 MB last-level cache between steps"}
        log("decode, state beyond the last-level cache ...")
        dh = bench_decode_hbm(dev)
        log(f"decode (HBM): {dh}")
        line["decode_hbm"] = {
            "workload": "recurrent decode, fp32, 4096 streams x H=8, D=M=64 (545 MB state), 32 steps",
            "tokens_per_s": round(dh["tokens_per_s"], 1), "us_per_step": round(dh["us_per_step"], 2),
            "bytes_per_step": dh["bytes_per_step"], "GBs": round(dh["GBs"], 1),
            "frac_hbm_peak": round(dh["GBs"] / HBM_PEAK_GBS, 4)}
        log("peak probes ...")
        cp = bench_probes(dev)
        log(f"probes: {cp}")
        line["hbm_copy"] = {
            "workload": "plain device-to-device copy of 1 GiB (the library's copy probe): attainable HBM rate",
            "bytes_moved": cp["bytes"], "us": round(cp["us"], 1), "GBs": round(cp["GBs"], 1),
            "frac_hbm_peak": round(cp["GBs"] / HBM_PEAK_GBS, 4), "torch_copy_GBs": round(cp["torch_GBs"], 1)}
        line["mfma_probe"] = {
            "workload": "dense MFMA loops, 8 independent chains per wavefront, 2048 workgroups of 4 wavefronts",
            "f32_TFs": round(cp["mfma_f32_TFs"], 1), "f32_frac_peak": round(cp["mfma_f32_TFs"] / FP32_MFMA_PEAK_TFS, 4),
            "bf16_TFs": round(cp["mfma_bf16_TFs"], 1),
            "bf16_frac_peak": round(cp["mfma_bf16_TFs"] / BF16_MFMA_PEAK_TFS, 4)}
        line["decode_hbm"]["frac_of_copy_rate"] = round(dh["GBs"] / cp["GBs"], 4)
        others = {}
        for name, outdt in (("prefill_bf16_b4h8_n3072_d64", "fp32"), ("prefill_bf16_b1h16_n65536_d128", "fp32"),
                            ("prefill_bf16_b4h8_n3072_d64", "bf16"), ("prefill_bf16_b1h16_n65536_d128", "bf16")):
            c = dict(synthetic.WORKLOADS[name])
            if outdt == "bf16":
                c["out"] = "bf16"
            key = name if outdt == "fp32" else name + "_bf16out"
            log(f"prefill {key} ...")
            r = bench_prefill(c, max(10, args.steps // 4), 5, dev)
            log(f"{key}: {r}")
            others[key] = {
                "workload": f"causal prefill bf16 in, {outdt} out, B={c['B']} H={c['H']} N={c['N']} D=M={c['D']}",
                "tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 5),
                "chunk": r["chunk"], "segments": r["segments"],
                "kernel_us": round(r["us_kernel"], 2),
                "kernel_GBs": round(r["bytes"] / (r["us_kernel"] * 1e-6) / 1e9, 1),
                "frac_hbm_peak_kernel": round(r["bytes"] / (r["us_kernel"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        line["other_workloads"] = others
        log("backward ...")
        bw = bench_backward(cfg, max(10, args.steps // 4), dev)
        log(f"backward: {bw}")
        line["backward"] = {
            "workload": "gradients dQ, dK, dV of causal attention, fp32, B=8 H=8 N=1024 D=M=64",
            "tokens_per_s": round(bw["tokens_per_s"], 1), "ms_per_step": round(bw["ms_per_step"], 5),
            "algorithmic_bytes": bw["bytes"], "GBs": round(bw["GBs"], 1),
            "frac_hbm_peak": round(bw["GBs"] / HBM_PEAK_GBS, 4), "buffer_sets": bw["nsets"],
            "note": "one la_backward_chunked call = five kernels; time between events around the calls"}
        log("decode steps ...")
        ds = bench_decode_steps(dcfg, 16, 200, dev)
        log(f"decode steps: {ds}")
        line["decode_steps"] = {
            "workload": "recurrent decode, 16 tokens per call, fp32, 256 streams x H=8, D=M=64",
            "tokens_per_s": round(ds["tokens_per_s"], 1), "us_per_call": round(ds["us_per_call"], 2),
            "bytes_per_call": ds["bytes_per_call"], "GBs": round(ds["GBs"], 1),
            "frac_hbm_peak": round(ds["GBs"] / HBM_PEAK_GBS, 4)}

        log("softmax scan ...")
        sm = bench_softmax_scan(cfg, max(10, args.steps // 4), dev)
        log(f"softmax scan: {sm}")
        line["softmax_scan"] = {
            "workload": "softmax attention of one query per head over every prefix (RNN form), fp32, "
                        "B=8 H=8 N=1024 D=M=64",
            "tokens_per_s": round(sm["tokens_per_s"], 1), "kernel_us": round(sm["us_kernel"], 2),
            "algorithmic_bytes": sm["bytes"], "GBs": round(sm["GBs"], 1),
            "frac_hbm_peak": round(sm["GBs"] / HBM_PEAK_GBS, 4), "buffer_sets": sm["nsets"]}

        log("random features ...")
        fcfg = dict(synthetic.WORKLOADS["prefill_prf16_f32_b8h8_n1024_d64"])
        fe = bench_features(fcfg, max(10, args.steps // 4), dev)
        log(f"features: {fe}")
        line["features"] = {
            "workload": "16 positive random features (orthogonal projection) of q, k, then causal linear "
                        "attention on them, fp32, B=8 H=8 N=1024 D=M=64",
            "tokens_per_s": round(fe["tokens_per_s"], 1), "us_per_step": round(fe["us_fused"], 2),
            "fused_kernel_us": round(fe["us_fused"], 2), "fused_bytes": fe["fused_bytes"],
            "fused_GBs": round(fe["fused_bytes"] / (fe["us_fused"] * 1e-6) / 1e9, 1),
            "fused_frac_hbm_peak": round(fe["fused_bytes"] / (fe["us_fused"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "two_launch_us_per_step": round(fe["us_two"], 2),
            "two_launch_tokens_per_s": round(fe["two_launch_tokens_per_s"], 1),
            "feature_map_us": round(fe["us_map"], 2), "attention_us": round(fe["us_attn"], 2),
            "feature_map_GBs": round(fe["map_bytes"] / (fe["us_map"] * 1e-6) / 1e9, 1),
            "attention_GBs": round(fe["attn_bytes"] / (fe["us_attn"] * 1e-6) / 1e9, 1),
            "feature_map_bytes": fe["map_bytes"], "attention_bytes": fe["attn_bytes"],
            "buffer_sets": fe["nsets"]}

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(dict(synthetic.WORKLOADS["prefill_f32_b8h8_n1024_d64"]))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
