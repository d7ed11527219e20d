#!/usr/bin/env python3
"""Throughput of causal kernelized linear attention on one MI355X.

Method: "Transformers are RNNs: Fast Autoregressive Transformers with Linear
Attention" (Katharopoulos et al., 2020) -- parallel (chunked prefill) mode and
recurrent (decode) mode, both through the C ABI of liblinattn.so.

Headline (`value`): prefill tokens/s of the largest single-GPU workload, bf16
inputs with fp32 accumulation and fp32 outputs, B=1 H=16 N=65536 D=M=128 (one
token = one position across all 16 heads).  A step is one la_forward_chunked
call (one kernel launch) over that batch, inputs resident in HBM (1.34 GB of
algorithmic traffic per call, far beyond the 256 MB last-level cache).  The
timed region is K back-to-back steps between HIP events on the stream the
library launches on; the kernel's average duration is that region / K.

The same JSON line carries, for every workload of the benchmark set (the
64-position fp32 case, B=8 H=8 N=1024 fp32, B=4 H=8 N=3072 bf16, the headline,
the 256x8-head decode over 4096 steps, and a decode whose state lives in HBM)
a roofline object (algorithmic bytes / kernel time against 8 TB/s, the MFMA
fraction at the minimum flop count beside its ceiling, and, when the kernel
sources are those the committed profiles were taken on, the rocprofv3 average,
the HBM traffic and the MFMA-busy counter) and the fp64 CPU oracle's rate on
a bounded sample of it; then the NEXT workloads (backward, multi-token decode,
softmax scan, random features, bf16 outputs) and the peak probes.

Prints exactly one JSON line on stdout; progress goes to stderr.
`--mode profile --workload NAME` runs only a few untimed launches of one
workload (for rocprofv3 runs).
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

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FP32_MFMA_PEAK_TFS = 157.3   # dense fp32 matrix
BF16_MFMA_PEAK_TFS = 2516.6  # dense bf16 matrix
LLC_BYTES = 256 << 20        # Infinity Cache

METRIC = "causal linear-attention tokens/sec (prefill, decode) and % of MFMA/HBM roofline"

HEADLINE = "prefill_bf16_b1h16_n65536_d128"
PREFILLS = ["prefill_f32_n64_d16", "prefill_f32_b8h8_n1024_d64", "prefill_bf16_b4h8_n3072_d64", HEADLINE]
DECODE = "decode_f32_256x8_t4096_d64"
DECODE_HBM = dict(kind="decode", B=4096, H=8, T=32, D=64, M=64, sigma=1.0, dtype="f32")

# the committed rocprofv3 summary of each workload (profiles/<file>)
PROFILE_FILES = {
    "prefill_f32_n64_d16": "prefill_f32_B1H1N64_D16M16.md",
    "prefill_f32_b8h8_n1024_d64": "prefill_f32_B8H8N1024_D64M64.md",
    "prefill_bf16_b4h8_n3072_d64": "prefill_bf16_B4H8N3072_D64M64.md",
    HEADLINE: "prefill_bf16_B1H16N65536_D128M128.md",
    DECODE: "decode_f32_256x8_D64M64.md",
    "decode_hbm": "decode_f32_4096x8_D64M64.md",
    "backward": "backward_f32_B8H8N1024_D64M64.md",
    "decode_steps": "decode_steps_f32_256x8_T16_D64M64.md",
    "softmax_scan": "softmax_scan_f32_B8H8N1024_D64M64.md",
    "features": "features_prf16_f32_B8H8N1024_D64M64.md",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def csrc_sha256_16() -> str:
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "efficient_transformer_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profile_fields(workload: str) -> dict:
    """Figures of a workload's committed rocprofv3 summary (kernel average, HBM traffic per
    launch, MFMA-busy fraction), or {} when the kernel sources changed since it was taken."""
    name = PROFILE_FILES.get(workload)
    if name is None:
        return {}
    try:
        text = open(os.path.join(ROOT, "profiles", name)).read()
    except OSError:
        return {}
    f = {}
    for line in text.splitlines():
        if ": " in line and line.split(": ", 1)[0] in (
                "rocprof_avg_us", "traffic_bytes_per_launch", "mfma_busy_frac", "csrc_sha256_16", "kernel"):
            k, v = line.split(": ", 1)
            f[k] = v.strip()
    if f.get("csrc_sha256_16") != csrc_sha256_16():
        return {}
    out = {"profile": f"profiles/{name}"}
    if "rocprof_avg_us" in f:
        out["rocprof_avg_us"] = float(f["rocprof_avg_us"])
    if "traffic_bytes_per_launch" in f:
        out["traffic"] = int(f["traffic_bytes_per_launch"])
    if "mfma_busy_frac" in f:
        out["mfma_busy_frac_counter"] = float(f["mfma_busy_frac"])
    return out


# ---------------------------------------------------------------------------
# algorithmic work (bytes and the minimum flop count per head-token)
# ---------------------------------------------------------------------------

def prefill_bytes(cfg) -> int:
    """Read Q, K, V once, write out once (fp32, or bf16 when cfg["out"] == "bf16")."""
    s = 4 if cfg["dtype"] == "f32" else 2
    so = 2 if cfg.get("out") == "bf16" else 4
    BH, N, D, M = cfg["B"] * cfg["H"], cfg["N"], cfg["D"], cfg["M"]
    return BH * N * ((2 * D + M) * s + so * M)


def flops_min(BH, N, D, M) -> int:
    """Per head-token: state update 2DM, read-out 2DM, normaliser 4D, divide M."""
    return BH * N * (4 * D * M + 4 * D + M)


def decode_bytes_per_step(cfg) -> int:
    """Per step: S and z read and written, q k v read, out written (all fp32)."""
    BH, D, M = cfg["B"] * cfg["H"], cfg["D"], cfg["M"]
    return BH * (2 * 4 * D * M + 2 * 4 * D + 4 * (2 * D + M) + 4 * M)


def mfma_ceiling(nbytes, flops, mfma_peak_tfs) -> float:
    """The MFMA fraction reachable at the HBM peak: arithmetic intensity / ridge point."""
    ridge = mfma_peak_tfs * 1e12 / (HBM_PEAK_GBS * 1e9)
    return min(1.0, flops / nbytes / ridge)


def roofline(workload, nbytes, us, flops=None, mfma_peak=None, mfma_dtype=None, **extra) -> dict:
    achieved = nbytes / (us * 1e-6) / 1e9
    r = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
             frac=round(achieved / HBM_PEAK_GBS, 4), traffic=None, algorithmic_bytes=int(nbytes),
             kernel_us=round(us, 3))
    pf = profile_fields(workload)
    r["traffic"] = pf.pop("traffic", None)
    if flops is not None:
        tfs = flops / (us * 1e-6) / 1e12
        r["mfma"] = dict(dtype=mfma_dtype, flops_min=int(flops), achieved_TFs=round(tfs, 2), peak_TFs=mfma_peak,
                         frac=round(tfs / mfma_peak, 4),
                         ceiling_frac_at_hbm_peak=round(mfma_ceiling(nbytes, flops, mfma_peak), 4))
        if "mfma_busy_frac_counter" in pf:
            r["mfma"]["busy_frac_counter"] = pf.pop("mfma_busy_frac_counter")
    r.update(pf)
    r.update(extra)
    return r


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

# Upper bound on the untimed warm-up calls of `timed`; profile mode lowers it (a counter
# profiler serialises every dispatch, so 0.3 s of calls would take minutes there).
WARM_CALLS_MAX = 1 << 30


def timed(step, steps, warmup, stream, warm_s=0.3):
    """Average ms of one step over `steps` back-to-back steps between events on `stream`, after
    untimed steps for at least `warm_s` seconds (the clocks settle on the workload's own kernels:
    a few warm-up calls left the backward 4 % slow) and then `warmup` more."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < warm_s and i < WARM_CALLS_MAX:
        step(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def make_prefill_sets(cfg, nsets, dev, seed0=0):
    import torch
    import synthetic
    sets = []
    for r in range(nsets):
        shp = (cfg["B"], cfg["H"], cfg["N"])
        Q = synthetic.draw_torch(seed0 + r, synthetic.TID_Q, shp + (cfg["D"],), cfg["sigma"], cfg["dtype"], dev)
        K = synthetic.draw_torch(seed0 + r, synthetic.TID_K, shp + (cfg["D"],), cfg["sigma"], cfg["dtype"], dev)
        V = synthetic.draw_torch(seed0 + r, synthetic.TID_V, shp + (cfg["M"],), cfg["sigma"], cfg["dtype"], dev)
        odt = torch.bfloat16 if cfg.get("out") == "bf16" else torch.float32
        sets.append((Q, K, V, torch.empty(shp + (cfg["M"],), dtype=odt, device=dev)))
    torch.cuda.synchronize()
    return sets


MAX_SETS = 64  # a launch-bound workload gains nothing from more rotation


def prefill_runner(cfg, dev, nsets=None):
    """(step function, plan) of a causal prefill workload; inputs rotate over enough buffer
    sets that the last-level cache cannot hold them (at most MAX_SETS), or over `nsets`."""
    import torch
    import efficient_transformer_amd as ea
    from efficient_transformer_amd import linattn as L
    code = L.LA_F32 if cfg["dtype"] == "f32" else L.LA_BF16
    B, H, N, D, M = cfg["B"], cfg["H"], cfg["N"], cfg["D"], cfg["M"]
    C, G, wsb = ea.forward_plan(B, H, N, D, M, True, code, cfg.get("chunk", 0))
    nbytes = prefill_bytes(cfg)
    if nsets is None:
        nsets = min(MAX_SETS, max(1, math.ceil(1.25 * LLC_BYTES / nbytes)))
    sets = make_prefill_sets(cfg, nsets, dev)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)  # zeroed once; each call leaves it ready
    stream = torch.cuda.current_stream(dev)

    def step(i):
        Q, K, V, out = sets[i % nsets]
        ea.forward_chunked(Q, K, V, causal=True, chunk=C, out=out, workspace=ws, stream=stream)

    return step, dict(chunk=C, segments=G, buffer_sets=nsets, ws=ws, stream=stream, sets=sets)


def causal_kernel_name(cfg, chunk, segments) -> str:
    n_chunks = -(-cfg["N"] // chunk)
    cps = -(-n_chunks // segments)
    kind = "onepass_causal_kernel" if cps <= 4 else "fused_causal_kernel"
    t = "float" if cfg["dtype"] == "f32" else "bf16"
    ot = "bf16" if cfg.get("out") == "bf16" else "float"
    extra = f", 0, {t}" if kind == "onepass_causal_kernel" else ""
    if kind == "fused_causal_kernel" and t == "bf16" and cfg["D"] == cfg["M"] == 128 and chunk == 64:
        return f"fused_causal32_kernel<{ot}>"  # the 32x32x16 engine for this shape
    return f"{kind}<{t}, {cfg['D']}, {cfg['M']}, {chunk}, true, {ot}{extra}>"


def bench_prefill(name, cfg, steps, warmup, dev):
    import torch
    step, plan = prefill_runner(cfg, dev)
    ms = timed(step, steps, warmup, plan["stream"])
    lat = None
    if cfg["N"] * cfg["B"] * cfg["H"] <= 4096:
        # a launch-bound workload: also the latency of one call (events around single calls)
        per = []
        for i in range(50):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(plan["stream"])
            step(i)
            e1.record(plan["stream"])
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3)
        lat = sorted(per)[len(per) // 2]
    bf16 = cfg["dtype"] == "bf16"
    BH = cfg["B"] * cfg["H"]
    rl = roofline(name, prefill_bytes(cfg), ms * 1e3, flops_min(BH, cfg["N"], cfg["D"], cfg["M"]),
                  BF16_MFMA_PEAK_TFS if bf16 else FP32_MFMA_PEAK_TFS, "bf16" if bf16 else "f32",
                  kernel=causal_kernel_name(cfg, plan["chunk"], plan["segments"]))
    res = dict(workload=f"causal prefill, {cfg['dtype']} in, fp32 out, B={cfg['B']} H={cfg['H']} N={cfg['N']} "
                        f"D={cfg['D']} M={cfg['M']}",
               tokens_per_s=round(cfg["B"] * cfg["N"] / (ms * 1e-3), 1), ms_per_step=round(ms, 5),
               chunk=plan["chunk"], segments=plan["segments"], buffer_sets=plan["buffer_sets"], roofline=rl)
    if lat is not None:
        res["latency_us_single_call"] = round(lat, 2)
        res["roofline"]["note"] = "launch-bound: 16 KB of algorithmic traffic; the figure of merit is latency"
    del plan
    torch.cuda.empty_cache()
    return res


def bench_decode_loop(cfg, dev, reps=3, seed=0):
    """The whole T-step loop of la_decode_step from a zero state, best of `reps`; per-step
    time = loop time / T (one kernel launch per step)."""
    import torch
    import efficient_transformer_amd as ea
    import synthetic
    B, H, D, M, T = cfg["B"], cfg["H"], cfg["D"], cfg["M"], cfg["T"]
    q = synthetic.draw_torch(seed, synthetic.TID_DQ, (T, B, H, D), cfg["sigma"], cfg["dtype"], dev)
    k = synthetic.draw_torch(seed, synthetic.TID_DK, (T, B, H, D), cfg["sigma"], cfg["dtype"], dev)
    v = synthetic.draw_torch(seed, synthetic.TID_DV, (T, B, H, M), cfg["sigma"], cfg["dtype"], dev)
    S = torch.zeros((B, H, D, M), device=dev)
    z = torch.zeros((B, H, D), device=dev)
    out = torch.empty((B, H, M), device=dev)
    stream = torch.cuda.current_stream(dev)
    for t in range(min(T, 64)):
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
    del q, k, v, S, z
    torch.cuda.empty_cache()
    return best


def bench_decode(name, cfg, dev, note):
    ms = bench_decode_loop(cfg, dev)
    T, BH = cfg["T"], cfg["B"] * cfg["H"]
    us = ms * 1e3 / T
    rl = roofline(name, decode_bytes_per_step(cfg), us, kernel=f"decode_kernel<float, {cfg['D']}, {cfg['M']}, true, 0>",
                  note=note)
    return dict(workload=f"recurrent decode, fp32, {cfg['B']} streams x H={cfg['H']}, D=M={cfg['D']}, {T} steps "
                         "from a zero state",
                tokens_per_s=round(cfg["B"] * T / (ms * 1e-3), 1), us_per_step=round(us, 3),
                state_bytes=BH * (cfg["D"] * cfg["M"] + cfg["D"]) * 4, roofline=rl)


# ---------------------------------------------------------------------------
# the fp64 CPU oracle on bounded samples
# ---------------------------------------------------------------------------

def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        return ""


def _repeat(fn, target_s):
    t0 = time.perf_counter()
    reps = 0
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 10000:
            return reps, el


def oracle_prefill(cfg, target_s, one_thread_s=0.0):
    """Tokens/s of the oracle's causal running sums over a bounded sample of a prefill
    workload: all heads, the first n positions (per-position work does not depend on the
    position), repeated for about target_s seconds on every host core; optionally also one
    thread on one head."""
    import oracle
    import synthetic
    oracle.build(force=False)
    threads = len(os.sched_getaffinity(0))
    B, H, N, D, M, dt = cfg["B"], cfg["H"], cfg["N"], cfg["D"], cfg["M"], cfg["dtype"]
    BH = B * H
    n = min(N, max(64, int(2 ** 32 // max(1, BH * (4 * D * M)))))  # about 4 GFLOP per pass

    def rows(tid, width):
        return [synthetic.as_f64(synthetic.prefill_head_rows(cfg, 0, tid, h, 0, n, width), dt) for h in range(BH)]

    import numpy as np
    Q = np.stack(rows(synthetic.TID_Q, D)).reshape(B, H, n, D)
    K = np.stack(rows(synthetic.TID_K, D)).reshape(B, H, n, D)
    V = np.stack(rows(synthetic.TID_V, M)).reshape(B, H, n, M)
    reps, el = _repeat(lambda: oracle.causal(Q, K, V, threads=threads), target_s)
    res = dict(value=round(B * n * reps / el, 1), unit="tokens/s", cores=threads, kind="oracle",
               sample=f"{reps} passes of the fp64 causal running sums over the first {n} of {N} positions of all "
                      f"{BH} heads (B={B} H={H} D={D} M={M}, {dt} inputs widened exactly), {el:.1f} s on {threads} "
                      f"threads; a token is one position of all {H} heads")
    if one_thread_s > 0:
        Q1, K1, V1 = Q[:1, :1], K[:1, :1], V[:1, :1]
        r1, e1 = _repeat(lambda: oracle.causal(Q1, K1, V1, threads=1), one_thread_s)
        res["one_thread_value"] = round(n * r1 / e1 / H, 1)
        res["one_thread_sample"] = (f"{r1} passes over one head, {n} positions, one thread, {e1:.1f} s; "
                                    f"tokens/s counts a token as all {H} heads")
    return res


def oracle_decode(cfg, target_s):
    """Tokens/s of the oracle's recurrent step over every head of a decode workload."""
    import numpy as np
    import oracle
    import synthetic
    oracle.build(force=False)
    threads = len(os.sched_getaffinity(0))
    B, H, D, M = cfg["B"], cfg["H"], cfg["D"], cfg["M"]
    T = 64
    q, k, v = (x.reshape(T, B * H, -1).astype(np.float64) for x in synthetic.decode_inputs(cfg, 0, 0, T))
    S = np.zeros((B * H, D, M))
    z = np.zeros((B * H, D))
    t0 = time.perf_counter()
    steps = 0
    while True:
        oracle.decode_step(S, z, q[steps % T], k[steps % T], v[steps % T], threads=threads)
        steps += 1
        el = time.perf_counter() - t0
        if el >= target_s or steps >= 100000:
            break
    return dict(value=round(B * steps / el, 1), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{steps} fp64 recurrent steps of all {B * H} heads ({B} streams x H={H}, D=M={D}), "
                       f"{el:.1f} s on {threads} threads")


# ---------------------------------------------------------------------------
# NEXT workloads and probes (timed region: back-to-back calls between events)
# ---------------------------------------------------------------------------

def backward_bytes(cfg) -> int:
    """Read q, k, v, out, dout; write dq, dk, dv."""
    s_in = 4 if cfg["dtype"] == "f32" else 2
    D, M = cfg["D"], cfg["M"]
    return cfg["B"] * cfg["H"] * cfg["N"] * ((2 * D + M) * s_in + 8 * M + 8 * D + 4 * M)


def bench_backward(cfg, steps, dev):
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
        sets.append((Q, K, V, ea.forward_chunked(Q, K, V), dO))
    need = int(ea.linattn.lib().la_backward_workspace_bytes(B, H, N, D, M, 0 if cfg["dtype"] == "f32" else 1))
    ws = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ms = timed(lambda i: ea.backward(*sets[i % nsets], workspace=ws, stream=stream), steps, 3, stream)
    del sets
    torch.cuda.empty_cache()
    return dict(workload=f"gradients dQ, dK, dV of causal attention, {cfg['dtype']}, B={B} H={H} N={N} D=M={D}",
                tokens_per_s=round(B * N / (ms * 1e-3), 1), ms_per_step=round(ms, 5), buffer_sets=nsets,
                roofline=roofline("backward", nbytes, ms * 1e3, note="one la_backward_chunked call = five kernels"))


def bench_decode_steps(cfg, T, calls, dev):
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
    ms = timed(lambda i: ea.decode_steps(S, z, q, k, v, out=out, stream=stream), calls, 5, stream)
    per_call = B * H * ((8 * D * M + 8 * D) + T * (4 * (2 * D + M) + 4 * M))
    return dict(workload=f"recurrent decode, {T} tokens per call, fp32, {B} streams x H={H}, D=M={D}",
                tokens_per_s=round(B * T / (ms * 1e-3), 1), us_per_call=round(ms * 1e3, 2),
                roofline=roofline("decode_steps", per_call, ms * 1e3))


def bench_softmax_scan(cfg, steps, dev):
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

    def step(i):
        q, K, V, o = sets[i % nsets]
        ea.softmax_scan(q, K, V, out=o, workspace=ws, stream=stream)

    ms = timed(step, steps, 5, stream)
    del sets
    torch.cuda.empty_cache()
    return dict(workload="softmax attention of one query per head over every prefix (RNN form), "
                         f"{cfg['dtype']}, B={B} H={H} N={N} D=M={D}",
                tokens_per_s=round(B * N / (ms * 1e-3), 1), ms_per_step=round(ms, 5), buffer_sets=nsets,
                roofline=roofline("softmax_scan", nbytes, ms * 1e3))


def bench_features(cfg, steps, dev):
    """16 positive random features then causal attention: one fused launch per step, and the
    two launches (feature map, attention on features) for comparison."""
    import torch
    import efficient_transformer_amd as ea
    import synthetic
    B, H, N, D, M, F = (cfg[k] for k in ("B", "H", "N", "D", "M", "F"))
    map_bytes = B * H * N * (2 * D * 4 + 2 * F * 4)
    attn_bytes = B * H * N * ((2 * F + M) * 4 + 4 * M)
    fused_bytes = B * H * N * (2 * D + 2 * M) * 4
    nsets = max(1, math.ceil(1.25 * LLC_BYTES / (map_bytes + attn_bytes)))
    W = torch.from_numpy(ea.draw_projection(F, D, "orthogonal", 0)).to(dev)
    sets = []
    for i in range(nsets):
        Xq = synthetic.draw_torch(30 + i, synthetic.TID_Q, (B, H, N, D), cfg["sigma"], "f32", dev)
        Xk = synthetic.draw_torch(30 + i, synthetic.TID_K, (B, H, N, D), cfg["sigma"], "f32", dev)
        V = synthetic.draw_torch(30 + i, synthetic.TID_V, (B, H, N, M), 1.0, "f32", dev)
        sets.append((Xq, Xk, V, torch.empty((B, H, N, F), device=dev), torch.empty((B, H, N, F), device=dev),
                     torch.empty((B, H, N, M), device=dev)))
    stream = torch.cuda.current_stream(dev)

    def fused(i):
        Xq, Xk, V, _, _, o = sets[i % nsets]
        ea.forward_features(Xq, Xk, V, W, F, cfg["feature"], out=o, stream=stream)

    def two(i):
        Xq, Xk, V, fq, fk, o = sets[i % nsets]
        ea.feature_map(Xq, W, F, cfg["feature"], out=fq, X2=Xk, out2=fk, stream=stream)
        ea.forward_chunked(fq, fk, V, causal=True, out=o, stream=stream, features=True)

    ms_f = timed(fused, steps, 5, stream)
    ms_2 = timed(two, steps, 5, stream)
    del sets
    torch.cuda.empty_cache()
    return dict(workload="16 positive random features (orthogonal projection) of q, k, then causal linear "
                         f"attention on them, fp32, B={B} H={H} N={N} D=M={D}",
                tokens_per_s=round(B * N / (ms_f * 1e-3), 1), us_per_step=round(ms_f * 1e3, 2),
                roofline=roofline("features", fused_bytes, ms_f * 1e3,
                                  note="one la_forward_features launch; algorithmic bytes: raw q, k, v read, "
                                       "out written"),
                two_launch_us_per_step=round(ms_2 * 1e3, 2),
                two_launch_tokens_per_s=round(B * N / (ms_2 * 1e-3), 1),
                two_launch_bytes=map_bytes + attn_bytes)


def bench_probes(dev, nbytes=1 << 30, reps=5):
    """Attainable peaks: the library's copy probe (read + written bytes per second), its
    read-only and write-only stream probes, torch's copy kernel, and the fp32 / bf16 MFMA
    loops (8 independent chains per wavefront, 4 for the bf16 32x32x16 shape; 8 wavefronts
    per SIMD).  Best of several launches."""
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
    part = torch.empty(int(ea.linattn.lib().la_probe_read_partials()), device=dev)
    ms_copy = best_ms(lambda: ea.probe_copy(b, a))
    ms_read = best_ms(lambda: ea.probe_read(a, out=part))
    ms_write = best_ms(lambda: ea.probe_write(b, 1.0))
    ms_torch = best_ms(lambda: b.copy_(a))
    del a, b
    torch.cuda.empty_cache()
    blocks = 256 * 8
    out = torch.empty(blocks * 256, device=dev)
    mfma = {}
    for kind in ("f32", "bf16", "bf16_32x32"):
        flops = ea.probe_mfma(kind, blocks, 2048, out=out)[1]
        mfma[kind] = flops / (best_ms(lambda: ea.probe_mfma(kind, blocks, 2048, out=out)) * 1e-3) / 1e12
    copy_gbs = 2 * nbytes / (ms_copy * 1e-3) / 1e9
    read_gbs = nbytes / (ms_read * 1e-3) / 1e9
    write_gbs = nbytes / (ms_write * 1e-3) / 1e9
    return dict(
        hbm_copy=dict(workload="device-to-device copy of 1 GiB (nontemporal 16-byte loads and stores): "
                               "attainable read + write rate",
                      bytes_moved=2 * nbytes, us=round(ms_copy * 1e3, 1), GBs=round(copy_gbs, 1),
                      frac_hbm_peak=round(copy_gbs / HBM_PEAK_GBS, 4),
                      torch_copy_GBs=round(2 * nbytes / (ms_torch * 1e-3) / 1e9, 1)),
        hbm_read=dict(workload="read-only stream over 1 GiB (nontemporal 16-byte loads): attainable read rate",
                      bytes_read=nbytes, us=round(ms_read * 1e3, 1), GBs=round(read_gbs, 1),
                      frac_hbm_peak=round(read_gbs / HBM_PEAK_GBS, 4)),
        hbm_write=dict(workload="write-only stream over 1 GiB (nontemporal 16-byte stores): attainable write rate",
                       bytes_written=nbytes, us=round(ms_write * 1e3, 1), GBs=round(write_gbs, 1),
                       frac_hbm_peak=round(write_gbs / HBM_PEAK_GBS, 4)),
        mfma_probe=dict(workload="dense MFMA loops, 8 independent chains per wavefront (4 for the bf16 32x32x16 "
                                 "shape), 2048 workgroups of 4 wavefronts",
                        bf16_32x32_TFs=round(mfma["bf16_32x32"], 1),
                        bf16_32x32_frac_peak=round(mfma["bf16_32x32"] / BF16_MFMA_PEAK_TFS, 4),
                        f32_TFs=round(mfma["f32"], 1), f32_frac_peak=round(mfma["f32"] / FP32_MFMA_PEAK_TFS, 4),
                        bf16_TFs=round(mfma["bf16"], 1),
                        bf16_frac_peak=round(mfma["bf16"] / BF16_MFMA_PEAK_TFS, 4)))


# ---------------------------------------------------------------------------
# profile mode: untimed launches of one workload, for rocprofv3
# ---------------------------------------------------------------------------

def warm_clocks(dev, seconds=0.3):
    """Untimed device work (torch's own elementwise kernels, not the library's) until the clocks have
    settled, so that a profiler's kernel averages see the same clocks as the timed bench."""
    import torch
    x = torch.ones(1 << 26, device=dev)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            x.mul_(1.0)
        torch.cuda.synchronize()
    del x


def profile_run(workload, dev, launches=16):
    import torch
    import efficient_transformer_amd as ea
    import synthetic
    if workload in synthetic.WORKLOADS and synthetic.WORKLOADS[workload]["kind"] == "prefill":
        # as the timed bench: the kernel itself for 0.3 s (at most 256 launches) first; after an idle
        # spell the long-head kernel runs up to 30 % slow for its first few dozen launches
        # the bench's input rotation (at most 8 sets: under a counter profiler every dispatch,
        # the input generator's included, is collected one at a time)
        cfg = dict(synthetic.WORKLOADS[workload])
        nsets = min(8, max(1, math.ceil(1.25 * LLC_BYTES / prefill_bytes(cfg))))
        step, plan = prefill_runner(cfg, dev, nsets=nsets)
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < 0.3 and i < 256:
            step(i)
            i += 1
            if i % 16 == 0:
                torch.cuda.synchronize()
        for i in range(launches):
            step(i)
        torch.cuda.synchronize()
        log(f"profile run of {workload} done")
        return
    global WARM_CALLS_MAX
    WARM_CALLS_MAX = 256  # the timed functions below warm up on their own calls, as in the bench
    warm_clocks(dev)
    if workload == DECODE:
        bench_decode_loop(dict(synthetic.WORKLOADS[DECODE], T=256), dev, reps=1)
    elif workload == "decode_hbm":
        bench_decode_loop(dict(DECODE_HBM, T=16), dev, reps=1)
    elif workload == "backward":
        bench_backward(dict(synthetic.WORKLOADS["prefill_f32_b8h8_n1024_d64"]), 4, dev)
    elif workload == "decode_steps":
        bench_decode_steps(dict(synthetic.WORKLOADS[DECODE]), 16, 4, dev)
    elif workload == "softmax_scan":
        bench_softmax_scan(dict(synthetic.WORKLOADS["prefill_f32_b8h8_n1024_d64"]), 4, dev)
    elif workload == "features":  # the fused launch only
        c = dict(synthetic.WORKLOADS["prefill_prf16_f32_b8h8_n1024_d64"])
        B, H, N, D, M, F = (c[k] for k in ("B", "H", "N", "D", "M", "F"))
        W = torch.from_numpy(ea.draw_projection(F, D, "orthogonal", 0)).to(dev)
        X = [synthetic.draw_torch(30, t, (B, H, N, D if t < 2 else M), c["sigma"] if t < 2 else 1.0, "f32", dev)
             for t in range(3)]
        o = torch.empty((B, H, N, M), device=dev)
        timed(lambda i: ea.forward_features(X[0], X[1], X[2], W, F, c["feature"], out=o), 8, 0,
              torch.cuda.current_stream(dev))
    elif workload == "copy512":
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            ea.probe_copy(dst, src)
    else:
        raise SystemExit(f"unknown workload {workload!r}")
    torch.cuda.synchronize()
    log(f"profile run of {workload} done")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the headline workload")
    ap.add_argument("--mode", choices=["bench", "profile"], default="bench")
    ap.add_argument("--workload", default=HEADLINE, help="profile mode: which workload to launch")
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
        profile_run(args.workload, dev)
        return

    cfg = dict(synthetic.WORKLOADS[HEADLINE])
    log(f"headline prefill {cfg}")
    head = bench_prefill(HEADLINE, cfg, args.steps, args.warmup, dev)
    log(f"headline: {head}")
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal linear attention prefill (phi = elu + 1), bf16 inputs, fp32 accumulate and "
                               "output, B=1 H=16 N=65536 D=M=128",
                   "B": cfg["B"], "H": cfg["H"], "N": cfg["N"], "D": cfg["D"], "M": cfg["M"],
                   "chunk": head["chunk"], "segments": head["segments"], "parallelism": "single GPU"},
        "roofline": head["roofline"],
    }
    configs = {HEADLINE: {k: v for k, v in head.items() if k != "roofline"}}
    configs[HEADLINE]["roofline"] = "see the top-level roofline"

    if not args.no_extras:
        for name in PREFILLS[:-1]:
            c = dict(synthetic.WORKLOADS[name])
            log(f"prefill {name} ...")
            configs[name] = bench_prefill(name, c, max(args.steps, 50), args.warmup, dev)
            log(f"{name}: {configs[name]}")
        log("decode ...")
        configs[DECODE] = bench_decode(DECODE, dict(synthetic.WORKLOADS[DECODE]), dev,
                                       "cache-assisted: the 34 MB state stays in the 256 MB last-level cache "
                                       "between steps")
        log(f"decode: {configs[DECODE]}")
        log("decode, state in HBM ...")
        configs["decode_hbm"] = bench_decode("decode_hbm", DECODE_HBM, dev,
                                             "the 545 MB state cannot stay in the last-level cache: HBM-resident")
        log(f"decode (HBM): {configs['decode_hbm']}")
    line["configs"] = configs

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = oracle_prefill(cfg, 10.0)
        line["cpu_baseline"]["cpu_model"] = _cpu_model()
        if not args.no_extras:
            for name, t, t1 in (("prefill_f32_n64_d16", 1.0, 1.0), ("prefill_f32_b8h8_n1024_d64", 3.0, 1.5),
                                ("prefill_bf16_b4h8_n3072_d64", 3.0, 1.5)):
                configs[name]["cpu_baseline"] = oracle_prefill(dict(synthetic.WORKLOADS[name]), t, t1)
            configs[HEADLINE]["cpu_baseline"] = "see the top-level cpu_baseline"
            configs[DECODE]["cpu_baseline"] = oracle_decode(dict(synthetic.WORKLOADS[DECODE]), 3.0)
            log("oracle timings done")

    if not args.no_extras:
        extras = {}
        base = dict(synthetic.WORKLOADS["prefill_f32_b8h8_n1024_d64"])
        log("backward ...")
        extras["backward"] = bench_backward(base, max(10, args.steps), dev)
        log("decode steps ...")
        extras["decode_steps"] = bench_decode_steps(dict(synthetic.WORKLOADS[DECODE]), 16, 200, dev)
        log("softmax scan ...")
        extras["softmax_scan"] = bench_softmax_scan(base, max(10, args.steps), dev)
        log("random features ...")
        extras["features"] = bench_features(dict(synthetic.WORKLOADS["prefill_prf16_f32_b8h8_n1024_d64"]),
                                            max(10, args.steps), dev)
        for name in ("prefill_bf16_b4h8_n3072_d64", HEADLINE):
            c = dict(synthetic.WORKLOADS[name], out="bf16")
            log(f"{name} with bf16 outputs ...")
            r = bench_prefill(name + "_bf16out", c, max(10, args.steps), args.warmup, dev)
            r["workload"] = r["workload"].replace("fp32 out", "bf16 out")
            extras[name + "_bf16out"] = r
        log("probes ...")
        extras.update(bench_probes(dev))
        line["next"] = extras
        cp = extras["hbm_copy"]["GBs"]
        for k in ("decode_hbm",):
            configs[k]["roofline"]["frac_of_copy_probe"] = round(configs[k]["roofline"]["achieved"] / cp, 4)
        line["roofline"]["frac_of_copy_probe"] = round(line["roofline"]["achieved"] / cp, 4)
        line["roofline"]["frac_of_read_probe"] = round(line["roofline"]["achieved"] / extras["hbm_read"]["GBs"], 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
