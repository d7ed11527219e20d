"""Seeded synthetic inputs shared by the HIP-path tests, the oracle tests and the bench.

This module holds no arithmetic of the attention method: it only draws numbers.
Every value is a pure function of (seed, tensor_id, flat_index), so any block of
any tensor can be regenerated on its own (a sampled check of a 65536-token head,
or one decode step of one stream, needs no other part of the tensor).

Generator (counter based, all integer arithmetic modulo 2**64):
  * SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
    number generators", OOPSLA 2014): z += 0x9E3779B97F4A7C15, then two
    xor-shift-multiply rounds and a final xor-shift.
  * base = splitmix64(seed * 0x9E3779B97F4A7C15 + tensor_id)
  * u_a, u_b = top 53 bits of splitmix64(base ^ (2*i)) and splitmix64(base ^ (2*i+1)),
    scaled to [0, 1)
  * Box-Muller: g = sqrt(-2 ln(1 - u_a)) * cos(2 pi u_b), in float64
  * value = float32(sigma * g); the bfloat16 variant rounds that float32 to
    nearest-even on its top 16 bits.

The pages evaluate on image and speech datasets that are not available here; the
tensors drawn here have the shapes of those workloads (for example 3072 = 32*32*3
positions, one per sub-pixel of a CIFAR-10 image) but i.i.d. normal content.
"""
from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# tensor ids: prefill Q, K, V; decode q, k, v over all steps ([T, B, H, width])
TID_Q, TID_K, TID_V = 0, 1, 2
TID_DQ, TID_DK, TID_DV = 3, 4, 5


def splitmix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output function applied elementwise to uint64 counters."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = x + _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _base(seed: int, tensor_id: int) -> np.uint64:
    with np.errstate(over="ignore"):
        s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) * _GOLDEN + np.uint64(tensor_id)
    return splitmix64(np.array([s], dtype=np.uint64))[0]


def normal_f64(seed: int, tensor_id: int, index: np.ndarray) -> np.ndarray:
    """Standard normal draws (float64) at the given flat indices."""
    idx = np.asarray(index, dtype=np.uint64)
    base = _base(seed, tensor_id)
    two = np.uint64(2)
    with np.errstate(over="ignore"):
        ra = splitmix64(base ^ (two * idx))
        rb = splitmix64(base ^ (two * idx + np.uint64(1)))
    scale = 2.0 ** -53
    ua = (ra >> np.uint64(11)).astype(np.float64) * scale
    ub = (rb >> np.uint64(11)).astype(np.float64) * scale
    return np.sqrt(-2.0 * np.log1p(-ua)) * np.cos(2.0 * np.pi * ub)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    # keep NaN payloads quiet (never produced by the generator, kept for completeness)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(seed: int, tensor_id: int, shape, sigma: float = 1.0, dtype: str = "f32",
         start: int = 0, chunk: int = 1 << 22) -> np.ndarray:
    """A tensor of i.i.d. N(0, sigma^2) values.

    dtype "f32" returns float32; "bf16" returns the uint16 bit patterns of the
    bfloat16 values (view them with bf16_bits_to_f32). `start` offsets the flat
    index, so draw(..., shape=(n,), start=s) equals elements [s, s+n) of a larger
    tensor drawn from the same (seed, tensor_id).
    """
    n = int(np.prod(shape)) if len(shape) else 1
    out32 = np.empty(n, dtype=np.float32)

    def fill(lo: int) -> None:
        hi = min(n, lo + chunk)
        idx = np.arange(start + lo, start + hi, dtype=np.uint64)
        out32[lo:hi] = (sigma * normal_f64(seed, tensor_id, idx)).astype(np.float32)

    blocks = list(range(0, n, chunk))
    if len(blocks) > 1:
        # numpy releases the GIL inside these ufuncs, so threads help on big tensors
        import os
        from concurrent.futures import ThreadPoolExecutor
        workers = min(len(blocks), max(1, min(16, len(os.sched_getaffinity(0)))))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, blocks))
    else:
        for lo in blocks:
            fill(lo)
    out32 = out32.reshape(shape)
    if dtype == "f32":
        return out32
    if dtype == "bf16":
        return f32_to_bf16_bits(out32).reshape(shape)
    raise ValueError(f"unknown dtype {dtype!r}")


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 image of a drawn tensor (bf16 patterns are widened exactly)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# The five workloads, named by what they are (shapes and distributions of the pages experiments, i.i.d. content).
WORKLOADS = {
    "prefill_f32_n64_d16": dict(kind="prefill", B=1, H=1, N=64, D=16, M=16, sigma=1.0, dtype="f32", chunk=16),
    "prefill_f32_b8h8_n1024_d64": dict(kind="prefill", B=8, H=8, N=1024, D=64, M=64, sigma=1.0, dtype="f32", chunk=0),
    "prefill_bf16_b4h8_n3072_d64": dict(kind="prefill", B=4, H=8, N=3072, D=64, M=64, sigma=0.5, dtype="bf16", chunk=0),
    "prefill_bf16_b1h16_n65536_d128": dict(kind="prefill", B=1, H=16, N=65536, D=128, M=128, sigma=1.0, dtype="bf16", chunk=0),
    "decode_f32_256x8_t4096_d64": dict(kind="decode", B=256, H=8, T=4096, D=64, M=64, sigma=1.0, dtype="f32"),
    # random features: q, k with sigma = D^(-1/4) (unit-variance q . k), 16 positive random features
    "prefill_prf16_f32_b8h8_n1024_d64": dict(kind="features", B=8, H=8, N=1024, D=64, M=64, F=16, feature="prf",
                                             sigma=64 ** -0.25, dtype="f32", chunk=0),
}


def prefill_inputs(cfg: dict, seed: int = 0):
    """Q, K ([B,H,N,D]) and V ([B,H,N,M]) for a prefill workload."""
    B, H, N, D, M = cfg["B"], cfg["H"], cfg["N"], cfg["D"], cfg["M"]
    s, dt = cfg["sigma"], cfg["dtype"]
    Q = draw(seed, TID_Q, (B, H, N, D), s, dt)
    K = draw(seed, TID_K, (B, H, N, D), s, dt)
    V = draw(seed, TID_V, (B, H, N, M), s, dt)
    return Q, K, V


def prefill_head_rows(cfg: dict, seed: int, tensor_id: int, bh: int, n0: int, n1: int, width: int):
    """Rows [n0, n1) of head bh (flattened b*H+h) of one prefill tensor, without drawing the rest."""
    N = cfg["N"]
    start = (bh * N + n0) * width
    return draw(seed, tensor_id, (n1 - n0, width), cfg["sigma"], cfg["dtype"], start=start)


def decode_inputs(cfg: dict, seed: int, t0: int, t1: int):
    """q, k ([t1-t0, B, H, D]) and v ([t1-t0, B, H, M]) for decode steps t0..t1-1."""
    B, H, D, M = cfg["B"], cfg["H"], cfg["D"], cfg["M"]
    s, dt = cfg["sigma"], cfg["dtype"]
    T = t1 - t0
    q = draw(seed, TID_DQ, (T, B, H, D), s, dt, start=t0 * B * H * D)
    k = draw(seed, TID_DK, (T, B, H, D), s, dt, start=t0 * B * H * D)
    v = draw(seed, TID_DV, (T, B, H, M), s, dt, start=t0 * B * H * M)
    return q, k, v


def decode_step_inputs(cfg: dict, seed: int, step: int, heads=None):
    """q, k ([B,H,D]) and v ([B,H,M]) for decode step `step` (or [len(heads), width] for some flat heads)."""
    B, H, D, M = cfg["B"], cfg["H"], cfg["D"], cfg["M"]
    s, dt = cfg["sigma"], cfg["dtype"]
    if heads is None:
        q, k, v = decode_inputs(cfg, seed, step, step + 1)
        return q[0], k[0], v[0]
    heads = list(heads)
    BH = B * H
    q = np.stack([draw(seed, TID_DQ, (D,), s, dt, start=(step * BH + h) * D) for h in heads])
    k = np.stack([draw(seed, TID_DK, (D,), s, dt, start=(step * BH + h) * D) for h in heads])
    v = np.stack([draw(seed, TID_DV, (M,), s, dt, start=(step * BH + h) * M) for h in heads])
    return q, k, v


def draw_torch(seed: int, tensor_id: int, shape, sigma: float = 1.0, dtype: str = "f32", device="cuda:0",
               start: int = 0, chunk: int = 1 << 26):
    """The same generator in torch int64/float64 arithmetic on `device` (for large benchmark inputs).

    Integer steps are exact (two's-complement wraparound equals arithmetic modulo
    2**64); the float64 log/cos may differ from numpy's in the last place, so an
    occasional float32 value can differ by one ulp from draw().  Parity tests use
    draw(); this variant only feeds timing runs.
    """
    import torch

    def c64(x: int) -> int:  # uint64 constant as the int64 with the same bits
        return x - (1 << 64) if x >= (1 << 63) else x

    def lsr(x, s: int):
        return (x >> s) & ((1 << (64 - s)) - 1)

    def mix(x):
        z = x + c64(0x9E3779B97F4A7C15)
        z = (z ^ lsr(z, 30)) * c64(0xBF58476D1CE4E5B9)
        z = (z ^ lsr(z, 27)) * c64(0x94D049BB133111EB)
        return z ^ lsr(z, 31)

    base = int(_base(seed, tensor_id))
    base = c64(base)
    n = 1
    for s_ in shape:
        n *= int(s_)
    out = torch.empty(n, dtype=torch.float32, device=device)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        idx = torch.arange(start + lo, start + hi, dtype=torch.int64, device=device)
        ra = mix(base ^ (2 * idx))
        rb = mix(base ^ (2 * idx + 1))
        ua = lsr(ra, 11).to(torch.float64) * 2.0 ** -53
        ub = lsr(rb, 11).to(torch.float64) * 2.0 ** -53
        g = torch.sqrt(-2.0 * torch.log1p(-ua)) * torch.cos(2.0 * torch.pi * ub)
        out[lo:hi] = (sigma * g).to(torch.float32)
    out = out.view(*shape)
    if dtype == "f32":
        return out
    if dtype == "bf16":
        return out.to(torch.bfloat16)  # round to nearest even
    raise ValueError(dtype)
