"""Parity of the HIP prefill path (la_forward_chunked and its stages) with the fp64 oracle.

Every case draws seeded inputs, runs the C ABI on cuda:0 and compares element by
element with the oracle at the tolerance of the input type (fp32 1e-4, bf16 2e-2,
row-wise relative; see gpu_helpers).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import TOL, rowwise_rel, to_dev, whole_rel

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def run_prefill(ea, cfg, seed, causal=True, chunk=None, with_state=False):
    Q, K, V = synthetic.prefill_inputs(cfg, seed)
    dt = cfg["dtype"]
    Qd, Kd, Vd = to_dev(Q, dt), to_dev(K, dt), to_dev(V, dt)
    S = z = None
    if with_state:
        B, H, D, M = cfg["B"], cfg["H"], cfg["D"], cfg["M"]
        S = torch.full((B, H, D, M), float("nan"), device=DEV)
        z = torch.full((B, H, D), float("nan"), device=DEV)
    out = ea.forward_chunked(Qd, Kd, Vd, causal=causal, chunk=cfg.get("chunk", 0) if chunk is None else chunk,
                             S_out=S, z_out=z)
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    if with_state:
        return (Q, K, V), res, S.cpu().numpy(), z.cpu().numpy()
    return (Q, K, V), res


def f64(x, dt):
    return synthetic.as_f64(x, dt)


def small_cfg(dtype, B, H, N, D, M, sigma=1.0):
    return dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=sigma, dtype=dtype, chunk=0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefill_f32_n64_d16_parity(ea, seed):
    cfg = synthetic.WORKLOADS["prefill_f32_n64_d16"]
    (Q, K, V), out = run_prefill(ea, cfg, seed)
    ref, _, _ = oracle.causal(f64(Q, "f32"), f64(K, "f32"), f64(V, "f32"))
    err = rowwise_rel(out, ref)
    assert err <= TOL["f32"], f"rowwise_rel {err:.3e}"


SHAPES = [(16, 16), (32, 64), (64, 32), (64, 64), (128, 128), (16, 128), (128, 16)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", SHAPES)
@pytest.mark.parametrize("N", [1, 33, 300])
@pytest.mark.parametrize("chunk", [0, 16, 32, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_small_parity(ea, dtype, D, M, N, chunk, causal):
    if chunk and not ea.linattn.lib().la_forward_plan(1, 1, max(N, 1), D, M, int(causal),
                                                      0 if dtype == "f32" else 1, chunk, None, None, None) == 0:
        pytest.skip("chunk does not fit LDS for this shape")
    cfg = small_cfg(dtype, 2, 3, N, D, M)
    (Q, K, V), out = run_prefill(ea, cfg, seed=N + D + M, causal=causal, chunk=chunk)
    Qf, Kf, Vf = f64(Q, dtype), f64(K, dtype), f64(V, dtype)
    ref = oracle.causal(Qf, Kf, Vf)[0] if causal else oracle.noncausal(Qf, Kf, Vf)
    err = rowwise_rel(out, ref)
    assert err <= TOL[dtype], f"row-wise rel err {err:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [1, 100, 1000])
def test_final_state(ea, dtype, causal, N):
    cfg = small_cfg(dtype, 2, 2, N, 64, 32)
    (Q, K, V), out, S, z = run_prefill(ea, cfg, seed=7, causal=causal, with_state=True)
    _, S_ref, z_ref = oracle.causal(f64(Q, dtype), f64(K, dtype), f64(V, dtype))
    # fp32 state sums; the bf16 path rounds phi(K) to bf16 before its MFMA, which bounds
    # the state's accuracy by the bf16 input tolerance
    tol = 1e-5 if dtype == "f32" else TOL["bf16"]
    err = whole_rel(S, S_ref)
    assert err <= tol, f"whole_rel {err:.3e} > {tol}"
    err = whole_rel(z, z_ref)
    assert err <= tol, f"whole_rel {err:.3e} > {tol}"


def test_empty_sequence_writes_zero_state(ea):
    Q = torch.empty((2, 3, 0, 16), device=DEV)
    V = torch.empty((2, 3, 0, 32), device=DEV)
    S = torch.full((2, 3, 16, 32), 5.0, device=DEV)
    z = torch.full((2, 3, 16), 5.0, device=DEV)
    out = ea.forward_chunked(Q, Q, V, S_out=S, z_out=z)
    torch.cuda.synchronize()
    assert out.shape == (2, 3, 0, 32)
    assert torch.count_nonzero(S).item() == 0 and torch.count_nonzero(z).item() == 0


def test_prefill_f32_b8h8_n1024_full(ea):
    cfg = synthetic.WORKLOADS["prefill_f32_b8h8_n1024_d64"]
    (Q, K, V), out = run_prefill(ea, cfg, 0)
    ref, _, _ = oracle.causal(f64(Q, "f32"), f64(K, "f32"), f64(V, "f32"))
    err = rowwise_rel(out, ref)
    print(f"b8h8 n1024 row-wise rel err {err:.3e}")
    assert err <= TOL["f32"], f"{err:.3e}"


def test_prefill_bf16_b4h8_n3072_full(ea):
    cfg = synthetic.WORKLOADS["prefill_bf16_b4h8_n3072_d64"]
    (Q, K, V), out = run_prefill(ea, cfg, 0)
    ref, _, _ = oracle.causal(f64(Q, "bf16"), f64(K, "bf16"), f64(V, "bf16"))
    err = rowwise_rel(out, ref)
    print(f"b4h8 n3072 row-wise rel err {err:.3e}")
    assert err <= TOL["bf16"], f"{err:.3e}"


def test_prefill_bf16_n65536_d128_full(ea):
    """The long-sequence workload at full size (B=1 H=16 N=65536 D=M=128, bf16), in the
    plan and launch that bench.py times: every row of all 16 heads and the final state
    against the oracle's running sums."""
    cfg = synthetic.WORKLOADS["prefill_bf16_b1h16_n65536_d128"]
    B, H, N, D, M = (cfg[k] for k in ("B", "H", "N", "D", "M"))
    Q, K, V = synthetic.prefill_inputs(cfg, 0)
    S = torch.empty((B, H, D, M), device=DEV)
    z = torch.empty((B, H, D), device=DEV)
    out = ea.forward_chunked(to_dev(Q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16"), S_out=S, z_out=z)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref, S_ref, z_ref = oracle.causal(f64(Q, "bf16"), f64(K, "bf16"), f64(V, "bf16"))
    for h in range(H):
        err = rowwise_rel(out[0, h], ref[0, h])
        print(f"n65536 head {h} row-wise rel err {err:.3e}")
        assert err <= TOL["bf16"], f"head {h}: {err:.3e}"
    assert whole_rel(S.cpu().numpy(), S_ref) <= TOL["bf16"]
    assert whole_rel(z.cpu().numpy(), z_ref) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ones_invariant(ea, dtype):
    cfg = small_cfg(dtype, 2, 2, 700, 64, 64)
    Q, K, _ = synthetic.prefill_inputs(cfg, 3)
    ones = np.ones((2, 2, 700, 64), np.float32)
    Vd = to_dev(ones if dtype == "f32" else synthetic.f32_to_bf16_bits(ones), dtype)
    out = ea.forward_chunked(to_dev(Q, dtype), to_dev(K, dtype), Vd)
    torch.cuda.synchronize()
    err = np.abs(out.cpu().numpy() - 1.0).max()
    assert err <= (1e-5 if dtype == "f32" else 1e-2), f"{err:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_first_row_and_last_row(ea, dtype):
    cfg = small_cfg(dtype, 1, 4, 333, 32, 64)
    Q, K, V = synthetic.prefill_inputs(cfg, 4)
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    c = ea.forward_chunked(Qd, Kd, Vd, causal=True).cpu().numpy()
    nc = ea.forward_chunked(Qd, Kd, Vd, causal=False).cpu().numpy()
    v0 = f64(V, dtype)[:, :, 0]
    err = rowwise_rel(c[:, :, 0], v0)
    assert err <= 1e-6, f"rowwise_rel {err:.3e} > {1e-6}"
    err = rowwise_rel(c[:, :, -1], nc[:, :, -1])
    assert err <= TOL[dtype], f"rowwise_rel {err:.3e}"


def test_stage_path_bitwise_repeatable(ea):
    """The three-stage path sums states in a fixed order: repeated calls agree bit for bit."""
    cfg = synthetic.WORKLOADS["prefill_bf16_b4h8_n3072_d64"]
    Q, K, V = synthetic.prefill_inputs(cfg, 1)
    Qd, Kd, Vd = to_dev(Q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16")
    B, H, N, D, M = cfg["B"], cfg["H"], cfg["N"], cfg["D"], cfg["M"]
    C, G = 64, 12
    ws = torch.empty(B * H * (G + 1) * (D * M + D) * 4, dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(2):
        out = torch.empty((B, H, N, M), device=DEV)
        ea.segment_states(Kd, Vd, ws, C, G, G - 1)
        ea.segment_scan(ws, B, H, D, M, G, G - 1)
        ea.segment_outputs(Qd, Kd, Vd, out, ws, C, G)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_fused_repeat_on_one_workspace(ea):
    """Consecutive causal calls reuse one workspace (its epoch advances each call); the
    look-back may sum the prefix in a different order, so results agree to rounding."""
    cfg = synthetic.WORKLOADS["prefill_bf16_b4h8_n3072_d64"]
    Q, K, V = synthetic.prefill_inputs(cfg, 1)
    Qd, Kd, Vd = to_dev(Q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16")
    ref = oracle.causal(f64(Q, "bf16"), f64(K, "bf16"), f64(V, "bf16"))[0]
    B, H, N, D, M = cfg["B"], cfg["H"], cfg["N"], cfg["D"], cfg["M"]
    nbytes = max(ea.fused_workspace_bytes(B, H, D, M, 24), ea.fused_workspace_bytes(B, H, D, M, 48))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ea.workspace_init(ws)
    outs = [ea.forward_fused(Qd, Kd, Vd, 64, 24, workspace=ws) for _ in range(4)]
    torch.cuda.synchronize()
    for o in outs:
        err = rowwise_rel(o.cpu().numpy(), ref)
        assert err <= TOL["bf16"], f"{err:.3e}"
    err = rowwise_rel(outs[3].cpu().numpy(), outs[0].cpu().numpy())
    assert err <= 1e-2, f"{err:.3e}"
    # the same memory with another plan, after re-initialisation
    ea.workspace_init(ws)
    outs = [ea.forward_fused(Qd, Kd, Vd, 32, 48, workspace=ws) for _ in range(2)]
    torch.cuda.synchronize()
    for o in outs:
        err = rowwise_rel(o.cpu().numpy(), ref)
        assert err <= TOL["bf16"], f"{err:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk,segments", [(64, 1), (64, 2), (64, 3), (64, 16), (32, 32), (16, 63), (16, 21)])
def test_fused_segments(ea, dtype, chunk, segments):
    """The fused causal kernel over explicit segment counts, with the final state."""
    B, H, N, D, M = 2, 2, 1000, 64, 32
    cfg = small_cfg(dtype, B, H, N, D, M)
    Q, K, V = synthetic.prefill_inputs(cfg, 8)
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    S = torch.full((B, H, D, M), float("nan"), device=DEV)
    z = torch.full((B, H, D), float("nan"), device=DEV)
    out = ea.forward_fused(Qd, Kd, Vd, chunk, segments, S_out=S, z_out=z)
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal(f64(Q, dtype), f64(K, dtype), f64(V, dtype))
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= TOL[dtype], f"out {err:.3e}"
    stol = 1e-5 if dtype == "f32" else TOL["bf16"]
    err = whole_rel(S.cpu().numpy(), S_ref)
    assert err <= stol, f"S {err:.3e}"
    err = whole_rel(z.cpu().numpy(), z_ref)
    assert err <= stol, f"z {err:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", SHAPES)
def test_fused_shapes(ea, dtype, D, M):
    """The two-phase fused kernel (phase A, look-back, phase B) on every shape."""
    cfg = small_cfg(dtype, 1, 2, 300, D, M)
    Q, K, V = synthetic.prefill_inputs(cfg, 12)
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    out = ea.forward_fused(Qd, Kd, Vd, 32, 3)  # 10 chunks: segments of 4, 4, 2
    torch.cuda.synchronize()
    ref = oracle.causal(f64(Q, dtype), f64(K, dtype), f64(V, dtype))[0]
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= TOL[dtype], f"{err:.3e}"


# ---- one-pass kernel (segments of at most four chunks) ----------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", SHAPES)
def test_onepass_shapes(ea, dtype, D, M):
    cfg = small_cfg(dtype, 1, 2, 300, D, M)
    Q, K, V = synthetic.prefill_inputs(cfg, 13)
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    S = torch.full((1, 2, D, M), float("nan"), device=DEV)
    z = torch.full((1, 2, D), float("nan"), device=DEV)
    try:
        out = ea.forward_onepass(Qd, Kd, Vd, 32, 3, S_out=S, z_out=z)  # 10 chunks: segments of 4, 4, 2
    except ea.LinAttnError as e:
        # the planner only picks the one-pass kernel where its LDS fits
        assert e.status == 2 and D > M, str(e)
        pytest.skip("one-pass phi(Q) tiles do not fit in LDS for this shape")
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal(f64(Q, dtype), f64(K, dtype), f64(V, dtype))
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= TOL[dtype], f"out {err:.3e}"
    stol = 1e-5 if dtype == "f32" else TOL["bf16"]
    assert whole_rel(S.cpu().numpy(), S_ref) <= stol
    assert whole_rel(z.cpu().numpy(), z_ref) <= stol


ONEPASS_PLANS = [(1000, 32, 8), (1000, 32, 11), (1000, 32, 16), (1000, 32, 32), (1000, 16, 16), (1000, 16, 63),
                 (100, 32, 1), (97, 16, 2), (1, 16, 1)]
# 64-position chunks: bf16 only (fp32 tiles of 64 rows do not fit twice per CU)
ONEPASS_PLANS_BF16 = [(1000, 64, 4), (1000, 64, 6), (1000, 64, 8), (1000, 64, 16), (200, 64, 1)]


@pytest.mark.parametrize("dtype,N,chunk,segments", [("f32",) + p for p in ONEPASS_PLANS] +
                         [("bf16",) + p for p in ONEPASS_PLANS + ONEPASS_PLANS_BF16])
def test_onepass_segments(ea, dtype, N, chunk, segments):
    """Explicit segment counts (1 to 4 chunks per segment, ragged tails), with the final state."""
    B, H, D, M = 2, 2, 64, 32
    cfg = small_cfg(dtype, B, H, N, D, M)
    Q, K, V = synthetic.prefill_inputs(cfg, 14)
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    S = torch.full((B, H, D, M), float("nan"), device=DEV)
    z = torch.full((B, H, D), float("nan"), device=DEV)
    out = ea.forward_onepass(Qd, Kd, Vd, chunk, segments, S_out=S, z_out=z)
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal(f64(Q, dtype), f64(K, dtype), f64(V, dtype))
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= TOL[dtype], f"out {err:.3e}"
    stol = 1e-5 if dtype == "f32" else TOL["bf16"]
    assert whole_rel(S.cpu().numpy(), S_ref) <= stol
    assert whole_rel(z.cpu().numpy(), z_ref) <= stol


def test_onepass_long_lookback(ea):
    """One chunk per segment, 512 segments per head."""
    B, H, N, D, M = 1, 3, 8192, 32, 32
    cfg = small_cfg("f32", B, H, N, D, M)
    Q, K, V = synthetic.prefill_inputs(cfg, 15)
    Qd, Kd, Vd = to_dev(Q, "f32"), to_dev(K, "f32"), to_dev(V, "f32")
    out = ea.forward_onepass(Qd, Kd, Vd, 16, 512)
    torch.cuda.synchronize()
    ref = oracle.causal(f64(Q, "f32"), f64(K, "f32"), f64(V, "f32"))[0]
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= TOL["f32"], f"{err:.3e}"


def test_onepass_repeat_on_one_workspace(ea):
    """Repeated one-pass calls on one workspace, then the two-phase kernel on the same
    (re-initialised) memory: every result matches the oracle."""
    cfg = synthetic.WORKLOADS["prefill_f32_b8h8_n1024_d64"]
    Q, K, V = synthetic.prefill_inputs(cfg, 2)
    Qd, Kd, Vd = to_dev(Q, "f32"), to_dev(K, "f32"), to_dev(V, "f32")
    ref = oracle.causal(f64(Q, "f32"), f64(K, "f32"), f64(V, "f32"))[0]
    B, H, N, D, M = cfg["B"], cfg["H"], cfg["N"], cfg["D"], cfg["M"]
    ws = torch.empty(ea.fused_workspace_bytes(B, H, D, M, 8), dtype=torch.uint8, device=DEV)
    ea.workspace_init(ws)
    outs = [ea.forward_onepass(Qd, Kd, Vd, 32, 8, workspace=ws) for _ in range(3)]
    ea.workspace_init(ws)
    outs.append(ea.forward_fused(Qd, Kd, Vd, 32, 8, workspace=ws))
    torch.cuda.synchronize()
    for o in outs:
        err = rowwise_rel(o.cpu().numpy(), ref)
        assert err <= TOL["f32"], f"{err:.3e}"


def test_fused_long_lookback(ea):
    """Many short segments per head: long look-back chains."""
    B, H, N, D, M = 1, 3, 8192, 32, 32
    cfg = small_cfg("f32", B, H, N, D, M)
    Q, K, V = synthetic.prefill_inputs(cfg, 9)
    Qd, Kd, Vd = to_dev(Q, "f32"), to_dev(K, "f32"), to_dev(V, "f32")
    out = ea.forward_fused(Qd, Kd, Vd, 16, 512)
    torch.cuda.synchronize()
    ref = oracle.causal(f64(Q, "f32"), f64(K, "f32"), f64(V, "f32"))[0]
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= TOL["f32"], f"{err:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stages_match_oracle(ea, dtype):
    """The three stage kernels run by hand, and the fused default, both against the oracle."""
    from efficient_transformer_amd import linattn as L
    cfg = small_cfg(dtype, 2, 2, 1000, 64, 64)
    Q, K, V = synthetic.prefill_inputs(cfg, 5)
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    C, G = 64, 4
    ws = torch.empty(2 * 2 * (G + 1) * (64 * 64 + 64) * 4, dtype=torch.uint8, device=DEV)
    out = torch.empty((2, 2, 1000, 64), device=DEV)
    ea.segment_states(Kd, Vd, ws, C, G, G - 1)
    ea.segment_scan(ws, 2, 2, 64, 64, G, G - 1)
    ea.segment_outputs(Qd, Kd, Vd, out, ws, C, G)
    fused = ea.forward_chunked(Qd, Kd, Vd)
    torch.cuda.synchronize()
    ref = oracle.causal(f64(Q, dtype), f64(K, dtype), f64(V, dtype))[0]
    for got in (out, fused):
        err = rowwise_rel(got.cpu().numpy(), ref)
        assert err <= TOL[dtype], f"{err:.3e}"


@pytest.mark.parametrize("segments", [1, 2, 3, 4, 6, 16])
def test_segment_counts(ea, segments):
    """Any split of the chunks into segments gives the oracle's result."""
    dtype = "f32"
    cfg = small_cfg(dtype, 1, 3, 1000, 32, 32)
    Q, K, V = synthetic.prefill_inputs(cfg, 6)
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    C = 64
    E = 32 * 32 + 32
    ws = torch.empty(3 * (segments + 1) * E * 4, dtype=torch.uint8, device=DEV)
    out = torch.empty((1, 3, 1000, 32), device=DEV)
    S = torch.empty((1, 3, 32, 32), device=DEV)
    z = torch.empty((1, 3, 32), device=DEV)
    ea.segment_states(Kd, Vd, ws, C, segments, segments)
    ea.segment_scan(ws, 1, 3, 32, 32, segments, segments)
    ea.segment_outputs(Qd, Kd, Vd, out, ws, C, segments, causal=True, S_out=S, z_out=z)
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal(f64(Q, dtype), f64(K, dtype), f64(V, dtype))
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= TOL[dtype], f"rowwise_rel {err:.3e}"
    err = whole_rel(S.cpu().numpy(), S_ref)
    assert err <= 1e-5, f"whole_rel {err:.3e} > {1e-5}"
