"""bf16 outputs (dtype LA_BF16 | LA_OUT_BF16) of the prefill entry points: against
the fp64 oracle at the bf16 tolerance, and against the same call with fp32 output
rounded to bf16 (the arithmetic is the same, only the final store differs)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import TOL, rowwise_rel, to_dev

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SHAPES = [(16, 16), (32, 64), (64, 32), (64, 64), (128, 128), (16, 128), (128, 16)]


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def inputs(B, H, N, D, M, seed):
    cfg = dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype="bf16", chunk=0)
    Q, K, V = synthetic.prefill_inputs(cfg, seed)
    return (Q, K, V), tuple(to_dev(x, "bf16") for x in (Q, K, V))


def as_f64(x):
    return synthetic.as_f64(x, "bf16")


def check_rounding(got_bf16, ref_f32):
    """got == ref rounded to nearest even, up to one bf16 ulp (the two calls may sum a
    look-back prefix in a different order)."""
    g = got_bf16.float().cpu().numpy().astype(np.float64)
    r32 = ref_f32.cpu()
    r = r32.to(torch.bfloat16).float().numpy().astype(np.float64)
    ulp = np.abs(r) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(g - r) <= ulp), float(np.max(np.abs(g - r) / ulp))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D,M", SHAPES)
@pytest.mark.parametrize("N", [1, 33, 300])
def test_bf16_output_parity(ea, causal, D, M, N):
    (Q, K, V), (Qd, Kd, Vd) = inputs(1, 3, N, D, M, 70)
    out = ea.forward_chunked(Qd, Kd, Vd, causal=causal, out_dtype=torch.bfloat16)
    ref32 = ea.forward_chunked(Qd, Kd, Vd, causal=causal)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    want = (oracle.causal if causal else oracle.noncausal)(as_f64(Q), as_f64(K), as_f64(V))
    want = want[0] if causal else want
    assert rowwise_rel(out.float().cpu().numpy(), want) <= TOL["bf16"]
    check_rounding(out, ref32)


@pytest.mark.parametrize("segments,chunk", [(4, 64), (12, 16), (32, 16)])
def test_bf16_output_explicit_plans(ea, segments, chunk):
    B, H, N, D, M = 2, 2, 1500, 64, 64
    (Q, K, V), (Qd, Kd, Vd) = inputs(B, H, N, D, M, 71)
    want = oracle.causal(as_f64(Q), as_f64(K), as_f64(V))[0]
    n_chunks = -(-N // chunk)
    cps = -(-n_chunks // segments)
    outs = [ea.forward_fused(Qd, Kd, Vd, chunk, segments, out_dtype=torch.bfloat16)]
    if cps <= 4:
        outs.append(ea.forward_onepass(Qd, Kd, Vd, chunk, segments, out_dtype=torch.bfloat16))
    torch.cuda.synchronize()
    for o in outs:
        assert rowwise_rel(o.float().cpu().numpy(), want) <= TOL["bf16"]


def test_bf16_output_continue_and_state(ea):
    """Continuation with bf16 outputs: the final state stays fp32 and equals the fp32-output call's."""
    B, H, n0, n1, D, M = 2, 2, 200, 300, 64, 64
    (Q, K, V), (Qd, Kd, Vd) = inputs(B, H, n0 + n1, D, M, 72)
    S0 = torch.empty((B, H, D, M), device=DEV)
    z0 = torch.empty((B, H, D), device=DEV)
    ea.forward_chunked(Qd[:, :, :n0].contiguous(), Kd[:, :, :n0].contiguous(), Vd[:, :, :n0].contiguous(),
                       S_out=S0, z_out=z0)
    S1, z1 = torch.empty_like(S0), torch.empty_like(z0)
    S2, z2 = torch.empty_like(S0), torch.empty_like(z0)
    rest = [x[:, :, n0:].contiguous() for x in (Qd, Kd, Vd)]
    o16 = ea.forward_continue(*rest, S0, z0, S_out=S1, z_out=z1, out_dtype=torch.bfloat16)
    o32 = ea.forward_continue(*rest, S0, z0, S_out=S2, z_out=z2)
    torch.cuda.synchronize()
    want = oracle.causal(as_f64(Q), as_f64(K), as_f64(V))[0][:, :, n0:]
    assert rowwise_rel(o16.float().cpu().numpy(), want) <= TOL["bf16"]
    check_rounding(o16, o32)
    assert torch.allclose(S1, S2, rtol=1e-6, atol=0) and torch.allclose(z1, z2, rtol=1e-6, atol=0)


def test_bf16_output_stage_path(ea):
    """la_segment_outputs with a bf16 output after fp32 segment states."""
    B, H, N, D, M, C, G = 1, 2, 640, 64, 32, 32, 4
    (Q, K, V), (Qd, Kd, Vd) = inputs(B, H, N, D, M, 73)
    E = D * M + D
    ws = torch.zeros(B * H * (G + 1) * E, device=DEV)
    ea.segment_states(Kd, Vd, ws, C, G, G)
    ea.segment_scan(ws, B, H, D, M, G, G)
    out = torch.empty((B, H, N, M), dtype=torch.bfloat16, device=DEV)
    ea.segment_outputs(Qd, Kd, Vd, out, ws, C, G, causal=False)
    torch.cuda.synchronize()
    want = oracle.noncausal(as_f64(Q), as_f64(K), as_f64(V))
    assert rowwise_rel(out.float().cpu().numpy(), want) <= TOL["bf16"]


def test_bf16_output_workload(ea):
    """The bf16 image workload (B=4, H=8, N=3072, D=M=64) with bf16 outputs: every row
    within the bf16 tolerance of the fp32-output call and within one ulp of its rounding."""
    cfg = synthetic.WORKLOADS["prefill_bf16_b4h8_n3072_d64"]
    Q, K, V = synthetic.prefill_inputs(cfg, 0)
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    o16 = ea.forward_chunked(Qd, Kd, Vd, out_dtype=torch.bfloat16)
    o32 = ea.forward_chunked(Qd, Kd, Vd)
    torch.cuda.synchronize()
    check_rounding(o16, o32)
    want = oracle.causal(as_f64(Q[:1, :2]), as_f64(K[:1, :2]), as_f64(V[:1, :2]))[0]
    assert rowwise_rel(o16[:1, :2].float().cpu().numpy(), want) <= TOL["bf16"]
