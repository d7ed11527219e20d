"""Continuing a sequence from a carried state: la_forward_continue (both causal
kernels), the explicit-plan entry points with S_in, and la_decode_steps, all
against the fp64 oracle's continued running sums (page "Transformers are RNNs",
Proposed method: the causal model is an RNN whose memories S and z carry every
earlier position)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import TOL, rowwise_rel, to_dev, whole_rel

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SHAPES = [(16, 16), (32, 64), (64, 32), (64, 64), (128, 128), (16, 128), (128, 16)]


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def pcfg(dtype, B, H, N, D, M):
    return dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype=dtype, chunk=0)


def carried_state(B, H, D, M, n0, seed):
    """The state a real prefix of n0 positions leaves (fp64 oracle, then fp32 for the GPU)."""
    cfg = pcfg("f32", B, H, n0, D, M)
    Q, K, V = synthetic.prefill_inputs(cfg, seed)
    _, S, z = oracle.causal(Q, K, V)
    return S.astype(np.float32), z.astype(np.float32)


def check(out, S, z, ref, S_ref, z_ref, dtype):
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= TOL[dtype], f"out {err:.3e}"
    stol = 1e-5 if dtype == "f32" else TOL["bf16"]
    assert whole_rel(S.cpu().numpy(), S_ref) <= stol
    assert whole_rel(z.cpu().numpy(), z_ref) <= stol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", SHAPES)
def test_continue_parity(ea, dtype, D, M):
    B, H, N = 1, 3, 300
    S0, z0 = carried_state(B, H, D, M, 77, 21)
    Q, K, V = synthetic.prefill_inputs(pcfg(dtype, B, H, N, D, M), 22)
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    Sin, zin = torch.from_numpy(S0).to(DEV), torch.from_numpy(z0).to(DEV)
    S = torch.full((B, H, D, M), float("nan"), device=DEV)
    z = torch.full((B, H, D), float("nan"), device=DEV)
    out = ea.forward_continue(Qd, Kd, Vd, Sin, zin, S_out=S, z_out=z)
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal_from(synthetic.as_f64(Q, dtype), synthetic.as_f64(K, dtype),
                                           synthetic.as_f64(V, dtype), S0.astype(np.float64), z0.astype(np.float64))
    check(out, S, z, ref, S_ref, z_ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kernel,chunk,segments", [("onepass", 32, 3), ("onepass", 16, 19), ("onepass", 32, 1),
                                                   ("fused", 32, 3), ("fused", 16, 7), ("fused", 64, 1)])
def test_explicit_plans_with_initial_state(ea, dtype, kernel, chunk, segments):
    B, H, N, D, M = 2, 2, 300, 64, 32
    if kernel == "onepass" and segments == 1:
        N = 100  # a single segment of at most four chunks
    S0, z0 = carried_state(B, H, D, M, 50, 23)
    Q, K, V = synthetic.prefill_inputs(pcfg(dtype, B, H, N, D, M), 24)
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    Sin, zin = torch.from_numpy(S0).to(DEV), torch.from_numpy(z0).to(DEV)
    S = torch.full((B, H, D, M), float("nan"), device=DEV)
    z = torch.full((B, H, D), float("nan"), device=DEV)
    fn = ea.forward_onepass if kernel == "onepass" else ea.forward_fused
    out = fn(Qd, Kd, Vd, chunk, segments, S_out=S, z_out=z, S_in=Sin, z_in=zin)
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal_from(synthetic.as_f64(Q, dtype), synthetic.as_f64(K, dtype),
                                           synthetic.as_f64(V, dtype), S0.astype(np.float64), z0.astype(np.float64))
    check(out, S, z, ref, S_ref, z_ref, dtype)


def test_continue_long_two_phase_in_place(ea):
    """Enough positions that the planner takes the two-phase kernel (segments of more
    than four chunks); the state is updated in place (S_out is S_in)."""
    B, H, N, D, M = 2, 8, 8192, 64, 32
    S0, z0 = carried_state(B, H, D, M, 500, 25)
    Q, K, V = synthetic.prefill_inputs(pcfg("f32", B, H, N, D, M), 26)
    Qd, Kd, Vd = to_dev(Q, "f32"), to_dev(K, "f32"), to_dev(V, "f32")
    C, G, _ = ea.forward_plan(B, H, N, D, M, True, 0, 0)
    n_chunks = -(-N // C)
    assert -(-n_chunks // G) > 4, "expected the two-phase kernel's plan"
    S = torch.from_numpy(S0).to(DEV)
    z = torch.from_numpy(z0).to(DEV)
    out = ea.forward_continue(Qd, Kd, Vd, S, z, S_out=S, z_out=z)
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal_from(Q, K, V, S0.astype(np.float64), z0.astype(np.float64))
    check(out, S, z, ref, S_ref, z_ref, "f32")


def test_prefill_in_pieces(ea):
    """A sequence prefilled in three pieces equals the one-call prefill."""
    B, H, N, D, M = 2, 2, 900, 64, 64
    Q, K, V = synthetic.prefill_inputs(pcfg("f32", B, H, N, D, M), 27)
    Qd, Kd, Vd = to_dev(Q, "f32"), to_dev(K, "f32"), to_dev(V, "f32")
    whole = ea.forward_chunked(Qd, Kd, Vd)
    S = torch.zeros((B, H, D, M), device=DEV)
    z = torch.zeros((B, H, D), device=DEV)
    parts = []
    for a, b in ((0, 250), (250, 251), (251, 900)):
        sl = lambda t: t[:, :, a:b].contiguous()
        parts.append(ea.forward_continue(sl(Qd), sl(Kd), sl(Vd), S, z, S_out=S, z_out=z))
    torch.cuda.synchronize()
    got = torch.cat(parts, dim=2).cpu().numpy()
    ref = oracle.causal(Q, K, V)[0]
    assert rowwise_rel(got, ref) <= TOL["f32"]
    assert rowwise_rel(got, whole.cpu().numpy()) <= 1e-5


def test_continue_empty_copies_the_state(ea):
    B, H, D, M = 1, 2, 32, 16
    S0, z0 = carried_state(B, H, D, M, 10, 28)
    Sin, zin = torch.from_numpy(S0).to(DEV), torch.from_numpy(z0).to(DEV)
    Q = torch.empty((B, H, 0, D), device=DEV)
    V = torch.empty((B, H, 0, M), device=DEV)
    S = torch.full((B, H, D, M), float("nan"), device=DEV)
    z = torch.full((B, H, D), float("nan"), device=DEV)
    ea.forward_continue(Q, Q, V, Sin, zin, S_out=S, z_out=z)
    torch.cuda.synchronize()
    assert torch.equal(S, Sin) and torch.equal(z, zin)


# ---- several recurrent steps per call ----------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", SHAPES)
@pytest.mark.parametrize("T", [1, 5, 16, 17, 40])
def test_decode_steps_parity(ea, dtype, D, M, T):
    B, H = 3, 2
    S0, z0 = carried_state(B, H, D, M, 30, 29)
    q, k, v = synthetic.prefill_inputs(pcfg(dtype, B, H, T, D, M), 30)
    S = torch.from_numpy(S0).to(DEV)
    z = torch.from_numpy(z0).to(DEV)
    out = ea.decode_steps(S, z, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype))
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal_from(synthetic.as_f64(q, dtype), synthetic.as_f64(k, dtype),
                                           synthetic.as_f64(v, dtype), S0.astype(np.float64), z0.astype(np.float64))
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= 1e-4, f"out {err:.3e}"  # fp32 state and arithmetic for both input types
    assert whole_rel(S.cpu().numpy(), S_ref) <= 1e-5
    assert whole_rel(z.cpu().numpy(), z_ref) <= 1e-5


@pytest.mark.parametrize("dtype,D,M,T", [("f32", 64, 64, 12), ("f32", 64, 64, 33), ("f32", 128, 128, 12),
                                         ("f32", 16, 128, 16), ("f32", 32, 32, 16), ("f32", 16, 16, 32),
                                         ("f32", 128, 64, 40), ("bf16", 64, 64, 16)])
def test_decode_steps_chunked_path(ea, dtype, D, M, T):
    """512 heads: one segment per head, so fp32 calls of 12+ tokens run the chunked
    kernel with the state carried in and out in place (bf16 inputs stay on the fp32
    register recurrence)."""
    B, H = 64, 8
    S0, z0 = carried_state(B, H, D, M, 20, 32)
    q, k, v = synthetic.prefill_inputs(pcfg(dtype, B, H, T, D, M), 33)
    S = torch.from_numpy(S0).to(DEV)
    z = torch.from_numpy(z0).to(DEV)
    out = ea.decode_steps(S, z, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype))
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal_from(synthetic.as_f64(q, dtype), synthetic.as_f64(k, dtype),
                                           synthetic.as_f64(v, dtype), S0.astype(np.float64), z0.astype(np.float64))
    assert rowwise_rel(out.cpu().numpy(), ref) <= 1e-4
    assert whole_rel(S.cpu().numpy(), S_ref) <= 1e-5
    assert whole_rel(z.cpu().numpy(), z_ref) <= 1e-5


def test_decode_steps_equals_single_steps(ea):
    """T steps in one call and T calls of la_decode_step agree to rounding."""
    B, H, D, M, T = 4, 2, 64, 64, 33
    q, k, v = synthetic.prefill_inputs(pcfg("f32", B, H, T, D, M), 31)
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    S1 = torch.zeros((B, H, D, M), device=DEV)
    z1 = torch.zeros((B, H, D), device=DEV)
    S2, z2 = S1.clone(), z1.clone()
    many = ea.decode_steps(S1, z1, qd, kd, vd)
    single = torch.stack([ea.decode_step(S2, z2, qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                         vd[:, :, t].contiguous()) for t in range(T)], dim=2)
    torch.cuda.synchronize()
    assert rowwise_rel(many.cpu().numpy(), single.cpu().numpy()) <= 1e-5
    assert whole_rel(S1.cpu().numpy(), S2.cpu().numpy()) <= 1e-6


def test_decode_steps_empty_is_a_no_op(ea):
    S = torch.ones((1, 1, 16, 16), device=DEV)
    z = torch.ones((1, 1, 16), device=DEV)
    q = torch.empty((1, 1, 0, 16), device=DEV)
    out = ea.decode_steps(S, z, q, q, q)
    torch.cuda.synchronize()
    assert out.shape == (1, 1, 0, 16)
    assert torch.all(S == 1) and torch.all(z == 1)
