"""Seeded random shapes through the prefill, continuation and multi-token decode entry
points, against the fp64 oracle (page "Transformers are RNNs", Proposed method: one
result from the cumulative sums, whatever the chunking and segmentation).

Each case draws the batch, heads, length (1 .. 700, lengths next to chunk and segment
boundaries favoured), widths (multiples of 16 up to 128, padded widths included), input
type, causal or not, the chunk (planner's choice, 16, 32 or 64) and whether the call
continues from a carried state.  The draw is fixed by the case number, so every run
checks the same cases; each is held to the tolerance of its input type in the row-wise
metric, and the final states as in the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import TOL, rowwise_rel, to_dev, whole_rel

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NCASES = 160


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def draw_case(i):
    r = np.random.default_rng(1000 + i)
    B, H = int(r.integers(1, 4)), int(r.integers(1, 5))
    if r.random() < 0.4:  # next to a chunk or segment boundary
        N = max(1, int(r.choice([16, 32, 64, 128, 256])) * int(r.integers(1, 4)) + int(r.integers(-1, 2)))
    else:
        N = int(r.integers(1, 701))
    D, M = 16 * int(r.integers(1, 9)), 16 * int(r.integers(1, 9))
    dtype = str(r.choice(["f32", "bf16"]))
    causal = bool(r.random() < 0.75)
    carry = causal and bool(r.random() < 0.4)
    chunk = int(r.choice([0, 16, 32, 64]))
    n0 = int(r.integers(1, 200))
    return B, H, N, D, M, dtype, causal, carry, chunk, n0


def pcfg(dtype, B, H, N, D, M):
    return dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype=dtype, chunk=0)


@pytest.mark.parametrize("case", range(NCASES))
def test_random_shape(ea, case):
    from efficient_transformer_amd import linattn as L
    B, H, N, D, M, dtype, causal, carry, chunk, n0 = draw_case(case)
    code = L.LA_F32 if dtype == "f32" else L.LA_BF16
    try:
        ea.forward_plan(B, H, N, D, M, causal, code, chunk)
    except L.LinAttnError:
        chunk = 0  # that chunk has no kernel at these widths: the planner's choice instead
    print(f"case {case}: B={B} H={H} N={N} D={D} M={M} {dtype} causal={causal} carry={carry} chunk={chunk}",
          flush=True)
    Q, K, V = synthetic.prefill_inputs(pcfg(dtype, B, H, N, D, M), 500 + case)
    Qf, Kf, Vf = (synthetic.as_f64(x, dtype) for x in (Q, K, V))
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    S = torch.full((B, H, D, M), float("nan"), device=DEV)
    z = torch.full((B, H, D), float("nan"), device=DEV)
    S0 = z0 = None
    if carry:  # the state a real prefix of n0 positions leaves
        P = synthetic.prefill_inputs(pcfg("f32", B, H, n0, D, M), 900 + case)
        _, S0, z0 = oracle.causal(*P)
        S0, z0 = S0.astype(np.float32), z0.astype(np.float32)
        out = ea.forward_continue(Qd, Kd, Vd, torch.from_numpy(S0).to(DEV), torch.from_numpy(z0).to(DEV),
                                  chunk=chunk, S_out=S, z_out=z)
        ref, S_ref, z_ref = oracle.causal_from(Qf, Kf, Vf, S0.astype(np.float64), z0.astype(np.float64))
    elif causal:
        out = ea.forward_chunked(Qd, Kd, Vd, causal=True, chunk=chunk, S_out=S, z_out=z)
        ref, S_ref, z_ref = oracle.causal(Qf, Kf, Vf)
    else:
        out = ea.forward_chunked(Qd, Kd, Vd, causal=False, chunk=chunk, S_out=S, z_out=z)
        ref = oracle.noncausal(Qf, Kf, Vf)
        _, S_ref, z_ref = oracle.causal(Qf, Kf, Vf)  # the final sums are those of the whole sequence
    torch.cuda.synchronize()
    assert tuple(out.shape) == (B, H, N, M)
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= TOL[dtype], f"out {err:.3e}"
    stol = 1e-5 if dtype == "f32" else TOL["bf16"]
    assert whole_rel(S.cpu().numpy(), S_ref) <= stol
    assert whole_rel(z.cpu().numpy(), z_ref) <= stol
    if causal and N <= 80:
        # the same positions as recurrent steps in one call, from the same state (fp32
        # arithmetic for both input types)
        Sd = torch.from_numpy(S0).to(DEV) if carry else torch.zeros((B, H, D, M), device=DEV)
        zd = torch.from_numpy(z0).to(DEV) if carry else torch.zeros((B, H, D), device=DEV)
        steps = ea.decode_steps(Sd, zd, Qd, Kd, Vd)
        torch.cuda.synchronize()
        assert rowwise_rel(steps.cpu().numpy(), ref) <= TOL["f32"]
        assert whole_rel(Sd.cpu().numpy(), S_ref) <= 1e-5
        assert whole_rel(zd.cpu().numpy(), z_ref) <= 1e-5
