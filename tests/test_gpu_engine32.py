"""Parity of the long-head two-phase kernel on 32x32x16 tiles (bf16, D = M = 128, chunk 64)
against the fp64 oracle, through the explicit plan (la_forward_fused), at sizes that reach
every branch of its chunk loops: a ragged last chunk, odd and even chunk counts per segment
(the loops run pairs of chunks), one-chunk segments, one segment advancing its own final
state, a carried initial state and bf16 outputs (page "Transformers are RNNs", Proposed
method: one result from the cumulative sums, whatever the chunking and segmentation)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import TOL, rowwise_rel, to_dev, whole_rel

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
B, H, D, M = 1, 2, 128, 128


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def inputs(N, seed):
    cfg = dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype="bf16", chunk=0)
    Q, K, V = synthetic.prefill_inputs(cfg, seed)
    return (Q, K, V), tuple(to_dev(x, "bf16") for x in (Q, K, V)), tuple(synthetic.as_f64(x, "bf16") for x in (Q, K, V))


def carried_state(n0, seed):
    _, _, (Qf, Kf, Vf) = inputs(n0, seed)
    _, S0, z0 = oracle.causal(Qf, Kf, Vf)
    return S0.astype(np.float32), z0.astype(np.float32)


# N = 1000: 16 chunks, the last one 40 rows.  Segments 1 (one segment of 16 chunks, its
# own final state), 2 (8 + 8), 3 (6 + 6 + 4), 6 (3 x 5 + 1: odd counts and a one-chunk
# segment), 16 (one chunk each).
@pytest.mark.parametrize("segments", [1, 2, 3, 6, 16])
@pytest.mark.parametrize("carry", [False, True])
def test_engine32_segments(ea, segments, carry):
    N = 1000
    print(f"engine32 N={N} segments={segments} carry={carry}", flush=True)
    _, (Qd, Kd, Vd), (Qf, Kf, Vf) = inputs(N, 40 + segments)
    S = torch.full((B, H, D, M), float("nan"), device=DEV)
    z = torch.full((B, H, D), float("nan"), device=DEV)
    if carry:
        S0, z0 = carried_state(150, 7)
        out = ea.forward_fused(Qd, Kd, Vd, 64, segments, S_out=S, z_out=z, S_in=torch.from_numpy(S0).to(DEV),
                               z_in=torch.from_numpy(z0).to(DEV))
        ref, S_ref, z_ref = oracle.causal_from(Qf, Kf, Vf, S0.astype(np.float64), z0.astype(np.float64))
    else:
        out = ea.forward_fused(Qd, Kd, Vd, 64, segments, S_out=S, z_out=z)
        ref, S_ref, z_ref = oracle.causal(Qf, Kf, Vf)
    torch.cuda.synchronize()
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= TOL["bf16"], f"out {err:.3e}"
    assert whole_rel(S.cpu().numpy(), S_ref) <= TOL["bf16"]
    assert whole_rel(z.cpu().numpy(), z_ref) <= TOL["bf16"]


@pytest.mark.parametrize("N,segments", [(64, 1), (65, 2), (127, 2), (320, 5), (449, 4)])
def test_engine32_short(ea, N, segments):
    """Short heads: one chunk, a one-row second chunk, and segment counts next to the chunk count."""
    print(f"engine32 N={N} segments={segments}", flush=True)
    _, (Qd, Kd, Vd), (Qf, Kf, Vf) = inputs(N, N)
    S = torch.full((B, H, D, M), float("nan"), device=DEV)
    z = torch.full((B, H, D), float("nan"), device=DEV)
    out = ea.forward_fused(Qd, Kd, Vd, 64, segments, S_out=S, z_out=z)
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal(Qf, Kf, Vf)
    assert rowwise_rel(out.cpu().numpy(), ref) <= TOL["bf16"]
    assert whole_rel(S.cpu().numpy(), S_ref) <= TOL["bf16"]


@pytest.mark.parametrize("segments", [1, 3, 6])
def test_engine32_bf16_out(ea, segments):
    """bf16 outputs: the rows rounded to bf16 (nearest even), compared at the bf16 tolerance."""
    N = 1000
    print(f"engine32 bf16 out segments={segments}", flush=True)
    _, (Qd, Kd, Vd), (Qf, Kf, Vf) = inputs(N, 90 + segments)
    out = ea.forward_fused(Qd, Kd, Vd, 64, segments, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    ref = oracle.causal(Qf, Kf, Vf)[0]
    assert rowwise_rel(out.float().cpu().numpy(), ref) <= TOL["bf16"]
