"""la_forward_chunked_noalloc (the entry point for callers that cannot allocate) through
the C ABI: its outputs and final states equal la_forward_chunked's on the same inputs, on
two calls in a row with the second smaller, for causal plans with a look-back (two-phase
and one-pass kernels), a non-causal plan and a padded width; a plan beyond the scratch
is refused before anything runs.  The bar is that of the parity tests (row-wise, the
input type's tolerance), and both calls are also held against the fp64 oracle."""
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


def pcfg(dtype, B, H, N, D, M):
    return dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype=dtype, chunk=0)


def both(ea, dtype, B, H, N, D, M, causal, seed, oracle_heads=None):
    Q, K, V = synthetic.prefill_inputs(pcfg(dtype, B, H, N, D, M), seed)
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    out = torch.full((B, H, N, M), float("nan"), device=DEV)
    S = torch.full((B, H, D, M), float("nan"), device=DEV)
    z = torch.full((B, H, D), float("nan"), device=DEV)
    ea.forward_chunked_noalloc(Qd, Kd, Vd, out, causal=causal, S_out=S, z_out=z)
    S2 = torch.empty_like(S)
    z2 = torch.empty_like(z)
    want = ea.forward_chunked(Qd, Kd, Vd, causal=causal, S_out=S2, z_out=z2)
    torch.cuda.synchronize()
    o, w = out.cpu().numpy(), want.cpu().numpy()
    assert rowwise_rel(o, w) <= TOL[dtype]
    stol = 1e-5 if dtype == "f32" else TOL["bf16"]
    assert whole_rel(S.cpu().numpy(), S2.cpu().numpy()) <= stol
    assert whole_rel(z.cpu().numpy(), z2.cpu().numpy()) <= stol
    # and against the oracle (all heads, or the given ones for the long workload)
    hs = slice(None) if oracle_heads is None else oracle_heads
    f = lambda x: synthetic.as_f64(x[:, hs], dtype)
    ref = oracle.causal(f(Q), f(K), f(V))[0] if causal else oracle.noncausal(f(Q), f(K), f(V))
    assert rowwise_rel(o[:, hs], ref) <= TOL[dtype]


def test_noalloc_two_calls_second_smaller(ea):
    # a long-head bf16 call (two-phase kernel, 16 segments per head, about 34 MB of scratch)
    both(ea, "bf16", 1, 16, 65536, 128, 128, True, 0, oracle_heads=[0, 7, 15])
    # then a smaller fp32 call with another plan (one-pass kernel, 8 segments per head)
    both(ea, "f32", 8, 8, 1024, 64, 64, True, 1)


def test_noalloc_other_plans(ea):
    both(ea, "f32", 2, 3, 5000, 64, 32, False, 2)   # non-causal stages
    both(ea, "bf16", 2, 2, 3000, 48, 112, True, 3)  # a padded width (copies in the scratch)
    both(ea, "f32", 1, 1, 64, 16, 16, True, 4)      # one segment: no look-back, no scratch


def test_noalloc_refuses_a_plan_beyond_the_scratch(ea):
    limit = ea.noalloc_scratch_bytes()
    assert limit == 64 << 20
    B, H, N, D, M = 1, 16, 65536, 112, 112  # padded copies of Q, K, V and out: about 1.3 GB
    assert ea.workspace_bytes(B, H, N, D, M, True, 1, 0) > limit
    st = ea.linattn.lib().la_forward_chunked_noalloc(0x10000, 0x10000, 0x10000, 0x10000, B, H, N, D, M, 1, 1, 0,
                                                      None, None, None)
    assert st == ea.linattn.LA_ERR_WORKSPACE
