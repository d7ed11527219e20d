"""Softmax attention as an RNN (la_softmax_scan, la_softmax_step) against the fp64
oracle (page "Attention as an RNN", Proposed method: many-to-many outputs of the
attention RNN by a prefix scan; one learned query per head)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import rowwise_rel, to_dev, whole_rel

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SHAPES = [(16, 16), (32, 64), (64, 32), (64, 64), (128, 128), (16, 128), (128, 16)]
TOL = 1e-4  # fp32 arithmetic on exactly represented inputs, for both input types


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def inputs(dtype, B, H, N, D, M, seed, qscale=1.0):
    cfg = dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype=dtype)
    _, K, V = synthetic.prefill_inputs(cfg, seed)
    q = synthetic.draw(seed, 9, (B, H, D), qscale, dtype)
    return q, K, V


def run(ea, dtype, B, H, N, D, M, seed, qscale=1.0, with_state=False):
    q, K, V = inputs(dtype, B, H, N, D, M, seed, qscale)
    st = None
    if with_state:
        st = (torch.full((B, H), float("nan"), device=DEV), torch.full((B, H), float("nan"), device=DEV),
              torch.full((B, H, M), float("nan"), device=DEV))
    out = ea.softmax_scan(to_dev(q, dtype), to_dev(K, dtype), to_dev(V, dtype),
                          m_out=st[0] if st else None, u_out=st[1] if st else None, w_out=st[2] if st else None)
    torch.cuda.synchronize()
    ref = oracle.softmax_scan(synthetic.as_f64(q, dtype), synthetic.as_f64(K, dtype), synthetic.as_f64(V, dtype))
    return out.cpu().numpy(), ref, st


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", SHAPES)
@pytest.mark.parametrize("N", [1, 31, 33, 128, 129, 300])
def test_softmax_scan_parity(ea, dtype, D, M, N):
    got, ref, _ = run(ea, dtype, 2, 2, N, D, M, 60)
    err = rowwise_rel(got, ref[0])
    assert err <= TOL, f"{err:.3e}"


@pytest.mark.parametrize("qscale", [0.0, 4.0, 40.0])
def test_softmax_scan_score_range(ea, qscale):
    """q = 0 (uniform weights: prefix means) up to scores of several hundred (beyond exp's range)."""
    got, ref, _ = run(ea, "f32", 1, 3, 1000, 64, 64, 61, qscale)
    assert np.all(np.isfinite(got))
    err = rowwise_rel(got, ref[0])
    assert err <= TOL, f"{err:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_softmax_scan_final_state(ea, dtype):
    got, ref, st = run(ea, dtype, 2, 3, 777, 64, 128, 62, with_state=True)
    _, m, u, w = ref
    mg, ug, wg = (x.cpu().numpy() for x in st)
    assert np.max(np.abs(mg - m)) <= 1e-5 * max(1.0, np.max(np.abs(m)))
    # u and w share the scale exp(-m): compare w / u (the last output) and u itself
    assert whole_rel(ug, u) <= 1e-4
    assert whole_rel(wg, w) <= 1e-4


def test_softmax_scan_long_lookback(ea):
    """512 groups of 128 rows per head (look-back beyond 64 groups)."""
    got, ref, _ = run(ea, "f32", 1, 2, 65536, 32, 64, 63, 2.0)
    err = rowwise_rel(got, ref[0])
    assert err <= TOL, f"{err:.3e}"


def test_softmax_scan_workspace_reuse(ea):
    q, K, V = inputs("f32", 4, 8, 3000, 64, 64, 64)
    qd, Kd, Vd = to_dev(q, "f32"), to_dev(K, "f32"), to_dev(V, "f32")
    ws = torch.empty(int(ea.linattn.lib().la_softmax_scan_workspace_bytes(4, 8, 3000, 64, 64)), dtype=torch.uint8,
                     device=DEV)
    ea.workspace_init(ws)
    outs = [ea.softmax_scan(qd, Kd, Vd, workspace=ws) for _ in range(4)]
    torch.cuda.synchronize()
    ref = oracle.softmax_scan(q, K, V)[0]
    for o in outs:
        assert rowwise_rel(o.cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(16, 16), (64, 64), (128, 128), (32, 128)])
def test_softmax_step_matches_scan_and_continues_it(ea, dtype, D, M):
    """Token-by-token steps reproduce the scan; a scan's final state continued by steps
    gives the rows of the longer sequence."""
    B, H, N, n1 = 2, 3, 40, 25
    q, K, V = inputs(dtype, B, H, N, D, M, 65)
    qd, Kd, Vd = to_dev(q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    ref = oracle.softmax_scan(synthetic.as_f64(q, dtype), synthetic.as_f64(K, dtype), synthetic.as_f64(V, dtype))[0]
    m = torch.full((B, H), float("-inf"), device=DEV)
    u = torch.zeros((B, H), device=DEV)
    w = torch.zeros((B, H, M), device=DEV)
    steps = torch.stack([ea.softmax_step(m, u, w, qd, Kd[:, :, t].contiguous(), Vd[:, :, t].contiguous())
                         for t in range(N)], dim=2)
    # scan of the first n1 positions, then steps for the rest
    m2 = torch.empty((B, H), device=DEV)
    u2 = torch.empty((B, H), device=DEV)
    w2 = torch.empty((B, H, M), device=DEV)
    ea.softmax_scan(qd, Kd[:, :, :n1].contiguous(), Vd[:, :, :n1].contiguous(), m_out=m2, u_out=u2, w_out=w2)
    rest = torch.stack([ea.softmax_step(m2, u2, w2, qd, Kd[:, :, t].contiguous(), Vd[:, :, t].contiguous())
                        for t in range(n1, N)], dim=2)
    torch.cuda.synchronize()
    assert rowwise_rel(steps.cpu().numpy(), ref) <= TOL
    assert rowwise_rel(rest.cpu().numpy(), ref[:, :, n1:]) <= TOL
