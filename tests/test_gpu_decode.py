"""Parity of the HIP recurrent decode step (la_decode_step) with the fp64 oracle,
and its equivalence with the parallel mode (page "Transformers are RNNs",
Proposed method: the causal model is an RNN with memories S and z)."""
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


def dcfg(dtype, B, H, D, M, sigma=1.0):
    return dict(kind="decode", B=B, H=H, D=D, M=M, sigma=sigma, dtype=dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(16, 16), (64, 64), (32, 128), (128, 32), (128, 128), (64, 128), (128, 64)])
def test_decode_parity(ea, dtype, D, M):
    cfg = dcfg(dtype, 3, 2, D, M)
    T = 40
    q, k, v = synthetic.decode_inputs(cfg, 0, 0, T)
    S = torch.zeros((3, 2, D, M), device=DEV)
    z = torch.zeros((3, 2, D), device=DEV)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    outs = [ea.decode_step(S, z, qd[t], kd[t], vd[t]) for t in range(T)]
    torch.cuda.synchronize()
    got = torch.stack(outs).cpu().numpy()
    So = np.zeros((3, 2, D, M))
    zo = np.zeros((3, 2, D))
    ref = np.stack([oracle.decode_step(So, zo, synthetic.as_f64(q[t], dtype), synthetic.as_f64(k[t], dtype),
                                       synthetic.as_f64(v[t], dtype)) for t in range(T)])
    err = rowwise_rel(got, ref)
    assert err <= 1e-4, f"rowwise_rel {err:.3e}"  # fp32 state and arithmetic for both input types
    err = whole_rel(S.cpu().numpy(), So)
    assert err <= 1e-5, f"whole_rel {err:.3e} > {1e-5}"
    err = whole_rel(z.cpu().numpy(), zo)
    assert err <= 1e-5, f"whole_rel {err:.3e} > {1e-5}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_equals_prefill(ea, dtype):
    """Decode step t reproduces causal prefill row t; the states agree at the end."""
    B, H, N, D, M = 2, 3, 150, 64, 64
    cfg = dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype=dtype)
    Q, K, V = synthetic.prefill_inputs(cfg, 9)
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    Sp = torch.empty((B, H, D, M), device=DEV)
    zp = torch.empty((B, H, D), device=DEV)
    pre = ea.forward_chunked(Qd, Kd, Vd, S_out=Sp, z_out=zp)
    S = torch.zeros((B, H, D, M), device=DEV)
    z = torch.zeros((B, H, D), device=DEV)
    dec = torch.stack([ea.decode_step(S, z, Qd[:, :, t].contiguous(), Kd[:, :, t].contiguous(),
                                      Vd[:, :, t].contiguous()) for t in range(N)], dim=2)
    torch.cuda.synchronize()
    # the bf16 prefill rounds its MFMA operands (phi(K), phi(Q), A, S) to bf16; decode keeps fp32
    tol = 1e-4 if dtype == "f32" else TOL["bf16"]
    stol = 1e-5 if dtype == "f32" else TOL["bf16"]
    err = rowwise_rel(dec.cpu().numpy(), pre.cpu().numpy())
    assert err <= tol, f"rowwise_rel {err:.3e} > {tol}"
    err = whole_rel(S.cpu().numpy(), Sp.cpu().numpy())
    assert err <= stol, f"whole_rel {err:.3e} > {stol}"
    err = whole_rel(z.cpu().numpy(), zp.cpu().numpy())
    assert err <= stol, f"whole_rel {err:.3e} > {stol}"


def test_prefill_then_decode_continues_the_sequence(ea):
    """State handed from the parallel mode to the recurrent mode continues exactly."""
    B, H, N, D, M, T = 1, 4, 500, 64, 64, 20
    cfg = dict(kind="prefill", B=B, H=H, N=N + T, D=D, M=M, sigma=1.0, dtype="f32")
    Q, K, V = synthetic.prefill_inputs(cfg, 10)
    S = torch.empty((B, H, D, M), device=DEV)
    z = torch.empty((B, H, D), device=DEV)
    Qd, Kd, Vd = to_dev(Q, "f32"), to_dev(K, "f32"), to_dev(V, "f32")
    ea.forward_chunked(Qd[:, :, :N].contiguous(), Kd[:, :, :N].contiguous(), Vd[:, :, :N].contiguous(),
                       S_out=S, z_out=z)
    outs = [ea.decode_step(S, z, Qd[:, :, N + t].contiguous(), Kd[:, :, N + t].contiguous(),
                           Vd[:, :, N + t].contiguous()) for t in range(T)]
    torch.cuda.synchronize()
    got = torch.stack(outs, dim=2).cpu().numpy()
    ref, _, _ = oracle.causal(synthetic.as_f64(Q, "f32"), synthetic.as_f64(K, "f32"), synthetic.as_f64(V, "f32"))
    err = rowwise_rel(got, ref[:, :, N:])
    assert err <= 1e-4, f"rowwise_rel {err:.3e} > {1e-4}"


def test_decode_resume_is_bitwise(ea):
    """The state is the whole history: a copy to host and back resumes bit for bit."""
    cfg = dcfg("f32", 4, 2, 64, 64)
    T, t0 = 30, 11
    q, k, v = synthetic.decode_inputs(cfg, 1, 0, T)
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    S = torch.zeros((4, 2, 64, 64), device=DEV)
    z = torch.zeros((4, 2, 64), device=DEV)
    full = [ea.decode_step(S, z, qd[t], kd[t], vd[t]) for t in range(T)]
    S2 = torch.zeros_like(S)
    z2 = torch.zeros_like(z)
    for t in range(t0):
        ea.decode_step(S2, z2, qd[t], kd[t], vd[t])
    torch.cuda.synchronize()
    S_host, z_host = S2.cpu().clone(), z2.cpu().clone()
    S3, z3 = S_host.to(DEV), z_host.to(DEV)
    rest = [ea.decode_step(S3, z3, qd[t], kd[t], vd[t]) for t in range(t0, T)]
    torch.cuda.synchronize()
    for a, b in zip(full[t0:], rest):
        assert torch.equal(a, b)
    assert torch.equal(S, S3) and torch.equal(z, z3)


def test_decode_256x8_t4096_full(ea):
    """Full decode workload (256 streams x 8 heads, D=M=64, 4096 steps from a zero state):
    every head's output at every step, and every head's final state, against the oracle's
    recurrence (fp64), in blocks of 256 steps."""
    cfg = synthetic.WORKLOADS["decode_f32_256x8_t4096_d64"]
    B, H, D, M, T = cfg["B"], cfg["H"], cfg["D"], cfg["M"], cfg["T"]
    BH = B * H
    S = torch.zeros((B, H, D, M), device=DEV)
    z = torch.zeros((B, H, D), device=DEV)
    block = 256
    hist = torch.empty((block, B, H, M), device=DEV)
    So = np.zeros((BH, D, M))
    zo = np.zeros((BH, D))
    worst = 0.0
    for t0 in range(0, T, block):
        q, k, v = synthetic.decode_inputs(cfg, 0, t0, t0 + block)
        qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
        for i in range(block):
            ea.decode_step(S, z, qd[i], kd[i], vd[i], out=hist[i])
        torch.cuda.synchronize()
        got = hist.view(block, BH, M).cpu().numpy()
        q, k, v = (x.reshape(block, BH, -1).astype(np.float64) for x in (q, k, v))
        for i in range(block):
            ref = oracle.decode_step(So, zo, q[i], k[i], v[i])
            err = rowwise_rel(got[i], ref)
            worst = max(worst, err)
            assert err <= TOL["f32"], f"step {t0 + i}: {err:.3e}"
    print(f"256x8 t4096 all heads, every step: row-wise rel err {worst:.3e}")
    assert whole_rel(S.view(BH, D, M).cpu().numpy(), So) <= 1e-5
    assert whole_rel(z.view(BH, D).cpu().numpy(), zo) <= 1e-5
