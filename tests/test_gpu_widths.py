"""Widths without a kernel of their own (D or M of 48, 80, 96, 112) through the C ABI,
against the fp64 oracle (page "Transformers are RNNs", Proposed method: the
similarity is phi(q)^T phi(k) for feature vectors of any length).

Prefill and continuation run on copies padded to the next kernel width (Q, K
columns -inf so that phi maps them to 0, V columns 0); decode runs one generic
kernel.  Each case is held to the tolerance of its input type in the row-wise
metric, and the final states as in the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import TOL, rowwise_rel, to_dev, whole_rel

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
WIDTHS = [(48, 48), (112, 112), (48, 112), (80, 96), (96, 16), (16, 80), (128, 48), (48, 128)]


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def pcfg(dtype, B, H, N, D, M):
    return dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype=dtype, chunk=0)


def f64(x, dtype):
    return synthetic.as_f64(x, dtype)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 33, 300])
@pytest.mark.parametrize("D,M", WIDTHS)
def test_prefill_widths(ea, D, M, N, dtype, causal):
    B, H = 2, 3
    Q, K, V = synthetic.prefill_inputs(pcfg(dtype, B, H, N, D, M), 40 + D + M + N)
    S = torch.full((B, H, D, M), float("nan"), device=DEV)
    z = torch.full((B, H, D), float("nan"), device=DEV)
    out = ea.forward_chunked(to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype), causal=causal,
                             S_out=S, z_out=z)
    torch.cuda.synchronize()
    Qf, Kf, Vf = f64(Q, dtype), f64(K, dtype), f64(V, dtype)
    if causal:
        ref, S_ref, z_ref = oracle.causal(Qf, Kf, Vf)
    else:
        ref = oracle.noncausal(Qf, Kf, Vf)
        _, S_ref, z_ref = oracle.causal(Qf, Kf, Vf)  # the final sums are those of the whole sequence
    assert tuple(out.shape) == (B, H, N, M)
    err = rowwise_rel(out.cpu().numpy(), ref)
    assert err <= TOL[dtype], f"out {err:.3e}"
    stol = 1e-5 if dtype == "f32" else TOL["bf16"]
    assert whole_rel(S.cpu().numpy(), S_ref) <= stol
    assert whole_rel(z.cpu().numpy(), z_ref) <= stol


@pytest.mark.parametrize("D,M", [(48, 48), (112, 80)])
def test_prefill_widths_explicit_chunks_and_long_heads(ea, D, M):
    """Every chunk length, and a head long enough for several segments (two-phase kernel)."""
    for N, chunks in ((300, (16, 32, 64)), (20000, (0,))):
        B, H = 1, 2
        Q, K, V = synthetic.prefill_inputs(pcfg("f32", B, H, N, D, M), 7)
        ref, _, _ = oracle.causal(Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64))
        for c in chunks:
            out = ea.forward_chunked(to_dev(Q, "f32"), to_dev(K, "f32"), to_dev(V, "f32"), chunk=c)
            torch.cuda.synchronize()
            err = rowwise_rel(out.cpu().numpy(), ref)
            assert err <= TOL["f32"], f"N {N} chunk {c}: {err:.3e}"


@pytest.mark.parametrize("D,M", [(48, 48), (80, 112)])
def test_prefill_widths_bf16_out(ea, D, M):
    B, H, N = 2, 2, 129
    Q, K, V = synthetic.prefill_inputs(pcfg("bf16", B, H, N, D, M), 9)
    out = ea.forward_chunked(to_dev(Q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16"), out_dtype=torch.bfloat16)
    o32 = ea.forward_chunked(to_dev(Q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16"))
    torch.cuda.synchronize()
    ref, _, _ = oracle.causal(f64(Q, "bf16"), f64(K, "bf16"), f64(V, "bf16"))
    assert out.dtype == torch.bfloat16
    assert rowwise_rel(out.float().cpu().numpy(), ref) <= TOL["bf16"]
    assert torch.equal(out, o32.to(torch.bfloat16))  # the fp32 result rounded to nearest even


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(48, 48), (112, 96), (16, 112)])
def test_continue_widths(ea, D, M, dtype):
    """A sequence in two pieces, the second continued in place from the state of the first."""
    B, H, N0, N1 = 1, 3, 77, 300
    Q, K, V = synthetic.prefill_inputs(pcfg(dtype, B, H, N0 + N1, D, M), 11)
    dev = [to_dev(x, dtype) for x in (Q, K, V)]
    S = torch.empty((B, H, D, M), device=DEV)
    z = torch.empty((B, H, D), device=DEV)
    ea.forward_chunked(*(x[:, :, :N0].contiguous() for x in dev), S_out=S, z_out=z)
    out = ea.forward_continue(*(x[:, :, N0:].contiguous() for x in dev), S, z, S_out=S, z_out=z)
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal(f64(Q, dtype), f64(K, dtype), f64(V, dtype))
    assert rowwise_rel(out.cpu().numpy(), ref[:, :, N0:]) <= TOL[dtype]
    stol = 1e-5 if dtype == "f32" else TOL["bf16"]
    assert whole_rel(S.cpu().numpy(), S_ref) <= stol
    assert whole_rel(z.cpu().numpy(), z_ref) <= stol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", WIDTHS)
def test_decode_widths(ea, D, M, dtype):
    """A prefill's final state continued by single steps and by one multi-token call."""
    B, H, N0, T = 2, 5, 40, 12
    Q, K, V = synthetic.prefill_inputs(pcfg(dtype, B, H, N0 + 2 * T, D, M), 13 + D)
    dev = [to_dev(x, dtype) for x in (Q, K, V)]
    S = torch.empty((B, H, D, M), device=DEV)
    z = torch.empty((B, H, D), device=DEV)
    ea.forward_chunked(*(x[:, :, :N0].contiguous() for x in dev), S_out=S, z_out=z)
    outs = [ea.decode_step(S, z, *(x[:, :, N0 + t].contiguous() for x in dev)) for t in range(T)]
    out_steps = ea.decode_steps(S, z, *(x[:, :, N0 + T:].contiguous() for x in dev))
    torch.cuda.synchronize()
    ref, S_ref, z_ref = oracle.causal(f64(Q, dtype), f64(K, dtype), f64(V, dtype))
    got = torch.stack(outs, dim=2).cpu().numpy()
    assert rowwise_rel(got, ref[:, :, N0:N0 + T]) <= TOL[dtype]
    assert rowwise_rel(out_steps.cpu().numpy(), ref[:, :, N0 + T:]) <= TOL[dtype]
    stol = 1e-5 if dtype == "f32" else TOL["bf16"]
    assert whole_rel(S.cpu().numpy(), S_ref) <= stol
    assert whole_rel(z.cpu().numpy(), z_ref) <= stol


def test_decode_widths_from_zero(ea):
    """From an empty history (zero state) the first step returns v itself."""
    B, H, D, M = 3, 4, 80, 48
    q = torch.randn(B, H, D, device=DEV)
    k = torch.randn(B, H, D, device=DEV)
    v = torch.randn(B, H, M, device=DEV)
    S = torch.zeros(B, H, D, M, device=DEV)
    z = torch.zeros(B, H, D, device=DEV)
    out = ea.decode_step(S, z, q, k, v)
    torch.cuda.synchronize()
    assert torch.allclose(out, v, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("D,M", [(48, 48), (96, 112)])
def test_feature_inputs_widths(ea, D, M):
    """Inputs that already hold features are padded with zeros (no map)."""
    B, H, N = 1, 2, 200
    rng = np.random.default_rng(3)
    Fq = rng.uniform(0.1, 2.0, (B, H, N, D)).astype(np.float32)
    Fk = rng.uniform(0.1, 2.0, (B, H, N, D)).astype(np.float32)
    V = rng.standard_normal((B, H, N, M)).astype(np.float32)
    out = ea.forward_chunked(*(torch.from_numpy(x).to(DEV) for x in (Fq, Fk, V)), features=True)
    torch.cuda.synchronize()
    ref, _, _ = oracle.attention_mapped(Fq.astype(np.float64), Fk.astype(np.float64), V.astype(np.float64))
    assert rowwise_rel(out.cpu().numpy(), ref) <= TOL["f32"]
