"""Parity of the HIP backward (la_backward_chunked) with the fp64 oracle's
gradients (page "Transformers are RNNs", Proposed method: linear-time gradients
by running sums).  The GPU forward's output is fed to the GPU backward, as in
training; the oracle recomputes everything in fp64."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import TOL, to_dev

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


def run(ea, dtype, B, H, N, D, M, seed):
    Q, K, V = synthetic.prefill_inputs(pcfg(dtype, B, H, N, D, M), seed)
    dO = synthetic.draw(seed + 1000, 7, (B, H, N, M), 1.0, "f32")
    Qd, Kd, Vd = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    dOd = torch.from_numpy(np.ascontiguousarray(dO)).to(DEV)
    out = ea.forward_chunked(Qd, Kd, Vd)
    dQ, dK, dV = ea.backward(Qd, Kd, Vd, out, dOd)
    torch.cuda.synchronize()
    ref = oracle.causal_backward(synthetic.as_f64(Q, dtype), synthetic.as_f64(K, dtype),
                                 synthetic.as_f64(V, dtype), dO.astype(np.float64))
    return (dQ.cpu().numpy(), dK.cpu().numpy(), dV.cpu().numpy()), ref


def check(got, ref, tol):
    """The row-wise metric on every (b, h, i) row of dQ, dK and dV: max over rows of
    max_m |x - y| / max_m |y|.  Rows whose exact value is zero are held absolutely
    against the tensor's scale instead (max |x| <= tol * max |y|): dq at position 0
    (out_0 = v_0 whatever q_0 is) and, for a one-position sequence, dk at position 0."""
    N = got[0].shape[2]
    for name, x, y in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(x)), name
        zero = np.zeros(N, dtype=bool)
        if name == "dQ" or (name == "dK" and N == 1):
            zero[0] = True
        if (~zero).any():
            num = np.abs(x - y)[:, :, ~zero].max(axis=-1)
            den = np.abs(y)[:, :, ~zero].max(axis=-1)
            err = float((num / den).max())
            assert err <= tol, f"{name} row-wise relative error {err:.3e} > {tol}"
        if zero.any():
            scale = max(float(np.abs(y).max()), 1e-30) if (~zero).any() else 1.0
            err0 = float(np.abs(x[:, :, zero]).max() / scale)
            assert err0 <= tol, f"{name} exact-zero rows: {err0:.3e} > {tol}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", SHAPES)
@pytest.mark.parametrize("N", [1, 33, 300])
def test_backward_parity(ea, dtype, D, M, N):
    got, ref = run(ea, dtype, 1, 2, N, D, M, 40)
    # fp32 arithmetic throughout; bf16 inputs carry the bf16 forward output's error into c_i
    check(got, ref, 1e-4 if dtype == "f32" else TOL["bf16"])


def test_backward_first_row_has_no_query_gradient(ea):
    """out_0 = v_0 whatever q_0 and k_0 are: dq_0 vanishes up to fp32 rounding
    (r_0 . v_0 + c_0 cancels)."""
    got, _ = run(ea, "f32", 1, 2, 50, 64, 64, 41)
    dq = got[0]
    assert np.max(np.abs(dq[:, :, 0])) <= 1e-5 * np.max(np.abs(dq))


def test_backward_value_gradients_sum_to_output_gradients(ea):
    B, H, N, D, M = 2, 2, 200, 32, 64
    Q, K, V = synthetic.prefill_inputs(pcfg("f32", B, H, N, D, M), 42)
    dO = synthetic.draw(42, 7, (B, H, N, M), 1.0, "f32")
    Qd, Kd, Vd = to_dev(Q, "f32"), to_dev(K, "f32"), to_dev(V, "f32")
    dOd = torch.from_numpy(np.ascontiguousarray(dO)).to(DEV)
    out = ea.forward_chunked(Qd, Kd, Vd)
    _, _, dV = ea.backward(Qd, Kd, Vd, out, dOd)
    torch.cuda.synchronize()
    s = dV.double().sum(dim=2).cpu().numpy()
    assert np.max(np.abs(s - dO.astype(np.float64).sum(axis=2))) <= 1e-3 * np.max(np.abs(s))


def test_backward_headline_shape(ea):
    """B=8 H=8 N=1024 D=M=64 fp32 (many segments per head)."""
    got, ref = run(ea, "f32", 8, 8, 1024, 64, 64, 43)
    check(got, ref, 1e-4)


def test_backward_long_sequence(ea):
    """N=8192 with D=M=128 bf16: long reverse and forward segment scans."""
    got, ref = run(ea, "bf16", 1, 2, 8192, 128, 128, 44)
    check(got, ref, TOL["bf16"])


def test_backward_repeatable(ea):
    """The backward uses no atomics or look-back: bitwise repeatable."""
    B, H, N, D, M = 2, 3, 700, 64, 64
    Q, K, V = synthetic.prefill_inputs(pcfg("f32", B, H, N, D, M), 45)
    dO = synthetic.draw(45, 7, (B, H, N, M), 1.0, "f32")
    Qd, Kd, Vd = to_dev(Q, "f32"), to_dev(K, "f32"), to_dev(V, "f32")
    dOd = torch.from_numpy(np.ascontiguousarray(dO)).to(DEV)
    out = ea.forward_chunked(Qd, Kd, Vd)
    a = ea.backward(Qd, Kd, Vd, out, dOd)
    b = ea.backward(Qd, Kd, Vd, out, dOd)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
