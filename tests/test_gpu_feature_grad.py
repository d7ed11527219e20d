"""Gradients through random-feature maps on the GPU against the fp64 oracle.

Two pieces, chained as in training: la_backward_chunked on LA_F32_FEATURES inputs (the
gradients with respect to the features phi(q), phi(k) and to v; page "Transformers are RNNs",
Proposed method: linear-time gradients by running sums) and la_feature_map_backward (the
chain rule through the PRF, TRF and elu maps, with and without row normalisation; page
"Stable, Fast and Accurate: Kernelized Attention with Relative Positional Encoding", Proposed
method).  The oracle's counterparts are pinned by autograd and central differences of its
forward functions.  Errors use the row-wise metric of the other parity tests; the arithmetic
is fp32 throughout, so the fp32 tolerance applies."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from efficient_transformer_amd.features import draw_projection
from gpu_helpers import TOL, rowwise_rel, to_dev

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def features(seed, shape):
    """Positive features with the spread of PRF features (a log-normal draw)."""
    x = synthetic.draw(seed, 11, shape, 0.5, "f32").astype(np.float64)
    return np.exp(x).astype(np.float32)


def check_grads(got, ref, tol):
    """Row-wise on every row.  Rows whose exact value is zero -- dq at position 0 (out_0 = v_0
    whatever q_0 is) and, for a one-position sequence, dk at position 0 -- are held absolutely
    against the scale of the other rows (1 when there are none: the inputs are of order 1)."""
    for name, x, y in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(x)), name
        N = x.shape[2]
        zero = np.zeros(N, dtype=bool)
        if name == "dQ" or (name == "dK" and N == 1):
            zero[0] = True
        if (~zero).any():
            err = rowwise_rel(x[:, :, ~zero], y[:, :, ~zero])
            assert err <= tol, f"{name}: {err:.3e}"
        if zero.any():
            scale = float(np.abs(y[:, :, ~zero]).max()) if (~zero).any() else 1.0
            err0 = float(np.abs(x[:, :, zero]).max()) / scale
            assert err0 <= tol, f"{name} exact-zero rows: {err0:.3e}"


@pytest.mark.parametrize("F,M", [(16, 64), (32, 32), (64, 16), (128, 128), (16, 128)])
@pytest.mark.parametrize("N", [1, 33, 300])
def test_backward_on_features(ea, F, M, N):
    B, H = 1, 2
    Fq, Fk = features(10 + N, (B, H, N, F)), features(20 + N, (B, H, N, F))
    V = synthetic.draw(30 + N, 2, (B, H, N, M), 1.0, "f32")
    dO = synthetic.draw(40 + N, 7, (B, H, N, M), 1.0, "f32")
    Fqd, Fkd, Vd, dOd = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (Fq, Fk, V, dO))
    out = ea.forward_chunked(Fqd, Fkd, Vd, features=True)
    dFq, dFk, dV = ea.backward(Fqd, Fkd, Vd, out, dOd, features=True)
    torch.cuda.synchronize()
    ref = oracle.backward_mapped(Fq, Fk, V, dO)
    check_grads((dFq.cpu().numpy(), dFk.cpu().numpy(), dV.cpu().numpy()), ref, TOL["f32"])


def test_backward_on_features_long(ea):
    """Several segments per head (the forward and reverse segment scans)."""
    B, H, N, F, M = 2, 2, 5000, 16, 64
    Fq, Fk = features(1, (B, H, N, F)), features(2, (B, H, N, F))
    V = synthetic.draw(3, 2, (B, H, N, M), 1.0, "f32")
    dO = synthetic.draw(4, 7, (B, H, N, M), 1.0, "f32")
    Fqd, Fkd, Vd, dOd = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (Fq, Fk, V, dO))
    out = ea.forward_chunked(Fqd, Fkd, Vd, features=True)
    got = [t.cpu().numpy() for t in ea.backward(Fqd, Fkd, Vd, out, dOd, features=True)]
    check_grads(got, oracle.backward_mapped(Fq, Fk, V, dO), TOL["f32"])


def test_elu_features_match_the_elu_backward(ea):
    """Features phi(Q), phi(K) formed by the elu map: the feature gradients times phi' are the
    gradients of the elu path (both on the GPU, within the fp32 tolerance)."""
    B, H, N, D, M = 1, 2, 300, 64, 32
    Q, K, V = synthetic.prefill_inputs(dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype="f32",
                                            chunk=0), 5)
    dO = synthetic.draw(6, 7, (B, H, N, M), 1.0, "f32")
    Qd, Kd, Vd, dOd = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (Q, K, V, dO))
    dQ, dK, dV = ea.backward(Qd, Kd, Vd, ea.forward_chunked(Qd, Kd, Vd), dOd)
    Fq, Fk = ea.feature_map(Qd, None, D, "elu", X2=Kd)
    dFq, dFk, dVf = ea.backward(Fq, Fk, Vd, ea.forward_chunked(Fq, Fk, Vd, features=True), dOd, features=True)
    gq = ea.feature_map_backward(Qd, dFq, None, D, "elu")
    gk = ea.feature_map_backward(Kd, dFk, None, D, "elu")
    torch.cuda.synchronize()
    for name, x, y in (("dQ", gq, dQ), ("dK", gk, dK), ("dV", dVf, dV)):
        x, y = x.cpu().numpy()[:, :, 1:], y.cpu().numpy()[:, :, 1:]
        assert rowwise_rel(x, y) <= TOL["f32"], name


KINDS = [("prf", False), ("prf", True), ("trf", False), ("trf", True), ("elu", False), ("elu", True)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind,normalize", KINDS)
@pytest.mark.parametrize("D,F", [(16, 16), (64, 16), (64, 64), (32, 128), (128, 32), (128, 128)])
def test_feature_map_backward(ea, D, F, kind, normalize, dtype):
    if kind == "elu" and D != F:
        pytest.skip("the elementwise map keeps the width")
    rows = 300
    X = synthetic.draw(50 + D + F, 3, (rows, D), 1.0 / np.sqrt(np.sqrt(D)), dtype)
    X[7] = 0  # a zero row (zero gradient under normalisation)
    P = F if kind != "trf" else F // 2
    W = draw_projection(P, D, "orthogonal", 3) if kind != "elu" else None
    g = synthetic.draw(60 + D + F, 4, (rows, F), 1.0, "f32")
    Xd = to_dev(X, dtype)
    Wd = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).to(DEV) if W is not None else None
    gd = torch.from_numpy(np.ascontiguousarray(g)).to(DEV)
    got = ea.feature_map_backward(Xd, gd, Wd, F, kind, normalize).cpu().numpy()
    Xf = synthetic.as_f64(X, dtype)
    ref = oracle.feature_map_backward(Xf, None if W is None else W.astype(np.float32).astype(np.float64), g, F,
                                      kind, normalize)
    nz = np.abs(ref).max(axis=-1) > 0
    assert np.all(np.isfinite(got))
    assert rowwise_rel(got[nz], ref[nz]) <= 1e-5
    if normalize:
        assert np.all(got[7] == 0.0)


@pytest.mark.parametrize("kind,F,normalize", [("prf", 16, False), ("prf", 32, True), ("trf", 128, True)])
def test_gradient_through_features_end_to_end(ea, kind, F, normalize):
    """dL/dQ, dL/dK, dL/dV of attention on random features of raw rows: GPU feature maps, forward,
    feature backward and map backward against the oracle's fp64 chain.  TRF features take both
    signs, so their denominators are sums that can cancel; with unit rows and 64 projections the
    estimate of exp(q . k) stays within about 15 % and the denominators stay well away from zero
    (with 8 projections of raw rows they do not, and fp32 rounding is amplified accordingly)."""
    B, H, N, D, M = 1, 2, 300, 64, 64
    cfg = dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=D ** -0.25, dtype="f32", chunk=0)
    Q, K, V = synthetic.prefill_inputs(cfg, 8)
    V = synthetic.draw(9, 2, (B, H, N, M), 1.0, "f32")
    dO = synthetic.draw(10, 7, (B, H, N, M), 1.0, "f32")
    P = F if kind == "prf" else F // 2
    W = draw_projection(P, D, "orthogonal", 4)
    Qd, Kd, Vd, dOd = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (Q, K, V, dO))
    Wd = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).to(DEV)
    Fq, Fk = ea.feature_map(Qd, Wd, F, kind, normalize, X2=Kd)
    out = ea.forward_chunked(Fq, Fk, Vd, features=True)
    dFq, dFk, dV = ea.backward(Fq, Fk, Vd, out, dOd, features=True)
    dQ = ea.feature_map_backward(Qd, dFq, Wd, F, kind, normalize)
    dK = ea.feature_map_backward(Kd, dFk, Wd, F, kind, normalize)
    torch.cuda.synchronize()
    W64 = W.astype(np.float32).astype(np.float64)
    Q64, K64 = Q.astype(np.float64), K.astype(np.float64)
    rq, rk = oracle.feature_map(Q64, W64, F, kind, normalize), oracle.feature_map(K64, W64, F, kind, normalize)
    rdFq, rdFk, rdV = oracle.backward_mapped(rq, rk, V, dO)
    rdQ = oracle.feature_map_backward(Q64, W64, rdFq, F, kind, normalize)
    rdK = oracle.feature_map_backward(K64, W64, rdFk, F, kind, normalize)
    check_grads((dQ.cpu().numpy(), dK.cpu().numpy(), dV.cpu().numpy()), (rdQ, rdK, rdV), TOL["f32"])
