"""Projection matrices of the random-feature maps (host-side set-up, page "Stable,
Fast and Accurate: Kernelized Attention with Relative Positional Encoding": PRF,
ORF, Sphere-PRF), checked against what the mathematics fixes: orthogonal rows in
blocks of D, row lengths, and unbiasedness of the orthogonal estimator of
exp(q . k) (computed with the fp64 oracle's feature map)."""
import numpy as np

import oracle
from efficient_transformer_amd.features import draw_projection


def test_gaussian_rows():
    W = draw_projection(4096, 8, "gaussian", 1)
    assert W.shape == (4096, 8) and W.dtype == np.float32
    assert abs(W.mean()) < 0.02 and abs(W.var() - 1.0) < 0.03


def test_orthogonal_blocks():
    D = 16
    W = draw_projection(40, D, "orthogonal", 2).astype(np.float64)
    for b0 in range(0, 40, D):
        blk = W[b0:b0 + D]
        G = blk @ blk.T
        off = G - np.diag(np.diag(G))
        assert np.max(np.abs(off)) <= 1e-5 * np.max(np.diag(G))
    # lengths of N(0, I_D) vectors: E|w|^2 = D
    lengths2 = (draw_projection(4096, D, "orthogonal", 3).astype(np.float64) ** 2).sum(1)
    assert abs(lengths2.mean() / D - 1.0) < 0.03


def test_sphere_rows():
    D = 32
    W = draw_projection(100, D, "sphere", 4).astype(np.float64)
    assert np.allclose(np.linalg.norm(W, axis=1), np.sqrt(D), rtol=1e-6)


def test_orthogonal_estimator_is_unbiased():
    D = 4
    q = np.array([0.3, -0.2, 0.5, 0.1])
    k = np.array([-0.4, 0.1, 0.2, 0.3])
    est = []
    for seed in range(3000):
        W = draw_projection(D, D, "orthogonal", seed).astype(np.float64)
        fq = oracle.feature_map(q[None], W, D, "prf")
        fk = oracle.feature_map(k[None], W, D, "prf")
        est.append(float(fq[0] @ fk[0]))
    est = np.array(est)
    want = np.exp(q @ k)
    assert abs(est.mean() - want) <= 5 * est.std() / np.sqrt(est.size)


def test_rows_are_c_contiguous():
    for kind in ("gaussian", "orthogonal", "sphere"):
        assert draw_projection(40, 16, kind, 0).flags.c_contiguous
