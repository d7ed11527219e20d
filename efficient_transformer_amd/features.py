"""Projection matrices W of the random-feature maps (host-side set-up, drawn once).

Page "Stable, Fast and Accurate: Kernelized Attention with Relative Positional
Encoding", Proposed method and Main findings: kernelized attention with the
feature maps PRF, TRF, Sphere-PRF and ORF.  The maps themselves run on the GPU
(feature_map, la_feature_map); they differ only in how the rows of W are drawn:

  "gaussian"    rows w ~ N(0, I_D)                     (PRF, TRF)
  "orthogonal"  blocks of D mutually orthogonal rows, each row rescaled to the
                length of an independent N(0, I_D) vector, so every row is still
                N(0, I_D) on its own                    (ORF)
  "sphere"      directions uniform on the sphere, every row of length sqrt(D)
                                                        (Sphere-PRF)

W is a parameter of the layer, drawn once (or redrawn between training steps),
not part of the per-token work.
"""
from __future__ import annotations

import numpy as np

KINDS = ("gaussian", "orthogonal", "sphere")


def draw_projection(rows: int, D: int, kind: str = "gaussian", seed: int = 0) -> np.ndarray:
    """W [rows, D] float32; rows = F for PRF, F / 2 for TRF."""
    if kind not in KINDS:
        raise ValueError(f"kind must be one of {KINDS}")
    rng = np.random.default_rng(seed)
    if kind == "gaussian":
        return np.ascontiguousarray(rng.standard_normal((rows, D)), dtype=np.float32)
    if kind == "sphere":
        G = rng.standard_normal((rows, D))
        return np.ascontiguousarray(G / np.linalg.norm(G, axis=1, keepdims=True) * np.sqrt(D), dtype=np.float32)
    blocks = []
    for _ in range((rows + D - 1) // D):
        Qm, R = np.linalg.qr(rng.standard_normal((D, D)))
        Qm = Qm * np.sign(np.diag(R))[None, :]  # a uniformly random orthogonal matrix
        blocks.append(Qm.T)                      # its rows are orthonormal
    W = np.concatenate(blocks, axis=0)[:rows]
    lengths = np.linalg.norm(rng.standard_normal((rows, D)), axis=1)
    return np.ascontiguousarray(W * lengths[:, None], dtype=np.float32)
