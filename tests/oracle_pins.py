"""Pins of the fp64 oracle against facts outside it.

Helpers, not a test module: `run_all(o)` runs every pin against an oracle build
`o` (oracle.Oracle) and returns the list of failures.  tests/test_oracle.py runs
it on the real build (no failure allowed) and on deliberately broken copies of
oracle.c (each must be caught), so that the pins are known to bite.

What pins what (page: "Transformers are RNNs", Katharopoulos et al. 2020):
  * golden/*.json  -- hand-derived exact values (phi, causal, non-causal, state,
                      decode), D != M so that a transposed state shows;
  * brute force    -- the quadratic masked form tril(phi(Q) phi(K)^T) V,
                      row-normalised, in numpy (Proposed method: the
                      associativity rewrite leaves this result unchanged);
  * mpmath         -- the definition at 50 digits on tiny inputs;
  * invariants     -- V = 1 gives 1; out_0 = v_0; causal last row = non-causal
                      row; affine equivariance in V; outputs in the convex hull
                      of the visible values; no dependence on future positions or
                      on other queries; key-order invariance of the non-causal form;
  * RNN form       -- decode steps reproduce causal rows and the final state
                      (Proposed method: the causal model is an RNN with memories S, z);
  * chunked algebra -- a blockwise fp64 evaluation (the form the GPU kernels
                      use) agrees with the recurrence for chunk 1, 3, 16 and N.
"""
from __future__ import annotations

import glob
import json
import os
import re

import mpmath
import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def np_phi(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def brute_causal(Q, K, V):
    """Quadratic masked form for one head: W = tril(phi(Q) phi(K)^T); out = W V / W 1."""
    W = np.tril(np_phi(Q) @ np_phi(K).T)
    return (W @ V) / W.sum(axis=1, keepdims=True)


def brute_noncausal(Q, K, V):
    W = np_phi(Q) @ np_phi(K).T
    return (W @ V) / W.sum(axis=1, keepdims=True)


def chunked_causal(Q, K, V, C):
    """Blockwise evaluation: intra-chunk masked quadratic term plus the state of earlier chunks."""
    N, D = Q.shape
    M = V.shape[1]
    FQ, FK = np_phi(Q), np_phi(K)
    S = np.zeros((D, M))
    z = np.zeros(D)
    out = np.empty((N, M))
    for c0 in range(0, N, C):
        c1 = min(N, c0 + C)
        A = np.tril(FQ[c0:c1] @ FK[c0:c1].T)
        num = A @ V[c0:c1] + FQ[c0:c1] @ S
        den = A.sum(axis=1) + FQ[c0:c1] @ z
        out[c0:c1] = num / den[:, None]
        S = S + FK[c0:c1].T @ V[c0:c1]
        z = z + FK[c0:c1].sum(axis=0)
    return out, S, z


_NUM = re.compile(r"(?<![A-Za-z_])(\d+\.?\d*(?:[eE][-+]?\d+)?)")


def _mp_eval(expr: str):
    """Evaluate an exact expression (numbers, + - * /, exp) at 50 digits."""
    mpmath.mp.dps = 50
    src = _NUM.sub(lambda m: f"mpf('{m.group(1)}')", expr)
    return eval(src, {"__builtins__": {}, "exp": mpmath.exp, "mpf": mpmath.mpf}, {})


def _expect(arr):
    return np.array([[float(_mp_eval(e)) for e in row] for row in arr]) if isinstance(arr[0], list) \
        else np.array([float(_mp_eval(e)) for e in arr])


def _close(name, got, want, rtol, fails):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if got.shape != want.shape:
        fails.append(f"{name}: shape {got.shape} != {want.shape}")
        return
    if not np.all(np.isfinite(got)):
        fails.append(f"{name}: non-finite values")
        return
    err = np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-300)) if got.size else 0.0
    # absolute floor for exact zeros
    abs_err = np.max(np.abs(got - want)) if got.size else 0.0
    if not (err <= rtol or abs_err <= rtol * 1e-3):
        fails.append(f"{name}: max rel err {err:.3e} > {rtol:.1e}")


def pin_golden(o, fails):
    with open(os.path.join(GOLDEN, "phi_values.json")) as f:
        g = json.load(f)
    xs = np.array([float(a) for a, _ in g["cases"]])
    want = np.array([float(_mp_eval(b)) for _, b in g["cases"]])
    _close("golden phi (vector)", o.phi(xs), want, 1e-15, fails)
    _close("golden phi (scalar)", [o.L.oracle_phi1(float(x)) for x in xs], want, 1e-15, fails)
    for path in sorted(glob.glob(os.path.join(GOLDEN, "causal_*.json"))):
        name = os.path.basename(path)
        with open(path) as f:
            g = json.load(f)
        Q, K, V = (np.array(g[k], dtype=np.float64) for k in ("Q", "K", "V"))
        out, S, z = o.causal(Q[None], K[None], V[None])
        _close(f"{name} causal", out[0], _expect(g["causal"]), 1e-14, fails)
        _close(f"{name} state S", S[0], _expect(g["S"]), 1e-14, fails)
        _close(f"{name} state z", z[0], _expect(g["z"]), 1e-14, fails)
        rows = o.causal_rows(Q, K, V, np.arange(Q.shape[0]))
        _close(f"{name} causal_rows", rows, _expect(g["causal"]), 1e-14, fails)
        _close(f"{name} noncausal", o.noncausal(Q[None], K[None], V[None])[0],
               _expect(g["noncausal"]), 1e-14, fails)
        D, M = K.shape[1], V.shape[1]
        Sd = np.zeros((1, D, M))
        zd = np.zeros((1, D))
        outs = [o.decode_step(Sd, zd, Q[i][None], K[i][None], V[i][None])[0] for i in range(Q.shape[0])]
        _close(f"{name} decode outputs", np.array(outs), _expect(g["causal"]), 1e-14, fails)
        _close(f"{name} decode state S", Sd[0], _expect(g["S"]), 1e-14, fails)
        _close(f"{name} decode state z", zd[0], _expect(g["z"]), 1e-14, fails)


def _rand(rng, N, D, M, scale=1.0):
    return (rng.normal(size=(N, D)) * scale, rng.normal(size=(N, D)) * scale, rng.normal(size=(N, M)))


SHAPES = [(1, 1, 1), (2, 1, 3), (3, 2, 1), (7, 3, 2), (16, 16, 3), (64, 3, 16), (33, 16, 16), (64, 2, 5)]


def pin_bruteforce(o, fails):
    rng = np.random.default_rng(1234)
    for (N, D, M) in SHAPES:
        for scale in (0.5, 1.0, 3.0):
            Q, K, V = _rand(rng, N, D, M, scale)
            want = brute_causal(Q, K, V)
            out, S, z = o.causal(Q[None], K[None], V[None])
            _close(f"brute causal N{N} D{D} M{M} s{scale}", out[0], want, 1e-11, fails)
            _close(f"brute causal_rows N{N} D{D} M{M} s{scale}",
                   o.causal_rows(Q, K, V, np.arange(N)), want, 1e-11, fails)
            _close(f"brute noncausal N{N} D{D} M{M} s{scale}",
                   o.noncausal(Q[None], K[None], V[None])[0], brute_noncausal(Q, K, V), 1e-11, fails)
            _close(f"brute final S N{N} D{D} M{M}", S[0], np_phi(K).T @ V, 1e-11, fails)
            _close(f"brute final z N{N} D{D} M{M}", z[0], np_phi(K).sum(axis=0), 1e-12, fails)
    # several heads at once: each head independent of the others
    Q = rng.normal(size=(3, 2, 9, 4))
    K = rng.normal(size=(3, 2, 9, 4))
    V = rng.normal(size=(3, 2, 9, 5))
    out, _, _ = o.causal(Q, K, V)
    for b in range(3):
        for h in range(2):
            _close(f"brute multihead b{b} h{h}", out[b, h], brute_causal(Q[b, h], K[b, h], V[b, h]), 1e-11, fails)


def pin_mpmath(o, fails):
    mpmath.mp.dps = 50
    rng = np.random.default_rng(99)
    for (N, D, M) in [(1, 1, 1), (4, 2, 3), (6, 3, 2), (8, 1, 2)]:
        Q, K, V = _rand(rng, N, D, M, 2.0)

        def ph(x):
            x = mpmath.mpf(float(x))
            return x + 1 if x > 0 else mpmath.exp(x)

        want = np.zeros((N, M))
        for i in range(N):
            num = [mpmath.mpf(0)] * M
            den = mpmath.mpf(0)
            for j in range(i + 1):
                w = mpmath.fsum(ph(Q[i, d]) * ph(K[j, d]) for d in range(D))
                den += w
                for m in range(M):
                    num[m] += w * mpmath.mpf(float(V[j, m]))
            for m in range(M):
                want[i, m] = float(num[m] / den)
        out, _, _ = o.causal(Q[None], K[None], V[None])
        err = np.max(np.abs(out[0] - want) / np.maximum(np.abs(want).max(axis=1, keepdims=True), 1e-300))
        if not err <= 1e-13:
            fails.append(f"mpmath N{N} D{D} M{M}: row-relative err {err:.3e} > 1e-13")


def pin_invariants(o, fails):
    rng = np.random.default_rng(7)
    for (N, D, M) in [(13, 4, 6), (40, 8, 3), (64, 16, 16)]:
        Q, K, V = _rand(rng, N, D, M, 1.5)
        out, S, z = o.causal(Q[None], K[None], V[None])
        out = out[0]
        ones = o.causal(Q[None], K[None], np.ones((1, N, M)))[0][0]
        if not np.max(np.abs(ones - 1.0)) <= 1e-14:
            fails.append(f"ones invariant N{N}: {np.max(np.abs(ones - 1.0)):.3e}")
        nc_ones = o.noncausal(Q[None], K[None], np.ones((1, N, M)))[0]
        if not np.max(np.abs(nc_ones - 1.0)) <= 1e-14:
            fails.append(f"non-causal ones invariant N{N}")
        _close(f"first row N{N}", out[0], V[0], 1e-14, fails)
        nc = o.noncausal(Q[None], K[None], V[None])[0]
        _close(f"last row causal=noncausal N{N}", out[-1], nc[-1], 1e-12, fails)
        a, c = -2.5, rng.normal(size=M)
        aff = o.causal(Q[None], K[None], (a * V + c)[None])[0][0]
        _close(f"affine equivariance N{N}", aff, a * out + c, 1e-11, fails)
        lo = np.minimum.accumulate(V, axis=0)
        hi = np.maximum.accumulate(V, axis=0)
        if not (np.all(out >= lo - 1e-12) and np.all(out <= hi + 1e-12)):
            fails.append(f"convex hull N{N}")
        # causality: changing positions after i leaves rows <= i unchanged
        i = N // 2
        Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
        Q2[i + 1:] += 1.0
        K2[i + 1:] -= 0.7
        V2[i + 1:] *= 3.0
        out2 = o.causal(Q2[None], K2[None], V2[None])[0][0]
        if not np.array_equal(out2[: i + 1], out[: i + 1]):
            fails.append(f"causality N{N}")
        if np.allclose(out2[i + 1:], out[i + 1:]):
            fails.append(f"future positions ignored entirely N{N}")
        # row i depends on q only through q_i
        Q3 = Q.copy()
        Q3[:i] += 0.9
        out3 = o.causal(Q3[None], K[None], V[None])[0][0]
        if not np.array_equal(out3[i:], out[i:]):
            fails.append(f"query locality N{N}")
        # non-causal: order of keys does not matter, query order permutes rows
        perm = rng.permutation(N)
        ncp = o.noncausal(Q[None], K[perm][None], V[perm][None])[0]
        _close(f"non-causal key permutation N{N}", ncp, nc, 1e-12, fails)
        ncq = o.noncausal(Q[perm][None], K[None], V[None])[0]
        _close(f"non-causal query permutation N{N}", ncq, nc[perm], 1e-12, fails)


def pin_rnn(o, fails):
    rng = np.random.default_rng(5)
    for (BH, N, D, M) in [(3, 20, 4, 6), (2, 50, 16, 8)]:
        Q = rng.normal(size=(BH, N, D))
        K = rng.normal(size=(BH, N, D))
        V = rng.normal(size=(BH, N, M))
        out, S, z = o.causal(Q, K, V)
        Sd = np.zeros((BH, D, M))
        zd = np.zeros((BH, D))
        dec = np.stack([o.decode_step(Sd, zd, Q[:, t], K[:, t], V[:, t]) for t in range(N)], axis=1)
        _close(f"decode == causal rows BH{BH} N{N}", dec, out, 1e-12, fails)
        _close(f"decode state == causal state BH{BH} N{N}", Sd, S, 1e-12, fails)
        _close(f"decode z == causal z BH{BH} N{N}", zd, z, 1e-12, fails)
        # resume from a copied state (the state is the whole history)
        t0 = N // 3
        S1 = np.zeros((BH, D, M))
        z1 = np.zeros((BH, D))
        for t in range(t0):
            o.decode_step(S1, z1, Q[:, t], K[:, t], V[:, t])
        S2, z2 = S1.copy(), z1.copy()
        res = np.stack([o.decode_step(S2, z2, Q[:, t], K[:, t], V[:, t]) for t in range(t0, N)], axis=1)
        _close(f"decode resume BH{BH}", res, out[:, t0:], 1e-12, fails)


def pin_chunked(o, fails):
    rng = np.random.default_rng(11)
    for (N, D, M) in [(64, 8, 5), (100, 16, 16)]:
        Q, K, V = _rand(rng, N, D, M)
        out, S, z = o.causal(Q[None], K[None], V[None])
        for C in (1, 3, 16, N):
            co, cS, cz = chunked_causal(Q, K, V, C)
            _close(f"chunked C{C} N{N}", co, out[0], 1e-12, fails)
            _close(f"chunked state C{C} N{N}", cS, S[0], 1e-12, fails)


def pin_continue(o, fails):
    """A sequence cut in two: the second part continued from the state of the first
    (computed here with numpy, phi(K1)^T V1 and the column sums of phi(K1)) gives the
    rows of the whole sequence, checked against the quadratic masked form."""
    rng = np.random.default_rng(17)
    for (N, n1, D, M) in [(9, 4, 3, 2), (30, 1, 2, 5), (40, 25, 16, 3), (20, 19, 4, 4)]:
        Q, K, V = _rand(rng, N, D, M)
        want = brute_causal(Q, K, V)
        S0 = np_phi(K[:n1]).T @ V[:n1]
        z0 = np_phi(K[:n1]).sum(axis=0)
        out, S, z = o.causal_from(Q[None, n1:], K[None, n1:], V[None, n1:], S0[None], z0[None])
        _close(f"continue rows N{N} n1={n1}", out[0], want[n1:], 1e-11, fails)
        _close(f"continue final S N{N} n1={n1}", S[0], np_phi(K).T @ V, 1e-11, fails)
        _close(f"continue final z N{N} n1={n1}", z[0], np_phi(K).sum(axis=0), 1e-12, fails)
        # from the zero state it is plain causal attention
        zo = o.causal_from(Q[None], K[None], V[None], np.zeros((1, D, M)), np.zeros((1, D)))[0]
        _close(f"continue from zero N{N}", zo[0], want, 1e-11, fails)


def pin_backward(o, fails):
    """Gradients against (a) fp64 autograd through the quadratic masked form (torch CPU),
    (b) central finite differences of the oracle's forward, (c) closed forms: the value
    gradients sum to the output gradients (outputs are convex combinations of values),
    and row 0 does not depend on q_0 (out_0 = v_0)."""
    import torch
    rng = np.random.default_rng(41)

    def quad(Qt, Kt, Vt):
        ph = lambda x: torch.where(x > 0, x + 1, torch.exp(x))
        W = torch.tril(ph(Qt) @ ph(Kt).T)
        return (W @ Vt) / W.sum(dim=1, keepdim=True)

    for (N, D, M) in [(1, 2, 3), (5, 3, 2), (16, 4, 7), (33, 16, 16)]:
        for scale in (0.5, 2.0):
            Q, K, V = _rand(rng, N, D, M, scale)
            dO = rng.normal(size=(N, M))
            dQ, dK, dV = o.causal_backward(Q[None], K[None], V[None], dO[None])
            Qt, Kt, Vt = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V)]
            (quad(Qt, Kt, Vt) * torch.tensor(dO)).sum().backward()
            for nm, got, want in (("dQ", dQ[0], Qt.grad.numpy()), ("dK", dK[0], Kt.grad.numpy()),
                                  ("dV", dV[0], Vt.grad.numpy())):
                err = np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-3)  # exact zeros at N = 1
                if not err <= 1e-11:
                    fails.append(f"backward autograd {nm} N{N} D{D} M{M} s{scale}: {err:.3e}")
            _close(f"backward sum dV N{N}", dV[0].sum(axis=0), dO.sum(axis=0), 1e-11, fails)
            if not np.max(np.abs(dQ[0, 0])) <= 1e-12:
                fails.append(f"backward dq_0 != 0 N{N}")
    # central differences of the forward on a tiny case
    N, D, M = 6, 3, 4
    Q, K, V = _rand(rng, N, D, M, 1.0)
    dO = rng.normal(size=(N, M))
    dQ, dK, dV = o.causal_backward(Q[None], K[None], V[None], dO[None])
    loss = lambda Q_, K_, V_: float(np.sum(o.causal(Q_[None], K_[None], V_[None])[0][0] * dO))
    h = 1e-6
    for nm, X, G in (("Q", Q, dQ[0]), ("K", K, dK[0]), ("V", V, dV[0])):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = [Q, K, V]
            args_m = [Q, K, V]
            pos = "QKV".index(nm)
            args_p[pos], args_m[pos] = Xp, Xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.max(np.abs(num - G)) / max(np.max(np.abs(G)), 1e-300)
        if not err <= 1e-6:
            fails.append(f"backward finite differences d{nm}: {err:.3e}")


def pin_softmax_scan(o, fails):
    """Softmax attention of one query over every prefix: against scipy's softmax on each
    prefix (library routine), 50-digit mpmath, closed forms (V = 1; q = 0 gives prefix means;
    out_0 = v_0; the final state), scores far beyond exp's range, and the one-token RNN."""
    from scipy.special import softmax as sp_softmax
    rng = np.random.default_rng(51)
    for (N, D, M, scale) in [(1, 3, 2, 1.0), (9, 4, 3, 1.0), (40, 16, 5, 3.0), (33, 8, 8, 30.0)]:
        q = rng.normal(size=D) * scale
        K = rng.normal(size=(N, D))
        V = rng.normal(size=(N, M))
        out, m, u, w = o.softmax_scan(q[None], K[None], V[None])
        sc = K @ q
        want = np.stack([sp_softmax(sc[:k + 1]) @ V[:k + 1] for k in range(N)])
        _close(f"softmax scan N{N} D{D} M{M} s{scale}", out[0], want, 1e-11, fails)
        _close(f"softmax final m N{N}", np.array([m[0]]), np.array([sc.max()]), 1e-14, fails)
        e = np.exp(sc - sc.max())
        _close(f"softmax final u N{N}", np.array([u[0]]), np.array([e.sum()]), 1e-12, fails)
        _close(f"softmax final w N{N}", w[0], e @ V, 1e-12, fails)
        ones = o.softmax_scan(q[None], K[None], np.ones((1, N, M)))[0][0]
        if not np.max(np.abs(ones - 1.0)) <= 1e-14:
            fails.append(f"softmax ones invariant N{N}")
        zq = o.softmax_scan(np.zeros((1, D)), K[None], V[None])[0][0]
        _close(f"softmax q=0 prefix means N{N}", zq, np.cumsum(V, axis=0) / np.arange(1, N + 1)[:, None], 1e-12,
               fails)
        _close(f"softmax first row N{N}", out[0, 0], V[0], 1e-14, fails)
        # the one-token RNN reproduces every row and the state
        ms, us, ws = np.full(1, -np.inf), np.zeros(1), np.zeros((1, M))
        steps = np.stack([o.softmax_step(ms, us, ws, q[None], K[None, i], V[None, i]) for i in range(N)], axis=1)
        _close(f"softmax step == scan N{N}", steps[0], out[0], 1e-12, fails)
        _close(f"softmax step state N{N}", ws[0], w[0], 1e-12, fails)
    # scores beyond the range of exp: stays finite, equals the shifted definition
    q = np.array([800.0, -800.0])
    K = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 0.1], [-1.0, 0.0]])
    V = rng.normal(size=(4, 3))
    out = o.softmax_scan(q[None], K[None], V[None])[0][0]
    sc = K @ q
    want = np.stack([sp_softmax(sc[:k + 1]) @ V[:k + 1] for k in range(4)])
    if not np.all(np.isfinite(out)):
        fails.append("softmax scan overflow")
    _close("softmax scan extreme scores", out, want, 1e-12, fails)
    # 50-digit evaluation of the definition
    mpmath.mp.dps = 50
    N, D, M = 6, 3, 2
    q = rng.normal(size=D) * 4
    K = rng.normal(size=(N, D))
    V = rng.normal(size=(N, M))
    out = o.softmax_scan(q[None], K[None], V[None])[0][0]
    for k in range(N):
        ws_ = [mpmath.exp(mpmath.fsum(mpmath.mpf(float(q[d])) * mpmath.mpf(float(K[i, d])) for d in range(D)))
               for i in range(k + 1)]
        tot = mpmath.fsum(ws_)
        for j in range(M):
            val = float(mpmath.fsum(ws_[i] * mpmath.mpf(float(V[i, j])) for i in range(k + 1)) / tot)
            if not abs(out[k, j] - val) <= 1e-13 * max(1.0, abs(val)):
                fails.append(f"softmax mpmath row {k} col {j}")


def pin_features(o, fails):
    """Random-feature maps (page "Stable, Fast and Accurate: Kernelized Attention with Relative
    Positional Encoding": PRF, TRF and their variants) and linear attention on mapped features.

    * unbiasedness: over w ~ N(0, I) the mean of phi(q) . phi(k) is exp(q . k) for PRF and TRF
      (Monte Carlo with 2^17 features, bound from the sample variance);
    * exact identities that hold for ANY W and are computed another way:
      PRF  phi(x) . phi(y) = mean_f exp(w_f . (x + y) - (|x|^2 + |y|^2) / 2),
      TRF  phi(x) . phi(y) = exp((|x|^2 + |y|^2) / 2) mean_p cos(w_p . (x - y)),
      so  TRF phi(x) . phi(x) = exp(|x|^2);  W = 0 gives PRF exp(-(|x|^2+|y|^2)/2);
    * normalisation: phi(c x) = phi(x) for c > 0, and equals phi(x / |x|) without it;
    * the elu kind is phi (pinned above);
    * attention on mapped features: the quadratic masked form in numpy (causal and not),
      the final sums, the elu features reproduce the causal oracle, and with many PRF
      features linear attention approaches softmax attention."""
    rng = np.random.default_rng(71)
    # unbiasedness
    D = 3
    q = np.array([0.3, -0.5, 0.2])
    k = np.array([-0.1, 0.4, 0.6])
    F = 1 << 17
    W = rng.normal(size=(F, D))
    want = np.exp(q @ k)
    fq, fk = o.feature_map(q[None], W, F, "prf"), o.feature_map(k[None], W, F, "prf")
    per = fq[0] * fk[0] * F  # one estimate per feature
    if not abs(per.mean() - want) <= 6 * per.std() / np.sqrt(F):
        fails.append(f"prf unbiased: {per.mean():.6f} vs {want:.6f}")
    P = F // 2
    Wt = W[:P]
    fq, fk = o.feature_map(q[None], Wt, F, "trf"), o.feature_map(k[None], Wt, F, "trf")
    per = (fq[0, :P] * fk[0, :P] + fq[0, P:] * fk[0, P:]) * P
    if not abs(per.mean() - want) <= 6 * per.std() / np.sqrt(P):
        fails.append(f"trf unbiased: {per.mean():.6f} vs {want:.6f}")
    # exact identities for arbitrary W
    for (D, F) in [(4, 8), (16, 16), (7, 32)]:
        X = rng.normal(size=(5, D)) * 0.7
        Y = rng.normal(size=(5, D)) * 0.7
        W = rng.normal(size=(F, D))
        fx, fy = o.feature_map(X, W, F, "prf"), o.feature_map(Y, W, F, "prf")
        nx, ny = (X * X).sum(1), (Y * Y).sum(1)
        want = np.exp((X + Y) @ W.T - 0.5 * (nx + ny)[:, None]).mean(axis=1)
        _close(f"prf identity D{D} F{F}", (fx * fy).sum(1), want, 1e-12, fails)
        if not np.all(fx > 0):
            fails.append("prf features not positive")
        f0 = o.feature_map(X, np.zeros((F, D)), F, "prf")
        _close(f"prf W=0 D{D}", f0, np.repeat(np.exp(-0.5 * nx)[:, None] / np.sqrt(F), F, axis=1), 1e-13, fails)
        Wt = W[:F // 2]
        tx, ty = o.feature_map(X, Wt, F, "trf"), o.feature_map(Y, Wt, F, "trf")
        want = np.exp(0.5 * (nx + ny)) * np.cos((X - Y) @ Wt.T).mean(axis=1)
        _close(f"trf identity D{D} F{F}", (tx * ty).sum(1), want, 1e-11, fails)
        _close(f"trf self D{D} F{F}", (tx * tx).sum(1), np.exp(nx), 1e-12, fails)
        for kind, Wk in (("prf", W), ("trf", Wt)):
            a = o.feature_map(X * 3.7, Wk, F, kind, normalize=True)
            b = o.feature_map(X, Wk, F, kind, normalize=True)
            c = o.feature_map(X / np.sqrt(nx)[:, None], Wk, F, kind)
            _close(f"{kind} normalised scale D{D}", a, b, 1e-12, fails)
            _close(f"{kind} normalised = unit rows D{D}", b, c, 1e-12, fails)
        _close(f"elu kind D{D}", o.feature_map(X, None, D, "elu"), o.phi(X), 0.0, fails)
    # attention on mapped features
    for (N, F, M) in [(1, 4, 3), (9, 5, 2), (40, 16, 7)]:
        Fq = np.abs(rng.normal(size=(2, N, F))) + 0.05
        Fk = np.abs(rng.normal(size=(2, N, F))) + 0.05
        V = rng.normal(size=(2, N, M))
        out, S, z = o.attention_mapped(Fq, Fk, V, causal=True)
        outn, Sn, zn = o.attention_mapped(Fq, Fk, V, causal=False)
        for h in range(2):
            A = Fq[h] @ Fk[h].T
            L = np.tril(A)
            _close(f"mapped causal N{N} F{F}", out[h], (L @ V[h]) / L.sum(1, keepdims=True), 1e-12, fails)
            _close(f"mapped non-causal N{N} F{F}", outn[h], (A @ V[h]) / A.sum(1, keepdims=True), 1e-12, fails)
            for nm, SS, zz in (("causal", S, z), ("non-causal", Sn, zn)):
                _close(f"mapped {nm} S N{N}", SS[h], Fk[h].T @ V[h], 1e-12, fails)
                _close(f"mapped {nm} z N{N}", zz[h], Fk[h].sum(0), 1e-12, fails)
    Q, K, V = rng.normal(size=(2, 30, 6)), rng.normal(size=(2, 30, 6)), rng.normal(size=(2, 30, 4))
    _close("mapped elu = causal", o.attention_mapped(o.phi(Q), o.phi(K), V)[0], o.causal(Q, K, V)[0], 1e-12, fails)
    # many PRF features: linear attention approaches softmax attention
    N, D, M, F = 6, 4, 3, 1 << 16
    Q, K, V = rng.normal(size=(N, D)) * 0.4, rng.normal(size=(N, D)) * 0.4, rng.normal(size=(N, M))
    W = rng.normal(size=(F, D))
    got = o.attention_mapped(o.feature_map(Q, W, F, "prf")[None], o.feature_map(K, W, F, "prf")[None], V[None])[0][0]
    E = np.tril(np.exp(Q @ K.T))
    soft = (E @ V) / E.sum(1, keepdims=True)
    if not np.max(np.abs(got - soft)) <= 2e-2 * np.max(np.abs(soft)):
        fails.append(f"prf attention vs softmax: {np.max(np.abs(got - soft)):.3e}")


def _central_diff(loss, X, h):
    """Central differences of a scalar function of the array X, element by element."""
    g = np.zeros_like(X)
    for idx in np.ndindex(X.shape):
        Xp, Xm = X.copy(), X.copy()
        Xp[idx] += h
        Xm[idx] -= h
        g[idx] = (loss(Xp) - loss(Xm)) / (2 * h)
    return g


def pin_feature_gradients(o, fails):
    """Gradients through random-feature maps:

    * attention on mapped features: fp64 autograd through the quadratic masked form on the
      features (torch CPU), central differences of the (pinned) mapped forward, and the chain
      rule back to the elu path: with features phi(Q), phi(K) the gradients times phi' are the
      causal backward's (pinned above);
    * the feature maps: central differences of the (pinned) forward map for elu, PRF and TRF,
      with and without row normalisation, and a zero row under normalisation gets zero."""
    import torch
    rng = np.random.default_rng(83)

    def quad(Gt, Ft, Vt):
        A = torch.tril(Gt @ Ft.T)
        return (A @ Vt) / A.sum(dim=1, keepdim=True)

    for (N, F, M) in [(1, 3, 2), (7, 5, 3), (20, 16, 6)]:
        Fq = np.abs(rng.normal(size=(N, F))) + 0.1
        Fk = np.abs(rng.normal(size=(N, F))) + 0.1
        V = rng.normal(size=(N, M))
        dO = rng.normal(size=(N, M))
        dFq, dFk, dV = o.backward_mapped(Fq[None], Fk[None], V[None], dO[None])
        Gt, Ft, Vt = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Fq, Fk, V)]
        (quad(Gt, Ft, Vt) * torch.tensor(dO)).sum().backward()
        for nm, got, want in (("dFq", dFq[0], Gt.grad.numpy()), ("dFk", dFk[0], Ft.grad.numpy()),
                              ("dV", dV[0], Vt.grad.numpy())):
            err = np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-3)
            if not err <= 1e-11:
                fails.append(f"mapped backward autograd {nm} N{N} F{F} M{M}: {err:.3e}")
    N, F, M = 5, 3, 2
    Fq, Fk = np.abs(rng.normal(size=(N, F))) + 0.2, np.abs(rng.normal(size=(N, F))) + 0.2
    V, dO = rng.normal(size=(N, M)), rng.normal(size=(N, M))
    dFq, dFk, dV = o.backward_mapped(Fq[None], Fk[None], V[None], dO[None])
    args = [Fq, Fk, V]
    for pos, (nm, G) in enumerate((("Fq", dFq[0]), ("Fk", dFk[0]), ("V", dV[0]))):
        def loss(X, pos=pos):
            a = list(args)
            a[pos] = X
            return float(np.sum(o.attention_mapped(a[0][None], a[1][None], a[2][None])[0][0] * dO))
        num = _central_diff(loss, args[pos], 1e-6)
        err = np.max(np.abs(num - G)) / max(np.max(np.abs(G)), 1e-300)
        if not err <= 1e-6:
            fails.append(f"mapped backward finite differences d{nm}: {err:.3e}")
    Q, K, V = rng.normal(size=(2, 12, 4)), rng.normal(size=(2, 12, 4)), rng.normal(size=(2, 12, 3))
    dO = rng.normal(size=(2, 12, 3))
    dFq, dFk, dVm = o.backward_mapped(o.phi(Q), o.phi(K), V, dO)
    dQ, dK, dV = o.causal_backward(Q, K, V, dO)
    dphi = lambda x: np.where(x > 0, 1.0, np.exp(x))
    _close("mapped backward chain dQ", dFq * dphi(Q), dQ, 1e-12, fails)
    _close("mapped backward chain dK", dFk * dphi(K), dK, 1e-12, fails)
    _close("mapped backward chain dV", dVm, dV, 1e-12, fails)
    # the feature maps
    for (D, F) in [(3, 4), (5, 8)]:
        X = rng.normal(size=(3, D)) * 0.6
        W = rng.normal(size=(F, D))
        for kind, Wk, Fk_ in (("elu", None, D), ("prf", W, F), ("trf", W[:F // 2], F)):
            for normalize in (False, True):
                dOut = rng.normal(size=(3, Fk_))
                got = o.feature_map_backward(X, Wk, dOut, Fk_, kind, normalize)
                loss = lambda Xv: float(np.sum(o.feature_map(Xv, Wk, Fk_, kind, normalize) * dOut))
                num = _central_diff(loss, X, 1e-6)
                err = np.max(np.abs(num - got)) / max(np.max(np.abs(got)), 1e-300)
                if not err <= 1e-6:
                    fails.append(f"feature map backward {kind} norm={normalize} D{D} F{Fk_}: {err:.3e}")
        Z = np.zeros((2, D))
        for kind, Wk, Fk_ in (("prf", W, F), ("trf", W[:F // 2], F)):
            g = o.feature_map_backward(Z, Wk, rng.normal(size=(2, Fk_)), Fk_, kind, True)
            if not np.all(g == 0.0):
                fails.append(f"feature map backward {kind}: zero row not zero under normalisation")


ALL_PINS = [pin_golden, pin_bruteforce, pin_mpmath, pin_invariants, pin_rnn, pin_chunked, pin_continue,
            pin_backward, pin_softmax_scan, pin_features, pin_feature_gradients]


def run_all(o, pins=ALL_PINS):
    fails = []
    for p in pins:
        try:
            p(o, fails)
        except Exception as e:  # a crash in a pin is a failure of the oracle under test
            fails.append(f"{p.__name__}: raised {type(e).__name__}: {e}")
    return fails
