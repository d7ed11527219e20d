"""fp64 CPU oracle for causal kernelized linear attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The HIP path (efficient_transformer_amd) never imports it, and the
two share no code.  The arithmetic lives in oracle.c (plain C, float64, OpenMP
over independent heads); this module only builds that file and marshals numpy
arrays into it.

Method: "Transformers are RNNs: Fast Autoregressive Transformers with Linear
Attention" (Katharopoulos et al., 2020), page of that title, Proposed method and
Main findings.  phi(x) = elu(x) + 1; S_i = sum_{j<=i} phi(k_j) v_j^T;
z_i = sum_{j<=i} phi(k_j); out_i = phi(q_i)^T S_i / phi(q_i)^T z_i.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def compile_lib(src: str, dst: str) -> str:
    """gcc -O3 (no fast-math) with OpenMP; the build used for the oracle and for test mutants."""
    tmp = dst + ".tmp"
    cmd = ["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, dst)
    return dst


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so."""
    if force or not os.path.exists(LIB_PATH):
        compile_lib(_SRC, LIB_PATH)
    return LIB_PATH


class Oracle:
    """ctypes bindings of one build of oracle.c (the default build, or a test's mutant)."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        L.oracle_phi1.restype = ctypes.c_double
        L.oracle_phi1.argtypes = [ctypes.c_double]
        L.oracle_phi.argtypes = [_dp, _dp, _i64]
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_causal.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, ctypes.c_int]
        L.oracle_causal_from.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64,
                                         ctypes.c_int]
        L.oracle_causal_rows.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64,
                                         ctypes.POINTER(_i64), _i64, _dp, ctypes.c_int]
        L.oracle_noncausal.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, ctypes.c_int]
        L.oracle_decode_step.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_int]
        L.oracle_softmax_scan.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, ctypes.c_int]
        L.oracle_softmax_step.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_int]
        L.oracle_causal_backward.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64,
                                             ctypes.c_int]
        L.oracle_feature_map.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.oracle_attention_mapped.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, ctypes.c_int,
                                              ctypes.c_int]
        L.oracle_backward_mapped.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64,
                                             ctypes.c_int]
        L.oracle_feature_map_backward.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int]
        self.L = L
        self.path = path

    def max_threads(self) -> int:
        return int(self.L.oracle_max_threads())

    def phi(self, x) -> np.ndarray:
        x = _f64(x)
        y = np.empty_like(x)
        self.L.oracle_phi(_p(x), _p(y), x.size)
        return y

    def causal(self, Q, K, V, threads: int = 0):
        """Causal outputs by the running-sum recurrence.

        Q, K: [..., N, D]; V: [..., N, M] (leading dims are independent heads).
        Returns (out [..., N, M], S [..., D, M], z [..., D]); S, z are the final state.
        """
        Q, K, V = _f64(Q), _f64(K), _f64(V)
        *lead, N, D = Q.shape
        M = V.shape[-1]
        assert K.shape == Q.shape and tuple(V.shape[:-1]) == tuple(Q.shape[:-1])
        BH = int(np.prod(lead)) if lead else 1
        out = np.empty((*lead, N, M))
        S = np.empty((*lead, D, M))
        z = np.empty((*lead, D))
        self.L.oracle_causal(_p(Q), _p(K), _p(V), _p(out), _p(S), _p(z), BH, N, D, M, threads)
        return out, S, z

    def causal_from(self, Q, K, V, S0, z0, threads: int = 0):
        """Causal outputs continued from the carried state (S0 [..., D, M], z0 [..., D]).

        Returns (out [..., N, M], S [..., D, M], z [..., D]) like causal().
        """
        Q, K, V, S0, z0 = _f64(Q), _f64(K), _f64(V), _f64(S0), _f64(z0)
        *lead, N, D = Q.shape
        M = V.shape[-1]
        assert K.shape == Q.shape and tuple(V.shape[:-1]) == tuple(Q.shape[:-1])
        assert tuple(S0.shape) == (*lead, D, M) and tuple(z0.shape) == (*lead, D)
        BH = int(np.prod(lead)) if lead else 1
        out = np.empty((*lead, N, M))
        S = np.empty((*lead, D, M))
        z = np.empty((*lead, D))
        self.L.oracle_causal_from(_p(Q), _p(K), _p(V), _p(S0), _p(z0), _p(out), _p(S), _p(z), BH, N, D, M,
                                  threads)
        return out, S, z

    def causal_rows(self, Qh, Kh, Vh, rows, threads: int = 0) -> np.ndarray:
        """Selected output rows of ONE head, from the quadratic definition.

        Qh, Kh: [n, D]; Vh: [n, M] with n > max(rows) (row i reads rows 0..i only).
        """
        Qh, Kh, Vh = _f64(Qh), _f64(Kh), _f64(Vh)
        n, D = Qh.shape
        M = Vh.shape[1]
        r = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((r.size, M))
        self.L.oracle_causal_rows(_p(Qh), _p(Kh), _p(Vh), n, D, M,
                                  r.ctypes.data_as(ctypes.POINTER(_i64)), r.size, _p(out), threads)
        return out

    def noncausal(self, Q, K, V, threads: int = 0) -> np.ndarray:
        Q, K, V = _f64(Q), _f64(K), _f64(V)
        *lead, N, D = Q.shape
        M = V.shape[-1]
        BH = int(np.prod(lead)) if lead else 1
        out = np.empty((*lead, N, M))
        self.L.oracle_noncausal(_p(Q), _p(K), _p(V), _p(out), BH, N, D, M, threads)
        return out

    def decode_step(self, S, z, q, k, v, threads: int = 0) -> np.ndarray:
        """One recurrent step; S [..., D, M] and z [..., D] (float64, contiguous) update in place."""
        assert S.dtype == np.float64 and S.flags.c_contiguous
        assert z.dtype == np.float64 and z.flags.c_contiguous
        q, k, v = _f64(q), _f64(k), _f64(v)
        D, M = S.shape[-2], S.shape[-1]
        BH = S.size // (D * M)
        assert q.size == BH * D and k.size == BH * D and v.size == BH * M and z.size == BH * D
        out = np.empty(v.shape)
        self.L.oracle_decode_step(_p(S), _p(z), _p(q), _p(k), _p(v), _p(out), BH, D, M, threads)
        return out


    def causal_backward(self, Q, K, V, dO, threads: int = 0):
        """Gradients (dQ, dK, dV) of causal attention for the output gradient dO [..., N, M]."""
        Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
        *lead, N, D = Q.shape
        M = V.shape[-1]
        assert K.shape == Q.shape and V.shape == dO.shape and tuple(V.shape[:-1]) == tuple(Q.shape[:-1])
        BH = int(np.prod(lead)) if lead else 1
        dQ = np.empty(Q.shape)
        dK = np.empty(K.shape)
        dV = np.empty(V.shape)
        self.L.oracle_causal_backward(_p(Q), _p(K), _p(V), _p(dO), _p(dQ), _p(dK), _p(dV), BH, N, D, M, threads)
        return dQ, dK, dV


    def softmax_scan(self, q, K, V, threads: int = 0):
        """Softmax attention of one query per head over every prefix (q [..., D], K [..., N, D],
        V [..., N, M]).  Returns (out [..., N, M], m [...], u [...], w [..., M]), the last three
        the final state (max score, sum of exp, sum of exp-weighted values)."""
        q, K, V = _f64(q), _f64(K), _f64(V)
        *lead, N, D = K.shape
        M = V.shape[-1]
        assert tuple(q.shape) == (*lead, D) and tuple(V.shape[:-1]) == tuple(K.shape[:-1])
        BH = int(np.prod(lead)) if lead else 1
        out = np.empty((*lead, N, M))
        m = np.empty(tuple(lead))
        u = np.empty(tuple(lead))
        w = np.empty((*lead, M))
        self.L.oracle_softmax_scan(_p(q), _p(K), _p(V), _p(out), _p(m), _p(u), _p(w), BH, N, D, M, threads)
        return out, m, u, w

    def softmax_step(self, m, u, w, q, k, v, threads: int = 0) -> np.ndarray:
        """One token; m, u [...], w [..., M] (float64, contiguous) update in place."""
        for a in (m, u, w):
            assert a.dtype == np.float64 and a.flags.c_contiguous
        q, k, v = _f64(q), _f64(k), _f64(v)
        M = w.shape[-1]
        BH = m.size
        D = q.size // BH
        out = np.empty(v.shape)
        self.L.oracle_softmax_step(_p(m), _p(u), _p(w), _p(q), _p(k), _p(v), _p(out), BH, D, M, threads)
        return out


    FEATURE_KINDS = {"elu": 0, "prf": 1, "trf": 2}

    def feature_map(self, X, W, F: int, kind: str, normalize: bool = False, threads: int = 0) -> np.ndarray:
        """Features of every row of X [..., D]: kind "elu" (F = D, W unused), "prf" (W [F, D])
        or "trf" (W [F/2, D]); normalize scales each row to unit length first.  Returns [..., F]."""
        X = _f64(X)
        D = X.shape[-1]
        rows = X.size // D if D else 0
        k = self.FEATURE_KINDS[kind]
        if k == 0:
            assert F == D
            W = np.zeros(1)
        else:
            W = _f64(W)
            assert W.shape == ((F if k == 1 else F // 2), D)
        out = np.empty((*X.shape[:-1], F))
        self.L.oracle_feature_map(_p(X), _p(W), _p(out), rows, D, F, k, int(bool(normalize)), threads)
        return out

    def attention_mapped(self, Fq, Fk, V, causal: bool = True, threads: int = 0):
        """Linear attention on mapped features Fq, Fk [..., N, F] (no feature map applied).
        Returns (out [..., N, M], S [..., F, M], z [..., F]) with S, z the sums over all positions."""
        Fq, Fk, V = _f64(Fq), _f64(Fk), _f64(V)
        *lead, N, F = Fq.shape
        M = V.shape[-1]
        assert Fk.shape == Fq.shape and tuple(V.shape[:-1]) == tuple(Fq.shape[:-1])
        BH = int(np.prod(lead)) if lead else 1
        out = np.empty((*lead, N, M))
        S = np.empty((*lead, F, M))
        z = np.empty((*lead, F))
        self.L.oracle_attention_mapped(_p(Fq), _p(Fk), _p(V), _p(out), _p(S), _p(z), BH, N, F, M, int(bool(causal)),
                                       threads)
        return out, S, z


    def backward_mapped(self, Fq, Fk, V, dO, threads: int = 0):
        """Gradients (dFq, dFk, dV) of causal linear attention on mapped features Fq, Fk [..., N, F]
        (no feature map applied) for the output gradient dO [..., N, M]."""
        Fq, Fk, V, dO = _f64(Fq), _f64(Fk), _f64(V), _f64(dO)
        *lead, N, F = Fq.shape
        M = V.shape[-1]
        assert Fk.shape == Fq.shape and V.shape == dO.shape and tuple(V.shape[:-1]) == tuple(Fq.shape[:-1])
        BH = int(np.prod(lead)) if lead else 1
        dFq, dFk, dV = np.empty(Fq.shape), np.empty(Fk.shape), np.empty(V.shape)
        self.L.oracle_backward_mapped(_p(Fq), _p(Fk), _p(V), _p(dO), _p(dFq), _p(dFk), _p(dV), BH, N, F, M, threads)
        return dFq, dFk, dV

    def feature_map_backward(self, X, W, dOut, F: int, kind: str, normalize: bool = False,
                             threads: int = 0) -> np.ndarray:
        """Gradient with respect to X [..., D] of sum(dOut * feature_map(X, W, F, kind, normalize))."""
        X, dOut = _f64(X), _f64(dOut)
        D = X.shape[-1]
        rows = X.size // D if D else 0
        k = self.FEATURE_KINDS[kind]
        if k == 0:
            assert F == D
            W = np.zeros(1)
        else:
            W = _f64(W)
            assert W.shape == ((F if k == 1 else F // 2), D)
        assert dOut.shape == (*X.shape[:-1], F)
        dX = np.empty(X.shape)
        self.L.oracle_feature_map_backward(_p(X), _p(W), _p(dOut), _p(dX), rows, D, F, k, int(bool(normalize)),
                                           threads)
        return dX


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def max_threads() -> int:
    return default().max_threads()


def phi(x):
    return default().phi(x)


def causal(Q, K, V, threads: int = 0):
    return default().causal(Q, K, V, threads)


def causal_from(Q, K, V, S0, z0, threads: int = 0):
    return default().causal_from(Q, K, V, S0, z0, threads)


def causal_rows(Qh, Kh, Vh, rows, threads: int = 0):
    return default().causal_rows(Qh, Kh, Vh, rows, threads)


def noncausal(Q, K, V, threads: int = 0):
    return default().noncausal(Q, K, V, threads)


def decode_step(S, z, q, k, v, threads: int = 0):
    return default().decode_step(S, z, q, k, v, threads)


def causal_backward(Q, K, V, dO, threads: int = 0):
    return default().causal_backward(Q, K, V, dO, threads)


def softmax_scan(q, K, V, threads: int = 0):
    return default().softmax_scan(q, K, V, threads)


def softmax_step(m, u, w, q, k, v, threads: int = 0):
    return default().softmax_step(m, u, w, q, k, v, threads)


def feature_map(X, W, F: int, kind: str, normalize: bool = False, threads: int = 0):
    return default().feature_map(X, W, F, kind, normalize, threads)


def attention_mapped(Fq, Fk, V, causal: bool = True, threads: int = 0):
    return default().attention_mapped(Fq, Fk, V, causal, threads)


def backward_mapped(Fq, Fk, V, dO, threads: int = 0):
    return default().backward_mapped(Fq, Fk, V, dO, threads)


def feature_map_backward(X, W, dOut, F: int, kind: str, normalize: bool = False, threads: int = 0):
    return default().feature_map_backward(X, W, dOut, F, kind, normalize, threads)
