"""ctypes binding of liblinattn.so (include/linattn.h): marshalling only.

Every step of the computation runs in the library's HIP kernels; torch is used
to hold device memory and to name the stream.  If the library has not been
built, every call raises -- there is no fallback implementation.
"""
from __future__ import annotations

import collections
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblinattn.so")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE, LA_ERR_HIP, LA_ERR_GAVE_UP = range(6)
LA_F32, LA_BF16, LA_F32_FEATURES = 0, 1, 2
LA_OUT_BF16 = 16
LA_FEATURE_ELU, LA_FEATURE_PRF, LA_FEATURE_TRF = 0, 1, 2
LA_FEATURE_NORMALIZE = 1

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/linattn.h
SIGNATURES = {
    "la_status_str": (ctypes.c_char_p, [_int]),
    "la_version": (_int, []),
    "la_forward_plan": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _int, _int,
                               ctypes.POINTER(_int), ctypes.POINTER(_int), ctypes.POINTER(_sz)]),
    "la_forward_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _int, _int, _int]),
    "la_forward_chunked": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _int,
                                  _vp, _sz, _vp, _vp, _vp]),
    "la_workspace_init": (_int, [_vp, _sz, _vp]),
    "la_noalloc_scratch_bytes": (_sz, []),
    "la_forward_chunked_noalloc": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _int,
                                          _vp, _vp, _vp]),
    "la_workspace_status": (_int, [_vp, _sz, _vp]),
    "la_forward_continue": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp,
                                   _vp, _sz, _vp, _vp, _vp]),
    "la_forward_fused": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _int, _vp, _vp,
                                _vp, _sz, _vp, _vp, _vp]),
    "la_forward_onepass": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _int, _vp, _vp,
                                  _vp, _sz, _vp, _vp, _vp]),
    "la_segment_states": (_int, [_vp, _vp, _vp, _sz, _i64, _i64, _i64, _i64, _i64, _int, _int, _int, _int, _vp]),
    "la_segment_scan": (_int, [_vp, _sz, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp]),
    "la_segment_outputs": (_int, [_vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _i64, _i64, _i64, _int, _int, _int,
                                  _int, _vp, _vp, _vp]),
    "la_backward_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _int]),
    "la_backward_chunked": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int,
                                   _vp, _sz, _vp]),
    "la_softmax_scan_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "la_softmax_scan": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp, _vp, _vp,
                               _vp]),
    "la_softmax_step": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp]),
    "la_decode_step": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp]),
    "la_decode_steps": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _vp]),
    "la_feature_map": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _int, _vp, _i64, _int, _int, _vp]),
    "la_feature_map_backward": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _vp, _i64, _int, _int, _vp]),
    "la_decode_step_features": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp, _i64, _int,
                                       _int, _vp]),
    "la_forward_features_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64, _int]),
    "la_forward_features": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _i64, _int,
                                   _int, _vp, _sz, _vp, _vp, _vp, _vp, _vp]),
    "la_probe_copy": (_int, [_vp, _vp, _sz, _vp]),
    "la_probe_read_partials": (_sz, []),
    "la_probe_read": (_int, [_vp, _vp, _sz, _vp]),
    "la_probe_mfma": (_int, [_vp, _int, _i64, _int, ctypes.c_float, _vp]),
    "la_probe_write": (_int, [_vp, _sz, ctypes.c_float, _vp]),
    "la_probe_mfma32": (_int, [_vp, _i64, _int, ctypes.c_float, _vp]),
}


class LinAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


_lib = None


def lib_path() -> str:
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first (__graft_entry__.build() "
                "or python -m efficient_transformer_amd.build_lib); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().la_status_str(status).decode()


def version() -> int:
    return int(lib().la_version())


def _check(status: int, where: str) -> None:
    if status != LA_OK:
        raise LinAttnError(status, where)


def _dtype_code(t, features: bool = False) -> int:
    """LA_F32 / LA_BF16 from the tensor; features=True: fp32 rows that already hold phi(q), phi(k)."""
    import torch
    if features:
        if t.dtype != torch.float32:
            raise TypeError("feature inputs must be float32")
        return LA_F32_FEATURES
    if t.dtype == torch.float32:
        return LA_F32
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise TypeError(f"unsupported input dtype {t.dtype} (float32 or bfloat16)")


def _out_code(dt, out, out_dtype, shape, dev):
    """The output tensor (allocated when None) and the element-type code with the
    bf16-output flag when out is bfloat16 (bf16 inputs only)."""
    import torch
    want = out.dtype if out is not None else (out_dtype or torch.float32)
    if want not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    if want == torch.bfloat16:
        if dt != LA_BF16:
            raise TypeError("a bfloat16 output needs bfloat16 inputs")
        dt |= LA_OUT_BF16
    if out is None:
        out = torch.empty(shape, dtype=want, device=dev)
    _require(out, "out", shape, want, dev)
    return out, dt


def _torch_float32():
    import torch
    return torch.float32


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t, name, shape, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def forward_plan(B, H, N, D, M, causal=True, dtype=LA_F32, chunk=0):
    """(chunk, segments, workspace_bytes) chosen by the library for this problem."""
    c, g, w = _int(0), _int(0), _sz(0)
    _check(lib().la_forward_plan(B, H, N, D, M, int(bool(causal)), dtype, chunk,
                                 ctypes.byref(c), ctypes.byref(g), ctypes.byref(w)), "la_forward_plan")
    return c.value, g.value, w.value


def workspace_bytes(B, H, N, D, M, causal=True, dtype=LA_F32, chunk=0) -> int:
    return forward_plan(B, H, N, D, M, causal, dtype, chunk)[2]


# Workspaces made by the binding when the caller passes none: one per (device,
# stream, plan), at most WS_CACHE_PER_STREAM per (device, stream), the least
# recently used dropped first.  A cached buffer serves only the plan it was
# zeroed for, so the "zero before first use with a plan" rule of the look-back
# workspaces holds without re-zeroing.
WS_CACHE_PER_STREAM = 8
_ws_cache = collections.OrderedDict()

# When true (environment LA_CHECK_WAITS=1), every call that used a look-back
# workspace waits for its stream and raises LinAttnError(LA_ERR_GAVE_UP) if a
# wait for earlier segments gave up (see workspace_status).  Off by default: the
# check synchronises.
CHECK_WAITS = os.environ.get("LA_CHECK_WAITS", "0") == "1"


def workspace_init(ws, stream=None):
    """Zero a workspace before its first use (or before reuse with another plan)."""
    _check(lib().la_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream, ws.device)),
           "la_workspace_init")


def workspace_status(ws, stream=None) -> None:
    """Wait for `stream`, then raise LinAttnError (status LA_ERR_GAVE_UP) if a look-back wait
    gave up in a call that used `ws` since it was last zeroed; the outputs of such a call hold
    NaN rows and the workspace must be zeroed (workspace_init) before it is used again."""
    _check(lib().la_workspace_status(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream, ws.device)),
           "la_workspace_status")


def _after_call(ws, stream, check):
    if ws is not None and (CHECK_WAITS if check is None else check):
        workspace_status(ws, stream)


def _cached_workspace(nbytes, device, stream, key):
    """A zero-initialised workspace for one plan on one (device, stream); calls with one plan
    on one stream run in order, so they may share it."""
    import torch
    st = stream if stream is not None else torch.cuda.current_stream(device)
    dk = (str(device), st.cuda_stream)
    k = dk + (key,)
    ws = _ws_cache.get(k)
    if ws is not None and ws.numel() >= nbytes:
        _ws_cache.move_to_end(k)
        return ws
    with torch.cuda.stream(st):
        ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)
    _ws_cache[k] = ws
    same = [kk for kk in _ws_cache if kk[:2] == dk]
    for old in same[:max(0, len(same) - WS_CACHE_PER_STREAM)]:
        del _ws_cache[old]
    return ws


def forward_chunked(Q, K, V, causal=True, chunk=0, out=None, workspace=None, S_out=None, z_out=None,
                    stream=None, features=False, out_dtype=None, check=None):
    """Parallel-mode attention: Q, K [B,H,N,D], V [B,H,N,M] (float32 or bfloat16) -> out [B,H,N,M] float32.

    With S_out [B,H,D,M] and z_out [B,H,D] (float32) the final state is written too.
    A given `workspace` must have been zeroed (workspace_init) for this plan; by
    default a cached, zeroed one is used.  features=True: Q and K are float32
    features (feature_map), no feature map is applied and D is the feature dimension.
    A bfloat16 `out` (or out_dtype=torch.bfloat16) with bfloat16 inputs writes bf16 outputs.
    D and M may be any multiple of 16 up to 128 (widths other than 16, 32, 64, 128 run on padded
    copies in the workspace).  check=True (default: CHECK_WAITS) synchronises and raises if a
    look-back wait gave up.
    """
    import torch
    if Q.dim() != 4:
        raise ValueError("Q must be [B, H, N, D]")
    B, H, N, D = Q.shape
    M = V.shape[-1]
    dev = Q.device
    _require(Q, "Q", (B, H, N, D))
    _require(K, "K", (B, H, N, D), Q.dtype, dev)
    _require(V, "V", (B, H, N, M), Q.dtype, dev)
    dt = _dtype_code(Q, features)
    out, dt = _out_code(dt, out, out_dtype, (B, H, N, M), dev)
    if (S_out is None) != (z_out is None):
        raise ValueError("give both S_out and z_out, or neither")
    if S_out is not None:
        _require(S_out, "S_out", (B, H, D, M), torch.float32, dev)
        _require(z_out, "z_out", (B, H, D), torch.float32, dev)
    C, G, need = forward_plan(B, H, N, D, M, causal, dt, chunk)
    if workspace is None and need > 0:
        workspace = _cached_workspace(need, dev, stream, ("chunked", B * H, N, D, M, bool(causal), dt, C, G))
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().la_forward_chunked(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), B, H, N, D, M, int(bool(causal)), dt,
                                  chunk, _ptr(workspace), wbytes, _ptr(S_out), _ptr(z_out), _stream(stream, dev))
    _check(st, "la_forward_chunked")
    if causal:
        _after_call(workspace, stream, check)
    return out


def forward_chunked_noalloc(Q, K, V, out, causal=True, chunk=0, S_out=None, z_out=None, stream=None):
    """la_forward_chunked_noalloc: the same attention as forward_chunked with the library's
    static device scratch as workspace; the caller supplies `out` (and S_out, z_out), so
    nothing is allocated.  Calls that overlap in time on one device race on the scratch."""
    B, H, N, D = Q.shape
    M = V.shape[-1]
    dev = Q.device
    _require(K, "K", (B, H, N, D), Q.dtype, dev)
    _require(V, "V", (B, H, N, M), Q.dtype, dev)
    dt = _dtype_code(Q)
    out, dt = _out_code(dt, out, None, (B, H, N, M), dev)
    st = lib().la_forward_chunked_noalloc(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), B, H, N, D, M, int(bool(causal)),
                                          dt, chunk, _ptr(S_out), _ptr(z_out), _stream(stream, dev))
    _check(st, "la_forward_chunked_noalloc")
    return out


def noalloc_scratch_bytes() -> int:
    return int(lib().la_noalloc_scratch_bytes())


def fused_workspace_bytes(B, H, D, M, segments) -> int:
    if segments <= 1:
        return 0
    bhg = B * H * segments
    slot = (D * M + D + 63) // 64 * 64  # one exchanged state, padded to whole 256-byte blocks
    return (64 + 64 * ((bhg + 63) // 64)) * 4 + 2 * bhg * slot * 4


def forward_fused(Q, K, V, chunk, segments, out=None, workspace=None, S_out=None, z_out=None, stream=None,
                  S_in=None, z_in=None, features=False, out_dtype=None):
    """The causal two-phase fused kernel with an explicit plan (chunk, segments)."""
    return _forward_explicit("la_forward_fused", Q, K, V, chunk, segments, out, workspace, S_out, z_out, stream,
                             S_in, z_in, features, out_dtype)


def forward_onepass(Q, K, V, chunk, segments, out=None, workspace=None, S_out=None, z_out=None, stream=None,
                    S_in=None, z_in=None, features=False, out_dtype=None):
    """The causal one-pass kernel with an explicit plan (segments of at most 4 chunks)."""
    return _forward_explicit("la_forward_onepass", Q, K, V, chunk, segments, out, workspace, S_out, z_out, stream,
                             S_in, z_in, features, out_dtype)


def forward_continue(Q, K, V, S_in, z_in, out=None, chunk=0, workspace=None, S_out=None, z_out=None, stream=None,
                     features=False, out_dtype=None, check=None):
    """Causal attention continuing from the carried state (S_in [B,H,D,M], z_in [B,H,D], fp32)."""
    import torch
    B, H, N, D = Q.shape
    M = V.shape[-1]
    dev = Q.device
    _require(K, "K", (B, H, N, D), Q.dtype, dev)
    _require(V, "V", (B, H, N, M), Q.dtype, dev)
    if S_in is not None:
        _require(S_in, "S_in", (B, H, D, M), torch.float32, dev)
        _require(z_in, "z_in", (B, H, D), torch.float32, dev)
    dt = _dtype_code(Q, features)
    out, dt = _out_code(dt, out, out_dtype, (B, H, N, M), dev)
    C, G, need = forward_plan(B, H, N, D, M, True, dt & ~LA_OUT_BF16, chunk)
    if workspace is None and need > 0:
        workspace = _cached_workspace(need, dev, stream, ("chunked", B * H, N, D, M, True, dt, C, G))
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().la_forward_continue(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), B, H, N, D, M, dt, chunk, _ptr(S_in),
                                   _ptr(z_in), _ptr(workspace), wbytes, _ptr(S_out), _ptr(z_out),
                                   _stream(stream, dev))
    _check(st, "la_forward_continue")
    _after_call(workspace, stream, check)
    return out


def _forward_explicit(name, Q, K, V, chunk, segments, out, workspace, S_out, z_out, stream, S_in, z_in, features,
                      out_dtype=None):
    B, H, N, D = Q.shape
    M = V.shape[-1]
    dev = Q.device
    _require(K, "K", (B, H, N, D), Q.dtype, dev)
    _require(V, "V", (B, H, N, M), Q.dtype, dev)
    dt = _dtype_code(Q, features)
    out, dt = _out_code(dt, out, out_dtype, (B, H, N, M), dev)
    need = fused_workspace_bytes(B, H, D, M, segments)
    if workspace is None and need > 0:
        workspace = _cached_workspace(need, dev, stream, (name, B * H, N, D, M, dt & ~LA_OUT_BF16, chunk,
                                                          segments))
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = getattr(lib(), name)(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), B, H, N, D, M, dt, chunk,
                              segments, _ptr(S_in), _ptr(z_in), _ptr(workspace), wbytes, _ptr(S_out), _ptr(z_out),
                              _stream(stream, dev))
    _check(st, name)
    _after_call(workspace, stream, None)
    return out


def segment_states(K, V, ws, chunk, segments, nstates, stream=None, features=False):
    B, H, N, D = K.shape
    M = V.shape[-1]
    st = lib().la_segment_states(_ptr(K), _ptr(V), _ptr(ws), ws.numel() * ws.element_size(), B, H, N, D, M,
                                 _dtype_code(K, features), chunk, segments, nstates, _stream(stream, K.device))
    _check(st, "la_segment_states")


def segment_scan(ws, B, H, D, M, segments, nstates, S_out=None, z_out=None, stream=None):
    st = lib().la_segment_scan(_ptr(ws), ws.numel() * ws.element_size(), B, H, D, M, segments, nstates,
                               _ptr(S_out), _ptr(z_out), _stream(stream, ws.device))
    _check(st, "la_segment_scan")


def segment_outputs(Q, K, V, out, ws, chunk, segments, causal=True, S_out=None, z_out=None, stream=None,
                    features=False):
    B, H, N, D = Q.shape
    M = out.shape[-1]
    dt = _dtype_code(Q, features)
    if out.dtype != _torch_float32():
        if dt != LA_BF16:
            raise TypeError("a bfloat16 output needs bfloat16 inputs")
        dt |= LA_OUT_BF16
    st = lib().la_segment_outputs(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                  B, H, N, D, M, int(bool(causal)), dt, chunk, segments,
                                  _ptr(S_out), _ptr(z_out), _stream(stream, Q.device))
    _check(st, "la_segment_outputs")


def decode_step(S, z, q, k, v, out=None, stream=None, features=False):
    """One recurrent step: S [B,H,D,M], z [B,H,D] (float32, updated in place); q, k [B,H,D]; v [B,H,M]."""
    import torch
    if S.dim() != 4:
        raise ValueError("S must be [B, H, D, M]")
    B, H, D, M = S.shape
    dev = S.device
    _require(S, "S", (B, H, D, M), torch.float32)
    _require(z, "z", (B, H, D), torch.float32, dev)
    _require(q, "q", (B, H, D), None, dev)
    _require(k, "k", (B, H, D), q.dtype, dev)
    _require(v, "v", (B, H, M), q.dtype, dev)
    if out is None:
        out = torch.empty((B, H, M), dtype=torch.float32, device=dev)
    _require(out, "out", (B, H, M), torch.float32, dev)
    st = lib().la_decode_step(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, D, M,
                              _dtype_code(q, features), _stream(stream, dev))
    _check(st, "la_decode_step")
    return out


def decode_steps(S, z, q, k, v, out=None, stream=None, features=False):
    """T recurrent steps in one call: S [B,H,D,M], z [B,H,D] (float32, updated in place);
    q, k [B,H,T,D]; v [B,H,T,M]; returns out [B,H,T,M]."""
    import torch
    if S.dim() != 4 or q.dim() != 4:
        raise ValueError("S must be [B, H, D, M] and q [B, H, T, D]")
    B, H, D, M = S.shape
    T = q.shape[2]
    dev = S.device
    _require(S, "S", (B, H, D, M), torch.float32)
    _require(z, "z", (B, H, D), torch.float32, dev)
    _require(q, "q", (B, H, T, D), None, dev)
    _require(k, "k", (B, H, T, D), q.dtype, dev)
    _require(v, "v", (B, H, T, M), q.dtype, dev)
    if out is None:
        out = torch.empty((B, H, T, M), dtype=torch.float32, device=dev)
    _require(out, "out", (B, H, T, M), torch.float32, dev)
    st = lib().la_decode_steps(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, T, D, M,
                               _dtype_code(q, features), _stream(stream, dev))
    _check(st, "la_decode_steps")
    return out


def backward(Q, K, V, out, dout, workspace=None, stream=None, features=False):
    """Gradients (dQ, dK, dV) of causal attention; out is the forward's output.
    features=True: Q, K (float32) hold features, and dQ, dK are the gradients with respect
    to them (feature_map_backward carries them on to the raw rows)."""
    import torch
    B, H, N, D = Q.shape
    M = V.shape[-1]
    dev = Q.device
    _require(K, "K", (B, H, N, D), Q.dtype, dev)
    _require(V, "V", (B, H, N, M), Q.dtype, dev)
    _require(out, "out", (B, H, N, M), torch.float32, dev)
    _require(dout, "dout", (B, H, N, M), torch.float32, dev)
    dt = _dtype_code(Q, features)
    need = int(lib().la_backward_workspace_bytes(B, H, N, D, M, dt))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dQ = torch.empty((B, H, N, D), dtype=torch.float32, device=dev)
    dK = torch.empty((B, H, N, D), dtype=torch.float32, device=dev)
    dV = torch.empty((B, H, N, M), dtype=torch.float32, device=dev)
    st = lib().la_backward_chunked(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(dout), _ptr(dQ), _ptr(dK), _ptr(dV),
                                   B, H, N, D, M, dt, _ptr(workspace), wbytes, _stream(stream, dev))
    _check(st, "la_backward_chunked")
    return dQ, dK, dV


def softmax_scan(q, K, V, out=None, workspace=None, m_out=None, u_out=None, w_out=None, stream=None):
    """Softmax attention of one query per head (q [B,H,D]) over every prefix of K, V."""
    import torch
    B, H, N, D = K.shape
    M = V.shape[-1]
    dev = K.device
    _require(q, "q", (B, H, D), K.dtype, dev)
    _require(V, "V", (B, H, N, M), K.dtype, dev)
    if out is None:
        out = torch.empty((B, H, N, M), dtype=torch.float32, device=dev)
    need = int(lib().la_softmax_scan_workspace_bytes(B, H, N, D, M))
    if workspace is None and need > 0:
        workspace = _cached_workspace(need, dev, stream, ("softmax_scan", B * H, N, D, M))
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().la_softmax_scan(_ptr(q), _ptr(K), _ptr(V), _ptr(out), B, H, N, D, M, _dtype_code(K), _ptr(workspace),
                               wbytes, _ptr(m_out), _ptr(u_out), _ptr(w_out), _stream(stream, dev))
    _check(st, "la_softmax_scan")
    _after_call(workspace, stream, None)
    return out


def softmax_step(m, u, w, q, k, v, out=None, stream=None):
    """One token: state m, u [B,H] and w [B,H,M] (float32, in place); q, k [B,H,D]; v [B,H,M]."""
    import torch
    B, H, M = w.shape
    D = q.shape[-1]
    dev = w.device
    _require(m, "m", (B, H), torch.float32, dev)
    _require(u, "u", (B, H), torch.float32, dev)
    _require(q, "q", (B, H, D), None, dev)
    _require(k, "k", (B, H, D), q.dtype, dev)
    _require(v, "v", (B, H, M), q.dtype, dev)
    if out is None:
        out = torch.empty((B, H, M), dtype=torch.float32, device=dev)
    st = lib().la_softmax_step(_ptr(m), _ptr(u), _ptr(w), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, D, M,
                               _dtype_code(q), _stream(stream, dev))
    _check(st, "la_softmax_step")
    return out


FEATURE_KINDS = {"elu": LA_FEATURE_ELU, "prf": LA_FEATURE_PRF, "trf": LA_FEATURE_TRF}


def feature_map_backward(X, dout, W, F, kind="prf", normalize=False, dX=None, stream=None):
    """Gradient with respect to X [..., D] (float32 or bfloat16) of sum(dout * feature_map(X, W, F, kind,
    normalize)), dout [..., F] float32 -> float32 [..., D]."""
    import torch
    D = X.shape[-1]
    dev = X.device
    _require(X, "X", tuple(X.shape), None, dev)
    k = FEATURE_KINDS[kind]
    if k != LA_FEATURE_ELU:
        _require(W, "W", ((F if k == LA_FEATURE_PRF else F // 2), D), torch.float32, dev)
    _require(dout, "dout", (*X.shape[:-1], F), torch.float32, dev)
    if dX is None:
        dX = torch.empty(tuple(X.shape), dtype=torch.float32, device=dev)
    _require(dX, "dX", tuple(X.shape), torch.float32, dev)
    rows = X.numel() // D if D else 0
    st = lib().la_feature_map_backward(_ptr(dX), _ptr(X), _ptr(dout), rows, D, _dtype_code(X),
                                       _ptr(W) if k != LA_FEATURE_ELU else None, F, k,
                                       LA_FEATURE_NORMALIZE if normalize else 0, _stream(stream, dev))
    _check(st, "la_feature_map_backward")
    return dX


def feature_map(X, W, F, kind="prf", normalize=False, out=None, X2=None, out2=None, stream=None):
    """Random features of every row of X [..., D] (float32 or bfloat16) -> float32 [..., F].

    kind "elu" (F = D, W unused), "prf" (W [F, D] float32) or "trf" (W [F/2, D]);
    normalize scales every row to unit length first.  X2 (same shape as X) is
    mapped into out2 in the same launch; returns out, or (out, out2) with X2.
    """
    import torch
    D = X.shape[-1]
    dev = X.device
    _require(X, "X", tuple(X.shape), None, dev)
    k = FEATURE_KINDS[kind]
    if k != LA_FEATURE_ELU:
        _require(W, "W", ((F if k == LA_FEATURE_PRF else F // 2), D), torch.float32, dev)
    shape = (*X.shape[:-1], F)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    _require(out, "out", shape, torch.float32, dev)
    if X2 is not None:
        _require(X2, "X2", tuple(X.shape), X.dtype, dev)
        if out2 is None:
            out2 = torch.empty(shape, dtype=torch.float32, device=dev)
        _require(out2, "out2", shape, torch.float32, dev)
    rows = X.numel() // D if D else 0
    st = lib().la_feature_map(_ptr(out), _ptr(X), _ptr(out2) if X2 is not None else None, _ptr(X2), rows, D,
                              _dtype_code(X), _ptr(W) if k != LA_FEATURE_ELU else None, F, k,
                              LA_FEATURE_NORMALIZE if normalize else 0, _stream(stream, dev))
    _check(st, "la_feature_map")
    return out if X2 is None else (out, out2)


def forward_features(Q, K, V, W, F, kind="prf", normalize=False, out=None, workspace=None, S_out=None,
                     z_out=None, stream=None, S_in=None, z_in=None, causal=True):
    """Causal attention over random features computed inside the attention kernel:
    Q, K [B,H,N,D], V [B,H,N,M] float32 or bfloat16 (raw rows; the map and the
    attention run in fp32 either way), W as for feature_map ("prf":
    [F, D], "trf": [F/2, D]) -> out [B,H,N,M] float32.  S_out [B,H,F,M] / z_out
    [B,H,F] receive the final state over the features; S_in / z_in (same shapes)
    continue from a carried state (S_out may be S_in); causal=False: every row
    attends to all N positions (no states).  Raises LinAttnError
    (LA_ERR_UNSUPPORTED) where the fused kernel does not run the shape; feature_map
    followed by forward_chunked(features=True) computes the same there.
    """
    import torch
    if Q.dim() != 4:
        raise ValueError("Q must be [B, H, N, D]")
    B, H, N, D = Q.shape
    M = V.shape[-1]
    dev = Q.device
    k = FEATURE_KINDS[kind]
    if k == LA_FEATURE_ELU:
        raise ValueError("forward_features takes 'prf' or 'trf' (elu+1 is forward_chunked itself)")
    _require(Q, "Q", (B, H, N, D))
    _require(K, "K", (B, H, N, D), Q.dtype, dev)
    _require(V, "V", (B, H, N, M), Q.dtype, dev)
    dt = _dtype_code(Q)
    _require(W, "W", ((F if k == LA_FEATURE_PRF else F // 2), D), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, N, M), dtype=torch.float32, device=dev)
    _require(out, "out", (B, H, N, M), torch.float32, dev)
    if (S_out is None) != (z_out is None):
        raise ValueError("give both S_out and z_out, or neither")
    if S_out is not None:
        _require(S_out, "S_out", (B, H, F, M), torch.float32, dev)
        _require(z_out, "z_out", (B, H, F), torch.float32, dev)
    if (S_in is None) != (z_in is None):
        raise ValueError("give both S_in and z_in, or neither")
    if S_in is not None:
        _require(S_in, "S_in", (B, H, F, M), torch.float32, dev)
        _require(z_in, "z_in", (B, H, F), torch.float32, dev)
    c = int(bool(causal))
    need = int(lib().la_forward_features_workspace_bytes(B, H, N, D, M, F, c))  # 0: the call refuses the shape
    if workspace is None and need > 0:
        workspace = _cached_workspace(need, dev, stream, ("features", B * H, N, D, M, F, c))
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().la_forward_features(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), B, H, N, D, M, c, dt, _ptr(W), F, k,
                                   LA_FEATURE_NORMALIZE if normalize else 0, _ptr(workspace), wbytes,
                                   _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out), _stream(stream, dev))
    _check(st, "la_forward_features")
    if causal:
        _after_call(workspace, stream, None)
    return out


def decode_step_features(S, z, q, k, v, W, F, kind="prf", normalize=False, out=None, stream=None):
    """One recurrent step on raw rows with the random-feature map formed in the kernel:
    S [B,H,F,M], z [B,H,F] (float32, updated in place); q, k [B,H,D] and v [B,H,M]
    (float32 or bfloat16); W as for feature_map.  Returns out [B,H,M] float32."""
    import torch
    if S.dim() != 4:
        raise ValueError("S must be [B, H, F, M]")
    B, H, Fs, M = S.shape
    if Fs != F:
        raise ValueError("S must hold F features per head")
    D = q.shape[-1]
    dev = S.device
    k_ = FEATURE_KINDS[kind]
    if k_ == LA_FEATURE_ELU:
        raise ValueError("decode_step_features takes 'prf' or 'trf' (elu+1 is decode_step itself)")
    _require(S, "S", (B, H, F, M), torch.float32, dev)
    _require(z, "z", (B, H, F), torch.float32, dev)
    _require(q, "q", (B, H, D), None, dev)
    _require(k, "k", (B, H, D), q.dtype, dev)
    _require(v, "v", (B, H, M), q.dtype, dev)
    _require(W, "W", ((F if k_ == LA_FEATURE_PRF else F // 2), D), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, M), dtype=torch.float32, device=dev)
    _require(out, "out", (B, H, M), torch.float32, dev)
    st = lib().la_decode_step_features(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, D, M,
                                       _dtype_code(q), _ptr(W), F, k_, LA_FEATURE_NORMALIZE if normalize else 0,
                                       _stream(stream, dev))
    _check(st, "la_decode_step_features")
    return out


def probe_copy(dst, src, stream=None):
    """Plain device copy src -> dst (same byte size) by the library's copy probe."""
    if dst.numel() * dst.element_size() != src.numel() * src.element_size():
        raise ValueError("probe_copy: dst and src differ in size")
    if not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("probe_copy: tensors must be contiguous")
    _check(lib().la_probe_copy(_ptr(dst), _ptr(src), src.numel() * src.element_size(), _stream(stream, src.device)),
           "la_probe_copy")
    return dst


def probe_read(src, out=None, stream=None):
    """Read-only stream probe: per-thread partial sums of src's fp32 words (returns them)."""
    import torch
    n = int(lib().la_probe_read_partials())
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=src.device)
    if out.numel() != n or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError(f"probe_read: out must be contiguous float32 with {n} elements")
    if not src.is_contiguous():
        raise ValueError("probe_read: src must be contiguous")
    _check(lib().la_probe_read(_ptr(out), _ptr(src), src.numel() * src.element_size(), _stream(stream, src.device)),
           "la_probe_read")
    return out


def probe_write(dst, value: float = 0.0, stream=None):
    """Write-only stream probe: fills dst (contiguous) with the fp32 value by nontemporal stores."""
    if not dst.is_contiguous():
        raise ValueError("probe_write: dst must be contiguous")
    _check(lib().la_probe_write(_ptr(dst), dst.numel() * dst.element_size(), value, _stream(stream, dst.device)),
           "la_probe_write")
    return dst


def probe_mfma(kind: str, blocks: int, iters: int, x: float = 0.5, out=None, stream=None, device=None):
    """MFMA throughput probe ("f32": 16x16x4, "bf16": 16x16x32, "bf16_32x32": 32x32x16); returns
    (out, flops of the launch)."""
    import torch
    if kind not in ("f32", "bf16", "bf16_32x32"):
        raise ValueError(f"probe_mfma: unknown kind {kind!r}")
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device=device or "cuda")
    if out.dtype != torch.float32 or out.numel() < blocks * 256 or not out.is_contiguous():
        raise ValueError("probe_mfma: out must be contiguous float32 with blocks * 256 elements")
    if kind == "bf16_32x32":
        _check(lib().la_probe_mfma32(_ptr(out), blocks, iters, x, _stream(stream, out.device)), "la_probe_mfma32")
        return out, blocks * 4 * iters * 4 * 32768
    dt = {"f32": LA_F32, "bf16": LA_BF16}[kind]
    _check(lib().la_probe_mfma(_ptr(out), dt, blocks, iters, x, _stream(stream, out.device)), "la_probe_mfma")
    return out, blocks * 4 * iters * 8 * (2048 if kind == "f32" else 16384)
