"""The C-ABI library on the CPU: it loads, exports what include/linattn.h declares,
plans as documented, and rejects bad arguments before touching the GPU.

Only calls that the library answers from its argument checks are made here (they
return before any HIP runtime call), so no GPU is needed.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")


@pytest.fixture(scope="module")
def L():
    from efficient_transformer_amd import build_lib, linattn
    if not os.path.exists(linattn.LIB_PATH):
        build_lib.build(force=True)
    return linattn


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"LA_API\s+[\w\s\*]+?\b(la_\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ("la_forward_chunked", "la_decode_step", "la_forward_workspace_bytes", "la_forward_plan",
              "la_status_str", "la_segment_states", "la_segment_scan", "la_segment_outputs", "la_version",
              "la_forward_fused", "la_forward_onepass", "la_forward_continue", "la_workspace_init",
              "la_backward_chunked", "la_decode_steps", "la_softmax_scan", "la_softmax_step", "la_feature_map",
              "la_forward_features", "la_forward_features_workspace_bytes", "la_workspace_status"):
        assert s in syms


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    for s in declared_symbols():
        assert hasattr(lib, s), s
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(la_\w+)", out))
    assert set(declared_symbols()) == exported, "exports differ from the header"
    assert set(L.SIGNATURES) == set(declared_symbols()), "binding signatures differ from the header"


def test_status_strings(L):
    for code in range(6):
        assert L.status_str(code).startswith(["LA_OK", "LA_ERR_INVALID_ARG", "LA_ERR_UNSUPPORTED",
                                              "LA_ERR_WORKSPACE", "LA_ERR_HIP", "LA_ERR_GAVE_UP"][code])
    assert L.status_str(99) == "unknown status"
    assert L.version() >= 100


@pytest.mark.parametrize("B,H,N,D,M,causal,dtype,chunk", [
    (1, 1, 64, 16, 16, 1, 0, 16), (8, 8, 1024, 64, 64, 1, 0, 0), (4, 8, 3072, 64, 64, 1, 1, 0),
    (1, 16, 65536, 128, 128, 1, 1, 0), (2, 3, 257, 32, 128, 0, 0, 32), (1, 1, 1, 128, 16, 1, 1, 64),
    (3, 1, 100, 16, 64, 1, 0, 0), (1, 2, 5000, 128, 128, 1, 0, 0)])
def test_plan_covers_the_sequence(L, B, H, N, D, M, causal, dtype, chunk):
    C, G, ws = L.forward_plan(B, H, N, D, M, causal, dtype, chunk)
    if chunk:
        assert C == chunk
    assert C in (16, 32, 64)
    n_chunks = -(-N // C)
    cps = -(-n_chunks // G)
    assert 1 <= G <= n_chunks
    assert (G - 1) * cps < n_chunks <= G * cps  # every segment owns at least one chunk
    E = D * M + D
    if causal:
        bhg = B * H * G
        P = (E + 63) // 64 * 64
        assert ws == (0 if G == 1 else (64 + 64 * ((bhg + 63) // 64)) * 4 + 2 * bhg * P * 4)
    else:
        assert ws == B * H * (G + 1) * E * 4
    assert L.workspace_bytes(B, H, N, D, M, causal, dtype, chunk) == ws


@pytest.mark.parametrize("dtype", [0, 1])
def test_plan_default_chunk(L, dtype):
    for D in (16, 32, 64, 128):
        for M in (16, 32, 64, 128):
            C, _, _ = L.forward_plan(1, 1, 4096, D, M, 1, dtype, 0)
            assert C == (32 if dtype == 0 and D * M <= 4096 else 64)


def _fwd(L, Q=None, K=None, V=None, out=None, B=1, H=1, N=64, D=16, M=16, causal=1, dtype=0, chunk=0,
         ws=None, ws_bytes=0, S=None, z=None):
    return L.lib().la_forward_chunked(Q, K, V, out, B, H, N, D, M, causal, dtype, chunk, ws, ws_bytes, S, z, None)


FAKE = 0x10000  # aligned, never dereferenced: every call below fails its checks first


@pytest.mark.parametrize("kw,status", [
    (dict(D=40), 2), (dict(M=8), 2), (dict(D=256), 2), (dict(D=144), 2), (dict(M=120), 2), (dict(dtype=3), 1), (dict(causal=2), 1),
    (dict(chunk=128), 2), (dict(chunk=8), 2), (dict(N=-1), 1), (dict(B=-1), 1), (dict(H=-3), 1),
    (dict(Q=None), 1), (dict(out=None), 1), (dict(V=FAKE + 4), 1), (dict(S=FAKE), 1),
])
def test_forward_rejects_bad_arguments(L, kw, status):
    args = dict(Q=FAKE, K=FAKE, V=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    assert _fwd(L, **args) == status


def _round256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("D,M", [(48, 64), (64, 48), (112, 112), (80, 96), (48, 16), (96, 128), (16, 112)])
@pytest.mark.parametrize("causal,dtype", [(1, 0), (1, 1), (0, 0), (1, 17), (1, 2)])
def test_padded_widths_plan(L, D, M, causal, dtype):
    """Widths without a kernel of their own plan like the next kernel width up, with the
    padded copies of Q, K, V, out and the state after the kernels' own workspace."""
    B, H, N = 2, 3, 1000
    up = lambda x: 16 if x <= 16 else 32 if x <= 32 else 64 if x <= 64 else 128
    Dk, Mk = up(D), up(M)
    C, G, ws = L.forward_plan(B, H, N, D, M, causal, dtype, 0)
    Ck, Gk, wsk = L.forward_plan(B, H, N, Dk, Mk, causal, dtype, 0)
    assert (C, G) == (Ck, Gk)
    s_in = 2 if dtype & ~16 == 1 else 4
    s_out = 2 if dtype & 16 else 4
    rows = B * H * N
    want = (_round256(max(wsk, 256)) + 2 * _round256(rows * Dk * s_in) + _round256(rows * Mk * s_in)
            + _round256(rows * Mk * s_out) + _round256(B * H * Dk * Mk * 4) + _round256(B * H * Dk * 4))
    assert ws == want
    assert L.workspace_bytes(B, H, N, D, M, causal, dtype, 0) == ws
    # empty problems need no workspace
    assert L.forward_plan(B, H, 0, D, M, causal, dtype, 0)[2] == 0
    assert L.forward_plan(0, H, N, D, M, causal, dtype, 0)[2] == 0


def test_padded_widths_need_their_workspace(L):
    need = L.workspace_bytes(1, 1, 64, 48, 48, 1, 0, 0)
    assert need > 0
    assert _fwd(L, Q=FAKE, K=FAKE, V=FAKE, out=FAKE, N=64, D=48, M=48, ws=None, ws_bytes=0) == L.LA_ERR_WORKSPACE
    assert _fwd(L, Q=FAKE, K=FAKE, V=FAKE, out=FAKE, N=64, D=48, M=48, ws=FAKE,
                ws_bytes=need - 1) == L.LA_ERR_WORKSPACE
    # the explicit-plan and stage entry points keep the kernel widths
    f = L.lib().la_forward_fused
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 48, 48, 0, 16, 1, None, None, None, 0, None, None,
             None) == L.LA_ERR_UNSUPPORTED


def test_workspace_status_checks(L):
    f = L.lib().la_workspace_status
    assert f(None, 1024, None) == L.LA_ERR_INVALID_ARG
    assert f(FAKE + 4, 1024, None) == L.LA_ERR_INVALID_ARG
    assert f(FAKE, 8, None) == L.LA_ERR_INVALID_ARG


def test_forward_workspace_checks(L):
    need = L.workspace_bytes(1, 1, 4096, 64, 64, 1, 0, 0)
    assert need > 0
    assert _fwd(L, Q=FAKE, K=FAKE, V=FAKE, out=FAKE, N=4096, D=64, M=64, ws=None, ws_bytes=0) == L.LA_ERR_WORKSPACE
    assert _fwd(L, Q=FAKE, K=FAKE, V=FAKE, out=FAKE, N=4096, D=64, M=64, ws=FAKE,
                ws_bytes=need - 1) == L.LA_ERR_WORKSPACE
    assert _fwd(L, Q=FAKE, K=FAKE, V=FAKE, out=FAKE, N=4096, D=64, M=64, ws=FAKE + 8,
                ws_bytes=need) == L.LA_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op(L):
    # B*H == 0 returns before any pointer or HIP use
    assert _fwd(L, B=0, H=4, N=64) == L.LA_OK
    assert L.lib().la_decode_step(None, None, None, None, None, None, 0, 8, 64, 64, 0, None) == L.LA_OK


def test_decode_rejects_bad_arguments(L):
    f = L.lib().la_decode_step
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 40, 64, 0, None) == L.LA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 144, 0, None) == L.LA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 64, 3, None) == L.LA_ERR_INVALID_ARG
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 64, 0, None) == L.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE, 2, 2, 64, 64, 0, None) == L.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 2, 64, 64, 0, None) == L.LA_ERR_INVALID_ARG


def test_stage_entry_points_check_plans(L):
    lib = L.lib()
    # segments must each own a chunk: 4 chunks cannot make 5 non-empty segments
    assert lib.la_segment_states(FAKE, FAKE, FAKE, 1 << 30, 2, 1, 256, 64, 64, 0, 64, 5, 5,
                                 None) == L.LA_ERR_UNSUPPORTED
    assert lib.la_segment_states(FAKE, FAKE, FAKE, 16, 2, 1, 256, 64, 64, 0, 64, 2, 2, None) == L.LA_ERR_WORKSPACE
    assert lib.la_segment_states(FAKE, FAKE, FAKE, 1 << 30, 2, 1, 256, 64, 64, 0, 64, 2, 0,
                                 None) == L.LA_ERR_INVALID_ARG
    assert lib.la_segment_scan(FAKE, 16, 2, 1, 64, 64, 2, 1, None, None, None) == L.LA_ERR_WORKSPACE
    assert lib.la_segment_scan(FAKE, 1 << 30, 2, 1, 64, 64, 2, 1, FAKE, None, None) == L.LA_ERR_INVALID_ARG
    assert lib.la_segment_outputs(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 2, 1, 256, 64, 64, 3, 0, 64, 2,
                                  None, None, None) == L.LA_ERR_INVALID_ARG


def test_fused_entry_point_checks(L):
    f = L.lib().la_forward_fused
    need = L.fused_workspace_bytes(2, 2, 64, 64, 4)
    # 1000 positions in chunks of 64: 16 chunks; 4 segments of 4 chunks
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 64, 4, None, None, FAKE, need - 4, None, None, None) == L.LA_ERR_WORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 64, 5, None, None, FAKE, 1 << 30, None, None, None) == L.LA_ERR_UNSUPPORTED  # a segment would own no chunk
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 48, 4, None, None, FAKE, need, None, None, None) == L.LA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 64, 0, None, None, FAKE, need, None, None, None) == L.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 64, 4, None, None, FAKE + 4, need, None, None, None) == L.LA_ERR_INVALID_ARG
    assert f(None, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 64, 4, None, None, FAKE, need, None, None, None) == L.LA_ERR_INVALID_ARG
    w = L.lib().la_workspace_init
    assert w(None, 0, None) == L.LA_OK
    assert w(None, 64, None) == L.LA_ERR_INVALID_ARG
    assert w(FAKE + 4, 64, None) == L.LA_ERR_INVALID_ARG
    assert w(FAKE, 66, None) == L.LA_ERR_INVALID_ARG


def test_onepass_entry_point_checks(L):
    f = L.lib().la_forward_onepass
    need = L.fused_workspace_bytes(2, 2, 64, 64, 2)
    # 1000 positions in chunks of 64: 16 chunks; 2 segments would hold 8 chunks each (> 4)
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 64, 2, None, None, FAKE, need, None, None, None) == L.LA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 64, 17, None, None, FAKE, 1 << 30, None, None, None) == L.LA_ERR_UNSUPPORTED  # a segment would own no chunk
    need4 = L.fused_workspace_bytes(2, 2, 64, 64, 4)
    bf16 = 1
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, bf16, 64, 4, None, None, FAKE, need4 - 4, None, None, None) == L.LA_ERR_WORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, bf16, 64, 0, None, None, FAKE, need4, None, None, None) == L.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, bf16, 64, 4, None, None, FAKE, need4, FAKE, None, None) == L.LA_ERR_INVALID_ARG  # S_out without z_out
    # fp32 operands with 64-position chunks: the segment's phi(Q) tiles do not fit in LDS
    # (two workgroups per CU for D = M = 64, one for D = M = 128)
    for d in (64, 128):
        assert f(FAKE, FAKE, FAKE, FAKE, 1, 1, 256, d, d, 0, 64, 1, None, None, None, 0, None, None, None) == L.LA_ERR_UNSUPPORTED


def test_continue_entry_point_checks(L):
    f = L.lib().la_forward_continue
    need = L.lib().la_forward_workspace_bytes(2, 2, 1000, 64, 64, 1, 0, 0)
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 0, FAKE, None, FAKE, need, None, None,
             None) == L.LA_ERR_INVALID_ARG  # S_in without z_in
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 0, FAKE + 4, FAKE, FAKE, need, None, None,
             None) == L.LA_ERR_INVALID_ARG  # misaligned S_in
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 0, FAKE, FAKE, FAKE, need - 4, None, None,
             None) == L.LA_ERR_WORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 40, 64, 0, 0, FAKE, FAKE, FAKE, need, None, None,
             None) == L.LA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 3, 0, FAKE, FAKE, FAKE, need, None, None,
             None) == L.LA_ERR_INVALID_ARG  # dtype
    assert f(None, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, 0, FAKE, FAKE, FAKE, need, None, None,
             None) == L.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 2, 1000, 64, 64, 0, 0, FAKE, FAKE, None, 0, None, None, None) == L.LA_OK


def test_decode_steps_checks(L):
    f = L.lib().la_decode_steps
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, -1, 64, 64, 0, None) == L.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 8, 40, 64, 0, None) == L.LA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 8, 64, 64, 3, None) == L.LA_ERR_INVALID_ARG
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 8, 64, 64, 0, None) == L.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE + 4, FAKE, FAKE, FAKE, FAKE, 2, 2, 8, 64, 64, 0, None) == L.LA_ERR_INVALID_ARG
    assert f(None, None, None, None, None, None, 2, 2, 0, 64, 64, 0, None) == L.LA_OK  # T = 0


def test_softmax_scan_checks(L):
    f = L.lib().la_softmax_scan
    need = L.lib().la_softmax_scan_workspace_bytes(2, 2, 1000, 64, 64)
    items = 2 * 2 * 8  # groups of 128 positions
    assert need == (64 + 64 * ((items + 63) // 64)) * 4 + 2 * items * 128 * 4
    assert L.lib().la_softmax_scan_workspace_bytes(2, 2, 128, 64, 64) == 0  # one group per head
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 48, 64, 0, FAKE, need, None, None, None, None) == L.LA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 2, FAKE, need, None, None, None, None) == L.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, FAKE, need - 4, None, None, None,
             None) == L.LA_ERR_WORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, FAKE, need, FAKE, None, None,
             None) == L.LA_ERR_INVALID_ARG  # m_out without u_out, w_out
    assert f(None, FAKE, FAKE, FAKE, 2, 2, 1000, 64, 64, 0, FAKE, need, None, None, None, None) == L.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 0, 64, 64, 0, None, 0, None, None, None, None) == L.LA_OK
    g = L.lib().la_softmax_step
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 48, 0, None) == L.LA_ERR_UNSUPPORTED
    assert g(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 64, 0, None) == L.LA_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 64, 0, None) == L.LA_ERR_INVALID_ARG


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "efficient_transformer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text and "liboracle" not in text, f


def test_binding_fails_loudly_without_the_library(tmp_path):
    code = ("import efficient_transformer_amd.linattn as L; L.LIB_PATH = '/nonexistent/liblinattn.so'; L._lib = None\n"
            "try:\n    L.version()\nexcept RuntimeError as e:\n    print('raised', 'no fallback' in str(e))\n")
    r = subprocess.run(["python", "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert "raised True" in r.stdout, r.stdout + r.stderr


def test_feature_map_checks(L):
    f = L.lib().la_feature_map
    # out, X, out2, X2, rows, D, dtype, W, F, kind, flags, stream
    assert f(FAKE, FAKE, None, None, 100, 64, 0, FAKE, 16, 3, 0, None) == L.LA_ERR_INVALID_ARG  # kind
    assert f(FAKE, FAKE, None, None, 100, 64, 0, FAKE, 16, 1, 2, None) == L.LA_ERR_INVALID_ARG  # flag
    assert f(FAKE, FAKE, None, None, 100, 64, 0, None, 32, 0, 0, None) == L.LA_ERR_INVALID_ARG  # elu: F != D
    assert f(FAKE, FAKE, None, None, 100, 64, 2, FAKE, 16, 1, 0, None) == L.LA_ERR_INVALID_ARG  # dtype
    assert f(FAKE, FAKE, None, None, 100, 48, 0, FAKE, 16, 1, 0, None) == L.LA_ERR_UNSUPPORTED  # D
    assert f(FAKE, FAKE, None, None, 100, 64, 0, FAKE, 24, 1, 0, None) == L.LA_ERR_UNSUPPORTED  # F
    assert f(FAKE, FAKE, FAKE, None, 100, 64, 0, FAKE, 16, 1, 0, None) == L.LA_ERR_INVALID_ARG  # out2 alone
    assert f(FAKE, FAKE, None, None, 100, 64, 0, None, 16, 1, 0, None) == L.LA_ERR_INVALID_ARG  # PRF needs W
    assert f(FAKE, FAKE + 4, None, None, 100, 64, 0, FAKE, 16, 1, 0, None) == L.LA_ERR_INVALID_ARG  # alignment
    assert f(FAKE, FAKE, None, None, -1, 64, 0, FAKE, 16, 1, 0, None) == L.LA_ERR_INVALID_ARG
    assert f(None, None, None, None, 0, 64, 0, None, 16, 1, 0, None) == L.LA_OK  # no rows


def test_feature_map_backward_checks(L):
    f = L.lib().la_feature_map_backward
    # dX, X, dOut, rows, D, dtype, W, F, kind, flags, stream
    assert f(FAKE, FAKE, FAKE, 100, 64, 0, FAKE, 16, 3, 0, None) == L.LA_ERR_INVALID_ARG  # kind
    assert f(FAKE, FAKE, FAKE, 100, 64, 0, FAKE, 16, 1, 2, None) == L.LA_ERR_INVALID_ARG  # flag
    assert f(FAKE, FAKE, FAKE, 100, 64, 0, None, 32, 0, 0, None) == L.LA_ERR_INVALID_ARG  # elu: F != D
    assert f(FAKE, FAKE, FAKE, 100, 64, 2, FAKE, 16, 1, 0, None) == L.LA_ERR_INVALID_ARG  # dtype
    assert f(FAKE, FAKE, FAKE, 100, 48, 0, FAKE, 16, 1, 0, None) == L.LA_ERR_UNSUPPORTED  # D
    assert f(FAKE, FAKE, FAKE, 100, 64, 0, FAKE, 24, 1, 0, None) == L.LA_ERR_UNSUPPORTED  # F
    assert f(FAKE, FAKE, FAKE, 100, 64, 0, None, 16, 1, 0, None) == L.LA_ERR_INVALID_ARG  # PRF needs W
    assert f(None, FAKE, FAKE, 100, 64, 0, FAKE, 16, 1, 0, None) == L.LA_ERR_INVALID_ARG  # dX
    assert f(FAKE, FAKE, FAKE, -1, 64, 0, FAKE, 16, 1, 0, None) == L.LA_ERR_INVALID_ARG
    assert f(None, None, None, 0, 64, 0, None, 16, 1, 0, None) == L.LA_OK  # no rows


def test_feature_inputs_dtype(L):
    """LA_F32_FEATURES plans like fp32 (forward and backward), is refused by the softmax scan."""
    for D in (16, 64, 128):
        for M in (16, 64, 128):
            assert L.forward_plan(2, 3, 1000, D, M, 1, L.LA_F32_FEATURES, 0) == \
                L.forward_plan(2, 3, 1000, D, M, 1, L.LA_F32, 0)
    lib = L.lib()
    for (N, D, M) in ((100, 64, 64), (5000, 16, 128), (70000, 128, 32)):
        want = lib.la_backward_workspace_bytes(2, 2, N, D, M, L.LA_F32)
        assert want > 0 and lib.la_backward_workspace_bytes(2, 2, N, D, M, L.LA_F32_FEATURES) == want
    # refused before anything runs: a workspace one byte short, and a width without kernels
    need = lib.la_backward_workspace_bytes(2, 2, 100, 64, 64, L.LA_F32_FEATURES)
    assert lib.la_backward_chunked(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 100, 64, 64,
                                   L.LA_F32_FEATURES, FAKE, need - 1, None) == L.LA_ERR_WORKSPACE
    assert lib.la_backward_chunked(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 100, 48, 64,
                                   L.LA_F32_FEATURES, FAKE, 1 << 30, None) == L.LA_ERR_UNSUPPORTED
    assert lib.la_softmax_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 64, L.LA_F32_FEATURES,
                               None) == L.LA_ERR_INVALID_ARG
    assert lib.la_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 40, 64, L.LA_F32_FEATURES,
                              None) == L.LA_ERR_UNSUPPORTED  # accepted type, unsupported D


def test_bf16_output_flag(L):
    """LA_BF16 | LA_OUT_BF16 plans like LA_BF16; the flag is refused on other input types and by
    the entry points that do not write prefill outputs."""
    lib = L.lib()
    for D in (16, 64, 128):
        for M in (16, 64, 128):
            assert L.forward_plan(2, 3, 5000, D, M, 1, L.LA_BF16 | L.LA_OUT_BF16, 0) == \
                L.forward_plan(2, 3, 5000, D, M, 1, L.LA_BF16, 0)
    for bad in (L.LA_F32 | L.LA_OUT_BF16, L.LA_F32_FEATURES | L.LA_OUT_BF16):
        assert _fwd(L, Q=FAKE, K=FAKE, V=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30, dtype=bad) == L.LA_ERR_INVALID_ARG
    assert lib.la_backward_chunked(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 100, 64, 64,
                                   L.LA_BF16 | L.LA_OUT_BF16, FAKE, 1 << 30, None) == L.LA_ERR_UNSUPPORTED
    assert lib.la_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 64, L.LA_BF16 | L.LA_OUT_BF16,
                              None) == L.LA_ERR_INVALID_ARG


def test_forward_features_checks(L):
    lib = L.lib()
    wsb = lib.la_forward_features_workspace_bytes
    f = lib.la_forward_features
    # Q, K, V, out, B, H, N, D, M, causal, dtype, W, F, kind, flags, ws, ws_bytes, S_in, z_in, S_out, z_out, stream
    need = wsb(8, 8, 1024, 64, 64, 16, 1)
    assert need > 0
    assert wsb(8, 8, 1024, 48, 64, 16, 1) == 0 and wsb(8, 8, 1024, 64, 64, 24, 1) == 0  # D, F
    # no fused one-pass instantiation (F = 128), long segments, one-pass LDS too small: the map
    # and the attention as two launches, the features in the workspace (rows * F * 8 bytes and
    # rows * M * 4 for widened values besides the attention's own workspace)
    rows = 8 * 8 * 1024
    assert wsb(8, 8, 1024, 64, 64, 128, 1) >= rows * (128 * 8 + 64 * 4)
    assert wsb(8, 8, 1024, 64, 64, 128, 0) == 0  # non-causal: stage kernels, F up to 64
    assert wsb(1, 1, 1 << 20, 64, 64, 16, 1) >= (1 << 20) * (16 * 8 + 64 * 4)
    assert wsb(8, 8, 1024, 64, 64, 64, 1) >= rows * (64 * 8 + 64 * 4)
    assert wsb(-1, 8, 1024, 64, 64, 16, 1) == 0 and wsb(8, 8, 1024, 64, 64, 16, 2) == 0
    assert wsb(8, 8, 1024, 64, 64, 16, 0) > 0  # non-causal: the stage path

    def call(**kw):
        a = dict(Q=FAKE, K=FAKE, V=FAKE, out=FAKE, B=8, H=8, N=1024, D=64, M=64, causal=1, dtype=0, W=FAKE, F=16,
                 kind=1, flags=0, ws=FAKE, ws_bytes=need, Si=None, zi=None, S=None, z=None)
        a.update(kw)
        return f(a["Q"], a["K"], a["V"], a["out"], a["B"], a["H"], a["N"], a["D"], a["M"], a["causal"], a["dtype"],
                 a["W"], a["F"], a["kind"], a["flags"], a["ws"], a["ws_bytes"], a["Si"], a["zi"], a["S"], a["z"], None)

    assert call(dtype=2) == L.LA_ERR_INVALID_ARG  # raw rows: LA_F32 or LA_BF16 only
    assert call(dtype=1, ws_bytes=need - 1) == L.LA_ERR_WORKSPACE  # bf16 rows: the same plan
    assert call(kind=0) == L.LA_ERR_INVALID_ARG  # elu+1 is la_forward_chunked
    assert call(kind=3) == L.LA_ERR_INVALID_ARG
    assert call(flags=2) == L.LA_ERR_INVALID_ARG
    assert call(D=48) == L.LA_ERR_UNSUPPORTED
    assert call(F=128, causal=0) == L.LA_ERR_UNSUPPORTED
    assert call(F=128) == L.LA_ERR_WORKSPACE  # supported (two launches), with a larger workspace
    assert call(N=-1) == L.LA_ERR_INVALID_ARG
    assert call(S=FAKE) == L.LA_ERR_INVALID_ARG  # S_out without z_out
    assert call(causal=2) == L.LA_ERR_INVALID_ARG
    assert call(causal=0, S=FAKE, z=FAKE) == L.LA_ERR_INVALID_ARG  # states only with causal = 1
    assert call(causal=0, ws_bytes=0) == L.LA_ERR_WORKSPACE
    assert call(Si=FAKE) == L.LA_ERR_INVALID_ARG  # S_in without z_in
    assert call(Si=FAKE + 4, zi=FAKE) == L.LA_ERR_INVALID_ARG  # alignment
    assert call(W=None) == L.LA_ERR_INVALID_ARG
    assert call(V=FAKE + 4) == L.LA_ERR_INVALID_ARG
    assert call(ws_bytes=need - 1) == L.LA_ERR_WORKSPACE
    assert call(ws=None) == L.LA_ERR_WORKSPACE
    assert call(B=0) == L.LA_OK  # no heads: nothing to do


def test_decode_step_features_checks(L):
    f = L.lib().la_decode_step_features
    # S, z, q, k, v, out, B, H, D, M, dtype, W, F, kind, flags, stream
    a = [FAKE] * 6 + [2, 2, 64, 64, 0, FAKE, 16, 1, 0, None]

    def call(i, val):
        b = list(a)
        b[i] = val
        return f(*b)

    assert call(10, 2) == L.LA_ERR_INVALID_ARG  # dtype: raw rows only
    assert call(13, 0) == L.LA_ERR_INVALID_ARG  # elu+1 is la_decode_step
    assert call(14, 2) == L.LA_ERR_INVALID_ARG  # flag
    assert call(12, 128) == L.LA_ERR_UNSUPPORTED  # F
    assert call(8, 48) == L.LA_ERR_UNSUPPORTED  # D
    assert call(11, None) == L.LA_ERR_INVALID_ARG  # W
    assert call(4, FAKE + 4) == L.LA_ERR_INVALID_ARG  # alignment
    assert call(6, 0) == L.LA_OK  # no heads


def test_probe_checks(L):
    lib = L.lib()
    assert lib.la_probe_copy(None, None, 0, None) == L.LA_OK
    assert lib.la_probe_copy(None, None, 20, None) == L.LA_ERR_INVALID_ARG
    assert lib.la_probe_copy(None, None, 32, None) == L.LA_ERR_INVALID_ARG
    assert lib.la_probe_copy(16, 17, 32, None) == L.LA_ERR_INVALID_ARG
    assert lib.la_probe_read_partials() == 1024 * 256
    assert lib.la_probe_read(None, None, 0, None) == L.LA_ERR_INVALID_ARG  # no out
    assert lib.la_probe_read(FAKE, None, 16, None) == L.LA_ERR_INVALID_ARG  # no src
    assert lib.la_probe_read(FAKE, FAKE, 20, None) == L.LA_ERR_INVALID_ARG  # not whole 16-byte words
    assert lib.la_probe_read(FAKE + 2, FAKE, 32, None) == L.LA_ERR_INVALID_ARG  # misaligned out
    assert lib.la_probe_read(FAKE, FAKE + 8, 32, None) == L.LA_ERR_INVALID_ARG  # misaligned src
    assert lib.la_probe_mfma(None, L.LA_F32, 0, 10, 0.5, None) == L.LA_OK
    assert lib.la_probe_mfma(None, L.LA_F32, 4, 10, 0.5, None) == L.LA_ERR_INVALID_ARG
    assert lib.la_probe_mfma(None, 7, 4, 10, 0.5, None) == L.LA_ERR_INVALID_ARG
    assert lib.la_probe_mfma(None, L.LA_BF16, -1, 10, 0.5, None) == L.LA_ERR_INVALID_ARG
    assert lib.la_probe_mfma(None, L.LA_BF16, 1 << 21, 10, 0.5, None) == L.LA_ERR_INVALID_ARG
    assert lib.la_probe_mfma(None, L.LA_BF16, 4, -1, 0.5, None) == L.LA_ERR_INVALID_ARG

