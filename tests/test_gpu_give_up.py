"""The give-up path of the bounded look-back waits, forced from the host: word 4
of the workspace header caps every wait at one poll, so workgroups whose
predecessors have not published yet give up.  Every kernel still ends; the
rows (and final states) that lost their prefix are NaN, the error word (word 3)
is set, every row that is not NaN equals the normal call's, and after the
workspace is zeroed again the next call is whole.  la_workspace_status (and the
binding's check after a call) reports the give-up exactly when the word is set."""
import pytest
import torch

import synthetic
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ERROR_WORD, CAP_WORD = 3, 4


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def check_rows(got, want, rows_ok):
    """Rows that are not NaN equal the normal result; returns the NaN row mask."""
    nan_rows = torch.isnan(got).any(dim=-1)
    assert not torch.isnan(got[~nan_rows]).any()
    assert torch.allclose(got[~nan_rows], want[~nan_rows], rtol=1e-5, atol=1e-6)
    assert not nan_rows[rows_ok].any()
    return nan_rows


@pytest.mark.parametrize("dtype,shape", [("f32", (8, 8, 1024, 64, 64)), ("f32", (1, 4, 8192, 64, 64)),
                                         ("f32", (1, 2, 65536, 64, 64)), ("bf16", (1, 2, 65536, 128, 128))])
def test_forward_gives_up_cleanly(ea, dtype, shape):
    """In-order look-back (8 segments per head), inclusive look-back (one-pass
    kernel with 128 segments), the two-phase kernel, and the two-phase kernel on
    32x32x16 tiles (bf16, D = M = 128: 128 segments of 8 chunks per head)."""
    B, H, N, D, M = shape
    print(f"give-up {dtype} {shape}", flush=True)
    cfg = dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype=dtype, chunk=0)
    Q, K, V = (to_dev(x, dtype) for x in synthetic.prefill_inputs(cfg, 90))
    code = ea.linattn.LA_F32 if dtype == "f32" else ea.linattn.LA_BF16
    C, G, need = ea.forward_plan(B, H, N, D, M, True, code, 0)
    assert G > 1
    if dtype == "bf16":
        assert C == 64 and -(-(-(-N // C)) // G) > 4  # segments of more than 4 chunks: the two-phase kernel
    want = ea.forward_chunked(Q, K, V)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    words = ws.view(torch.int32)
    words[CAP_WORD] = 1
    S = torch.empty((B, H, D, M), device=DEV)
    z = torch.empty((B, H, D), device=DEV)
    got = ea.forward_chunked(Q, K, V, workspace=ws, S_out=S, z_out=z)
    torch.cuda.synchronize()
    n_chunks = -(-N // C)
    first_rows = torch.zeros(N, dtype=torch.bool, device=DEV)
    first_rows[: min(N, C * (-(-n_chunks // G)))] = True  # segment 0 never waits
    nan_rows = check_rows(got, want, first_rows.expand(B, H, N))
    failed = int(words[ERROR_WORD].item()) != 0
    assert failed == bool(nan_rows.any())
    if not failed:
        pytest.skip("every predecessor had published at the first poll")
    # a head whose rows lost their prefix near the end also has a NaN final state
    last_nan = nan_rows[:, :, -1]
    assert torch.isnan(S).any(dim=(-1, -2)).eq(last_nan).all()
    # the C ABI reports it, and so does the binding's check after a call
    with pytest.raises(ea.LinAttnError) as info:
        ea.workspace_status(ws)
    assert info.value.status == ea.linattn.LA_ERR_GAVE_UP
    with pytest.raises(ea.LinAttnError):
        ea.forward_chunked(Q, K, V, workspace=ws, check=True)
    # zeroed again, the workspace serves a whole call
    ws.zero_()
    again = ea.forward_chunked(Q, K, V, workspace=ws, check=True)
    torch.cuda.synchronize()
    assert int(words[ERROR_WORD].item()) == 0
    ea.workspace_status(ws)
    assert torch.allclose(again, want, rtol=1e-5, atol=1e-6)


def test_softmax_scan_gives_up_cleanly(ea):
    B, H, N, D, M = 8, 8, 4096, 64, 64
    q = synthetic.draw_torch(6, 9, (B, H, D), 0.125, "f32", DEV)
    K = synthetic.draw_torch(6, synthetic.TID_K, (B, H, N, D), 1.0, "f32", DEV)
    V = synthetic.draw_torch(6, synthetic.TID_V, (B, H, N, M), 1.0, "f32", DEV)
    want = ea.softmax_scan(q, K, V)
    wsb = int(ea.linattn.lib().la_softmax_scan_workspace_bytes(B, H, N, D, M))
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    words = ws.view(torch.int32)
    words[CAP_WORD] = 1
    got = ea.softmax_scan(q, K, V, workspace=ws)
    torch.cuda.synchronize()
    first_rows = torch.zeros(N, dtype=torch.bool, device=DEV)
    first_rows[:128] = True  # the first group never waits
    nan_rows = check_rows(got, want, first_rows.expand(B, H, N))
    failed = int(words[ERROR_WORD].item()) != 0
    assert failed == bool(nan_rows.any())
    if not failed:
        pytest.skip("every earlier group had published at the first poll")
    with pytest.raises(ea.LinAttnError) as info:
        ea.workspace_status(ws)
    assert info.value.status == ea.linattn.LA_ERR_GAVE_UP
    ws.zero_()
    again = ea.softmax_scan(q, K, V, workspace=ws)
    torch.cuda.synchronize()
    ea.workspace_status(ws)
    assert torch.allclose(again, want, rtol=1e-5, atol=1e-6)


def test_status_of_a_clean_workspace(ea):
    """Normal calls leave the error word clear; the binding's check passes."""
    B, H, N, D, M = 2, 4, 8192, 64, 64
    cfg = dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype="f32", chunk=0)
    Q, K, V = (to_dev(x, "f32") for x in synthetic.prefill_inputs(cfg, 91))
    _, G, need = ea.forward_plan(B, H, N, D, M, True, 0, 0)
    assert G > 1
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for _ in range(3):
        ea.forward_chunked(Q, K, V, workspace=ws, check=True)
    ea.workspace_status(ws)
