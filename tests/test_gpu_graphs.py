"""The entry points under HIP graph capture: a captured call replayed several times,
with eager work (new inputs written by torch) and synchronisations between the
replays, must give every time what the same eager call gives.  The causal kernels
keep an epoch in their workspace (advanced by the kernels themselves), so a
replayed look-back never reads flags of an earlier replay; workspaces are zeroed
with a fill kernel, never a memset node."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import TOL, rowwise_rel, to_dev

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def inputs(B, H, N, D, M, seed, dtype="f32"):
    cfg = dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype=dtype, chunk=0)
    return synthetic.prefill_inputs(cfg, seed)


@pytest.mark.parametrize("shape", [(8, 8, 1024, 64, 64), (1, 4, 8192, 64, 64), (2, 2, 300, 32, 128)])
def test_forward_replays(ea, shape):
    """One captured la_forward_chunked call (one-pass or two-phase kernel, several
    segments per head: look-back and epoch), replayed with new inputs each time."""
    B, H, N, D, M = shape
    Qd = torch.empty((B, H, N, D), device=DEV)
    Kd = torch.empty((B, H, N, D), device=DEV)
    Vd = torch.empty((B, H, N, M), device=DEV)
    out = torch.empty((B, H, N, M), device=DEV)
    C, G, need = ea.forward_plan(B, H, N, D, M, True, 0, 0)
    assert G > 1
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV)
    Qd.copy_(to_dev(inputs(B, H, N, D, M, 80)[0], "f32"))
    Kd.copy_(Qd)
    Vd.normal_()
    ea.forward_chunked(Qd, Kd, Vd, out=out, workspace=ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ea.forward_chunked(Qd, Kd, Vd, out=out, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        Q, K, V = inputs(B, H, N, D, M, 81 + rep)
        Qd.copy_(to_dev(Q, "f32"))
        Kd.copy_(to_dev(K, "f32"))
        Vd.copy_(to_dev(V, "f32"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = ea.forward_chunked(Qd, Kd, Vd)
        torch.cuda.synchronize()
        assert rowwise_rel(got.cpu().numpy(), eager.cpu().numpy()) <= 1e-5, rep
        if rep == 0 and B * H <= 4:
            assert rowwise_rel(got.cpu().numpy(), oracle.causal(Q, K, V)[0]) <= TOL["f32"]


def test_forward_replays_long_head_bf16(ea):
    """A captured call of the two-phase kernel on 32x32x16 tiles (bf16, D = M = 128:
    128 segments of 8 chunks per head), replayed with new inputs each time."""
    B, H, N, D, M = 1, 2, 65536, 128, 128
    code = ea.linattn.LA_BF16
    C, G, need = ea.forward_plan(B, H, N, D, M, True, code, 0)
    assert C == 64 and -(-(-(-N // C)) // G) > 4
    Qd = torch.empty((B, H, N, D), device=DEV, dtype=torch.bfloat16)
    Kd = torch.empty_like(Qd)
    Vd = torch.empty((B, H, N, M), device=DEV, dtype=torch.bfloat16)
    out = torch.empty((B, H, N, M), device=DEV)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)

    def load(seed):
        Q, K, V = inputs(B, H, N, D, M, seed, "bf16")
        Qd.copy_(to_dev(Q, "bf16"))
        Kd.copy_(to_dev(K, "bf16"))
        Vd.copy_(to_dev(V, "bf16"))
        return Q, K, V

    load(85)
    ea.forward_chunked(Qd, Kd, Vd, out=out, workspace=ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ea.forward_chunked(Qd, Kd, Vd, out=out, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        print(f"long-head bf16 replay {rep}", flush=True)
        Q, K, V = load(86 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = ea.forward_chunked(Qd, Kd, Vd)
        torch.cuda.synchronize()
        assert rowwise_rel(got.cpu().numpy(), eager.cpu().numpy()) <= 1e-5, rep
        if rep == 0:  # the first 4096 rows of head 0 depend only on themselves
            n = 4096
            ref = oracle.causal(*(synthetic.as_f64(x[:, :1, :n], "bf16") for x in (Q, K, V)))[0]
            assert rowwise_rel(got[:, :1, :n].cpu().numpy(), ref) <= TOL["bf16"]


def test_decode_replays(ea):
    """A captured la_decode_step (state updated in place) replayed T times equals T
    eager steps; the inputs change between replays."""
    B, H, D, M, T = 16, 4, 64, 64, 12
    cfg = dict(kind="decode", B=B, H=H, D=D, M=M, sigma=1.0, dtype="f32")
    q, k, v = synthetic.decode_inputs(cfg, 3, 0, T)
    S1 = torch.zeros((B, H, D, M), device=DEV)
    z1 = torch.zeros((B, H, D), device=DEV)
    qd = torch.empty((B, H, D), device=DEV)
    kd = torch.empty((B, H, D), device=DEV)
    vd = torch.empty((B, H, M), device=DEV)
    out = torch.empty((B, H, M), device=DEV)
    graph = torch.cuda.CUDAGraph()
    Sw, zw = S1.clone(), z1.clone()
    ea.decode_step(Sw, zw, qd.zero_(), kd.zero_(), vd.zero_(), out=out)  # warm-up on scratch state
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        ea.decode_step(S1, z1, qd, kd, vd, out=out)
    S2, z2 = torch.zeros_like(S1), torch.zeros_like(z1)
    for t in range(T):
        qd.copy_(to_dev(q[t], "f32"))
        kd.copy_(to_dev(k[t], "f32"))
        vd.copy_(to_dev(v[t], "f32"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        want = ea.decode_step(S2, z2, qd, kd, vd)
        torch.cuda.synchronize()
        assert torch.equal(got, want), t  # the same kernel on the same state: bit for bit
    assert torch.equal(S1, S2) and torch.equal(z1, z2)


def test_softmax_scan_replays(ea):
    """The softmax scan keeps its epoch in the workspace as well."""
    B, H, N, D, M = 2, 4, 2000, 64, 64
    rng = np.random.default_rng(5)
    qd = torch.empty((B, H, D), device=DEV)
    Kd = torch.empty((B, H, N, D), device=DEV)
    Vd = torch.empty((B, H, N, M), device=DEV)
    out = torch.empty((B, H, N, M), device=DEV)
    wsb = int(ea.linattn.lib().la_softmax_scan_workspace_bytes(B, H, N, D, M))
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=DEV)
    qd.zero_()
    Kd.zero_()
    Vd.zero_()
    ea.softmax_scan(qd, Kd, Vd, out=out, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ea.softmax_scan(qd, Kd, Vd, out=out, workspace=ws)
    for rep in range(3):
        q = (rng.normal(size=(B, H, D)) * 0.125).astype(np.float32)
        K = rng.normal(size=(B, H, N, D)).astype(np.float32)
        V = rng.normal(size=(B, H, N, M)).astype(np.float32)
        qd.copy_(torch.from_numpy(q))
        Kd.copy_(torch.from_numpy(K))
        Vd.copy_(torch.from_numpy(V))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        want = oracle.softmax_scan(q, K, V)[0]
        assert rowwise_rel(got, want) <= TOL["f32"], rep


@pytest.mark.parametrize("N", [1024, 65536])
def test_forward_features_replays(ea, N):
    """A captured la_forward_features call (one-pass plan at N = 1024, two-phase at
    N = 65536; look-back and epoch in both) and a captured la_decode_step_features
    step, replayed with new raw rows written eagerly between the replays."""
    B, H, D, M, F = (8, 8, 64, 64, 16) if N == 1024 else (1, 2, 64, 64, 16)
    W = torch.from_numpy(ea.draw_projection(F, D, "orthogonal", 4)).to(DEV)
    Qd = torch.zeros((B, H, N, D), device=DEV)
    Kd = torch.zeros((B, H, N, D), device=DEV)
    Vd = torch.zeros((B, H, N, M), device=DEV)
    out = torch.empty((B, H, N, M), device=DEV)
    need = int(ea.linattn.lib().la_forward_features_workspace_bytes(B, H, N, D, M, F, 1))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    S = torch.empty((B, H, F, M), device=DEV)
    z = torch.empty((B, H, F), device=DEV)
    ea.forward_features(Qd, Kd, Vd, W, F, "prf", out=out, workspace=ws, S_out=S, z_out=z)  # warm-up
    qd = torch.zeros((B, H, D), device=DEV)
    kd = torch.zeros((B, H, D), device=DEV)
    vd = torch.zeros((B, H, M), device=DEV)
    y = torch.empty((B, H, M), device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ea.forward_features(Qd, Kd, Vd, W, F, "prf", out=out, workspace=ws, S_out=S, z_out=z)
        ea.decode_step_features(S, z, qd, kd, vd, W, F, "prf", out=y)
    torch.cuda.synchronize()
    s = 64 ** -0.25
    for rep in range(3):
        Qd.copy_(synthetic.draw_torch(120 + rep, synthetic.TID_Q, (B, H, N, D), s, "f32", DEV))
        Kd.copy_(synthetic.draw_torch(120 + rep, synthetic.TID_K, (B, H, N, D), s, "f32", DEV))
        Vd.copy_(synthetic.draw_torch(120 + rep, synthetic.TID_V, (B, H, N, M), 1.0, "f32", DEV))
        qd.copy_(synthetic.draw_torch(130 + rep, synthetic.TID_DQ, (B, H, D), s, "f32", DEV))
        kd.copy_(synthetic.draw_torch(130 + rep, synthetic.TID_DK, (B, H, D), s, "f32", DEV))
        vd.copy_(synthetic.draw_torch(130 + rep, synthetic.TID_DV, (B, H, M), 1.0, "f32", DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got, got_y, got_S = out.clone(), y.clone(), S.clone()
        S2 = torch.empty_like(S)
        z2 = torch.empty_like(z)
        want = ea.forward_features(Qd, Kd, Vd, W, F, "prf", S_out=S2, z_out=z2)
        want_y = ea.decode_step_features(S2, z2, qd, kd, vd, W, F, "prf")
        torch.cuda.synchronize()
        assert rowwise_rel(got.cpu().numpy(), want.cpu().numpy()) <= 1e-5, rep
        assert rowwise_rel(got_y.cpu().numpy(), want_y.cpu().numpy()) <= 1e-5, rep
        assert torch.allclose(got_S, S2, rtol=1e-5, atol=1e-6), rep
