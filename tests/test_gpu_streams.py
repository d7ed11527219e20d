"""Calls on two streams at once.  The binding keeps one cached workspace per
(device, stream, plan), so look-back calls that overlap on two streams never
share flags or slots; their workgroups only wait on earlier-dispatched
workgroups of their own call, so concurrent kernels cannot block each other.
Every result must equal the same call made alone."""
import pytest
import torch

import synthetic
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def prefill(seed, B=8, H=8, N=1024, D=64, M=64):
    cfg = dict(kind="prefill", B=B, H=H, N=N, D=D, M=M, sigma=1.0, dtype="f32", chunk=0)
    return tuple(to_dev(x, "f32") for x in synthetic.prefill_inputs(cfg, seed))


def test_prefill_on_two_streams(ea):
    """Headline-shaped calls (8 segments per head) and long-head calls (two-phase
    kernel) interleaved on two streams."""
    sets = [prefill(100), prefill(101), prefill(102, B=1, H=2, N=65536), prefill(103, B=1, H=2, N=65536)]
    alone = [ea.forward_chunked(*x) for x in sets]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    main = torch.cuda.current_stream()
    s1.wait_stream(main)
    s2.wait_stream(main)
    outs = [[], []]
    for rep in range(5):
        for i, x in enumerate(sets):
            st = s1 if i % 2 == 0 else s2
            with torch.cuda.stream(st):
                outs[i % 2].append((i, ea.forward_chunked(*x, stream=st)))
    torch.cuda.synchronize()
    for lst in outs:
        for i, o in lst:
            assert torch.allclose(o, alone[i], rtol=1e-5, atol=1e-6), i


def test_scan_and_features_on_two_streams(ea):
    B, H, N, D, M, F = 8, 8, 2048, 64, 64, 16
    q = synthetic.draw_torch(7, 9, (B, H, D), 0.125, "f32", DEV)
    K = synthetic.draw_torch(7, synthetic.TID_K, (B, H, N, D), 1.0, "f32", DEV)
    V = synthetic.draw_torch(7, synthetic.TID_V, (B, H, N, M), 1.0, "f32", DEV)
    Xq = K * (64 ** -0.25)
    W = torch.from_numpy(ea.draw_projection(F, D, "orthogonal", 3)).to(DEV)
    scan_alone = ea.softmax_scan(q, K, V)
    feat_alone = ea.forward_features(Xq, K * (64 ** -0.25), V, W, F, "prf")
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    main = torch.cuda.current_stream()
    s1.wait_stream(main)
    s2.wait_stream(main)
    scans, feats = [], []
    Kf = K * (64 ** -0.25)
    torch.cuda.synchronize()
    for rep in range(5):
        with torch.cuda.stream(s1):
            scans.append(ea.softmax_scan(q, K, V, stream=s1))
        with torch.cuda.stream(s2):
            feats.append(ea.forward_features(Xq, Kf, V, W, F, "prf", stream=s2))
    torch.cuda.synchronize()
    for o in scans:
        assert torch.allclose(o, scan_alone, rtol=1e-5, atol=1e-6)
    for o in feats:
        assert torch.allclose(o, feat_alone, rtol=1e-5, atol=1e-6)
