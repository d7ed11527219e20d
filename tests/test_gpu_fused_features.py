"""Causal attention with the random-feature map inside the attention kernel
(la_forward_features) against the fp64 oracle: oracle.feature_map forms the
features of the same raw rows with the same projection W, oracle.attention_mapped
the running sums over them (page "Stable, Fast and Accurate: Kernelized Attention
with Relative Positional Encoding": PRF and TRF features, Sphere-PRF and ORF
draws, normalised rows; page "Transformers are RNNs": the causal running sums).

Outputs are held to the fp32 tolerance 1e-4 row-wise, the final state S, z to
1e-5 over the whole tensor; against the two-launch path (la_feature_map then
la_forward_chunked on the features, the same fp32 arithmetic in another order)
to 1e-5 row-wise.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import TOL, rowwise_rel, to_dev, whole_rel

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
W_ROWS = {"prf": lambda F: F, "trf": lambda F: F // 2}
# TRF features can be negative; inputs at a fifth of the unit scale keep every
# denominator away from zero (cosines dominate), as the estimator needs.
KIND_SCALE = {"prf": 1.0, "trf": 0.2}


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ea


def supported(ea, B, H, N, D, M, F, causal=True):
    return int(ea.linattn.lib().la_forward_features_workspace_bytes(B, H, N, D, M, F, int(causal))) > 0


def case(ea, B, H, N, D, M, F, kind, seed, normalize=False, draw="gaussian", scale=None):
    """Seeded raw X_q, X_k, V and W -> device tensors and the fp64 oracle's
    (out, S, z) over the oracle's own features."""
    s = (KIND_SCALE[kind] if scale is None else scale) * D ** -0.25
    Xq = synthetic.draw(seed, synthetic.TID_Q, (B, H, N, D), s, "f32")
    Xk = synthetic.draw(seed, synthetic.TID_K, (B, H, N, D), s, "f32")
    V = synthetic.draw(seed, synthetic.TID_V, (B, H, N, M), 1.0, "f32")
    W = ea.draw_projection(W_ROWS[kind](F), D, draw, seed + 1)
    dev = tuple(to_dev(x, "f32") for x in (Xq, Xk, V)) + (torch.from_numpy(W).to(DEV),)
    return dev, (Xq, Xk, V, W)


def oracle_out(host, F, kind, normalize, causal=True):
    Xq, Xk, V, W = host
    W64 = W.astype(np.float64)
    Fq = oracle.feature_map(Xq.astype(np.float64), W64, F, kind, normalize)
    Fk = oracle.feature_map(Xk.astype(np.float64), W64, F, kind, normalize)
    return oracle.attention_mapped(Fq, Fk, V.astype(np.float64), causal)


def run(ea, dev, F, kind, normalize, with_state=True):
    Qd, Kd, Vd, Wd = dev
    B, H, N, D = Qd.shape
    M = Vd.shape[-1]
    S = torch.full((B, H, F, M), float("nan"), device=DEV) if with_state else None
    z = torch.full((B, H, F), float("nan"), device=DEV) if with_state else None
    out = ea.forward_features(Qd, Kd, Vd, Wd, F, kind, normalize, S_out=S, z_out=z)
    return out, S, z


def check(out, S, z, ref):
    torch.cuda.synchronize()
    ref_out, S_ref, z_ref = ref
    err = rowwise_rel(out.cpu().numpy(), ref_out)
    assert err <= TOL["f32"], f"out {err:.3e}"
    if S is not None:
        assert whole_rel(S.cpu().numpy(), S_ref) <= 1e-5
        assert whole_rel(z.cpu().numpy(), z_ref) <= 1e-5


@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("kind", ["prf", "trf"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("F,M", [(16, 64), (32, 32), (16, 128), (32, 16), (64, 16), (128, 64)])
def test_fused_features_parity(ea, normalize, kind, D, F, M):
    """N = 300: nine full chunks of 32 and a ragged one, several segments per head."""
    B, H, N = 1, 3, 300
    assert supported(ea, B, H, N, D, M, F)
    dev, host = case(ea, B, H, N, D, M, F, kind, 50 + D + F, normalize)
    out, S, z = run(ea, dev, F, kind, normalize)
    check(out, S, z, oracle_out(host, F, kind, normalize))


def test_supported_shapes(ea):
    """Every (D, F, M) of widths 16 .. 128 is supported causally: the fused one-pass kernel
    where it is instantiated (F up to 64) and its LDS fits, else the map and the attention
    kernels as two launches; non-causal attention has F up to 64."""
    for D in (16, 32, 64, 128):
        for F in (16, 32, 64, 128):
            for M in (16, 32, 64, 128):
                assert supported(ea, 8, 8, 1024, D, M, F), (D, F, M)
                assert supported(ea, 8, 8, 1024, D, M, F, causal=False) == (F <= 64), (D, F, M)


@pytest.mark.parametrize("N", [1, 31, 32, 33, 127, 128, 129])
def test_fused_features_short_and_ragged(ea, N):
    B, H, D, M, F = 2, 2, 64, 64, 16
    dev, host = case(ea, B, H, N, D, M, F, "prf", 60)
    out, S, z = run(ea, dev, F, "prf", False)
    check(out, S, z, oracle_out(host, F, "prf", False))


@pytest.mark.parametrize("draw", ["gaussian", "orthogonal", "sphere"])
def test_fused_features_draws(ea, draw):
    B, H, N, D, M, F = 2, 2, 500, 64, 32, 32
    dev, host = case(ea, B, H, N, D, M, F, "prf", 61, draw=draw)
    out, S, z = run(ea, dev, F, "prf", False)
    check(out, S, z, oracle_out(host, F, "prf", False))


@pytest.mark.parametrize("kind", ["prf", "trf"])
@pytest.mark.parametrize("normalize", [False, True])
def test_fused_matches_two_launches(ea, kind, normalize):
    """Against la_feature_map + la_forward_chunked(LA_F32_FEATURES) on the same rows."""
    B, H, N, D, M, F = 4, 4, 1000, 64, 64, 16
    dev, _ = case(ea, B, H, N, D, M, F, kind, 62, normalize)
    Qd, Kd, Vd, Wd = dev
    out, S, z = run(ea, dev, F, kind, normalize)
    fq, fk = ea.feature_map(Qd, Wd, F, kind, normalize, X2=Kd)
    S2 = torch.empty_like(S)
    z2 = torch.empty_like(z)
    two = ea.forward_chunked(fq, fk, Vd, causal=True, S_out=S2, z_out=z2, features=True)
    torch.cuda.synchronize()
    assert rowwise_rel(out.cpu().numpy(), two.cpu().numpy()) <= 1e-5
    assert whole_rel(S.cpu().numpy(), S2.cpu().numpy()) <= 1e-6
    assert whole_rel(z.cpu().numpy(), z2.cpu().numpy()) <= 1e-6


def test_fused_features_zero_rows_and_empty(ea):
    """A zero row under normalisation stays finite; N = 0 writes a zero state."""
    B, H, N, D, M, F = 1, 2, 200, 32, 32, 16
    dev, host = case(ea, B, H, N, D, M, F, "prf", 63, True)
    dev[0][0, 1, 17] = 0.0
    dev[1][0, 0, 5] = 0.0
    host[0][0, 1, 17] = 0.0
    host[1][0, 0, 5] = 0.0
    out, S, z = run(ea, dev, F, "prf", True)
    check(out, S, z, oracle_out(host, F, "prf", True))
    assert torch.isfinite(out).all()
    e = torch.empty((B, H, 0, D), device=DEV)
    S0 = torch.full((B, H, F, M), float("nan"), device=DEV)
    z0 = torch.full((B, H, F), float("nan"), device=DEV)
    ea.forward_features(e, e, torch.empty((B, H, 0, M), device=DEV), dev[3], F, "prf", S_out=S0, z_out=z0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S0).item() == 0 and torch.count_nonzero(z0).item() == 0


def test_fused_features_continue_with_decode(ea):
    """The fused prefill's state continued by decode steps on the two-launch features:
    every row equals the running sums over the whole sequence."""
    B, H, D, M, F = 2, 3, 64, 64, 16
    n0, n1 = 300, 20
    dev, host = case(ea, B, H, n0 + n1, D, M, F, "prf", 64)
    Qd, Kd, Vd, Wd = dev
    ref = oracle_out(host, F, "prf", False)[0]
    S = torch.empty((B, H, F, M), device=DEV)
    z = torch.empty((B, H, F), device=DEV)
    head = ea.forward_features(Qd[:, :, :n0].contiguous(), Kd[:, :, :n0].contiguous(), Vd[:, :, :n0].contiguous(),
                               Wd, F, "prf", S_out=S, z_out=z)
    fq, fk = ea.feature_map(Qd[:, :, n0:].contiguous(), Wd, F, "prf", X2=Kd[:, :, n0:].contiguous())
    tail = ea.decode_steps(S, z, fq, fk, Vd[:, :, n0:].contiguous(), features=True)
    torch.cuda.synchronize()
    assert rowwise_rel(head.cpu().numpy(), ref[:, :, :n0]) <= TOL["f32"]
    assert rowwise_rel(tail.cpu().numpy(), ref[:, :, n0:]) <= TOL["f32"]


def test_fused_features_workload(ea):
    """The random-feature workload (B=8, H=8, N=1024, D=M=64, 16 PRF features,
    orthogonal projection) in the launch configuration the benchmark times: two
    heads against the oracle, every head against the two-launch path."""
    cfg = synthetic.WORKLOADS["prefill_prf16_f32_b8h8_n1024_d64"]
    B, H, N, D, M, F = (cfg[k] for k in ("B", "H", "N", "D", "M", "F"))
    Xq = synthetic.draw(30, synthetic.TID_Q, (B, H, N, D), cfg["sigma"], "f32")
    Xk = synthetic.draw(30, synthetic.TID_K, (B, H, N, D), cfg["sigma"], "f32")
    V = synthetic.draw(30, synthetic.TID_V, (B, H, N, M), 1.0, "f32")
    W = ea.draw_projection(F, D, "orthogonal", 0)
    Qd, Kd, Vd = (to_dev(x, "f32") for x in (Xq, Xk, V))
    Wd = torch.from_numpy(W).to(DEV)
    out = ea.forward_features(Qd, Kd, Vd, Wd, F, "prf")
    fq, fk = ea.feature_map(Qd, Wd, F, "prf", X2=Kd)
    two = ea.forward_chunked(fq, fk, Vd, causal=True, features=True)
    torch.cuda.synchronize()
    assert rowwise_rel(out.cpu().numpy(), two.cpu().numpy()) <= 1e-5
    sel = (slice(3, 4), slice(5, 7))
    ref = oracle_out((Xq[sel], Xk[sel], V[sel], W), F, "prf", False)[0]
    assert rowwise_rel(out[sel].cpu().numpy(), ref) <= TOL["f32"]


def bf16_case(ea, B, H, N, D, M, F, kind, seed, normalize=False):
    """bf16 raw rows and V; the oracle gets their exact fp64 images."""
    s = KIND_SCALE[kind] * D ** -0.25
    Xq = synthetic.draw(seed, synthetic.TID_Q, (B, H, N, D), s, "bf16")
    Xk = synthetic.draw(seed, synthetic.TID_K, (B, H, N, D), s, "bf16")
    V = synthetic.draw(seed, synthetic.TID_V, (B, H, N, M), 1.0, "bf16")
    W = ea.draw_projection(W_ROWS[kind](F), D, "gaussian", seed + 1)
    dev = tuple(to_dev(x, "bf16") for x in (Xq, Xk, V)) + (torch.from_numpy(W).to(DEV),)
    host = tuple(synthetic.as_f64(x, "bf16") for x in (Xq, Xk, V)) + (W,)
    return dev, host


@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("kind", ["prf", "trf"])
@pytest.mark.parametrize("D,F,M", [(64, 16, 64), (32, 32, 32), (128, 16, 128), (16, 64, 16)])
def test_fused_features_bf16_rows(ea, normalize, kind, D, F, M):
    """bf16 raw rows: widened exactly, then the same fp32 map and attention (fp32
    tolerance against the oracle on the same bf16 values)."""
    B, H, N = 2, 2, 300
    if not supported(ea, B, H, N, D, M, F):
        pytest.skip(f"D={D} F={F} M={M}: the kernel's LDS does not fit two workgroups per CU")
    dev, host = bf16_case(ea, B, H, N, D, M, F, kind, 70 + D, normalize)
    out, S, z = run(ea, dev, F, kind, normalize)
    check(out, S, z, oracle_out(host, F, kind, normalize))


@pytest.mark.parametrize("kind", ["prf", "trf"])
def test_fused_features_bf16_equals_widened_f32(ea, kind):
    """The bf16 kernel on bf16 rows and the fp32 kernel on the same values widened
    to fp32 run identical arithmetic: bit-identical outputs and states."""
    B, H, N, D, M, F = 4, 4, 1000, 64, 64, 16
    dev, _ = bf16_case(ea, B, H, N, D, M, F, kind, 71)
    out16, S16, z16 = run(ea, dev, F, kind, False)
    wide = tuple(x.float().contiguous() for x in dev[:3]) + (dev[3],)
    out32, S32, z32 = run(ea, wide, F, kind, False)
    torch.cuda.synchronize()
    assert torch.equal(out16, out32)
    assert torch.equal(S16, S32) and torch.equal(z16, z32)


def plan_is_onepass(B, H, N):
    """Whether la_forward_features' plan (chunks of 32, segments sized for 512
    workgroups) has segments of at most four chunks."""
    n = -(-N // 32)
    cps = max(1, -(-(n * B * H) // 512))
    G = -(-n // cps)
    return -(-n // G) <= 4


LONG = [(1, 2, 65536, 64, 16, 64), (2, 1, 40000, 32, 32, 32), (1, 1, 80000, 128, 16, 128)]


def two_phase_case(ea, kind, normalize, B, H, N, D, F, M, rows=None):
    """Runs la_forward_features on a plan without the one-pass kernel (two launches
    inside the entry point); checks it against the caller's own two launches (on the
    rows selected by `rows`, a function of the oracle inputs, if given)."""
    if not supported(ea, B, H, N, D, M, F):
        pytest.skip(f"D={D} F={F} M={M}: the kernel's LDS does not fit")
    assert not plan_is_onepass(B, H, N)
    dev, host = case(ea, B, H, N, D, M, F, kind, 80 + D, normalize)
    out, S, z = run(ea, dev, F, kind, normalize)
    Qd, Kd, Vd, Wd = dev
    fq, fk = ea.feature_map(Qd, Wd, F, kind, normalize, X2=Kd)
    two = ea.forward_chunked(fq, fk, Vd, causal=True, features=True)
    torch.cuda.synchronize()
    a, b = out.cpu().numpy(), two.cpu().numpy()
    mask = rows(host) if rows is not None else np.ones(a.shape[:-1], dtype=bool)
    assert rowwise_rel(a[mask], b[mask]) <= 1e-5
    return out, S, z, host, mask


@pytest.mark.parametrize("kind,normalize", [("prf", False), ("prf", True), ("trf", False)])
@pytest.mark.parametrize("B,H,N,D,F,M", LONG)
def test_fused_features_two_phase(ea, kind, normalize, B, H, N, D, F, M):
    """Long heads: segments of more than four chunks (ragged last chunk in the second
    shape) run as two launches inside the entry point: against the oracle and against
    the caller's two-launch path."""
    out, S, z, host, _ = two_phase_case(ea, kind, normalize, B, H, N, D, F, M)
    check(out, S, z, oracle_out(host, F, kind, normalize))


KAPPA_MAX = 30.0


def well_conditioned(F, kind, normalize):
    """Rows whose denominator sum cancels little: kappa_i = (|phi(q_i)| . sum_{j<=i}
    |phi(k_j)|) / |phi(q_i) . sum_{j<=i} phi(k_j)| (an upper bound on the sum of
    absolute terms over the absolute sum) at most KAPPA_MAX."""
    def rows(host):
        Xq, Xk, _, W = host
        W64 = W.astype(np.float64)
        Fq = oracle.feature_map(Xq.astype(np.float64), W64, F, kind, normalize)
        Fk = oracle.feature_map(Xk.astype(np.float64), W64, F, kind, normalize)
        den = np.abs(np.einsum("...f,...f->...", Fq, np.cumsum(Fk, axis=-2)))
        bound = np.einsum("...f,...f->...", np.abs(Fq), np.cumsum(np.abs(Fk), axis=-2))
        return bound <= KAPPA_MAX * den
    return rows


@pytest.mark.parametrize("B,H,N,D,F,M", LONG)
def test_fused_features_two_phase_trf_normalized(ea, B, H, N, D, F, M):
    """TRF on unit-length rows: the normalisation undoes the input scale that keeps
    TRF denominators away from zero, so some rows are ill-conditioned (their
    denominator sums cancel) and any two fp32 summation orders differ there
    beyond 1e-4.  The well-conditioned rows (cancellation factor at most 30) are
    held to the oracle and to the two-launch path; at least nine rows in ten of
    every head must qualify."""
    rows = well_conditioned(F, "trf", True)
    out, S, z, host, mask = two_phase_case(ea, "trf", True, B, H, N, D, F, M, rows)
    assert mask.mean(axis=-1).min() >= 0.9
    want = oracle_out(host, F, "trf", True)[0]
    err = rowwise_rel(out.cpu().numpy()[mask], want[mask])
    assert err <= TOL["f32"], f"{err:.3e}"


def test_fused_features_two_phase_bf16_equals_widened_f32(ea):
    B, H, N, D, M, F = 1, 2, 65536, 64, 64, 16
    assert not plan_is_onepass(B, H, N)
    dev, _ = bf16_case(ea, B, H, N, D, M, F, "prf", 81)
    out16, S16, z16 = run(ea, dev, F, "prf", False)
    wide = tuple(x.float().contiguous() for x in dev[:3]) + (dev[3],)
    out32, S32, z32 = run(ea, wide, F, "prf", False)
    torch.cuda.synchronize()
    assert torch.equal(out16, out32)
    assert torch.equal(S16, S32) and torch.equal(z16, z32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind,normalize", [("prf", False), ("prf", True), ("trf", False)])
@pytest.mark.parametrize("D,F,M", [(64, 16, 64), (32, 32, 128), (128, 64, 16)])
def test_decode_step_features(ea, dtype, kind, normalize, D, F, M):
    """Prefill with the map fused (la_forward_features, final state out), then
    decode steps on raw rows with the map formed in the decode kernel
    (la_decode_step_features): every decoded row equals the running sums of the
    whole sequence (oracle), and each step equals la_feature_map +
    la_decode_step on features."""
    B, H, n0, T = 2, 3, 200, 12
    N = n0 + T
    if dtype == "f32":
        dev, host = case(ea, B, H, N, D, M, F, kind, 90 + D, normalize)
    else:
        dev, host = bf16_case(ea, B, H, N, D, M, F, kind, 90 + D, normalize)
    Qd, Kd, Vd, Wd = dev
    ref = oracle_out(host, F, kind, normalize)[0]
    S = torch.empty((B, H, F, M), device=DEV)
    z = torch.empty((B, H, F), device=DEV)
    ea.forward_features(Qd[:, :, :n0].contiguous(), Kd[:, :, :n0].contiguous(), Vd[:, :, :n0].contiguous(), Wd, F,
                        kind, normalize, S_out=S, z_out=z)
    S2, z2 = S.clone(), z.clone()
    steps, steps2 = [], []
    for t in range(n0, N):
        q, k, v = (x[:, :, t].contiguous() for x in (Qd, Kd, Vd))
        steps.append(ea.decode_step_features(S, z, q, k, v, Wd, F, kind, normalize))
        fq, fk = ea.feature_map(q, Wd, F, kind, normalize, X2=k)
        steps2.append(ea.decode_step(S2, z2, fq, fk, v.float().contiguous(), features=True))
    torch.cuda.synchronize()
    got = torch.stack(steps, dim=2).cpu().numpy()
    two = torch.stack(steps2, dim=2).cpu().numpy()
    assert rowwise_rel(got, ref[:, :, n0:]) <= TOL["f32"]
    assert rowwise_rel(got, two) <= 1e-5
    assert whole_rel(S.cpu().numpy(), S2.cpu().numpy()) <= 1e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,n0,n1,D,F,M", [(2, 3, 300, 200, 64, 16, 64), (1, 2, 40000, 30000, 32, 32, 32)])
def test_fused_features_continue(ea, dtype, B, H, n0, n1, D, F, M):
    """Continuation from a carried state: the second call's rows (one-pass or
    two-phase plan) equal the oracle's running sums over the whole sequence, and
    its final state equals one call over everything; then the same continuation
    in place (S_out = S_in)."""
    N = n0 + n1
    if dtype == "f32":
        dev, host = case(ea, B, H, N, D, M, F, "prf", 95 + D)
    else:
        dev, host = bf16_case(ea, B, H, N, D, M, F, "prf", 95 + D)
    Qd, Kd, Vd, Wd = dev
    ref, S_ref, z_ref = oracle_out(host, F, "prf", False)
    head = [x[:, :, :n0].contiguous() for x in (Qd, Kd, Vd)]
    tail = [x[:, :, n0:].contiguous() for x in (Qd, Kd, Vd)]
    S0 = torch.empty((B, H, F, M), device=DEV)
    z0 = torch.empty((B, H, F), device=DEV)
    ea.forward_features(*head, Wd, F, "prf", S_out=S0, z_out=z0)
    S1, z1 = torch.empty_like(S0), torch.empty_like(z0)
    rest = ea.forward_features(*tail, Wd, F, "prf", S_in=S0, z_in=z0, S_out=S1, z_out=z1)
    S2, z2 = S0.clone(), z0.clone()
    rest2 = ea.forward_features(*tail, Wd, F, "prf", S_in=S2, z_in=z2, S_out=S2, z_out=z2)
    torch.cuda.synchronize()
    assert rowwise_rel(rest.cpu().numpy(), ref[:, :, n0:]) <= TOL["f32"]
    assert whole_rel(S1.cpu().numpy(), S_ref) <= 1e-5 and whole_rel(z1.cpu().numpy(), z_ref) <= 1e-5
    assert rowwise_rel(rest2.cpu().numpy(), rest.cpu().numpy()) <= 1e-6
    assert whole_rel(S2.cpu().numpy(), S1.cpu().numpy()) <= 1e-6


def test_fused_features_multi_token_decode(ea):
    """T tokens per call with the map fused (a continuation on 16 new rows, state
    updated in place) equals T single fused decode steps."""
    B, H, D, M, F, n0, T = 4, 8, 64, 64, 16, 256, 16
    dev, host = case(ea, B, H, n0 + T, D, M, F, "trf", 97)
    Qd, Kd, Vd, Wd = dev
    S = torch.empty((B, H, F, M), device=DEV)
    z = torch.empty((B, H, F), device=DEV)
    ea.forward_features(*(x[:, :, :n0].contiguous() for x in (Qd, Kd, Vd)), Wd, F, "trf", S_out=S, z_out=z)
    S1, z1 = S.clone(), z.clone()
    multi = ea.forward_features(*(x[:, :, n0:].contiguous() for x in (Qd, Kd, Vd)), Wd, F, "trf", S_in=S, z_in=z,
                                S_out=S, z_out=z)
    single = [ea.decode_step_features(S1, z1, *(x[:, :, t].contiguous() for x in (Qd, Kd, Vd)), Wd, F, "trf")
              for t in range(n0, n0 + T)]
    torch.cuda.synchronize()
    ref = oracle_out(host, F, "trf", False)[0][:, :, n0:]
    assert rowwise_rel(multi.cpu().numpy(), ref) <= TOL["f32"]
    assert rowwise_rel(torch.stack(single, dim=2).cpu().numpy(), multi.cpu().numpy()) <= 1e-5
    assert whole_rel(S.cpu().numpy(), S1.cpu().numpy()) <= 1e-5



@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind,normalize", [("prf", False), ("prf", True), ("trf", False)])
@pytest.mark.parametrize("B,H,N,D,F,M", [(2, 3, 300, 64, 16, 64), (1, 2, 5000, 32, 32, 128), (2, 2, 33, 128, 64, 16)])
def test_fused_features_noncausal(ea, dtype, kind, normalize, B, H, N, D, F, M):
    """Non-causal attention with the map fused into both stage kernels: against
    the oracle (every row attends to all N positions) and the two-launch path."""
    assert supported(ea, B, H, N, D, M, F, causal=False)
    if dtype == "f32":
        dev, host = case(ea, B, H, N, D, M, F, kind, 110 + D, normalize)
    else:
        dev, host = bf16_case(ea, B, H, N, D, M, F, kind, 110 + D, normalize)
    Qd, Kd, Vd, Wd = dev
    out = ea.forward_features(Qd, Kd, Vd, Wd, F, kind, normalize, causal=False)
    fq, fk = ea.feature_map(Qd, Wd, F, kind, normalize, X2=Kd)
    two = ea.forward_chunked(fq, fk, Vd.float().contiguous(), causal=False, features=True)
    torch.cuda.synchronize()
    ref = oracle_out(host, F, kind, normalize, causal=False)
    ref = ref[0] if isinstance(ref, tuple) else ref
    assert rowwise_rel(out.cpu().numpy(), ref) <= TOL["f32"]
    assert rowwise_rel(out.cpu().numpy(), two.cpu().numpy()) <= 1e-5
