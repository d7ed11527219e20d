"""The seeded input generator: determinism, block regeneration and bf16 rounding (CPU only)."""
import numpy as np
import torch

import synthetic


def test_deterministic_and_blockwise():
    a = synthetic.draw(7, 1, (4, 3, 100, 16))
    b = synthetic.draw(7, 1, (4, 3, 100, 16))
    assert np.array_equal(a, b)
    flat = a.reshape(-1)
    part = synthetic.draw(7, 1, (5, 16), start=3 * 16)
    assert np.array_equal(part.reshape(-1), flat[48:48 + 80])
    # other seed / tensor id gives other values
    assert not np.array_equal(a, synthetic.draw(8, 1, a.shape))
    assert not np.array_equal(a, synthetic.draw(7, 2, a.shape))


def test_threaded_equals_serial():
    n = (1 << 16) + 123
    a = synthetic.draw(3, 0, (n,), chunk=1 << 12)
    b = synthetic.draw(3, 0, (n,), chunk=1 << 20)
    assert np.array_equal(a, b)


def test_moments():
    x = synthetic.draw(0, 0, (1 << 20,), sigma=0.5).astype(np.float64)
    assert abs(x.mean()) < 3e-3
    assert abs(x.std() - 0.5) < 3e-3


def test_bf16_round_to_nearest_even_matches_torch():
    x = synthetic.draw(1, 2, (1 << 16,), sigma=3.0)
    special = np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 65504.0, 1e-30, -3.3895314e38], dtype=np.float32)
    x = np.concatenate([x, special])
    ours = synthetic.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synthetic.bf16_bits_to_f32(ours)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)


def test_decode_head_subset_matches_full_draw():
    cfg = dict(synthetic.WORKLOADS["decode_f32_256x8_t4096_d64"], B=4, H=2)
    q, k, v = synthetic.decode_step_inputs(cfg, 0, step=5)
    qs, ks, vs = synthetic.decode_step_inputs(cfg, 0, step=5, heads=[1, 6])
    assert np.array_equal(qs, q.reshape(8, -1)[[1, 6]])
    assert np.array_equal(vs, v.reshape(8, -1)[[1, 6]])


def test_prefill_head_rows_match_full_draw():
    cfg = dict(synthetic.WORKLOADS["prefill_bf16_b4h8_n3072_d64"], B=1, H=2, N=50)
    Q, K, V = synthetic.prefill_inputs(cfg, seed=2)
    rows = synthetic.prefill_head_rows(cfg, 2, synthetic.TID_V, bh=1, n0=10, n1=20, width=cfg["M"])
    assert np.array_equal(rows, V[0, 1, 10:20])


def test_torch_generator_matches_numpy_on_cpu():
    a = synthetic.draw(5, 4, (3, 1000), sigma=0.5)
    b = synthetic.draw_torch(5, 4, (3, 1000), sigma=0.5, device="cpu").numpy()
    assert np.mean(a == b) > 0.999
    assert np.max(np.abs(a - b)) <= 1e-6
    a16 = synthetic.draw(5, 4, (2000,), dtype="bf16", start=77)
    b16 = synthetic.draw_torch(5, 4, (2000,), dtype="bf16", device="cpu", start=77).view(torch.int16).numpy()
    assert np.mean(a16 == b16.view(np.uint16)) > 0.999
