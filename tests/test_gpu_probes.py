"""The peak probes through the C ABI: the copy is bit-exact and every MFMA chain
reaches the value its closed form gives (sum of 32 accumulator values per lane,
each iters * K * x^2, with K = 4 for fp32 16x16x4 and 32 for bf16 16x16x32; 64 values per lane,
each iters * 16 * x^2, for bf16 32x32x16); the write-only stream is bit-exact."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    import efficient_transformer_amd as ea
    return ea


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000003, 1 << 26])
def test_copy_is_exact(ea, nbytes):
    print(f"probe_copy {nbytes}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(nbytes % 9973)
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g).cuda()
    dst = torch.full_like(src, 7)
    ea.probe_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_copy_leaves_the_rest(ea):
    src = torch.arange(64, dtype=torch.int32, device="cuda")
    dst = torch.full((80,), -1, dtype=torch.int32, device="cuda")
    ea.probe_copy(dst[:64], src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:64], src) and bool((dst[64:] == -1).all())


@pytest.mark.parametrize("nbytes", [0, 16, 4096, 16 * 1000003, 1 << 28])
def test_read_sums_exactly(ea, nbytes):
    print(f"probe_read {nbytes}", flush=True)
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    part = ea.probe_read(src)
    torch.cuda.synchronize()
    # every partial is a count of ones below 2^24: exact
    assert part.numel() == ea.linattn.lib().la_probe_read_partials()
    assert float(part.double().sum().item()) == nbytes // 4


@pytest.mark.parametrize("kind,K", [("f32", 4), ("bf16", 32)])
@pytest.mark.parametrize("blocks,iters,x", [(1, 1, 0.5), (3, 17, 0.5), (512, 64, 0.25), (7, 0, 0.5)])
def test_mfma_closed_form(ea, kind, K, blocks, iters, x):
    print(f"probe_mfma {kind} blocks={blocks} iters={iters} x={x}", flush=True)
    out, flops = ea.probe_mfma(kind, blocks, iters, x)
    torch.cuda.synchronize()
    want = 32.0 * iters * K * x * x
    assert flops == blocks * 4 * iters * 8 * (2048 if kind == "f32" else 16384)
    assert out.shape == (blocks * 256,)
    assert bool((out == want).all()), (out.min().item(), out.max().item(), want)


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000003, 1 << 26])
def test_write_is_exact(ea, nbytes):
    print(f"probe_write {nbytes}", flush=True)
    dst = torch.full((nbytes // 4 + 8,), -1.0, dtype=torch.float32, device="cuda")
    ea.probe_write(dst[:nbytes // 4], 1.5)
    torch.cuda.synchronize()
    assert bool((dst[:nbytes // 4] == 1.5).all()) and bool((dst[nbytes // 4:] == -1.0).all())


@pytest.mark.parametrize("blocks,iters,x", [(1, 1, 0.5), (3, 17, 0.5), (512, 64, 0.25), (7, 0, 0.5)])
def test_mfma32_closed_form(ea, blocks, iters, x):
    print(f"probe_mfma bf16_32x32 blocks={blocks} iters={iters} x={x}", flush=True)
    out, flops = ea.probe_mfma("bf16_32x32", blocks, iters, x)
    torch.cuda.synchronize()
    want = 64.0 * iters * 16 * x * x
    assert flops == blocks * 4 * iters * 4 * 32768
    assert out.shape == (blocks * 256,)
    assert bool((out == want).all()), (out.min().item(), out.max().item(), want)
