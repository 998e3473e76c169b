"""GPU: the reference copy used beside the nominal peak in the benchmark
moves every byte unchanged."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 257, (1 << 24) + 48])
def test_copy_reference_is_exact(nbytes):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes + 32,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros(nbytes + 32, dtype=torch.uint8, device="cuda")
    Z.zero_copy_reference(dst, src, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert int(dst[nbytes:].count_nonzero()) == 0          # nothing beyond the range is written


@pytest.mark.parametrize("src_bytes", [8, 4096, 8 * 257, (1 << 24) + 40])
def test_widening_copy_is_exact(src_bytes):
    """Each 8-byte word of src lands twice, as one 16-byte vector of dst."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    g = torch.Generator().manual_seed(src_bytes)
    src = torch.randint(-2**62, 2**62, (src_bytes // 8 + 4,), dtype=torch.int64, generator=g).cuda()
    dst = torch.zeros(2 * (src_bytes // 8) + 8, dtype=torch.int64, device="cuda")
    Z.zero_copy_widen_reference(dst, src, src_bytes)
    torch.cuda.synchronize()
    n = src_bytes // 8
    assert torch.equal(dst[:2 * n].view(n, 2), src[:n, None].expand(n, 2))
    assert int(dst[2 * n:].count_nonzero()) == 0           # nothing beyond the range is written
