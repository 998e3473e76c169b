"""GPU: physically contiguous device memory for a shard's streams.

The raw calls hand out and take back memory that the library's kernels
read and write correctly; a torch memory pool backed by the library's
allocator serves a shard whose step matches the oracle and, bit for bit,
the same step on buffers from torch's default allocator."""
import pytest

import oracle
import workloads as W

from parity import bits_of, check_norm, compare_step, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    return Z


@pytest.mark.parametrize("nbytes", [16, 4096, (1 << 21) + 48, 1 << 28])
def test_contiguous_memory_round_trip(Z, nbytes):
    p = Z.zero_device_alloc_contiguous(nbytes)
    try:
        assert p != 0 and p % 256 == 0
        g = torch.Generator().manual_seed(nbytes)
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
        back = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        Z.zero_copy_reference(p, src, nbytes)
        Z.zero_copy_reference(back, p, nbytes)
        torch.cuda.synchronize()
        assert torch.equal(back, src)
    finally:
        Z.zero_device_free(p)
    assert Z.zero_device_alloc_contiguous(0) == 0
    Z.zero_device_free(0)


def test_shard_from_contiguous_pool_matches_oracle(Z):
    w = W.GPT_100B_RANK
    n = 70_001
    p, m, v, g = W.shard_inputs(w, 3_000_017, n)
    hyper = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                 max_grad_norm=w.max_grad_norm)

    def run(pool):
        ctx = torch.cuda.use_mem_pool(pool) if pool is not None else None
        if ctx is not None:
            ctx.__enter__()
        try:
            P, M, V, G = to_device(p), to_device(m), to_device(v), to_device(g, "f16")
            par = torch.empty(n, dtype=torch.float16, device="cuda")
        finally:
            if ctx is not None:
                ctx.__exit__(None, None, None)
        opt = Z.ShardAdam(P, M, V, applied_steps=w.step - 1, device_state=True,
                          scaler=Z.LossScaler(scale=w.loss_scale), **hyper)
        opt.step(G, par)
        torch.cuda.synchronize()
        return opt, P, M, V, par

    pool = Z.contiguous_pool()
    assert Z.contiguous_pool() is pool                     # one pool per device
    opt, P, M, V, par = run(pool)
    _, P2, M2, V2, par2 = run(None)
    for a, b in ((P, P2), (M, M2), (V, V2)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(par.view(torch.int16), par2.view(torch.int16))
    inv = 1.0 / w.loss_scale
    ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(g, "f16", inv)
    assert not ref_ovf
    check_norm(opt.sqnorm.item(), ref_sq)
    ref = oracle.shard_step(p, m, v, g, "f16", "f16", global_sq=ref_sq, global_overflow=False, step=w.step,
                            inv_loss_scale=inv, **hyper)
    compare_step((P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par)), ref)
    assert opt.read_state().applied == w.step
