"""GPU: the allocation-free norm pass (zero_shard_unscale_norm_overflow_noalloc,
partials in the library's fixed per-GPU array) against the workspace entry
point zero_shard_unscale_norm_overflow on the same gradients: the same
kernels and grid, so the sum of squares and the flag agree bit for bit; both
within the bar of the oracle.  Two calls in a row on the shared array, the
second on a smaller gradient, then an overflow and an empty gradient."""
import math

import numpy as np
import pytest

import oracle
import workloads as W

from parity import check_norm

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    return Z


def _grad(w, n, step):
    g = W.fill(w, "grad", 7 * W.CHUNK + 1000, n, step=step)
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.grad_dtype]
    return g, torch.from_numpy(g.view(np.int16).copy()).cuda().view(dt)


def _both(Z, G, inv):
    sq_a = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
    ov_a = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    sq_b, ov_b = sq_a.clone(), ov_a.clone()
    ws = torch.empty(Z.zero_norm_workspace_bytes(G.numel()), dtype=torch.uint8, device="cuda")
    Z.zero_shard_unscale_norm_overflow_noalloc(G, inv, sq_a, ov_a)
    Z.zero_shard_unscale_norm_overflow(G, inv, sq_b, ov_b, ws)
    torch.cuda.synchronize()
    return (sq_a.item(), int(ov_a.item())), (sq_b.item(), int(ov_b.item()))


@pytest.mark.parametrize("wname", ["gpt2", "gpt1t"])
def test_noalloc_norm_equals_workspace_norm(Z, wname):
    w = W.get(wname)
    inv = 1.0 / w.loss_scale
    # the first call fills every one of the 512 partial slots, the second
    # (smaller: 40 blocks and a ragged tail) reuses the same array
    for n in (512 * 8192 + 4099, 40 * 8192 + 77):
        g, G = _grad(w, n, step=n % 97)
        a, b = _both(Z, G, inv)
        assert a[1] == b[1] == 0
        assert a[0] == b[0], (n, a, b)                 # same kernels, same order: bit-identical
        ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(g, w.grad_dtype, inv)
        assert not ref_ovf
        check_norm(a[0], ref_sq)


def test_noalloc_norm_overflow_and_empty(Z):
    w = W.GPT2_SMALL
    inv = 1.0 / w.loss_scale
    g, G = _grad(w, 100_003, step=3)
    G.view(torch.int16)[50_000] = 0x7C00                 # +inf in fp16
    a, b = _both(Z, G, inv)
    assert a == b and a[1] == 1 and math.isinf(a[0])
    g, G = _grad(w, 9, step=4)                            # one block, ragged
    a, b = _both(Z, G, inv)
    assert a == b and a[1] == 0
    check_norm(a[0], oracle.shard_sqnorm_overflow(g, "f16", inv)[0])
    a, b = _both(Z, G[:0], inv)
    assert a == b == (0.0, 0)
