"""GPU: a shard larger than one launch grid covers.

The elementwise passes launch at most 2^26 - 1 one-wave workgroups (grid
size times 64 work-items must stay below 2^32), 256 elements each; past
2^34 elements they stride over the remaining tasks.  This shard has
2^34 + 4099 elements (ragged), so the last tasks, and the tail, go through
that stride.  (The first micro-batch's accumulation takes two tasks, 512
elements, per workgroup: its grid covers this shard in one launch, and the
partial last group takes its per-lane path.  A later micro-batch's strides.)  The fp32 accumulation copy (69 GB) and one bf16 gradient
(34 GB) fit in one MI355X's HBM; the update's 16 B/element would not.

The gradient repeats a table of 251 bf16 values (g_i = T[i mod 251]), filled
on the device, so every expected value is known in closed form:
  * accumulate (first):       acc_i = T[i mod 251]
  * accumulate (later):       acc_i = 2 T[i mod 251]
  * reduce of two slices:     acc_i = 2 T[i mod 251]   (both slices the same buffer)
  * fused add + norm:         acc_i = 3 T[i mod 251], sum of squares
                              = 9 sum_r count_r T_r^2, formed exactly with
                              rational arithmetic and rounded once.
Checked: every element from the first strided task to the end, a million
random elements anywhere, the flags and the norm.
"""
from fractions import Fraction

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N = (1 << 34) + 4099
PERIOD = 251
FIRST_STRIDED = ((1 << 26) - 1) * 256          # first element of task 2^26 - 1 (the grid size)
CHUNK = 1 << 30


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < 130 * (1 << 30):
        pytest.skip(f"needs ~130 GB of free device memory, {free >> 30} GB free")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    return Z


def _table():
    rng = np.random.default_rng(2034)
    vals = (rng.standard_normal(PERIOD) * 2.0 ** rng.integers(-8, 4, PERIOD)).astype(np.float32)
    t = torch.from_numpy(vals).to(torch.bfloat16)             # exact bf16 values
    return t, t.to(torch.float64).numpy()


def _expected(T64, lo, hi, k):
    return (k * T64[np.arange(lo, hi) % PERIOD]).astype(np.float32)


def _check(A, T64, k, what):
    lo = FIRST_STRIDED - 1024
    got = A[lo:].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), _expected(T64, lo, N, k).view(np.uint32)), f"{what}: strided tail"
    idx = np.random.default_rng(7).integers(0, N, 1_000_000)
    got = A.index_select(0, torch.from_numpy(idx).cuda()).cpu().numpy()
    ref = (k * T64[idx % PERIOD]).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{what}: random samples"


def test_passes_beyond_one_grid(Z):
    Tb, T64 = _table()
    Td = Tb.cuda()
    G = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    A = torch.empty(N, dtype=torch.float32, device="cuda")
    ws = torch.empty(Z.zero_sum_norm_workspace_bytes(N), dtype=torch.uint8, device="cuda")
    try:
        for lo in range(0, N, CHUNK):
            hi = min(N, lo + CHUNK)
            G[lo:hi] = Td[torch.arange(lo, hi, device="cuda") % PERIOD]
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")

        Z.zero_shard_grad_accumulate(A, G, 1.0, first=True, overflow=flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        _check(A, T64, 1, "accumulate")

        Z.zero_shard_grad_accumulate(A, G, 1.0, first=False, overflow=flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        _check(A, T64, 2, "accumulate, later micro-batch")

        Z.zero_shard_grad_reduce(A, [G, G], 1.0, overflow=flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        _check(A, T64, 2, "reduce")

        sq = torch.empty(1, dtype=torch.float64, device="cuda")
        ovf = torch.empty(1, dtype=torch.int32, device="cuda")
        Z.zero_shard_grad_sum_norm(A, [G], True, 1.0, sq, ovf, ws)
        torch.cuda.synchronize()
        assert int(ovf.item()) == 0
        _check(A, T64, 3, "fused add and norm")
        # sum over i of (3 T[i mod 251])^2, exactly, then rounded once
        counts = [N // PERIOD + (1 if r < N % PERIOD else 0) for r in range(PERIOD)]
        ref = float(sum(c * Fraction(3.0 * t) ** 2 for c, t in zip(counts, T64)))
        assert abs(sq.item() - ref) <= 1e-5 * ref, (sq.item(), ref)
    finally:
        del A, G, ws
        torch.cuda.empty_cache()
