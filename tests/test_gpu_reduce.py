"""GPU parity for the reduction of the data-parallel ranks' gradient slices
of one partition (the local half of the gradient reduce-scatter) into the
fp32 gradient copy, then the norm pass and the fused AdamW pass on it,
against the oracle; and bit-identity with the accumulation kernel applied
slice by slice."""
import math

import numpy as np
import pytest

import oracle
import workloads as W

from parity import bits_of, check_norm, compare_step, to_device
from test_gpu_accumulate import _norm, ulp_distance32

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SIZES = [1, 3, 4, 255, 256, 257, 4099, 65536 + 3, 1_000_003]


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    return Z


def _slices(w, fmt, k, begin, n, inv):
    """Rank r's gradient of this partition: the workload's gradient draw r."""
    return [W.fill(w, "grad", begin, n, step=500 + r, loss_scale=1.0 / inv) for r in range(k)]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("k", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_reduce_matches_oracle_and_accumulation(Z, n, k, fmt):
    w = W.GPT2_SMALL if fmt == "f16" else W.LLAMA_7B
    inv = 1.0 / w.loss_scale
    sl = _slices(w, fmt, k, 333 * (n % 11), n, inv)
    D = [to_device(b, fmt) for b in sl]
    A = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.zero_shard_grad_reduce(A, D, inv, flag)
    B = torch.empty(n, dtype=torch.float32, device="cuda")
    for r, d in enumerate(D):
        Z.zero_shard_grad_accumulate(B, d, inv, first=(r == 0))
    torch.cuda.synchronize()
    ref, ovf = oracle.grad_reduce(sl, fmt, inv)
    got = A.cpu().numpy()
    assert flag.item() == 0 and not ovf
    assert ulp_distance32(got, ref).max() <= 1
    assert np.array_equal(got.view(np.uint32), B.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_reduce_then_step(Z, fmt):
    w = W.GPT2_SMALL if fmt == "f16" else W.LLAMA_7B
    n, k = 300_007, 8
    inv = 1.0 / (w.loss_scale * k)                  # mean over the 8 ranks, folded into the unscale
    sl = _slices(w, fmt, k, 0, n, inv)
    A = torch.empty(n, dtype=torch.float32, device="cuda")
    Z.zero_shard_grad_reduce(A, [to_device(b, fmt) for b in sl], inv)
    acc, _ = oracle.grad_reduce(sl, fmt, inv)
    sq, ovf = _norm(Z, A, 1.0)
    ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(acc, "f32", 1.0)
    assert ovf.item() == 0 and not ref_ovf
    check_norm(sq.item(), ref_sq)
    p, m, v, _ = W.shard_inputs(w, 0, n)
    P, M, V = to_device(p), to_device(m), to_device(v)
    par = torch.empty(n, dtype={"f16": torch.float16, "bf16": torch.bfloat16}[fmt], device="cuda")
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=0.05, step=21, inv_loss_scale=1.0)
    Z.zero_shard_adam_step(P, M, V, A, par, Z.AdamHyper(**hp), sq, ovf)
    torch.cuda.synchronize()
    ref = oracle.shard_step(p, m, v, acc, "f32", fmt, global_sq=ref_sq, global_overflow=False, **hp)
    compare_step((P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par)), ref)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("where,pos", [(0, "first"), (5, "middle"), (15, "tail")])
def test_overflow_in_one_slice(Z, fmt, where, pos):
    n = 4 * 256 + 3
    sl = _slices(W.GPT2_SMALL, fmt, 16, 0, n, 1.0 / 1024)
    i = {"first": 0, "middle": n // 2, "tail": n - 1}[pos]
    sl[where][i] = W.POS_INF_BITS[fmt]
    A = torch.empty(n, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.zero_shard_grad_reduce(A, [to_device(b, fmt) for b in sl], 1.0 / 1024, flag)
    torch.cuda.synchronize()
    assert flag.item() == 1
    got = A.cpu().numpy()
    assert not np.isfinite(got[i]) and np.isfinite(np.delete(got, i)).all()
    sq, ovf = _norm(Z, A, 1.0)
    assert ovf.item() == 1 and not math.isfinite(sq.item())


def test_shard_adam_with_reduction_trajectory(Z):
    """ShardAdam over 4 steps whose gradient is the reduction of 8 ranks'
    slices, with an inf in one rank's slice at step 2: skips, loss scale and
    t bit-exact; state in tolerance after every step."""
    w = W.Workload(**{**W.GPT_100B_RANK.__dict__})
    n, k = 100_003, 8
    p, m, v, _ = W.shard_inputs(w, 0, n)
    P, M, V = to_device(p), to_device(m), to_device(v)
    A = torch.empty(n, dtype=torch.float32, device="cuda")
    par = torch.empty(n, dtype=torch.float16, device="cuda")
    opt = Z.ShardAdam(P, M, V, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                      max_grad_norm=w.max_grad_norm, scaler=Z.LossScaler(scale=w.loss_scale))
    state, scaler, t = (p, m, v), oracle.LossScalerState(scale=w.loss_scale), 0
    for it in range(1, 5):
        scale = opt.scaler.scale
        sl = [W.fill(w, "grad", 0, n, step=2000 * it + r, loss_scale=scale) for r in range(k)]
        if it == 2:
            sl[3][n // 2] = W.POS_INF_BITS["f16"]
        opt.reduce(A, [to_device(b, "f16") for b in sl])
        acc, ovf_any = oracle.grad_reduce(sl, "f16", 1.0 / scale)
        skip = opt.step(A, par)
        sq, ovf = oracle.shard_sqnorm_overflow(acc, "f32", 1.0)
        assert ovf == ovf_any
        scaler, ref_skip = oracle.loss_scaler_update(scaler, ovf)
        assert skip == ref_skip == (it == 2)
        if not ref_skip:
            t += 1
            out = oracle.shard_step(*state, acc, "f32", "f16", global_sq=sq, global_overflow=False,
                                    inv_loss_scale=1.0, max_grad_norm=w.max_grad_norm, lr=w.lr, beta1=w.beta1,
                                    beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=t)
            state = out[:3]
            compare_step((P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par)), out, what=f"it{it} ")
        assert opt.t == t and opt.scaler.scale == scaler.scale
