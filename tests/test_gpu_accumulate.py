"""GPU parity for the fp32 gradient-accumulation path (16-bit micro-batch
gradients accumulated into an fp32 copy, then the norm pass and the fused
AdamW pass on that fp32 gradient), against the oracle."""
import math

import numpy as np
import pytest

import oracle
import workloads as W

from parity import bits_of, check_norm, compare_step, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SIZES = [1, 3, 4, 5, 255, 256, 257, 4099, 8192 * 3 + 1, 1_000_003]


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    return Z


def ulp_distance32(a, b):
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def _norm(Z, G, inv):
    sq = torch.empty(1, dtype=torch.float64, device="cuda")
    ovf = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(Z.zero_norm_workspace_bytes(G.numel()), dtype=torch.uint8, device="cuda")
    Z.zero_shard_unscale_norm_overflow(G, inv, sq, ovf, ws)
    torch.cuda.synchronize()
    return sq, ovf


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_accumulate_then_step(Z, n, fmt):
    w = W.GPT2_SMALL if fmt == "f16" else W.LLAMA_7B
    inv = 1.0 / w.loss_scale
    begin = 777 * (n % 5)
    A = torch.empty(n, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref_acc = None
    for mb in range(4):
        g = W.fill(w, "grad", begin, n, step=200 + mb)
        Z.zero_shard_grad_accumulate(A, to_device(g, fmt), inv, first=(mb == 0), overflow=flag)
        ref_acc, ovf = oracle.grad_accumulate(ref_acc, g, fmt, inv)
        assert not ovf
    torch.cuda.synchronize()
    got = A.cpu().numpy()
    assert flag.item() == 0
    assert ulp_distance32(got, ref_acc).max() <= 1
    # norm and step on the fp32 gradient
    sq, ovf = _norm(Z, A, 1.0)
    ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(ref_acc, "f32", 1.0)
    assert ovf.item() == 0 and not ref_ovf
    check_norm(sq.item(), ref_sq)
    p, m, v, _ = W.shard_inputs(w, begin, n)
    P, M, V = to_device(p), to_device(m), to_device(v)
    par = torch.empty(n, dtype={"f16": torch.float16, "bf16": torch.bfloat16}[fmt], device="cuda")
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=0.02, step=9, inv_loss_scale=1.0)
    Z.zero_shard_adam_step(P, M, V, A, par, Z.AdamHyper(**hp), sq, ovf)
    torch.cuda.synchronize()
    ref = oracle.shard_step(p, m, v, ref_acc, "f32", fmt, global_sq=ref_sq, global_overflow=False, **hp)
    compare_step((P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par)), ref)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("pos", ["first", "middle", "tail"])
def test_overflow_in_a_microbatch_skips_the_step(Z, fmt, pos):
    n = 3 * 256 + 3
    w = W.GPT2_SMALL
    A = torch.empty(n, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    i = {"first": 0, "middle": n // 2, "tail": n - 1}[pos]
    for mb in range(3):
        g = W.fill(w, "grad", 0, n, step=300 + mb)
        if mb == 1:
            g[i] = W.POS_INF_BITS[fmt]
        Z.zero_shard_grad_accumulate(A, to_device(g, fmt), 1.0 / 1024, first=(mb == 0), overflow=flag)
        torch.cuda.synchronize()
        assert flag.item() == (1 if mb >= 1 else 0)     # OR-accumulated, never cleared
    got = A.cpu().numpy()
    assert np.isinf(got[i]) and np.isfinite(np.delete(got, i)).all()
    sq, ovf = _norm(Z, A, 1.0)
    assert ovf.item() == 1 and math.isinf(sq.item())
    p, m, v, _ = W.shard_inputs(w, 0, n)
    P, M, V = to_device(p), to_device(m), to_device(v)
    Z.zero_shard_adam_step(P, M, V, A, None, Z.AdamHyper(max_grad_norm=1.0), sq, ovf)
    torch.cuda.synchronize()
    assert (P.cpu().numpy().view(np.uint32) == p.view(np.uint32)).all()


def test_f32_norm_nan_and_huge(Z):
    x = np.ones(1001, np.float32)
    x[500] = np.nan
    sq, ovf = _norm(Z, to_device(x), 1.0)
    assert ovf.item() == 1 and math.isnan(sq.item())
    y = np.full(9, 3e38, np.float32)                  # finite; squares overflow fp32 but not fp64
    sq, ovf = _norm(Z, to_device(y), 1.0)
    ref, _ = oracle.shard_sqnorm_overflow(y, "f32", 1.0)
    assert ovf.item() == 0
    check_norm(sq.item(), ref)


def test_shard_adam_with_accumulation_trajectory(Z):
    """ShardAdam over 4 steps of 3 micro-batches each, with an inf in one
    micro-batch of step 3: skips, loss scale, t bit-exact; state in tolerance."""
    w = W.Workload(**{**W.GPT_100B_RANK.__dict__})
    n = 200_003
    p, m, v, _ = W.shard_inputs(w, 0, n)
    P, M, V = to_device(p), to_device(m), to_device(v)
    A = torch.empty(n, dtype=torch.float32, device="cuda")
    par = torch.empty(n, dtype=torch.float16, device="cuda")
    opt = Z.ShardAdam(P, M, V, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                      max_grad_norm=w.max_grad_norm, scaler=Z.LossScaler(scale=w.loss_scale))
    state, scaler, t = (p, m, v), oracle.LossScalerState(scale=w.loss_scale), 0
    for it in range(1, 5):
        scale = opt.scaler.scale
        acc = None
        ovf_any = False
        for mb in range(3):
            g = W.fill(w, "grad", 0, n, step=1000 * it + mb, loss_scale=scale)
            if it == 3 and mb == 2:
                g[n // 3] = W.POS_INF_BITS["f16"]
            opt.accumulate(A, to_device(g, "f16"), first=(mb == 0))
            acc, o = oracle.grad_accumulate(acc, g, "f16", 1.0 / scale)
            ovf_any |= o
        skip = opt.step(A, par)
        sq, ovf = oracle.shard_sqnorm_overflow(acc, "f32", 1.0)
        assert ovf == ovf_any
        scaler, ref_skip = oracle.loss_scaler_update(scaler, ovf)
        assert skip == ref_skip == (it == 3)
        if not ref_skip:
            t += 1
            out = oracle.shard_step(*state, acc, "f32", "f16", global_sq=sq, global_overflow=False,
                                    inv_loss_scale=1.0, max_grad_norm=w.max_grad_norm, lr=w.lr, beta1=w.beta1,
                                    beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=t)
            state = out[:3]
            compare_step((P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par)), out, what=f"it{it} ")
        assert opt.t == t and opt.scaler.scale == scaler.scale
