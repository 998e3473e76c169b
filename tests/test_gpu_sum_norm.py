"""GPU: the fp32 gradient copy and its norm in one pass (zero_shard_grad_sum_norm)
against the separate kernels (the copy bit for bit), the oracle (norm within
1e-5, flags exact), run-to-run determinism, edge cases, and whole steps."""
import math

import numpy as np
import pytest

import oracle
import workloads as W

from parity import bits_of, check_norm, compare_step, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SIZES = [1, 3, 255, 256, 257, 4099, 65536 + 3, 1_000_003]


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    return Z


def _scalars():
    return torch.empty(1, dtype=torch.float64, device="cuda"), torch.empty(1, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("k,add", [(1, False), (1, True), (3, False), (8, False)])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_sum_norm_matches_separate_kernels_and_oracle(Z, n, k, add, fmt):
    w = W.GPT2_SMALL if fmt == "f16" else W.LLAMA_7B
    inv = 1.0 / w.loss_scale
    sl = [W.fill(w, "grad", 17 * (n % 13), n, step=600 + r) for r in range(k)]
    D = [to_device(b, fmt) for b in sl]
    base = W.fill(w, "master", 0, n) * 1e-3 if add else None            # an fp32 copy to add to
    A = to_device(base) if add else torch.full((n,), float("nan"), device="cuda")
    B = to_device(base) if add else torch.empty(n, device="cuda")
    sq, ovf = _scalars()
    ws = torch.empty(Z.zero_sum_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)              # NaN bytes: a partial slot that is read but never written shows as overflow
    Z.zero_shard_grad_sum_norm(A, D, add, inv, sq, ovf, ws)
    if add:
        for d in D:
            Z.zero_shard_grad_accumulate(B, d, inv, first=False)
    else:
        Z.zero_shard_grad_reduce(B, D, inv)
    torch.cuda.synchronize()
    got = A.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), B.cpu().numpy().view(np.uint32))
    ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(got, "f32", 1.0)
    assert ovf.item() == int(ref_ovf) == 0
    check_norm(sq.item(), ref_sq)
    first = sq.item()
    Z.zero_shard_grad_sum_norm(B, D, False, inv, sq, ovf, ws) if not add else None
    torch.cuda.synchronize()
    if not add:
        assert sq.item() == first                                          # run to run, bit for bit


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("bad,pos", [("inf", "first"), ("inf", "tail"), ("nan", "middle")])
def test_sum_norm_overflow(Z, fmt, bad, pos):
    n = 3 * 256 + 5
    sl = [W.fill(W.GPT2_SMALL, "grad", 0, n, step=700 + r) for r in range(4)]
    i = {"first": 0, "middle": n // 2, "tail": n - 1}[pos]
    sl[2][i] = W.POS_INF_BITS[fmt] if bad == "inf" else (0x7E00 if fmt == "f16" else 0x7FC0)
    A = torch.empty(n, device="cuda")
    sq, ovf = _scalars()
    ws = torch.empty(Z.zero_sum_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    Z.zero_shard_grad_sum_norm(A, [to_device(b, fmt) for b in sl], False, 1.0 / 1024, sq, ovf, ws)
    torch.cuda.synchronize()
    assert ovf.item() == 1
    assert (math.isnan(sq.item()) if bad == "nan" else sq.item() == math.inf)


def test_sum_norm_empty(Z):
    A = torch.empty(0, device="cuda")
    G = torch.empty(0, dtype=torch.float16, device="cuda")
    sq, ovf = _scalars()
    sq.fill_(5.0)
    ovf.fill_(3)
    ws = torch.empty(Z.zero_sum_norm_workspace_bytes(0), dtype=torch.uint8, device="cuda")
    Z.zero_shard_grad_sum_norm(A, [G], False, 1.0, sq, ovf, ws)
    torch.cuda.synchronize()
    assert sq.item() == 0.0 and ovf.item() == 0


@pytest.mark.parametrize("device_state", [False, True])
@pytest.mark.parametrize("mode", ["reduce", "accumulate"])
def test_steps_with_fused_norm_match_oracle(Z, device_state, mode):
    """4 steps with the fused pass (8-slice reduction, or 3 micro-batches whose
    last fuses the norm), an overflow in step 2: skips, scale, t exact; state
    within the bar of the oracle after every step."""
    w = W.GPT_100B_RANK
    n, k = 150_001, 8
    p, m, v, _ = W.shard_inputs(w, 0, n)
    P, M, V = to_device(p), to_device(m), to_device(v)
    A = torch.empty(n, device="cuda")
    par = torch.empty(n, dtype=torch.float16, device="cuda")
    opt = Z.ShardAdam(P, M, V, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                      max_grad_norm=w.max_grad_norm, scaler=Z.LossScaler(scale=w.loss_scale), device_state=device_state)
    state, scaler, t = (p, m, v), oracle.LossScalerState(scale=w.loss_scale), 0
    for it in range(1, 5):
        scale = opt.read_state().scaler.scale if device_state else opt.scaler.scale
        parts = [W.fill(w, "grad", 0, n, step=900 * it + r, loss_scale=scale) for r in range(k if mode == "reduce" else 3)]
        if it == 2:
            parts[-1][n // 3] = W.POS_INF_BITS["f16"]
        if mode == "reduce":
            opt.reduce(A, [to_device(b, "f16") for b in parts], with_norm=True)
            acc, ovf_any = oracle.grad_reduce(parts, "f16", 1.0 / scale)
        else:
            acc, ovf_any = None, False
            for j, b in enumerate(parts):
                opt.accumulate(A, to_device(b, "f16"), first=(j == 0), last=(j == len(parts) - 1))
                acc, o = oracle.grad_accumulate(acc, b, "f16", 1.0 / scale)
                ovf_any = ovf_any or o
        skip = opt.step(A, par, norm_done=True)
        if device_state:
            skip = bool(opt.read_state().last_overflow)
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


def test_fused_decision_equals_decide_kernel(Z):
    """The decision folded into the fused pass's final kernel writes the same
    coefficient block and state as the separate decision kernel."""
    n = 70_001
    w = W.GPT2_SMALL
    G = [to_device(W.fill(w, "grad", 0, n, step=5 + r), "f16") for r in range(2)]
    hp = Z.AdamHyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=1.0)
    outs = []
    for fused in (True, False):
        st = Z.StepState(Z.LossScaler(scale=w.loss_scale, growth_interval=4, good_steps=3), applied_steps=41)
        A = torch.empty(n, device="cuda")
        sq, ovf = _scalars()
        coef = torch.empty(Z.zero_adam_coef_bytes(), dtype=torch.uint8, device="cuda")
        ws = torch.empty(Z.zero_sum_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
        if fused:
            Z.zero_shard_grad_sum_norm_dev(A, G, False, st, sq, ovf, ws, hp=hp, d_coef=coef)
        else:
            Z.zero_shard_grad_sum_norm_dev(A, G, False, st, sq, ovf, ws)
            Z.zero_step_decide_dev(hp, torch.float32, st, ovf, coef)
        torch.cuda.synchronize()
        outs.append((coef.cpu().numpy().tobytes(), bytes(st.read()), sq.item()))
    assert outs[0] == outs[1]
