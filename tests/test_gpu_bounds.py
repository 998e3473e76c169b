"""GPU: no pass reads or writes past the n elements it is given.

Every buffer is allocated with GUARD extra elements after the n the call
sees.  The gradient guards hold +inf and the fp32-copy guards +inf, so a read
past n would show in the norm or the overflow flag.  Every output guard holds
a sentinel that must come back bit for bit, so a write past n shows there.
Sizes are ragged: single elements, partial vectors, one past a 256-element
task, and several tasks with a tail.  Results inside [0, n) are checked
against the oracle as well.
"""
import numpy as np
import pytest

import oracle
import workloads as W

from parity import bits_of, check_norm, compare_step

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GUARD = 512                       # two whole 256-element tasks
SIZES = [1, 3, 7, 9, 255, 257, 1025, 4099, 65539]
SENT32 = 0x4640E400               # 12345.0
SENT16 = 0x7BCD
INF32 = 0x7F800000
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    return Z


def _f32(vals, n, guard_bits):
    full = np.full(n + GUARD, guard_bits, dtype=np.uint32)
    full[:n] = np.asarray(vals, np.float32).view(np.uint32)
    return torch.from_numpy(full.view(np.int32)).cuda().view(torch.float32)


def _b16(bits, n, guard_bits, fmt):
    full = np.full(n + GUARD, guard_bits, dtype=np.uint16)
    full[:n] = bits
    return torch.from_numpy(full.view(np.int16)).cuda().view(TDT[fmt])


def _guard32(t, n, bits):
    """The GUARD elements after n still hold the 32-bit pattern `bits`."""
    return bool((t.view(torch.int32)[n:] == (bits - (1 << 32) if bits >= 1 << 31 else bits)).all().item())


def _guard16(t, n, bits):
    return bool((t.view(torch.int16)[n:] == (bits - (1 << 16) if bits >= 1 << 15 else bits)).all().item())


def _scalars():
    return torch.empty(1, dtype=torch.float64, device="cuda"), torch.zeros(1, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_norm_and_update_stay_within_n(Z, n, fmt):
    w = W.GPT2_SMALL if fmt == "f16" else W.LLAMA_7B
    inf16 = W.POS_INF_BITS[fmt]
    p, m, v, g = W.shard_inputs(w, 7 * n, n)
    inv = 1.0 / w.loss_scale
    G = _b16(g, n, inf16, fmt)
    sq, ovf = _scalars()
    ws = torch.empty(Z.zero_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    Z.zero_shard_unscale_norm_overflow(G[:n], inv, sq, ovf, ws)
    torch.cuda.synchronize()
    ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(g, fmt, inv)
    assert int(ovf.item()) == int(ref_ovf) == 0, "the norm pass read past n"
    check_norm(sq.item(), ref_sq)

    P, M, V = _f32(p, n, SENT32), _f32(m, n, SENT32), _f32(v, n, SENT32)
    par = _b16(np.zeros(n, np.uint16), n, SENT16, w.param_dtype)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=0.05, step=w.step, inv_loss_scale=inv)
    Z.zero_shard_adam_step(P[:n], M[:n], V[:n], G[:n], par[:n], Z.AdamHyper(**hp), sq, ovf)
    torch.cuda.synchronize()
    for name, t in (("master", P), ("exp_avg", M), ("exp_avg_sq", V)):
        assert _guard32(t, n, SENT32), f"the update wrote past n in {name}"
    assert _guard16(par, n, SENT16), "the update wrote past n in param_out"
    ref = oracle.shard_step(p, m, v, g, fmt, w.param_dtype, global_sq=ref_sq, global_overflow=False, **hp)
    compare_step((P[:n].cpu().numpy(), M[:n].cpu().numpy(), V[:n].cpu().numpy(), bits_of(par[:n])), ref)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_fp32_copy_passes_stay_within_n(Z, n, fmt):
    """Accumulation, reduction, the fused copy-and-norm pass, the norm pass
    over the fp32 copy and the update on it."""
    w = W.GPT2_SMALL if fmt == "f16" else W.LLAMA_7B
    inf16 = W.POS_INF_BITS[fmt]
    inv = 1.0 / w.loss_scale
    gs = [W.fill(w, "grad", 11 * n, n, step=700 + r) for r in range(3)]
    D = [_b16(b, n, inf16, fmt) for b in gs]
    A = _f32(np.zeros(n, np.float32), n, INF32)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    # accumulation: first, then two more micro-batches
    for r in range(3):
        Z.zero_shard_grad_accumulate(A[:n], D[r][:n], inv, first=(r == 0), overflow=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0, "accumulation read past n"
    assert _guard32(A, n, INF32), "accumulation wrote past n"
    ref = None
    for b in gs:
        ref, _ = oracle.grad_accumulate(ref, b, fmt, inv)
    got = A[:n].cpu().numpy().astype(np.float64)
    assert (np.abs(got - ref) <= np.abs(np.spacing(ref.astype(np.float32)))).all()

    # the norm pass over the fp32 copy, and the update taking it as gradient
    sq, ovf = _scalars()
    ws = torch.empty(Z.zero_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    Z.zero_shard_unscale_norm_overflow(A[:n], 1.0, sq, ovf, ws)
    torch.cuda.synchronize()
    assert int(ovf.item()) == 0, "the fp32 norm pass read past n"
    p, m, v, _ = W.shard_inputs(w, 5 * n, n)
    P, M, V = _f32(p, n, SENT32), _f32(m, n, SENT32), _f32(v, n, SENT32)
    par = _b16(np.zeros(n, np.uint16), n, SENT16, "bf16")
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=1.0, step=w.step, inv_loss_scale=1.0)
    Z.zero_shard_adam_step(P[:n], M[:n], V[:n], A[:n], par[:n], Z.AdamHyper(**hp), sq, ovf)
    torch.cuda.synchronize()
    for t in (P, M, V):
        assert _guard32(t, n, SENT32), "the fp32-gradient update wrote past n"
    assert _guard16(par, n, SENT16)

    # reduction of three slices
    B = _f32(np.zeros(n, np.float32), n, INF32)
    flag.zero_()
    Z.zero_shard_grad_reduce(B[:n], [d[:n] for d in D], inv, overflow=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0, "the reduction read past n"
    assert _guard32(B, n, INF32), "the reduction wrote past n"
    ref_r, _ = oracle.grad_reduce(gs, fmt, inv)
    got = B[:n].cpu().numpy().astype(np.float64)
    assert (np.abs(got - ref_r) <= np.abs(np.spacing(ref_r.astype(np.float32)))).all()

    # fused copy-and-norm: three slices into a fresh copy, and one added to A
    sws = torch.empty(Z.zero_sum_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    for C, slices, add in ((_f32(np.zeros(n, np.float32), n, INF32), D, False), (A, D[:1], True)):
        sq2, ovf2 = _scalars()
        Z.zero_shard_grad_sum_norm(C[:n], [d[:n] for d in slices], add, inv, sq2, ovf2, sws)
        torch.cuda.synchronize()
        assert int(ovf2.item()) == 0, "the fused pass read past n"
        assert _guard32(C, n, INF32), "the fused pass wrote past n"
        r_sq, r_ovf = oracle.shard_sqnorm_overflow(C[:n].cpu().numpy(), "f32", 1.0)
        assert not r_ovf
        check_norm(sq2.item(), r_sq)
