"""GPU: the step with its loss scaler and step counts in device memory.

The coefficient block the decision kernel forms from the device state must
equal the host's zero_adam_prepare block bit for bit, and the state must
advance as zero_loss_scaler_update does; whole trajectories (overflow,
back-off, growth) must match the host-scaled path bit for bit, also with
every step enqueued back to back without any host synchronisation."""
import ctypes
import itertools

import numpy as np
import pytest

import oracle
import workloads as W

from parity import bits_of, compare_step, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    return Z


def test_decision_kernel_coefficients_and_state(Z):
    E = torch.empty(0, dtype=torch.float32, device="cuda")
    G16 = torch.empty(0, dtype=torch.float16, device="cuda")
    sq = torch.tensor([4.0], dtype=torch.float64, device="cuda")
    coef = torch.empty(Z.zero_adam_coef_bytes(), dtype=torch.uint8, device="cuda")
    cases = itertools.product([0.0, 0.9, 0.95, 0.999], [0.0, 0.98, 0.999, 0.9999], [1, 2, 7, 100, 9999, 1_000_003],
                              [1.0, 65536.0, 3.0], [0.0, 1.0], [0, 1])
    checked = 0
    for b1, b2, t, scale, clip, flag in cases:
        if (b1, b2) == (0.0, 0.0) and t > 7:
            continue
        lr, wd, eps = 3e-4 * (1 + t % 3), 0.01 * (t % 5), 1e-8
        scaler = Z.LossScaler(scale=scale, min_scale=1.0, growth_interval=5, good_steps=t % 5)
        st = Z.StepState(scaler, applied_steps=t - 1)
        ovf = torch.tensor([flag], dtype=torch.int32, device="cuda")
        for grad in (G16, E):                                   # 16-bit gradient, or the unscaled fp32 copy
            s2 = Z.StepState(scaler, applied_steps=t - 1)
            hp = Z.AdamHyper(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, max_grad_norm=clip)
            Z.zero_shard_adam_step_dev(E, E, E, grad, None, hp, s2, sq, ovf, coef)
            got = coef.cpu().numpy().tobytes()
            inv = 1.0 if grad.dtype == torch.float32 else 1.0 / scale
            want = np.zeros(Z.zero_adam_coef_bytes(), np.uint8)
            Z.zero_adam_prepare(Z.AdamHyper(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, step=t,
                                            inv_loss_scale=inv, max_grad_norm=clip), want)
            assert got == want.tobytes(), (b1, b2, t, scale, clip, grad.dtype)
            after = s2.read()
            ref = Z.LossScaler(scale=scale, min_scale=1.0, growth_interval=5, good_steps=t % 5)
            skip = Z.zero_loss_scaler_update(ref, bool(flag))
            assert bytes(after.scaler) == bytes(ref.s)
            assert (after.applied, after.skipped, after.last_overflow) == (t - 1 + (not skip), int(skip), flag)
            checked += 1
        del st
    assert checked > 500


def _pair(Z, w, n, **kw):
    p, m, v, _ = W.shard_inputs(w, 0, n)
    hyper = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                 max_grad_norm=w.max_grad_norm)
    mk = lambda **x: Z.ShardAdam(to_device(p), to_device(m), to_device(v), applied_steps=w.step - 1,  # noqa: E731
                                 scaler=Z.LossScaler(scale=w.loss_scale, growth_interval=3), **hyper, **x)
    return (p, m, v), mk(), mk(device_state=True)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("wname,n", [("gpt100b", 300_007), ("gpt1t", 70_001), ("tiny", 1000)])
def test_trajectory_matches_host_scaled_path(Z, wname, n, split):
    """8 steps, overflow at step 3, growth every 3 clean steps: every buffer,
    the loss scale and the counts bit-identical to the host-scaled path; the
    decision folded into the norm pass (one rank) or made by its own kernel
    after a data-parallel reduction point (split)."""
    w = W.get(wname)
    _, host, dev = _pair(Z, w, n)
    pdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.param_dtype]
    par_h, par_d = torch.empty(n, dtype=pdt, device="cuda"), torch.empty(n, dtype=pdt, device="cuda")
    for it in range(1, 9):
        g = W.fill(w, "grad", 0, n, step=70 + it, loss_scale=host.scaler.scale)
        if it == 3:
            g[n // 2] = W.POS_INF_BITS[w.grad_dtype]
        G = to_device(g, w.grad_dtype)
        skip = host.step(G, par_h)
        assert dev.step(G, par_d, allreduce=(lambda sq, ovf: None) if split else None) is None
        st = dev.read_state()
        assert skip == bool(st.last_overflow) == (it == 3)
        assert dev.t == host.t and bytes(dev.scaler.s) == bytes(host.scaler.s)
        for a, b in ((host.master, dev.master), (host.exp_avg, dev.exp_avg), (host.exp_avg_sq, dev.exp_avg_sq)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"iteration {it}"
        assert torch.equal(par_h.view(torch.int16), par_d.view(torch.int16))
    assert st.skipped == 1 and st.applied == w.step - 1 + 7


def test_back_to_back_steps_without_synchronisation(Z):
    """Five steps enqueued with no host wait in between equal five host-scaled
    steps; and the result is within the bar of the oracle."""
    w = W.GPT_100B_RANK
    n = 200_003
    (p, m, v), host, dev = _pair(Z, w, n)
    par_h = torch.empty(n, dtype=torch.float16, device="cuda")
    par_d = torch.empty(n, dtype=torch.float16, device="cuda")
    grads = [to_device(W.fill(w, "grad", 0, n, step=90 + k, loss_scale=w.loss_scale), "f16") for k in range(5)]
    torch.cuda.synchronize()
    for G in grads:
        dev.step(G, par_d)                      # nothing here waits for the device
    for G in grads:
        host.step(G, par_h)
    st = dev.read_state()
    assert st.applied == host.t == w.step - 1 + 5 and st.skipped == 0
    for a, b in ((host.master, dev.master), (host.exp_avg, dev.exp_avg), (host.exp_avg_sq, dev.exp_avg_sq)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(par_h.view(torch.int16), par_d.view(torch.int16))
    state = (p, m, v)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=w.max_grad_norm)
    scaler = oracle.LossScalerState(scale=w.loss_scale, growth_interval=3)     # grows after 3 clean steps
    for k, G in enumerate(grads):
        g = G.view(torch.int16).cpu().numpy().view(np.uint16)
        inv = 1.0 / scaler.scale
        sq, ovf = oracle.shard_sqnorm_overflow(g, "f16", inv)
        out = oracle.shard_step(*state, g, "f16", "f16", global_sq=sq, global_overflow=ovf,
                                inv_loss_scale=inv, step=w.step + k, **hp)
        state = out[:3]
        scaler, _ = oracle.loss_scaler_update(scaler, ovf)
    assert st.scaler.scale == scaler.scale == 2 * w.loss_scale
    compare_step((dev.master.cpu().numpy(), dev.exp_avg.cpu().numpy(), dev.exp_avg_sq.cpu().numpy(),
                  bits_of(par_d)), out)


@pytest.mark.parametrize("scale", [1024.0, 3.0])
def test_accumulate_and_reduce_read_the_device_scale(Z, scale):
    n = 50_001
    w = W.GPT2_SMALL
    st = Z.StepState(Z.LossScaler(scale=scale))
    gs = [to_device(W.fill(w, "grad", 0, n, step=k, loss_scale=scale), "f16") for k in range(3)]
    A, B = torch.empty(n, device="cuda"), torch.empty(n, device="cuda")
    for k, G in enumerate(gs):
        Z.zero_shard_grad_accumulate_dev(A, G, st, first=(k == 0))
        Z.zero_shard_grad_accumulate(B, G, 1.0 / scale, first=(k == 0))
    torch.cuda.synchronize()
    assert torch.equal(A.view(torch.int32), B.view(torch.int32))
    Z.zero_shard_grad_reduce_dev(A, gs, st)
    Z.zero_shard_grad_reduce(B, gs, 1.0 / scale)
    torch.cuda.synchronize()
    assert torch.equal(A.view(torch.int32), B.view(torch.int32))
    sq_d, ovf_d = torch.empty(1, dtype=torch.float64, device="cuda"), torch.empty(1, dtype=torch.int32, device="cuda")
    sq_h, ovf_h = torch.empty_like(sq_d), torch.empty_like(ovf_d)
    ws = torch.empty(Z.zero_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    Z.zero_shard_unscale_norm_overflow_dev(gs[0], st, sq_d, ovf_d, ws)
    Z.zero_shard_unscale_norm_overflow(gs[0], 1.0 / scale, sq_h, ovf_h, ws)
    torch.cuda.synchronize()
    assert sq_d.item() == sq_h.item() and ovf_d.item() == ovf_h.item() == 0


def test_state_layout(Z):
    assert ctypes.sizeof(Z.zero_step_state) == 72
    st = Z.StepState(Z.LossScaler(scale=8.0, growth_interval=7, good_steps=2), applied_steps=41)
    r = st.read()
    assert (r.scaler.scale, r.scaler.growth_interval, r.scaler.good_steps, r.applied, r.skipped) == (8.0, 7, 2, 41, 0)
