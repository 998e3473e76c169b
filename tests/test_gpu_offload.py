"""GPU + host: the offloaded shard step (device gradient -> pinned host ->
host-core AdamW -> 16-bit parameters back to the device) against the oracle,
over a short trajectory with a skipped step."""
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


@pytest.mark.parametrize("wname,device_norm", [("gpt100b", True), ("gpt1t", True), ("gpt1t", False)])
def test_offload_trajectory(Z, wname, device_norm):
    w = W.get(wname)
    n = 1_000_003
    p, m, v, _ = W.shard_inputs(w, 4096, n)
    pin = lambda a: torch.from_numpy(a.copy()).pin_memory()  # noqa: E731
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
    opt = Z.OffloadShardAdam(pin(p), pin(m), pin(v), grad_dtype=tdt[w.grad_dtype], param_dtype=tdt[w.param_dtype],
                             lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                             max_grad_norm=w.max_grad_norm,
                             scaler=(Z.LossScaler(scale=w.loss_scale) if w.loss_scale != 1.0
                                     else Z.LossScaler.static(1.0)), applied_steps=3,
                             device_norm=device_norm, chunk=1 << 18)      # 9 pipelined chunks, ramped at both ends
    par_dev = torch.zeros(n, dtype=tdt[w.param_dtype], device="cuda")
    state, scaler, t = (p, m, v), oracle.LossScalerState(scale=opt.scaler.scale, backoff=opt.scaler.s.backoff,
                                                          growth=opt.scaler.s.growth,
                                                          min_scale=opt.scaler.s.min_scale), 3
    for it in range(1, 5):
        scale = opt.scaler.scale
        g = W.fill(w, "grad", 4096, n, step=40 + it, loss_scale=scale)
        if it == 2:
            g[n // 2] = W.POS_INF_BITS[w.grad_dtype]
        skip = opt.step(to_device(g, w.grad_dtype), par_dev)
        sq, ovf = oracle.shard_sqnorm_overflow(g, w.grad_dtype, 1.0 / scale)
        scaler, ref_skip = oracle.loss_scaler_update(scaler, ovf)
        assert skip == ref_skip == (it == 2)
        if not ref_skip:
            t += 1
            check_norm(opt.sqnorm, sq)
            out = oracle.shard_step(*state, g, w.grad_dtype, w.param_dtype, global_sq=sq, global_overflow=False,
                                    inv_loss_scale=1.0 / scale, max_grad_norm=w.max_grad_norm, lr=w.lr,
                                    beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=t)
            state = out[:3]
            compare_step((opt.master.numpy(), opt.exp_avg.numpy(), opt.exp_avg_sq.numpy(), bits_of(par_dev)),
                         out, what=f"it{it} ")
        assert opt.t == t and opt.scaler.scale == scaler.scale


@pytest.mark.parametrize("wname", ["gpt100b", "gpt1t"])
def test_device_and_host_steps_interchange(Z, wname):
    """A shard stepped 3 times on the device, then handed to the offloaded
    optimizer (state copied to pinned host memory) for 3 more steps, one of
    them skipped, ends bit-identical to 6 steps on the device: the host loop
    rounds exactly as the kernel does and both take the norm from the same
    device pass."""
    w = W.get(wname)
    n = 300_007
    p, m, v, _ = W.shard_inputs(w, 77, n)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
    kw = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=w.max_grad_norm)
    mk_scaler = lambda: Z.LossScaler(scale=w.loss_scale) if w.loss_scale != 1.0 else Z.LossScaler.static(1.0)  # noqa: E731
    grads = []
    for it in range(6):
        g = W.fill(w, "grad", 77, n, step=60 + it, loss_scale=w.loss_scale / (2 if it >= 4 else 1))
        if it == 3:
            g[n // 3] = W.POS_INF_BITS[w.grad_dtype]          # skipped (scale halves when it is dynamic)
        grads.append(to_device(g, w.grad_dtype))
    # all six on the device (host loss scaler, as the offloaded optimizer keeps it)
    dev = [to_device(a) for a in (p, m, v)]
    ref_par = torch.empty(n, dtype=tdt[w.param_dtype], device="cuda")
    opt = Z.ShardAdam(*dev, scaler=mk_scaler(), applied_steps=10, **kw)
    for g in grads:
        opt.step(g, ref_par)
    # three on the device, then three offloaded
    dev2 = [to_device(a) for a in (p, m, v)]
    par = torch.empty(n, dtype=tdt[w.param_dtype], device="cuda")
    opt2 = Z.ShardAdam(*dev2, scaler=mk_scaler(), applied_steps=10, **kw)
    for g in grads[:3]:
        opt2.step(g, par)
    torch.cuda.synchronize()
    host = [t.cpu().pin_memory() for t in dev2]
    off = Z.OffloadShardAdam(*host, grad_dtype=tdt[w.grad_dtype], param_dtype=tdt[w.param_dtype], scaler=opt2.scaler,
                             applied_steps=opt2.t, chunk=1 << 16, **kw)
    skips = [off.step(g, par) for g in grads[3:]]
    torch.cuda.synchronize()
    assert skips == [True, False, False] and off.t == opt.t == 15 and off.scaler.scale == opt.scaler.scale
    for a, b in zip(host, (opt.master, opt.exp_avg, opt.exp_avg_sq)):
        assert torch.equal(a.view(torch.int32), b.cpu().view(torch.int32))
    assert torch.equal(par.view(torch.int16), ref_par.view(torch.int16))
