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
