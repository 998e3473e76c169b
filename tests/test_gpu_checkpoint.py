"""GPU: checkpoint and resume of one rank's shard.  k steps, save, load into
fresh buffers, k more steps must give the same bits as 2k uninterrupted steps
(host-scaled and device-state paths; an overflow on each side of the save)."""
import numpy as np
import pytest

import workloads as W

from parity import to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    return Z


@pytest.mark.parametrize("device_state", [False, True])
def test_resume_is_bit_identical(Z, tmp_path, device_state):
    from zero_sharded_mixed_partition_amd import checkpoint
    w = W.GPT_100B_RANK
    n = 123_457
    p, m, v, _ = W.shard_inputs(w, 0, n)
    hyper = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                 max_grad_norm=w.max_grad_norm)

    def fresh():
        return Z.ShardAdam(to_device(p), to_device(m), to_device(v), scaler=Z.LossScaler(scale=w.loss_scale,
                           growth_interval=2), device_state=device_state, **hyper)

    def grad(it, scale):
        g = W.fill(w, "grad", 0, n, step=300 + it, loss_scale=scale)
        if it in (2, 5):
            g[it * 97] = W.POS_INF_BITS["f16"]
        return to_device(g, "f16")

    def scale_of(opt):
        return opt.read_state().scaler.scale if device_state else opt.scaler.scale

    ref = fresh()
    par_ref = torch.empty(n, dtype=torch.float16, device="cuda")
    for it in range(1, 7):
        ref.step(grad(it, scale_of(ref)), par_ref)
    a = fresh()
    par_a = torch.empty(n, dtype=torch.float16, device="cuda")
    for it in range(1, 4):
        a.step(grad(it, scale_of(a)), par_a)
    checkpoint.save(a, str(tmp_path / "ck"))
    del a
    b = Z.ShardAdam(torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda"),
                    device_state=device_state)
    checkpoint.load(b, str(tmp_path / "ck"))
    for it in range(4, 7):
        b.step(grad(it, scale_of(b)), par_a)
    for k in ("master", "exp_avg", "exp_avg_sq"):
        assert torch.equal(getattr(ref, k).view(torch.int32), getattr(b, k).view(torch.int32)), k
    assert torch.equal(par_ref.view(torch.int16), par_a.view(torch.int16))
    sa, sb = checkpoint.state_dict(ref), checkpoint.state_dict(b)
    assert sa["t"] == sb["t"] == 4 and sa["scaler"] == sb["scaler"] and sa["skipped"] == sb["skipped"]
    assert np.array_equal(sa["master"].view(np.uint32), sb["master"].view(np.uint32))
