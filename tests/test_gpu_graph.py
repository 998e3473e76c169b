"""GPU: the recorded step graph against the eager step and the oracle.

Two copies of one shard are stepped side by side, one eagerly and one by
replaying the recorded graph, with the program's own eager work and
synchronizations between replays; every replay must match the eager result
bit for bit (same kernels, same coefficients), and both must match the oracle.
The trajectory includes an overflow (skipped step and loss-scale change, so
the graph is recorded again) and a change of gradient buffer.
"""
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


@pytest.mark.parametrize("wname,n", [("tiny", 196_864), ("gpt2", 1_000_003), ("gpt1t", 4099)])
def test_graph_replays_match_eager_and_oracle(Z, wname, n):
    w = W.get(wname)
    p, m, v, _ = W.shard_inputs(w, 0, n)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
    scaler = (lambda: Z.LossScaler(scale=w.loss_scale)) if w.loss_scale != 1.0 else (lambda: Z.LossScaler.static(1.0))
    hyper = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                 max_grad_norm=w.max_grad_norm)
    eager = Z.ShardAdam(to_device(p), to_device(m), to_device(v), scaler=scaler(), applied_steps=w.step - 1, **hyper)
    graph = Z.ShardAdam(to_device(p), to_device(m), to_device(v), scaler=scaler(), applied_steps=w.step - 1,
                        graph=True, **hyper)
    par_e = torch.zeros(n, dtype=tdt[w.param_dtype], device="cuda")
    par_g = torch.zeros(n, dtype=tdt[w.param_dtype], device="cuda")
    grads = [torch.empty(n, dtype=tdt[w.grad_dtype], device="cuda") for _ in range(2)]
    s0 = eager.scaler.s
    state, t = (p, m, v), w.step - 1
    ref_scaler = oracle.LossScalerState(scale=s0.scale, min_scale=s0.min_scale, backoff=s0.backoff,
                                        growth=s0.growth, growth_interval=s0.growth_interval)
    side = torch.randn(1 << 20, device="cuda")
    for it in range(1, 9):
        scale = eager.scaler.scale
        g = W.fill(w, "grad", 0, n, step=60 + it, loss_scale=scale)
        if it == 3:
            g[n // 3] = W.POS_INF_BITS[w.grad_dtype]
        # steps 1-3 replay one recording; the overflow at step 3 changes the
        # loss scale (dynamic scaler) and step 5 changes the gradient buffer:
        # both record again, and later steps replay the new recording
        G = grads[0 if it < 5 else 1]
        G.copy_(to_device(g, w.grad_dtype))
        skip_e = eager.step(G, par_e)
        side.mul_(1.0001).add_(0.5)                # unrelated eager work between replays
        torch.cuda.synchronize()
        skip_g = graph.step(G, par_g)
        side.sqrt_()
        torch.cuda.synchronize()
        assert skip_e == skip_g and eager.t == graph.t and eager.scaler.scale == graph.scaler.scale
        for a, b in ((eager.master, graph.master), (eager.exp_avg, graph.exp_avg),
                     (eager.exp_avg_sq, graph.exp_avg_sq)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"iteration {it}"
        assert torch.equal(par_e.view(torch.int16), par_g.view(torch.int16))
        sq, ovf = oracle.shard_sqnorm_overflow(g, w.grad_dtype, 1.0 / scale)
        ref_scaler, ref_skip = oracle.loss_scaler_update(ref_scaler, ovf)
        assert skip_g == ref_skip == (it == 3)
        if it in (2, 3, 7, 8):
            assert not graph.recorded_this_step, f"iteration {it} should replay"
        if not ref_skip:
            t += 1
            out = oracle.shard_step(*state, g, w.grad_dtype, w.param_dtype, global_sq=sq, global_overflow=False,
                                    inv_loss_scale=1.0 / scale, step=t, **hyper)
            state = out[:3]
            compare_step((graph.master.cpu().numpy(), graph.exp_avg.cpu().numpy(), graph.exp_avg_sq.cpu().numpy(),
                          bits_of(par_g)), out, what=f"it{it} ")
        assert graph.t == t and graph.scaler.scale == ref_scaler.scale
    assert t == w.step - 1 + 7


def test_coef_entry_point_matches_by_value(Z):
    """zero_shard_adam_step_coef with a device copy of the block equals
    zero_shard_adam_step bit for bit."""
    w = W.GPT2_SMALL
    n = 300_001
    p, m, v, g = W.shard_inputs(w, 5, n)
    hp = Z.AdamHyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=77,
                     inv_loss_scale=1.0 / w.loss_scale, max_grad_norm=0.3)
    coef = np.zeros(Z.zero_adam_coef_bytes(), np.uint8)
    Z.zero_adam_prepare(hp, coef)
    d_coef = torch.from_numpy(coef).cuda()
    sq = torch.tensor([123.0], dtype=torch.float64, device="cuda")
    ovf = torch.zeros(1, dtype=torch.int32, device="cuda")
    G = to_device(g, "f16")
    outs = []
    for use_coef in (False, True):
        P, M, V = to_device(p), to_device(m), to_device(v)
        par = torch.empty(n, dtype=torch.float16, device="cuda")
        if use_coef:
            Z.zero_shard_adam_step_coef(P, M, V, G, par, d_coef, sq, ovf)
        else:
            Z.zero_shard_adam_step(P, M, V, G, par, hp, sq, ovf)
        torch.cuda.synchronize()
        outs.append([P.cpu().numpy().view(np.uint32), M.cpu().numpy().view(np.uint32),
                     V.cpu().numpy().view(np.uint32), bits_of(par)])
    for a, b in zip(*outs):
        assert (a == b).all()


@pytest.mark.parametrize("wname,n", [("tiny", 196_864), ("gpt100b", 500_003)])
def test_device_state_graph_replays_match_eager(Z, wname, n):
    """The recorded device-state step (kernels only) against the eager
    device-state step: 8 steps with an overflow, back-off and growth, torch
    work and synchronisations between replays, a gradient-buffer change (one
    re-recording); every replay bit-identical, scaler and counts equal."""
    w = W.get(wname)
    p, m, v, _ = W.shard_inputs(w, 0, n)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
    hyper = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                 max_grad_norm=w.max_grad_norm)
    mk = lambda g: Z.ShardAdam(to_device(p), to_device(m), to_device(v), applied_steps=w.step - 1,  # noqa: E731
                               scaler=Z.LossScaler(scale=w.loss_scale, growth_interval=3), device_state=True,
                               graph=g, **hyper)
    eager, graph = mk(False), mk(True)
    par_e = torch.zeros(n, dtype=tdt[w.param_dtype], device="cuda")
    par_g = torch.zeros(n, dtype=tdt[w.param_dtype], device="cuda")
    grads = [torch.empty(n, dtype=tdt[w.grad_dtype], device="cuda") for _ in range(2)]
    side = torch.randn(1 << 20, device="cuda")
    recorded = []
    for it in range(1, 9):
        scale = eager.read_state().scaler.scale
        g = W.fill(w, "grad", 0, n, step=40 + it, loss_scale=scale)
        if it == 3:
            g[n // 4] = W.POS_INF_BITS[w.grad_dtype]
        G = grads[0 if it < 6 else 1]
        G.copy_(to_device(g, w.grad_dtype))
        eager.step(G, par_e)
        side.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        graph.step(G, par_g)
        side.abs_().sqrt_()
        recorded.append(graph.recorded_this_step)
        se, sg = eager.read_state(), graph.read_state()
        assert bytes(se) == bytes(sg), f"iteration {it}"
        assert sg.last_overflow == (it == 3)
        for a, b in ((eager.master, graph.master), (eager.exp_avg, graph.exp_avg),
                     (eager.exp_avg_sq, graph.exp_avg_sq)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"iteration {it}"
        assert torch.equal(par_e.view(torch.int16), par_g.view(torch.int16))
    assert recorded == [True, False, False, False, False, True, False, False]
    assert sg.skipped == 1 and sg.applied == w.step - 1 + 7
