"""GPU: the local half of the scalars' all-reduce (zero_norm_combine_ranks).
The combined sum of squares equals the rank-order float64 sum of the slots bit
for bit (a plain sequential sum, as a host loop over ranks forms it), and the
flag is the OR of the slots, for 1 to 65,536 ranks and across staging
boundaries; and, on every rank of a small workload stepped on one GPU, the
combined scalars drive the update to the oracle's result."""
import numpy as np
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


def _host_sum(xs):
    total = 0.0
    for x in xs:                                # rank order, one float64 rounding per addition
        total += float(x)
    return total


@pytest.mark.parametrize("n_ranks", [1, 2, 7, 8, 400, 1023, 1024, 1025, 3000, 65536])
@pytest.mark.parametrize("flag_at", [None, "first", "last", "middle"])
def test_combine_equals_rank_order_sum(Z, n_ranks, flag_at):
    rng = np.random.default_rng(n_ranks)
    sq = rng.random(n_ranks) * 10.0 ** rng.integers(-6, 6, n_ranks)     # wide magnitudes: order matters
    ovf = np.zeros(n_ranks, np.int32)
    if flag_at is not None:
        ovf[{"first": 0, "last": n_ranks - 1, "middle": n_ranks // 2}[flag_at]] = 7
    gsq = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    govf = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    Z.zero_norm_combine_ranks(torch.from_numpy(sq).cuda(), torch.from_numpy(ovf).cuda(), gsq, govf)
    torch.cuda.synchronize()
    assert gsq.item() == _host_sum(sq)          # bit for bit
    assert govf.item() == (0 if flag_at is None else 1)


def test_all_ranks_of_gpt2_through_the_combine(Z):
    """Every rank of GPT-2 small (N_d = 8) on one GPU: each rank's norm pass
    writes into its slot, the combine forms the global scalars on the device,
    and each rank's update with them matches the oracle."""
    w = W.GPT2_SMALL
    _, S, padded = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    p, m, v, g = W.shard_inputs(w, 0, padded)
    P, M, V, G = to_device(p), to_device(m), to_device(v), to_device(g, w.grad_dtype)
    par = torch.empty(padded, dtype=torch.float16, device="cuda")
    inv = 1.0 / w.loss_scale
    slot_sq = torch.empty(w.n_d, dtype=torch.float64, device="cuda")
    slot_ovf = torch.empty(w.n_d, dtype=torch.int32, device="cuda")
    ws = torch.empty(Z.zero_norm_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    for r in range(w.n_d):
        Z.zero_shard_unscale_norm_overflow(G[r * S:(r + 1) * S], inv, slot_sq[r:r + 1], slot_ovf[r:r + 1], ws)
    gsq = torch.empty(1, dtype=torch.float64, device="cuda")
    govf = torch.empty(1, dtype=torch.int32, device="cuda")
    Z.zero_norm_combine_ranks(slot_sq, slot_ovf, gsq, govf)
    torch.cuda.synchronize()
    assert gsq.item() == _host_sum(slot_sq.cpu().numpy()) and govf.item() == 0
    ref_sq, ref_ovf = oracle.global_sqnorm_overflow([g[r * S:(r + 1) * S] for r in range(w.n_d)], w.grad_dtype, inv)
    assert not ref_ovf
    check_norm(gsq.item(), ref_sq)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=w.max_grad_norm, step=w.step, inv_loss_scale=inv)
    for r in range(w.n_d):
        sl = slice(r * S, (r + 1) * S)
        Z.zero_shard_adam_step(P[sl], M[sl], V[sl], G[sl], par[sl], Z.AdamHyper(**hp), gsq, govf)
    torch.cuda.synchronize()
    gp, gm, gv, gpar = P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par)
    for r in (0, 3, w.n_d - 1):
        sl = slice(r * S, (r + 1) * S)
        ref = oracle.shard_step(p[sl], m[sl], v[sl], g[sl], w.grad_dtype, w.param_dtype, global_sq=ref_sq,
                                global_overflow=False, **hp)
        compare_step((gp[sl], gm[sl], gv[sl], gpar[sl]), ref, what=f"rank{r} ")


def test_data_parallel_device_state_protocol(Z):
    """The data-parallel step with device-resident state, every rank on one
    GPU: each of 8 ranks (own ShardAdam, own step state) runs its norm pass;
    its (sum of squares, flag) lands in slot r; the combine forms the global
    pair; each rank then decides and updates.  Over 4 steps with an inf in one
    rank's gradient at step 2, every rank skips that step, the 8 states stay
    bit-identical, and the shards of ranks 0, 5 (the one with the inf) and 7
    match the oracle."""
    w = W.GPT2_SMALL
    _, S, padded = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    n_d = w.n_d
    p, m, v, _ = W.shard_inputs(w, 0, padded)
    P, M, V = to_device(p), to_device(m), to_device(v)
    par = torch.empty(padded, dtype=torch.float16, device="cuda")
    opts = [Z.ShardAdam(P[r * S:(r + 1) * S], M[r * S:(r + 1) * S], V[r * S:(r + 1) * S], lr=w.lr, beta1=w.beta1,
                        beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm,
                        scaler=Z.LossScaler(scale=w.loss_scale, growth_interval=1000), applied_steps=w.step - 1,
                        device_state=True) for r in range(n_d)]
    slot_sq = torch.empty(n_d, dtype=torch.float64, device="cuda")
    slot_ovf = torch.empty(n_d, dtype=torch.int32, device="cuda")
    gsq = torch.empty(1, dtype=torch.float64, device="cuda")
    govf = torch.empty(1, dtype=torch.int32, device="cuda")
    tracked = (0, 5, n_d - 1)                                        # ranks stepped by the oracle too
    ref = {r: (p[r * S:(r + 1) * S], m[r * S:(r + 1) * S], v[r * S:(r + 1) * S]) for r in tracked}
    outs = {}
    scaler, t = oracle.LossScalerState(scale=w.loss_scale), w.step - 1
    for it in range(1, 5):
        g = W.fill(w, "grad", 0, padded, step=300 + it, loss_scale=scaler.scale)
        if it == 2:
            g[5 * S + 123] = W.POS_INF_BITS[w.grad_dtype]              # one element on rank 5
        G = to_device(g, w.grad_dtype)
        for r, opt in enumerate(opts):                                  # every rank's norm pass into its slot
            opt.unscale_norm(G[r * S:(r + 1) * S])
            slot_sq[r:r + 1].copy_(opt.sqnorm)
            slot_ovf[r:r + 1].copy_(opt.overflow)
        Z.zero_norm_combine_ranks(slot_sq, slot_ovf, gsq, govf)         # the exchange's local half
        for r, opt in enumerate(opts):
            opt.apply(G[r * S:(r + 1) * S], par[r * S:(r + 1) * S], global_sqnorm=gsq, global_overflow=govf)
        states = [bytes(opt.read_state()) for opt in opts]
        assert all(s_ == states[0] for s_ in states), f"iteration {it}: the ranks' states diverged"
        inv = 1.0 / scaler.scale
        ref_sq, ref_ovf = oracle.global_sqnorm_overflow([g[r * S:(r + 1) * S] for r in range(n_d)],
                                                        w.grad_dtype, inv)
        assert int(govf.item()) == int(ref_ovf) == (it == 2)
        scaler, skip = oracle.loss_scaler_update(scaler, ref_ovf)
        st = opts[0].read_state()
        assert bool(st.last_overflow) == skip and st.scaler.scale == scaler.scale
        if skip:
            continue
        t += 1
        assert st.applied == t
        check_norm(gsq.item(), ref_sq)
        hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                  max_grad_norm=w.max_grad_norm, step=t, inv_loss_scale=inv)
        for r in tracked:
            out = oracle.shard_step(*ref[r], g[r * S:(r + 1) * S], w.grad_dtype, w.param_dtype, global_sq=ref_sq,
                                    global_overflow=False, **hp)
            ref[r] = out[:3]
            outs[r] = out
    gp, gm, gv, gpar = P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par)
    for r in tracked:
        sl = slice(r * S, (r + 1) * S)
        compare_step((gp[sl], gm[sl], gv[sl], gpar[sl]), outs[r], what=f"rank{r} after 4 iterations ")
