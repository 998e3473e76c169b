"""GPU parity at full workload sizes, in the launch configuration the
benchmark times.

Inputs are generated block by block on the host and copied into HBM; the
oracle computes the exact gradient norm over the whole shard from the same
host blocks and the update at sampled elements (the first and last elements,
the real/padding boundary and ~100k random positions).  Padding elements must
stay exactly zero.
"""
import numpy as np
import pytest

import oracle
import workloads as W

from parity import bits_of, check_norm, compare_step

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BLOCK = 8 * W.CHUNK        # host generation block (elements)
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    yield Z
    torch.cuda.empty_cache()


def _samples(S, real, k=100_000):
    idx = set(W.sample_indices(S, k).tolist())
    idx |= {i for i in range(real - 4, min(S, real + 4)) if 0 <= i < S}
    return np.array(sorted(idx), dtype=np.int64)


def _gather(t, idx_t):
    return t.index_select(0, idx_t)


def _upload(w, begin, S, idx, step):
    """Streams the shard's inputs into HBM; returns device tensors, the host
    values at the sampled indices, and the oracle's (sq, overflow)."""
    P = torch.empty(S, dtype=torch.float32, device="cuda")
    M = torch.empty_like(P)
    V = torch.empty_like(P)
    G = torch.empty(S, dtype=TDT[w.grad_dtype], device="cuda")
    host = {k: [] for k in ("p", "m", "v", "g")}

    def blocks():
        for lo in range(0, S, BLOCK):
            n = min(BLOCK, S - lo)
            p, m, v, g = W.shard_inputs(w, begin + lo, n, step=step)
            for dst, src in ((P, p), (M, m), (V, v)):
                dst[lo:lo + n].copy_(torch.from_numpy(src))
            G[lo:lo + n].copy_(torch.from_numpy(g.view(np.int16)).view(G.dtype))
            sel = idx[(idx >= lo) & (idx < lo + n)] - lo
            for k, a in (("p", p), ("m", m), ("v", v), ("g", g)):
                host[k].append(a[sel])
            yield g

    ref_sq, ref_ovf = oracle.global_sqnorm_overflow(blocks(), w.grad_dtype, 1.0 / w.loss_scale)
    return (P, M, V, G), {k: np.concatenate(a) for k, a in host.items()}, ref_sq, ref_ovf


@pytest.mark.parametrize("wname", ["gpt1t", "llama7b"])
def test_single_step_full_shard(Z, wname):
    w = W.get(wname)
    _, S, _ = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    begin = w.rank * S
    real = min(S, max(0, W.real_total(w) - begin))
    idx = _samples(S, real)
    (P, M, V, G), h, ref_sq, ref_ovf = _upload(w, begin, S, idx, w.step)
    par = torch.empty(S, dtype=TDT[w.param_dtype], device="cuda")
    inv = 1.0 / w.loss_scale
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=w.max_grad_norm, step=w.step, inv_loss_scale=inv)
    # the launch configuration bench.py times: step state in device memory, the
    # decision in the norm pass's last kernel, the update reading the device
    # coefficients; one rank's own sum of squares stands in for the all-reduced one
    opt = Z.ShardAdam(P, M, V, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                      max_grad_norm=w.max_grad_norm, applied_steps=w.step - 1, device_state=True,
                      scaler=Z.LossScaler.static(w.loss_scale))
    opt.step(G, par)
    st = opt.read_state()
    assert st.last_overflow == int(ref_ovf) == 0 and st.applied == w.step
    check_norm(opt.sqnorm.item(), ref_sq)
    idx_t = torch.from_numpy(idx).cuda()
    got = (_gather(P, idx_t).cpu().numpy(), _gather(M, idx_t).cpu().numpy(), _gather(V, idx_t).cpu().numpy(),
           bits_of(_gather(par, idx_t)))
    ref = oracle.shard_step(h["p"], h["m"], h["v"], h["g"], w.grad_dtype, w.param_dtype, global_sq=ref_sq,
                            global_overflow=False, **hp)
    compare_step(got, ref, what=f"{w.name} ")
    if real < S:                                   # padding stays exactly zero
        for t in (P, M, V):
            assert bool((t[real:] == 0).all().item())
        assert bool((par[real:].view(torch.int16) == 0).all().item())
    del P, M, V, G, par
    torch.cuda.empty_cache()


@pytest.mark.parametrize("device_state", [True, False])
def test_trajectory_with_overflow_full_shard(Z, device_state):
    """One rank's 250M-parameter shard of a 100B model over 20 steps with
    +inf injected into 0.1% of the gradient at iterations 5 and 12: skip
    decisions, loss scale and step counter bit-exact; norms and sampled
    state within tolerance after every applied step (step state in device
    memory, as bench.py runs it, and on the host)."""
    w = W.GPT_100B_RANK
    _, S, _ = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    begin = w.rank * S
    idx = _samples(S, S, k=50_000)
    idx_t = torch.from_numpy(idx).cuda()
    P = torch.empty(S, dtype=torch.float32, device="cuda")
    ref_p = []
    for lo in range(0, S, BLOCK):
        n = min(BLOCK, S - lo)
        p = W.fill(w, "master", begin + lo, n)
        P[lo:lo + n].copy_(torch.from_numpy(p))
        ref_p.append(p[idx[(idx >= lo) & (idx < lo + n)] - lo])
    ref_p = np.concatenate(ref_p)
    M = torch.zeros_like(P)
    V = torch.zeros_like(P)
    G = torch.empty(S, dtype=torch.float16, device="cuda")
    par = torch.empty(S, dtype=torch.float16, device="cuda")
    ref_m = np.zeros_like(ref_p)
    ref_v = np.zeros_like(ref_p)
    opt = Z.ShardAdam(P, M, V, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                      max_grad_norm=w.max_grad_norm, scaler=Z.LossScaler(scale=w.loss_scale),
                      device_state=device_state)
    scaler, t, skips = oracle.LossScalerState(scale=w.loss_scale), 0, []
    last = None
    for it in range(1, w.n_steps + 1):
        scale = opt.read_state().scaler.scale if device_state else opt.scaler.scale
        assert scale == scaler.scale
        g = W.grad_for_step(w, begin, S, it, scale)
        G.copy_(torch.from_numpy(g.view(np.int16)).view(torch.float16))
        skip = opt.step(G, par)
        if device_state:
            skip = bool(opt.read_state().last_overflow)
        ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(g, "f16", 1.0 / scale)
        scaler, ref_skip = oracle.loss_scaler_update(scaler, ref_ovf)
        assert skip == ref_skip and int(opt.overflow.item()) == int(ref_ovf)
        if ref_skip:
            skips.append(it)
            continue
        t += 1
        check_norm(opt.sqnorm.item(), ref_sq)
        last = oracle.shard_step(ref_p, ref_m, ref_v, g[idx], "f16", "f16", global_sq=ref_sq, global_overflow=False,
                                 inv_loss_scale=1.0 / scale, max_grad_norm=w.max_grad_norm, lr=w.lr,
                                 beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=t)
        ref_p, ref_m, ref_v = last[:3]
        assert opt.t == t and opt.scaler.scale == scaler.scale
    assert skips == [5, 12] and t == 18 and scaler.scale == w.loss_scale / 4
    got = (_gather(P, idx_t).cpu().numpy(), _gather(M, idx_t).cpu().numpy(), _gather(V, idx_t).cpu().numpy(),
           bits_of(_gather(par, idx_t)))
    compare_step(got, last, what="after 20 iterations ")
    del P, M, V, G, par
    torch.cuda.empty_cache()


def test_fp32_accumulation_full_shard(Z):
    """The 1T model's last-rank shard (976M params) with 4 micro-batches
    accumulated into the fp32 gradient copy, then the step on that copy: the
    oracle accumulates the same micro-batches, takes the norm over the whole
    fp32 copy and checks the update at sampled elements."""
    w = W.GPT_1T_LAST_RANK
    K = 4
    _, S, _ = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    begin = w.rank * S
    real = min(S, max(0, W.real_total(w) - begin))
    idx = _samples(S, real, k=50_000)
    P = torch.empty(S, dtype=torch.float32, device="cuda")
    M = torch.empty_like(P)
    V = torch.empty_like(P)
    Gs = [torch.empty(S, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    host = {k: [] for k in ("p", "m", "v", "acc")}
    inv = 1.0 / w.loss_scale

    def acc_blocks():
        for lo in range(0, S, BLOCK):
            n = min(BLOCK, S - lo)
            p, m, v, _ = W.shard_inputs(w, begin + lo, n)
            for dst, src in ((P, p), (M, m), (V, v)):
                dst[lo:lo + n].copy_(torch.from_numpy(src))
            acc = None
            for k in range(K):
                g = W.fill(w, "grad", begin + lo, n, step=500 + k)
                Gs[k][lo:lo + n].copy_(torch.from_numpy(g.view(np.int16)).view(torch.bfloat16))
                acc, _ = oracle.grad_accumulate(acc, g, "bf16", inv)
            sel = idx[(idx >= lo) & (idx < lo + n)] - lo
            for key, a in (("p", p), ("m", m), ("v", v), ("acc", acc)):
                host[key].append(a[sel])
            yield acc

    ref_sq, ref_ovf = oracle.global_sqnorm_overflow(acc_blocks(), "f32", 1.0)
    h = {k: np.concatenate(a) for k, a in host.items()}
    A = torch.empty(S, dtype=torch.float32, device="cuda")
    par = torch.empty(S, dtype=torch.bfloat16, device="cuda")
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=w.max_grad_norm, step=w.step, inv_loss_scale=1.0)
    # as bench.py --accum runs it: device step state, the last micro-batch
    # writing the copy and its norm in one pass
    opt = Z.ShardAdam(P, M, V, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                      max_grad_norm=w.max_grad_norm, applied_steps=w.step - 1, device_state=True,
                      scaler=Z.LossScaler.static(w.loss_scale))
    for k in range(K):
        opt.accumulate(A, Gs[k], first=(k == 0), last=(k == K - 1))
    opt.step(A, par, norm_done=True)
    st = opt.read_state()
    del Gs
    assert st.last_overflow == int(ref_ovf) == 0 and st.applied == w.step
    check_norm(opt.sqnorm.item(), ref_sq)
    idx_t = torch.from_numpy(idx).cuda()
    acc_got = _gather(A, idx_t).cpu().numpy()
    assert (np.abs(acc_got.astype(np.float64) - h["acc"]) <= np.abs(np.spacing(h["acc"]))).all()
    got = (_gather(P, idx_t).cpu().numpy(), _gather(M, idx_t).cpu().numpy(), _gather(V, idx_t).cpu().numpy(),
           bits_of(_gather(par, idx_t)))
    ref = oracle.shard_step(h["p"], h["m"], h["v"], h["acc"], "f32", w.param_dtype, global_sq=ref_sq,
                            global_overflow=False, **hp)
    compare_step(got, ref, what="accumulated ")
    if real < S:
        assert bool((A[real:] == 0).all().item()) and bool((P[real:] == 0).all().item())
    del P, M, V, A, par
    torch.cuda.empty_cache()
