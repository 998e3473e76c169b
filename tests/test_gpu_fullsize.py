"""GPU parity at full workload sizes, every element of the shard, in the
launch configuration the benchmark times.  Besides the oracle's bar, every
element of master, exp_avg and exp_avg_sq of the device steps must equal the
float32 model of the header's documented operation order (f32model) bit for
bit (the offloaded step's host loop follows the same order).

Inputs are drawn chunk by chunk on the host (a pool of threads, see
`fullshard`) and copied into HBM.  The oracle computes the exact gradient norm
over the whole shard and the step of every element from the same host chunks;
its results go to device memory beside the GPU's, and after the GPU step
every element of master, exp_avg, exp_avg_sq and the 16-bit parameter copy is
compared with them (the strict second-moment check as well on single steps).
Padding elements must stay exactly zero.
"""
import time

import numpy as np
import pytest

import f32model
import oracle
import workloads as W
import fullshard as F

from parity import check_norm

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    yield Z
    torch.cuda.empty_cache()


def _put(dst, lo: int, a: np.ndarray) -> None:
    """Host array -> dst[lo:lo+len(a)] (16-bit patterns go in as raw bits)."""
    if a.dtype == np.uint16:
        dst.view(torch.int16)[lo:lo + a.size].copy_(torch.from_numpy(a.view(np.int16)))
    else:
        dst[lo:lo + a.size].copy_(torch.from_numpy(a))


def _f32(S):
    return torch.empty(S, dtype=torch.float32, device="cuda")


def _hp(w, step, inv):
    return dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                max_grad_norm=w.max_grad_norm, step=step, inv_loss_scale=inv)


def _values(g: np.ndarray, fmt: str) -> np.ndarray:
    """Gradient values as float32: 16-bit patterns decoded exactly, or the fp32 copy."""
    if fmt == "f32":
        return np.asarray(g, np.float32)
    if fmt == "f16":
        return g.view(np.float16).astype(np.float32)
    return (g.astype(np.uint32) << 16).view(np.float32)


def _state_and_reference(w, begin, blocks, grad_host, gfmt, ref_sq, hp, dev, ref, model=None):
    """Draws master, exp_avg and exp_avg_sq chunk by chunk, runs the oracle's
    step on each chunk (gradient from grad_host, the whole shard's norm
    ref_sq), and moves the inputs into dev = (P, M, V) and the oracle's
    results into ref = (RP, RM, RV, RPAR).  With model = three host float32
    arrays, the float32 model of the documented operation order (f32model)
    is run on each chunk too, into them."""
    def task(b):
        lo, hi = b
        n = hi - lo
        p, m, v = (W.fill(w, a, begin + lo, n, threads=1) for a in ("master", "exp_avg", "exp_avg_sq"))
        out = (np.empty(n, np.float32), np.empty(n, np.float32), np.empty(n, np.float32), np.empty(n, np.uint16))
        for a, c in F.by_sub(n):
            g = grad_host[lo + a:lo + c]
            r = oracle.shard_step(p[a:c], m[a:c], v[a:c], g, gfmt, w.param_dtype,
                                  global_sq=ref_sq, global_overflow=False, **hp)
            for k in range(4):
                out[k][a:c] = r[k]
            if model is not None:
                for dst, x in zip(model, f32model.adam_update(p[a:c], m[a:c], v[a:c], _values(g, gfmt), ref_sq, **hp)):
                    dst[lo + a:lo + c] = x
        return (p, m, v), out

    for (lo, _), (ins, out) in F.pmap(task, blocks):
        for d, a in zip(dev, ins):
            _put(d, lo, a)
        for d, a in zip(ref, out):
            _put(d, lo, a)


def _compare(blocks, got, ref, what, pfmt, strict=True):
    """Every element of got = (P, M, V, param) against ref = (RP, RM, RV,
    RPAR) on the device, and the writeback against the device's own master;
    returns the tallies (all must be clean)."""
    P, M, V, par = got
    RP, RM, RV, RPAR = ref
    vs = "exp_avg_sq (strict)" if strict else "exp_avg_sq (strict, report only)"
    names = ["master", "exp_avg", "exp_avg_sq", vs, "param", "param = RNE(own master)"]
    tl = {k: F.Tally(what + k) for k in names}
    pb, rb = par.view(torch.int16), RPAR.view(torch.int16)
    for lo, hi in blocks:
        F.tally_f32(tl["master"], P[lo:hi], RP[lo:hi], lo)
        F.tally_f32(tl["exp_avg"], M[lo:hi], RM[lo:hi], lo)
        F.tally_f32(tl["exp_avg_sq"], V[lo:hi], RV[lo:hi], lo)
        F.tally_strict_v(tl[vs], V[lo:hi], RV[lo:hi], lo)
        F.tally_param(tl["param"], pb[lo:hi], rb[lo:hi], lo, pfmt)
        F.tally_writeback(tl["param = RNE(own master)"], P[lo:hi], pb[lo:hi], lo, pfmt)
    tl = list(tl.values())
    F.assert_all(tl)
    return tl


def _check_model(blocks, got, model, gpu_sq, ref_sq, hp):
    """Every element of the GPU's master, exp_avg and exp_avg_sq equals the
    float32 model bit for bit.  The model ran with the oracle's sum of
    squares; the gradient factor it gives must be the one the GPU's own sum
    gives, so the two ran the same arithmetic."""
    fac = lambda sq: f32model.gradient_factor(hp["inv_loss_scale"], hp["max_grad_norm"], sq)  # noqa: E731
    assert fac(gpu_sq) == fac(ref_sq), "gradient factor from the GPU's norm differs from the oracle's"
    bad = 0
    for lo, hi in blocks:
        for t, x in zip(got, model):
            bad += int((t[lo:hi].cpu().numpy().view(np.uint32) != x[lo:hi].view(np.uint32)).sum())
    assert bad == 0, f"{bad} elements differ from the float32 model"
    return bad


def _padding_zero(real, S, tensors, par):
    if real < S:
        for t in tensors:
            assert bool((t[real:] == 0).all().item())
        assert bool((par[real:].view(torch.int16) == 0).all().item())


@pytest.mark.parametrize("wname", ["gpt1t", "llama7b"])
def test_single_step_full_shard(Z, wname):
    """The 1T model's last-rank shard (976M, bf16, padded tail) and Llama-7B
    at N_d = 1 (6.7B, 108 GB of state): one step, every element."""
    w = W.get(wname)
    _, S, _ = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    begin = w.rank * S
    real = min(S, max(0, W.real_total(w) - begin))
    fmt, inv = w.grad_dtype, 1.0 / w.loss_scale
    blocks = F.chunk_blocks(begin, S)
    t0 = time.perf_counter()
    P, M, V = _f32(S), _f32(S), _f32(S)
    G = torch.empty(S, dtype=TDT[fmt], device="cuda")
    par = torch.empty(S, dtype=TDT[w.param_dtype], device="cuda")
    ghost = np.empty(S, np.uint16)

    def grad_task(b):
        lo, hi = b
        g = W.fill(w, "grad", begin + lo, hi - lo, step=w.step, threads=1)
        ghost[lo:hi] = g
        return oracle.sqnorm_terms(g, fmt, inv)

    terms = []
    for (lo, hi), tm in F.pmap(grad_task, blocks):
        _put(G, lo, ghost[lo:hi])
        terms.append(tm)
    ref_sq, ref_ovf = oracle.combine_sqnorm_terms(terms, fmt, inv)
    hp = _hp(w, w.step, inv)
    ref = (_f32(S), _f32(S), _f32(S), torch.empty(S, dtype=torch.int16, device="cuda"))
    model = tuple(np.empty(S, np.float32) for _ in range(3))
    _state_and_reference(w, begin, blocks, ghost, fmt, ref_sq, hp, (P, M, V), ref, model)
    del ghost
    t1 = time.perf_counter()
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
    tl = _compare(blocks, (P, M, V, par), ref, f"{w.name} ", w.param_dtype)
    _check_model(blocks, (P, M, V), model, opt.sqnorm.item(), ref_sq, hp)
    del model
    _padding_zero(real, S, (P, M, V), par)
    print(f"\n{w.name}: S={S} every element within the bar and equal to the float32 model: {tl}; host+upload {t1 - t0:.1f} s, "
          f"compare {time.perf_counter() - t1:.1f} s", flush=True)
    del P, M, V, G, par, ref, opt
    torch.cuda.empty_cache()


def test_trajectory_with_overflow_full_shard(Z):
    """One rank's 250M-parameter shard of a 100B model over 20 steps with
    +inf injected into 0.1% of the gradient at iterations 5 and 12, on both
    scaler paths at once (step state in device memory, as bench.py runs it,
    and on the host): skip decisions, loss scale and step counter bit-exact
    against the oracle's loss scaler; norms within the bar after every applied
    step; the two GPU paths bit-identical to each other; and every element of
    both against the oracle's own 20-iteration trajectory, which keeps its
    float32 state on the host, and bit for bit against the float32 model's
    own trajectory.  Each side rounds its own state every step, so
    after 18 applied steps the comparison is held to the bar (1e-5 / 1e-7,
    1 ulp), not to the tighter single-step check of the second moment."""
    w = W.GPT_100B_RANK
    _, S, _ = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    begin = w.rank * S
    blocks = F.chunk_blocks(begin, S)
    ref_p = np.empty(S, np.float32)
    ref_m = np.zeros(S, np.float32)
    ref_v = np.zeros(S, np.float32)
    ref_par = np.empty(S, np.uint16)
    mod_p, mod_m, mod_v = np.empty(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.float32)
    Pa, Pb = _f32(S), _f32(S)

    def master_task(b):
        lo, hi = b
        ref_p[lo:hi] = W.fill(w, "master", begin + lo, hi - lo, threads=1)
        mod_p[lo:hi] = ref_p[lo:hi]

    for (lo, hi), _ in F.pmap(master_task, blocks):
        _put(Pa, lo, ref_p[lo:hi])
    Pb.copy_(Pa)
    Ma, Va, Mb, Vb = (torch.zeros(S, dtype=torch.float32, device="cuda") for _ in range(4))
    G = torch.empty(S, dtype=torch.float16, device="cuda")
    par_a = torch.empty(S, dtype=torch.float16, device="cuda")
    par_b = torch.empty_like(par_a)
    kw = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=w.max_grad_norm)
    opt_a = Z.ShardAdam(Pa, Ma, Va, scaler=Z.LossScaler(scale=w.loss_scale), device_state=True, **kw)
    opt_b = Z.ShardAdam(Pb, Mb, Vb, scaler=Z.LossScaler(scale=w.loss_scale), device_state=False, **kw)
    scaler, t, skips = oracle.LossScalerState(scale=w.loss_scale), 0, []
    for it in range(1, w.n_steps + 1):
        scale = scaler.scale
        assert opt_a.read_state().scaler.scale == scale == opt_b.scaler.scale
        g = W.grad_for_step(w, begin, S, it, scale)
        _put(G, 0, g)
        opt_a.step(G, par_a)
        skip_b = opt_b.step(G, par_b)
        st = opt_a.read_state()
        inv = 1.0 / scale
        ref_sq, ref_ovf = oracle.combine_sqnorm_terms(
            [tm for _, tm in F.pmap(lambda b: oracle.sqnorm_terms(g[b[0]:b[1]], "f16", inv), blocks)], "f16", inv)
        scaler, ref_skip = oracle.loss_scaler_update(scaler, ref_ovf)
        assert bool(st.last_overflow) == skip_b == ref_skip
        assert int(opt_a.overflow.item()) == int(opt_b.overflow.item()) == int(ref_ovf)
        if ref_skip:
            skips.append(it)
            continue
        t += 1
        check_norm(opt_a.sqnorm.item(), ref_sq)
        check_norm(opt_b.sqnorm.item(), ref_sq)
        last = it == w.n_steps
        hp_t = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=t,
                    inv_loss_scale=inv, max_grad_norm=w.max_grad_norm)
        fac = lambda sq: f32model.gradient_factor(inv, w.max_grad_norm, sq)  # noqa: E731
        assert fac(opt_a.sqnorm.item()) == fac(ref_sq), "gradient factor from the GPU's norm differs"

        def step_task(b, t=t, ref_sq=ref_sq, inv=inv, last=last, hp_t=hp_t):
            lo, hi = b
            for a, c in F.by_sub(hi - lo):
                s = slice(lo + a, lo + c)
                r = oracle.shard_step(ref_p[s], ref_m[s], ref_v[s], g[s], "f16", "f16" if last else None,
                                      global_sq=ref_sq, global_overflow=False, inv_loss_scale=inv,
                                      max_grad_norm=w.max_grad_norm, lr=w.lr, beta1=w.beta1, beta2=w.beta2,
                                      eps=w.eps, weight_decay=w.weight_decay, step=t)
                ref_p[s], ref_m[s], ref_v[s] = r[0], r[1], r[2]
                if last:
                    ref_par[s] = r[3]
                # the float32 model carries its own state from step to step
                mod_p[s], mod_m[s], mod_v[s] = f32model.adam_update(mod_p[s], mod_m[s], mod_v[s],
                                                                     _values(g[s], "f16"), ref_sq, **hp_t)

        for _ in F.pmap(step_task, blocks):
            pass
        assert opt_a.read_state().applied == opt_b.t == t and opt_b.scaler.scale == scaler.scale
    assert skips == [5, 12] and t == 18 and scaler.scale == w.loss_scale / 4
    # the last iteration was applied, so ref_par holds its writeback
    for x, y in ((Pa, Pb), (Ma, Mb), (Va, Vb), (par_a, par_b)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), "scaler paths differ"
    ref = tuple(torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
                for a in (ref_p, ref_m, ref_v, ref_par))
    tl = _compare(blocks, (Pa, Ma, Va, par_a), ref, "after 20 iterations ", "f16", strict=False)
    bad = 0
    for lo, hi in blocks:
        for t_, x in ((Pa, mod_p), (Ma, mod_m), (Va, mod_v)):
            bad += int((t_[lo:hi].cpu().numpy().view(np.uint32) != x[lo:hi].view(np.uint32)).sum())
    assert bad == 0, f"{bad} elements differ from the float32 model's 20-iteration trajectory"
    print(f"\n100B rank shard, 20 iterations: every element within the bar and equal to the float32 model: {tl}",
          flush=True)
    del Pa, Pb, Ma, Mb, Va, Vb, G, par_a, par_b, ref, opt_a, opt_b
    torch.cuda.empty_cache()


def test_fp32_accumulation_full_shard(Z):
    """The 1T model's last-rank shard (976M params) with 4 micro-batches
    accumulated into the fp32 gradient copy, the last one forming the copy's
    norm in the same pass (as bench.py --accum 4 runs it), then the step on
    that copy: the oracle accumulates the same micro-batches, takes the norm
    over the whole fp32 copy, and every element of the copy (within 1 fp32
    ulp) and of the updated state is compared."""
    w = W.GPT_1T_LAST_RANK
    K = 4
    _, S, _ = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    begin = w.rank * S
    real = min(S, max(0, W.real_total(w) - begin))
    blocks = F.chunk_blocks(begin, S)
    inv = 1.0 / w.loss_scale
    P, M, V = _f32(S), _f32(S), _f32(S)
    Gs = [torch.empty(S, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    acc_host = np.empty(S, np.float32)

    def acc_task(b):
        lo, hi = b
        gs = [W.fill(w, "grad", begin + lo, hi - lo, step=500 + k, threads=1) for k in range(K)]
        for a, c in F.by_sub(hi - lo):
            acc = None
            for g in gs:
                acc, _ = oracle.grad_accumulate(acc, g[a:c], "bf16", inv)
            acc_host[lo + a:lo + c] = acc
        return gs, oracle.sqnorm_terms(acc_host[lo:hi], "f32", 1.0)

    terms = []
    for (lo, hi), (gs, tm) in F.pmap(acc_task, blocks):
        for k in range(K):
            _put(Gs[k], lo, gs[k])
        terms.append(tm)
    ref_sq, ref_ovf = oracle.combine_sqnorm_terms(terms, "f32", 1.0)
    ref = (_f32(S), _f32(S), _f32(S), torch.empty(S, dtype=torch.int16, device="cuda"))
    hp = _hp(w, w.step, 1.0)
    model = tuple(np.empty(S, np.float32) for _ in range(3))
    _state_and_reference(w, begin, blocks, acc_host, "f32", ref_sq, hp, (P, M, V), ref, model)
    A = _f32(S)
    par = torch.empty(S, dtype=torch.bfloat16, device="cuda")
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
    RA = torch.from_numpy(acc_host).cuda()
    ta = F.Tally("fp32 gradient copy (1 ulp)")
    for lo, hi in blocks:
        F.tally_ulp_f32(ta, A[lo:hi], RA[lo:hi], lo)
    F.assert_all([ta])
    tl = _compare(blocks, (P, M, V, par), ref, "accumulated ", w.param_dtype)
    _check_model(blocks, (P, M, V), model, opt.sqnorm.item(), ref_sq, hp)
    del model
    _padding_zero(real, S, (P, M, V, A), par)
    print(f"\n1T shard, 4 micro-batches: every element within the bar: {ta}; {tl}", flush=True)
    del P, M, V, A, RA, par, ref, opt
    torch.cuda.empty_cache()


def test_reduction_full_shard(Z):
    """The 1T model's last-rank shard (976M params) with its gradient formed
    as the reduction of 8 ranks' distinct bf16 slices into the fp32 copy, the
    copy's norm in the same pass (as bench.py --reduce 8 runs it), then the
    step on that copy: the oracle reduces the same slices in rank order, takes
    the norm over the whole fp32 copy, and every element of the copy (within
    1 fp32 ulp) and of the updated state is compared."""
    w = W.GPT_1T_LAST_RANK
    K = 8
    _, S, _ = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    begin = w.rank * S
    real = min(S, max(0, W.real_total(w) - begin))
    blocks = F.chunk_blocks(begin, S)
    inv = 1.0 / (K * w.loss_scale)                 # the mean over the ranks, folded into the unscale
    P, M, V = _f32(S), _f32(S), _f32(S)
    slices = [torch.empty(S, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    acc_host = np.empty(S, np.float32)

    def red_task(b):
        lo, hi = b
        gs = [W.fill(w, "grad", begin + lo, hi - lo, step=600 + k, threads=1) for k in range(K)]
        for a, c in F.by_sub(hi - lo):
            acc_host[lo + a:lo + c], ovf = oracle.grad_reduce([g[a:c] for g in gs], "bf16", inv)
            assert not ovf
        return gs, oracle.sqnorm_terms(acc_host[lo:hi], "f32", 1.0)

    terms = []
    for (lo, hi), (gs, tm) in F.pmap(red_task, blocks):
        for k in range(K):
            _put(slices[k], lo, gs[k])
        terms.append(tm)
    ref_sq, ref_ovf = oracle.combine_sqnorm_terms(terms, "f32", 1.0)
    ref = (_f32(S), _f32(S), _f32(S), torch.empty(S, dtype=torch.int16, device="cuda"))
    hp = _hp(w, w.step, 1.0)
    model = tuple(np.empty(S, np.float32) for _ in range(3))
    _state_and_reference(w, begin, blocks, acc_host, "f32", ref_sq, hp, (P, M, V), ref, model)
    A = _f32(S)
    par = torch.empty(S, dtype=torch.bfloat16, device="cuda")
    opt = Z.ShardAdam(P, M, V, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                      max_grad_norm=w.max_grad_norm, applied_steps=w.step - 1, device_state=True,
                      scaler=Z.LossScaler.static(K * w.loss_scale))
    opt.reduce(A, slices, with_norm=True)
    opt.step(A, par, norm_done=True)
    st = opt.read_state()
    del slices
    assert st.last_overflow == int(ref_ovf) == 0 and st.applied == w.step
    check_norm(opt.sqnorm.item(), ref_sq)
    RA = torch.from_numpy(acc_host).cuda()
    ta = F.Tally("fp32 gradient copy (1 ulp)")
    for lo, hi in blocks:
        F.tally_ulp_f32(ta, A[lo:hi], RA[lo:hi], lo)
    F.assert_all([ta])
    tl = _compare(blocks, (P, M, V, par), ref, "reduced ", w.param_dtype)
    _check_model(blocks, (P, M, V), model, opt.sqnorm.item(), ref_sq, hp)
    del model
    _padding_zero(real, S, (P, M, V, A), par)
    print(f"\n1T shard, 8 ranks' slices reduced: every element within the bar: {ta}; {tl}", flush=True)
    del P, M, V, A, RA, par, ref, opt
    torch.cuda.empty_cache()


def test_offload_full_shard(Z):
    """The 1T model's last-rank shard (976M params) stepped with its fp32
    state in pinned host memory (as bench.py --offload runs it: the norm on
    the device, the AdamW step on host cores, the 16-bit parameters back to
    the device): every element of the host state and of the device parameter
    copy against the oracle, and the host master and moments bit for bit
    against the float32 model (the host loop uses the device's operation
    order)."""
    w = W.GPT_1T_LAST_RANK
    _, S, _ = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    begin = w.rank * S
    real = min(S, max(0, W.real_total(w) - begin))
    fmt, inv = w.grad_dtype, 1.0 / w.loss_scale
    blocks = F.chunk_blocks(begin, S)
    host = [torch.empty(S, dtype=torch.float32, pin_memory=True) for _ in range(3)]
    G = torch.empty(S, dtype=TDT[fmt], device="cuda")
    ghost = np.empty(S, np.uint16)

    def grad_task(b):
        lo, hi = b
        ghost[lo:hi] = W.fill(w, "grad", begin + lo, hi - lo, step=w.step, threads=1)
        return oracle.sqnorm_terms(ghost[lo:hi], fmt, inv)

    terms = []
    for (lo, hi), tm in F.pmap(grad_task, blocks):
        _put(G, lo, ghost[lo:hi])
        terms.append(tm)
    ref_sq, ref_ovf = oracle.combine_sqnorm_terms(terms, fmt, inv)
    ref = (_f32(S), _f32(S), _f32(S), torch.empty(S, dtype=torch.int16, device="cuda"))
    hp = _hp(w, w.step, inv)
    model = tuple(np.empty(S, np.float32) for _ in range(3))
    _state_and_reference(w, begin, blocks, ghost, fmt, ref_sq, hp, host, ref, model)
    del ghost
    par = torch.empty(S, dtype=TDT[w.param_dtype], device="cuda")
    opt = Z.OffloadShardAdam(*host, grad_dtype=TDT[fmt], param_dtype=TDT[w.param_dtype], lr=w.lr, beta1=w.beta1,
                             beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm,
                             scaler=Z.LossScaler.static(w.loss_scale), applied_steps=w.step - 1)
    assert opt.step(G, par) is False and opt.t == w.step and not ref_ovf
    check_norm(opt.sqnorm, ref_sq)
    _check_model(blocks, host, model, opt.sqnorm, ref_sq, hp)      # the host loop rounds as the device does
    del model
    _padding_zero(real, S, host, par)
    got = tuple(t.cuda() for t in host) + (par,)          # compared on the device, as the other shards
    del host, opt
    tl = _compare(blocks, got, ref, "offloaded ", w.param_dtype)
    print(f"\n1T shard, CPU offload: every element within the bar and equal to the float32 model: {tl}", flush=True)
    del got, G, par, ref
    torch.cuda.empty_cache()
