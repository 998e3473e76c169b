"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
element by element, on seeded inputs.

Sizes here are ones the oracle finishes in seconds and that still span
several kernel tiles and norm blocks plus a ragged tail; the full-size
workloads are in test_gpu_fullsize.py.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W

from parity import bits_of, check_norm, compare_step, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FMT = {"f16": 1, "bf16": 2}


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()           # fails loudly if the library is missing
    return Z


def _dev_scalars():
    return (torch.empty(1, dtype=torch.float64, device="cuda"),
            torch.empty(1, dtype=torch.int32, device="cuda"))


def gpu_norm(Z, grad_t, inv_scale):
    sq, ovf = _dev_scalars()
    ws = torch.empty(max(1, Z.zero_norm_workspace_bytes(grad_t.numel())), dtype=torch.uint8, device="cuda")
    Z.zero_shard_unscale_norm_overflow(grad_t, inv_scale, sq, ovf, ws)
    torch.cuda.synchronize()
    return sq, ovf


def hp_of(w, step=None, inv=None, **over):
    d = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
             max_grad_norm=w.max_grad_norm, step=w.step if step is None else step,
             inv_loss_scale=1.0 / w.loss_scale if inv is None else inv)
    d.update(over)
    return d


def oracle_step(p, m, v, g, w, gsq, govf, param_fmt, **hp):
    return oracle.shard_step(p, m, v, g, w.grad_dtype, param_fmt, global_sq=gsq, global_overflow=govf, **hp)


# --------------------------------------------------------------------- all ranks of small workloads

@pytest.mark.parametrize("wname", ["tiny", "gpt2"])
def test_all_ranks_of_workload(Z, wname):
    """Every rank of the workload stepped on one GPU: per-rank norm pass, the
    data-parallel sum/OR done on the host in rank order (stand-in for the
    all-reduce), fused update per rank into the ZeRO-2 flat parameter buffer."""
    w = W.get(wname)
    _, S, padded = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    assert (S, padded) == oracle.partition_plan(w.shapes, w.n_d, w.align)[1:]
    p, m, v, g = W.shard_inputs(w, 0, padded)
    P, M, V, G = to_device(p), to_device(m), to_device(v), to_device(g, w.grad_dtype)
    param_full = torch.full((padded,), float("nan"), dtype=G.dtype, device="cuda")
    inv = 1.0 / w.loss_scale
    parts = [gpu_norm(Z, G[r * S:(r + 1) * S], inv) for r in range(w.n_d)]
    gsq = 0.0
    govf = 0
    for sq, ovf in parts:                          # rank order
        gsq += sq.item()
        govf |= int(ovf.item())
    ref_sq, ref_ovf = oracle.global_sqnorm_overflow([g[r * S:(r + 1) * S] for r in range(w.n_d)],
                                                    w.grad_dtype, inv)
    assert govf == int(ref_ovf) == 0
    check_norm(gsq, ref_sq)
    for r in range(w.n_d):
        sq_r, _ = oracle.shard_sqnorm_overflow(g[r * S:(r + 1) * S], w.grad_dtype, inv)
        check_norm(parts[r][0].item(), sq_r)
    d_gsq = torch.tensor([gsq], dtype=torch.float64, device="cuda")
    d_govf = torch.tensor([govf], dtype=torch.int32, device="cuda")
    hp = hp_of(w)
    for r in range(w.n_d):
        sl = slice(r * S, (r + 1) * S)
        Z.zero_shard_adam_step(P[sl], M[sl], V[sl], G[sl], param_full[sl], Z.AdamHyper(**hp), d_gsq, d_govf)
    torch.cuda.synchronize()
    gp, gm, gv, gpar = P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(param_full)
    for r in range(w.n_d):
        sl = slice(r * S, (r + 1) * S)
        ref = oracle_step(p[sl], m[sl], v[sl], g[sl], w, ref_sq, False, w.param_dtype, **hp)
        assert ref[4]
        compare_step((gp[sl], gm[sl], gv[sl], gpar[sl]), ref, what=f"rank{r} ")


# --------------------------------------------------------------------- sizes, tails, dtypes

SIZES = [1, 3, 7, 8, 9, 255, 256, 257, 1023, 1024, 1025, 2049, 4099, 8192, 8192 + 8 * 1023 + 7, 256 * 2 * 8 * 3 + 5, 16384 * 5 + 3, 262144 + 8, 1_000_002, 8192 * 600 + 5]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("gfmt,pfmt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16"), ("bf16", "f16")])
def test_sizes_and_dtypes(Z, n, gfmt, pfmt):
    base = W.GPT2_SMALL if gfmt == "f16" else W.LLAMA_7B
    w = W.Workload(**{**base.__dict__, "grad_dtype": gfmt, "param_dtype": pfmt})
    begin = 1_000_003 * (n % 7 + 1)              # different data per size
    p, m, v, g = W.shard_inputs(w, begin, n)
    P, M, V, G = to_device(p), to_device(m), to_device(v), to_device(g, gfmt)
    par = torch.empty(n, dtype={"f16": torch.float16, "bf16": torch.bfloat16}[pfmt], device="cuda")
    inv = 1.0 / w.loss_scale
    sq, ovf = gpu_norm(Z, G, inv)
    ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(g, gfmt, inv)
    assert int(ovf.item()) == int(ref_ovf)
    check_norm(sq.item(), ref_sq)
    hp = hp_of(w, step=37, max_grad_norm=0.05)    # clipping active
    Z.zero_shard_adam_step(P, M, V, G, par, Z.AdamHyper(**hp), sq, ovf)
    torch.cuda.synchronize()
    ref = oracle_step(p, m, v, g, w, ref_sq, False, pfmt, **hp)
    compare_step((P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par)), ref)


def test_empty_shard(Z):
    G = torch.empty(0, dtype=torch.float16, device="cuda")
    sq, ovf = _dev_scalars()
    sq.fill_(123.0)
    ovf.fill_(7)
    ws = torch.empty(Z.zero_norm_workspace_bytes(0), dtype=torch.uint8, device="cuda")
    Z.zero_shard_unscale_norm_overflow(G, 1.0, sq, ovf, ws)
    E = torch.empty(0, dtype=torch.float32, device="cuda")
    Z.zero_shard_adam_step(E, E, E, G, None, Z.AdamHyper(max_grad_norm=1.0), sq, ovf)
    torch.cuda.synchronize()
    assert sq.item() == 0.0 and ovf.item() == 0


def test_no_param_writeback_and_no_clip(Z):
    w = W.TINY
    n = 10_001
    p, m, v, g = W.shard_inputs(w, 0, n)
    P, M, V, G = to_device(p), to_device(m), to_device(v), to_device(g, "f16")
    hp = hp_of(w)
    Z.zero_shard_adam_step(P, M, V, G, None, Z.AdamHyper(**hp), None, None)
    torch.cuda.synchronize()
    ref = oracle_step(p, m, v, g, w, 0.0, False, None, **hp)
    compare_step((P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), None), ref)


def test_fp16_subnormal_and_extreme_grads(Z):
    rng = np.random.default_rng(21)
    n = 40_000 + 5
    bits = rng.integers(0, 0x7C00, n, dtype=np.uint64).astype(np.uint16)     # every finite positive fp16
    bits[rng.random(n) < 0.5] |= 0x8000
    bits[:1000] = rng.integers(0, 0x400, 1000).astype(np.uint16)             # subnormals
    w = W.GPT2_SMALL
    p, m, v, _ = W.shard_inputs(w, 77, n)
    G = to_device(bits, "f16")
    for inv in (1.0, 2.0**-16):
        sq, ovf = gpu_norm(Z, G, inv)
        ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(bits, "f16", inv)
        assert ovf.item() == 0 and not ref_ovf
        check_norm(sq.item(), ref_sq)
        P, M, V = to_device(p), to_device(m), to_device(v)
        par = torch.empty(n, dtype=torch.float16, device="cuda")
        hp = hp_of(w, inv=inv, max_grad_norm=1.0)
        Z.zero_shard_adam_step(P, M, V, G, par, Z.AdamHyper(**hp), sq, ovf)
        torch.cuda.synchronize()
        ref = oracle_step(p, m, v, bits, w, ref_sq, False, "f16", **hp)
        compare_step((P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par)), ref)


def test_bf16_huge_finite_not_overflow(Z):
    bits = W.to_bits16(np.array([3e38, -3e38] + [1.0] * 14, np.float32), "bf16")
    sq, ovf = gpu_norm(Z, to_device(bits, "bf16"), 1.0)
    ref_sq, _ = oracle.shard_sqnorm_overflow(bits, "bf16", 1.0)
    assert ovf.item() == 0 and math.isfinite(sq.item())
    check_norm(sq.item(), ref_sq)


# --------------------------------------------------------------------- overflow and skip

@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("kind", ["inf", "-inf", "nan"])
@pytest.mark.parametrize("where", ["first", "middle", "last", "tail"])
def test_overflow_detect_and_skip(Z, fmt, kind, where):
    n = 3 * 16384 + 5
    w = W.GPT2_SMALL if fmt == "f16" else W.LLAMA_7B
    p, m, v, g = W.shard_inputs(w, 4242, n)
    pos = {"first": 0, "middle": n // 2, "last": n - 1, "tail": n - 3}[where]
    inf = W.POS_INF_BITS[fmt]
    g[pos] = {"inf": inf, "-inf": inf | 0x8000, "nan": inf | (0x200 if fmt == "f16" else 0x40)}[kind]
    G = to_device(g, fmt)
    sq, ovf = gpu_norm(Z, G, 1.0)
    ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(g, fmt, 1.0)
    assert ref_ovf and ovf.item() == 1
    check_norm(sq.item(), ref_sq)                  # inf, or NaN when a NaN is present
    P, M, V = to_device(p), to_device(m), to_device(v)
    sentinel = torch.full((n,), 0x1234, dtype=torch.int16, device="cuda")
    par = sentinel.clone().view(G.dtype)
    Z.zero_shard_adam_step(P, M, V, G, par, Z.AdamHyper(**hp_of(w, max_grad_norm=1.0)), sq, ovf)
    torch.cuda.synchronize()
    # skipped: every buffer bit-identical, parameter copy untouched
    assert (P.cpu().numpy().view(np.uint32) == p.view(np.uint32)).all()
    assert (M.cpu().numpy().view(np.uint32) == m.view(np.uint32)).all()
    assert (V.cpu().numpy().view(np.uint32) == v.view(np.uint32)).all()
    assert (par.view(torch.int16) == sentinel).all().item()


def test_overflow_flag_null_never_skips(Z):
    """With no overflow flag the update runs (the caller opted out of skipping)."""
    n = 1000
    p, m, v, g = W.shard_inputs(W.TINY, 0, n)
    P, M, V, G = to_device(p), to_device(m), to_device(v), to_device(g, "f16")
    Z.zero_shard_adam_step(P, M, V, G, None, Z.AdamHyper(**hp_of(W.TINY)), None, None)
    torch.cuda.synchronize()
    assert not (P.cpu().numpy() == p).all()


# --------------------------------------------------------------------- invariants

def test_norm_deterministic(Z):
    w = W.GPT2_SMALL
    n = 5_000_003
    g = W.fill(w, "grad", 0, n, step=3)
    G = to_device(g, "f16")
    a = [gpu_norm(Z, G, 2.0**-16)[0].item() for _ in range(3)]
    assert a[0] == a[1] == a[2]


def test_concatenation_equals_unpartitioned(Z):
    """The N_d per-rank updates, concatenated, equal the N_d = 1 update of
    the whole flat buffer bit-exactly, given the same global norm."""
    w = W.TINY
    _, S, padded = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    p, m, v, g = W.shard_inputs(w, 0, padded)
    d_gsq = torch.tensor([37.5], dtype=torch.float64, device="cuda")
    d_govf = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp = Z.AdamHyper(**hp_of(w, step=5, weight_decay=0.01, max_grad_norm=1.0))
    outs = []
    for ranks in (w.n_d, 1):
        Sr = padded // ranks
        P, M, V, G = to_device(p), to_device(m), to_device(v), to_device(g, "f16")
        par = torch.empty(padded, dtype=torch.float16, device="cuda")
        for r in range(ranks):
            sl = slice(r * Sr, (r + 1) * Sr)
            Z.zero_shard_adam_step(P[sl], M[sl], V[sl], G[sl], par[sl], hp, d_gsq, d_govf)
        torch.cuda.synchronize()
        outs.append([P.cpu().numpy().view(np.uint32), M.cpu().numpy().view(np.uint32),
                     V.cpu().numpy().view(np.uint32), bits_of(par)])
    for a, b in zip(*outs):
        assert (a == b).all()


def test_loss_scale_invariance_bitexact(Z):
    """Gradients x 2^k with the loss scale x 2^k give bit-identical results."""
    w = W.GPT2_SMALL
    n = 100_000
    p, m, v, _ = W.shard_inputs(w, 0, n)
    x = (np.random.default_rng(1).standard_normal(n) * 1e-3).astype(np.float32)
    base = W.to_bits16(x * np.float32(16.0), "f16")
    vals = base.view(np.float16).astype(np.float32)
    res = []
    for k in (4, 10):
        bits = W.to_bits16(vals * np.float32(2.0**(k - 4)), "f16")
        G = to_device(bits, "f16")
        sq, ovf = gpu_norm(Z, G, 2.0**-k)
        P, M, V = to_device(p), to_device(m), to_device(v)
        par = torch.empty(n, dtype=torch.float16, device="cuda")
        Z.zero_shard_adam_step(P, M, V, G, par, Z.AdamHyper(**hp_of(w, inv=2.0**-k, max_grad_norm=0.01)), sq, ovf)
        torch.cuda.synchronize()
        res.append((sq.item(), P.cpu().numpy().view(np.uint32), M.cpu().numpy().view(np.uint32),
                    V.cpu().numpy().view(np.uint32), bits_of(par)))
    assert res[0][0] == res[1][0]
    for a, b in zip(res[0][1:], res[1][1:]):
        assert (a == b).all()


def test_shard_adam_loop_matches_oracle_trajectory(Z):
    """ShardAdam over 6 steps with overflow injected at step 3: flags, skip
    decisions, loss scale and step counter bit-exact; state within tolerance
    after every step."""
    w = W.Workload(**{**W.GPT_100B_RANK.__dict__, "inf_steps": (3,), "inf_fraction": 0.001})
    n = 300_007
    p, m, v, _ = W.shard_inputs(w, 0, n)
    P, M, V = to_device(p), to_device(m), to_device(v)
    par = torch.empty(n, dtype=torch.float16, device="cuda")
    opt = Z.ShardAdam(P, M, V, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                      max_grad_norm=w.max_grad_norm, scaler=Z.LossScaler(scale=w.loss_scale))
    ref_state = (p, m, v)
    ref_scaler, ref_t = oracle.LossScalerState(scale=w.loss_scale), 0
    for it in range(1, 7):
        scale = opt.scaler.scale
        assert scale == ref_scaler.scale
        g = W.grad_for_step(w, 0, n, it, scale)
        skip = opt.step(to_device(g, "f16"), par)
        sq, ovf = oracle.shard_sqnorm_overflow(g, "f16", 1.0 / scale)
        out = oracle.shard_step(*ref_state, g, "f16", "f16", global_sq=sq, global_overflow=ovf,
                                inv_loss_scale=1.0 / scale, max_grad_norm=w.max_grad_norm, lr=w.lr,
                                beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                                step=ref_t + 1)
        ref_scaler, ref_skip = oracle.loss_scaler_update(ref_scaler, ovf)
        assert skip == ref_skip == (it == 3)
        if not ref_skip:
            ref_t += 1
            ref_state = out[:3]
            compare_step((P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par)), out, what=f"it{it} ")
        assert opt.t == ref_t and opt.scaler.scale == ref_scaler.scale
    assert ref_t == 5
