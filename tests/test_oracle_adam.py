"""Pins for the oracle's norm/overflow, clipping, Adam/AdamW update and loss
scaler.  Each check is independent of oracle/adam.py's arithmetic: exactly
rounded sums (math.fsum), closed forms, torch's CPU optimizers and clipping
utility, and the concatenation invariant over partitions."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import (LossScalerState, adam_update, clip_coefficient, decode16,
                    global_sqnorm_overflow, loss_scaler_update, partition_plan,
                    shard_sqnorm_overflow, shard_step)

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _lib_vals(bits, fmt):
    """Library decode of 16-bit bits to float64 (independent of the oracle)."""
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def _rand_bits(rng, n, fmt, sigma):
    return W.to_bits16((rng.standard_normal(n) * sigma).astype(np.float32), fmt)


# ---------------------------------------------------------------- norm / overflow

@pytest.mark.parametrize("fmt,sigma,inv", [("f16", 65.0, 2.0**-16), ("bf16", 1e-3, 1.0),
                                           ("f16", 1e-4, 1.0), ("bf16", 1e30, 0.75)])
def test_sqnorm_is_exactly_rounded(fmt, sigma, inv):
    rng = np.random.default_rng(3)
    bits = _rand_bits(rng, 200_003, fmt, sigma)
    sq, ovf = shard_sqnorm_overflow(bits, fmt, inv)
    assert not ovf
    # fsum of exactly representable squares is the correctly rounded sum
    v = _lib_vals(bits, fmt)
    assert sq == math.fsum((v * v).tolist()) * inv * inv or \
        abs(sq - math.fsum(((v * inv) ** 2).tolist())) <= 1e-15 * sq
    assert abs(sq - np.linalg.norm(v * inv) ** 2) <= 1e-12 * sq


def test_sqnorm_closed_form():
    # n copies of c = 2^-k: sum of squares is n * 2^-2k exactly
    for fmt in ("f16", "bf16"):
        for k, n in ((3, 1000), (12, 77777), (0, 5)):
            bits = W.to_bits16(np.full(n, 2.0**-k, np.float32), fmt)
            sq, ovf = shard_sqnorm_overflow(bits, fmt, 0.5)
            assert not ovf and sq == n * 2.0**(-2 * k) * 0.25


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_sqnorm_every_pattern_exhaustive(fmt):
    """Every finite 16-bit pattern (both signs), and the subnormals alone:
    the oracle's sum of squares equals math.fsum of the library-decoded
    squares (both are the correctly rounded exact sum)."""
    allp = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = _lib_vals(allp, fmt)
    finite = np.isfinite(v)
    sq, ovf = shard_sqnorm_overflow(allp[finite], fmt, 1.0)
    assert not ovf and sq == math.fsum((v[finite] ** 2).tolist())
    sub = allp[(allp & 0x7FFF) < (0x400 if fmt == "f16" else 0x80)]
    vs = _lib_vals(sub, fmt)
    for inv in (1.0, 2.0**-16, 3.0):
        sq, _ = shard_sqnorm_overflow(sub, fmt, inv)
        assert sq == math.fsum(((vs * inv) ** 2).tolist()) or \
            abs(sq - math.fsum(((vs * inv) ** 2).tolist())) <= 1e-15 * sq


def test_sqnorm_empty_and_zero():
    assert shard_sqnorm_overflow(np.zeros(0, np.uint16), "f16", 1.0) == (0.0, False)
    assert shard_sqnorm_overflow(np.zeros(100, np.uint16), "bf16", 1.0) == (0.0, False)
    # -0 squared is 0
    assert shard_sqnorm_overflow(np.full(9, 0x8000, np.uint16), "f16", 1.0) == (0.0, False)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_overflow_positions(fmt):
    rng = np.random.default_rng(5)
    base = _rand_bits(rng, 1001, fmt, 1.0)
    inf = W.POS_INF_BITS[fmt]
    nan = {"f16": 0x7E00, "bf16": 0x7FC0}[fmt]
    for pos in (0, 500, 1000):
        b = base.copy(); b[pos] = inf
        assert shard_sqnorm_overflow(b, fmt, 1.0) == (math.inf, True)
        b[pos] = inf | 0x8000                      # -inf
        assert shard_sqnorm_overflow(b, fmt, 1.0) == (math.inf, True)
        b[pos] = nan
        sq, ovf = shard_sqnorm_overflow(b, fmt, 1.0)
        assert ovf and math.isnan(sq)


def test_bf16_huge_finite_is_not_overflow():
    # a finite bf16 whose square overflows float32 must not raise the flag
    bits = W.to_bits16(np.array([3e38, -3e38, 1.0], np.float32), "bf16")
    sq, ovf = shard_sqnorm_overflow(bits, "bf16", 1.0)
    assert not ovf and math.isfinite(sq) and sq > 1e77


def test_global_equals_whole():
    """Concatenation: the data-parallel sum over N_d shards equals the sum over
    the unpartitioned buffer (both exactly rounded)."""
    w = W.TINY
    _, S, padded = partition_plan(w.shapes, w.n_d, w.align)
    whole = W.fill(w, "grad", 0, padded, step=1)
    shards = [whole[r * S:(r + 1) * S] for r in range(w.n_d)]
    assert global_sqnorm_overflow(shards, "f16", 2.0**-10) == shard_sqnorm_overflow(whole, "f16", 2.0**-10)


_NAN16 = {"f16": 0x7E00, "bf16": 0x7FC0}


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_global_nonfinite_is_or_over_shards(fmt):
    """The data-parallel OR: one non-finite element in any one of several
    finite shards raises the global flag; the global sum is +inf when the
    shards hold an infinity (of either sign) and no NaN, NaN as soon as any
    shard holds a NaN, whichever shard comes first (IEEE: inf + x = inf,
    NaN + x = NaN)."""
    rng = np.random.default_rng(21)
    shards = [_rand_bits(rng, 997 + 13 * k, fmt, 1e-3) for k in range(5)]
    inf, nan = W.POS_INF_BITS[fmt], _NAN16[fmt]
    assert global_sqnorm_overflow(shards, fmt, 1.0)[1] is False
    for k in range(5):
        for bits, want in ((inf, math.inf), (inf | 0x8000, math.inf)):
            s = [a.copy() for a in shards]
            s[k][k * 7] = bits
            assert global_sqnorm_overflow(s, fmt, 1.0) == (want, True)
        s = [a.copy() for a in shards]
        s[k][-1] = nan
        sq, ovf = global_sqnorm_overflow(s, fmt, 0.5)
        assert ovf is True and math.isnan(sq)
    for i, j in ((0, 4), (4, 0), (2, 2)):            # a NaN with an inf: NaN
        s = [a.copy() for a in shards]
        s[i][3] = nan
        s[j][5] = inf
        sq, ovf = global_sqnorm_overflow(s, fmt, 1.0)
        assert ovf is True and math.isnan(sq)
    # a NaN-free shard list whose finite part is empty: still +inf
    assert global_sqnorm_overflow([np.array([inf], np.uint16), np.zeros(0, np.uint16)], fmt, 1.0) == \
        (math.inf, True)


def test_global_f32_shards_match_exact_sum():
    """fp32 gradient shards (the accumulated copy): every square of an fp32
    value times a power of two is exact in float64, so math.fsum over the
    concatenated squares is the correctly rounded global sum; the oracle's
    chunked sum lies within 1e-14 of it for any split into shards (it is
    documented to), and equals it exactly where the partial sums are all
    representable (equal powers of two)."""
    rng = np.random.default_rng(23)
    whole = (rng.standard_normal(300_007) * np.exp(rng.uniform(-8, 8, 300_007))).astype(np.float32)
    for inv in (1.0, 2.0**-16, 0.5):
        exact = math.fsum(((whole.astype(np.float64) * inv) ** 2).tolist())
        for cuts in ((), (1,), (150_000,), (5, 77_777, 200_000, 300_006)):
            shards = np.split(whole, list(cuts))
            sq, ovf = global_sqnorm_overflow(shards, "f32", inv)
            assert ovf is False and abs(sq - exact) <= 1e-14 * exact
    # n copies of 2^-k, split unevenly: exactly n * 2^-2k
    c = np.full(100_003, 2.0**-9, np.float32)
    assert global_sqnorm_overflow(np.split(c, [3, 60_000]), "f32", 0.25) == (100_003 * 2.0**-18 / 16, False)
    assert global_sqnorm_overflow([np.zeros(0, np.float32)], "f32", 1.0) == (0.0, False)


def test_global_f32_nonfinite_is_or_over_shards():
    rng = np.random.default_rng(25)
    shards = [rng.standard_normal(1000 + k).astype(np.float32) for k in range(4)]
    for k in range(4):
        for bad, want in ((np.inf, math.inf), (-np.inf, math.inf)):
            s = [a.copy() for a in shards]
            s[k][k] = bad
            assert global_sqnorm_overflow(s, "f32", 1.0) == (want, True)
        s = [a.copy() for a in shards]
        s[k][-1] = np.nan
        sq, ovf = global_sqnorm_overflow(s, "f32", 1.0)
        assert ovf is True and math.isnan(sq)
    s = [a.copy() for a in shards]
    s[0][0], s[3][0] = np.inf, np.nan
    sq, ovf = global_sqnorm_overflow(s, "f32", 1.0)
    assert ovf is True and math.isnan(sq)
    # a finite fp32 value whose square overflows float32 is not an overflow
    sq, ovf = shard_sqnorm_overflow(np.array([3e38, -3e38], np.float32), "f32", 1.0)
    assert ovf is False and sq == 2 * float(np.float32(3e38)) ** 2


# ---------------------------------------------------------------- clipping

def test_clip_matches_torch():
    rng = np.random.default_rng(11)
    bits = _rand_bits(rng, 50_000, "f16", 65.0)
    inv = 2.0**-16
    g = _lib_vals(bits, "f16") * inv
    sq, _ = shard_sqnorm_overflow(bits, "f16", inv)
    for max_norm in (0.01, 0.1, 1.0, 1e6):
        p = torch.nn.Parameter(torch.zeros(g.size, dtype=torch.float64))
        p.grad = torch.from_numpy(g.copy())
        torch.nn.utils.clip_grad_norm_([p], max_norm)
        ours = g * clip_coefficient(sq, max_norm)
        np.testing.assert_allclose(ours, p.grad.numpy(), rtol=1e-13, atol=0)
    assert clip_coefficient(sq, 0.0) == 1.0 and clip_coefficient(sq, -1.0) == 1.0


def test_clip_closed_form():
    sq = 400.0                                    # norm 20
    c = clip_coefficient(sq, 1.0)
    assert c == 1.0 / (20.0 + 1e-6)
    assert abs(c * 20.0 - 20.0 / (20.0 + 1e-6)) < 1e-15
    assert clip_coefficient(1e-4, 1.0) == 1.0     # below the max: untouched


# ---------------------------------------------------------------- Adam / AdamW

def _torch_adamw(p, g, m, v, step, lr, beta1, beta2, eps, weight_decay):
    """torch.optim.AdamW (single-tensor path) in float64 from a given state."""
    param = torch.nn.Parameter(torch.from_numpy(p.astype(np.float64)))
    opt = torch.optim.AdamW([param], lr=lr, betas=(beta1, beta2), eps=eps, weight_decay=weight_decay,
                            foreach=False, fused=False)
    param.grad = torch.from_numpy(g.copy())
    opt.state[param] = {"step": torch.tensor(float(step - 1), dtype=torch.float64),
                        "exp_avg": torch.from_numpy(m.astype(np.float64)),
                        "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    opt.step()
    st = opt.state[param]
    return param.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("step,wd,fmt", [(1, 0.0, "f16"), (100, 0.01, "f16"), (1000, 0.1, "bf16"),
                                         (10000, 0.1, "bf16"), (7, 0.5, "f16")])
def test_adamw_matches_torch(step, wd, fmt):
    rng = np.random.default_rng(step)
    n = 100_000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32) if step > 1 else np.zeros(n, np.float32)
    v = rng.uniform(1e-8, 1e-5, n).astype(np.float32) if step > 1 else np.zeros(n, np.float32)
    bits = _rand_bits(rng, n, fmt, 1e-3 * 1024)
    gscale = 2.0**-10 * 0.37
    out = adam_update(p, m, v, bits, fmt, gscale, step=step, weight_decay=wd, param_fmt=fmt, **HP)
    g = _lib_vals(bits, fmt) * gscale
    tp, tm, tv = _torch_adamw(p, g, m, v, step, weight_decay=wd, **HP)
    # the oracle rounds its float64 result once to float32; torch's float64
    # result rounded the same way must agree to 1 float32 ulp
    for ours, ref in ((out[0], tp), (out[1], tm), (out[2], tv)):
        ref32 = ref.astype(np.float32)
        ulp = np.abs(np.spacing(ref32))
        assert (np.abs(ours.astype(np.float64) - ref32.astype(np.float64)) <= ulp).all()
    # the 16-bit copy is the library cast of the stored master
    assert (out[3] == W.to_bits16(out[0], fmt)).all()


def test_adam_equals_adamw_without_decay():
    rng = np.random.default_rng(2)
    n = 10_000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = rng.uniform(1e-8, 1e-5, n).astype(np.float32)
    bits = _rand_bits(rng, n, "f16", 1.0)
    out = adam_update(p, m, v, bits, "f16", 1.0, step=5, weight_decay=0.0, **HP)
    param = torch.nn.Parameter(torch.from_numpy(p.astype(np.float64)))
    opt = torch.optim.Adam([param], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                           foreach=False)
    param.grad = torch.from_numpy(_lib_vals(bits, "f16"))
    opt.state[param] = {"step": torch.tensor(4.0, dtype=torch.float64),
                        "exp_avg": torch.from_numpy(m.astype(np.float64)),
                        "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    opt.step()
    np.testing.assert_allclose(out[0], param.detach().numpy().astype(np.float32), rtol=2e-7, atol=0)


def test_step1_closed_form():
    """t = 1, m = v = 0: m_hat = g and v_hat = g^2, so the step is
    -lr * g / (|g| + eps), i.e. about -lr * sign(g) when eps is tiny."""
    rng = np.random.default_rng(9)
    n = 50_000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    bits = _rand_bits(rng, n, "f16", 1e-2 * 1024)
    z = np.zeros(n, np.float32)
    lr, eps = 1e-3, 1e-8
    master, m1, v1, _ = adam_update(p, z, z, bits, "f16", 2.0**-10, lr=lr, beta1=0.9, beta2=0.999,
                                    eps=eps, weight_decay=0.0, step=1)
    g = _lib_vals(bits, "f16") * 2.0**-10
    expect = p.astype(np.float64) - lr * g / (np.abs(g) + eps)
    assert (master == expect.astype(np.float32)).all()
    nz = g != 0
    delta = master.astype(np.float64) - p
    # |delta + lr*sign(g)| <= lr*eps/|g| + float32 rounding of the master
    bound = lr * eps / np.abs(g[nz]) + np.abs(np.spacing(master[nz])).astype(np.float64)
    assert (np.abs(delta[nz] + lr * np.sign(g[nz])) <= bound).all()
    assert (m1 == (0.1 * g).astype(np.float32)).all()
    assert (v1 == (0.001 * g * g).astype(np.float32)).all()


def test_zero_grad_decay_only():
    """g = 0, m = v = 0: the update reduces to p * (1 - lr * wd) exactly."""
    p = np.array([0.5, -0.25, 0.02, 0.0], np.float32)
    z = np.zeros(4, np.float32)
    for wd in (0.0, 0.01, 0.1):
        master, m, v, _ = adam_update(p, z, z, np.zeros(4, np.uint16), "f16", 1.0,
                                      weight_decay=wd, step=3, **HP)
        assert (master == (p.astype(np.float64) * (1 - 1e-3 * wd)).astype(np.float32)).all()
        assert (m == 0).all() and (v == 0).all()


def test_zero_betas():
    """beta1 = beta2 = 0: step = -lr * (g / (|g| + eps) + wd * p) for any t."""
    rng = np.random.default_rng(4)
    p = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    m = rng.standard_normal(1000).astype(np.float32)
    v = rng.uniform(0, 1, 1000).astype(np.float32)
    bits = _rand_bits(rng, 1000, "bf16", 1.0)
    g = _lib_vals(bits, "bf16")
    for t in (1, 2, 50):
        master, *_ = adam_update(p, m, v, bits, "bf16", 1.0, lr=1e-2, beta1=0.0, beta2=0.0,
                                 eps=1e-8, weight_decay=0.1, step=t)
        expect = p - 1e-2 * (g / (np.abs(g) + 1e-8) + 0.1 * p.astype(np.float64))
        assert (master == expect.astype(np.float32)).all()


def test_lr_zero_is_identity():
    rng = np.random.default_rng(6)
    p = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    m = rng.standard_normal(1000).astype(np.float32) * 1e-3
    v = rng.uniform(1e-8, 1e-5, 1000).astype(np.float32)
    bits = _rand_bits(rng, 1000, "f16", 1.0)
    master, *_ = adam_update(p, m, v, bits, "f16", 1.0, lr=0.0, beta1=0.9, beta2=0.999,
                             eps=1e-8, weight_decay=0.1, step=10)
    assert (master == p).all()


def test_padding_stays_zero():
    z = np.zeros(16, np.float32)
    out = adam_update(z, z, z, np.zeros(16, np.uint16), "bf16", 0.3, weight_decay=0.1,
                      step=10000, param_fmt="bf16", **HP)
    for a in out:
        assert (a == 0).all() and not np.signbit(a.astype(np.float32)).any()


def test_partition_concatenation_bitexact():
    """Updating the N_d shards separately and concatenating equals updating
    the unpartitioned flat buffer, given the same gradient scale."""
    w = W.TINY
    _, S, padded = partition_plan(w.shapes, w.n_d, w.align)
    p, m, v, g = W.shard_inputs(w, 0, padded)
    kw = dict(weight_decay=0.01, step=3, param_fmt="f16", **HP)
    whole = adam_update(p, m, v, g, "f16", 2.0**-10, **kw)
    parts = [adam_update(p[r * S:(r + 1) * S], m[r * S:(r + 1) * S], v[r * S:(r + 1) * S],
                         g[r * S:(r + 1) * S], "f16", 2.0**-10, **kw) for r in range(w.n_d)]
    for k in range(4):
        assert (np.concatenate([x[k] for x in parts]) == whole[k]).all()


def test_loss_scale_invariance():
    """Grads x 2^k with scale x 2^k give bit-identical updates."""
    rng = np.random.default_rng(8)
    n = 20_000
    x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = rng.uniform(1e-8, 1e-5, n).astype(np.float32)
    outs = []
    base = W.to_bits16(x * np.float32(2.0**4), "f16")
    for k in (4, 10):
        # the same fp16 values scaled by 2^(k-4): exact (no rounding, no overflow)
        bits = W.to_bits16((_lib_vals(base, "f16") * 2.0**(k - 4)).astype(np.float32), "f16")
        sq, _ = shard_sqnorm_overflow(bits, "f16", 2.0**-k)
        outs.append(shard_step(p, m, v, bits, "f16", "f16", global_sq=sq, global_overflow=False,
                               inv_loss_scale=2.0**-k, max_grad_norm=0.01, weight_decay=0.01,
                               step=20, **HP))
    for a, b in zip(outs[0][:4], outs[1][:4]):
        assert (a == b).all()


def test_skip_leaves_state():
    p = np.ones(4, np.float32)
    out = shard_step(p, p, p, np.array([0x7C00, 0, 0, 0], np.uint16), "f16", "f16", global_sq=math.inf,
                     global_overflow=True, inv_loss_scale=1.0, max_grad_norm=1.0, weight_decay=0.1,
                     step=1, **HP)
    assert out[0] is p and out[3] is None and out[4] is False


# ---------------------------------------------------------------- loss scaler

def test_scaler_trajectory_inf_at_5_and_12():
    """20 iterations with overflow at iterations 5 and 12: those two are
    skipped, the scale halves twice and 18 steps are applied."""
    s, t, scales, skipped = LossScalerState(scale=65536.0), 0, [], []
    for it in range(1, 21):
        s, skip = loss_scaler_update(s, overflow=it in (5, 12))
        if skip:
            skipped.append(it)
        else:
            t += 1
        scales.append(s.scale)
    assert skipped == [5, 12] and t == 18
    assert scales[3] == 65536.0 and scales[4] == 32768.0 and scales[11] == 16384.0
    assert scales[-1] == 16384.0 and s.good_steps == 8


def test_scaler_growth_floor_static():
    s = LossScalerState(scale=8.0, growth_interval=3)
    for _ in range(3):
        s, _ = loss_scaler_update(s, False)
    assert s.scale == 16.0 and s.good_steps == 0
    s = LossScalerState(scale=1.0)
    s, skip = loss_scaler_update(s, True)
    assert skip and s.scale == 1.0                 # floored at min_scale
    st = LossScalerState(scale=1.0, backoff=1.0, growth=1.0)
    for ovf in (True, False, True):
        st, _ = loss_scaler_update(st, ovf)
    assert st.scale == 1.0


def test_decode_agrees_with_library_on_workload_grads():
    w = W.GPT2_SMALL
    g = W.fill(w, "grad", 0, 4096, step=w.step)
    assert (decode16(g, "f16") == _lib_vals(g, "f16")).all()


# ---------------------------------------------------------------- scalar brute force

def _f32(x: float) -> float:
    """Round a Python float to IEEE binary32 (round to nearest even) with struct."""
    import struct
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _half_bits(x: float) -> int:
    """IEEE binary16 bits of x, round to nearest even (struct's 'e' format)."""
    import struct
    return struct.unpack("<H", struct.pack("<e", x))[0]


def _decode_half(b: int) -> float:
    import struct
    return struct.unpack("<e", struct.pack("<H", b))[0]


def _scalar_step(p, m, v, gbits, inv, max_norm, lr, b1, b2, eps, wd, t):
    """The whole step element by element in plain Python floats (IEEE double),
    written from the textbook definitions with no vector code: unscale,
    exact sum of squares (math.fsum), clip coefficient, AdamW with bias
    correction, float32 storage, fp16 writeback."""
    g = [_decode_half(b) * inv for b in gbits]
    norm = math.sqrt(math.fsum(x * x for x in g))
    coef = min(1.0, max_norm / (norm + 1e-6)) if max_norm > 0 else 1.0
    out = []
    for pi, mi, vi, gi in zip(p, m, v, g):
        gi = gi * coef
        mi2 = b1 * mi + (1 - b1) * gi
        vi2 = b2 * vi + (1 - b2) * gi * gi
        mhat = mi2 / (1 - b1 ** t)
        vhat = vi2 / (1 - b2 ** t)
        pi2 = pi - lr * (mhat / (math.sqrt(vhat) + eps) + wd * pi)
        p32 = _f32(pi2)
        out.append((p32, _f32(mi2), _f32(vi2), _half_bits(p32)))
    return out


@pytest.mark.parametrize("n,t,max_norm", [(1, 1, 0.0), (7, 3, 1.0), (64, 100, 0.05), (64, 1, 1e9)])
def test_scalar_loop_equals_vectorised(n, t, max_norm):
    """Brute force on tiny shards: a per-element pure-Python step equals the
    vectorised oracle (state to 1 float32 ulp, parameters bit for bit)."""
    rng = np.random.default_rng(n * 31 + t)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = rng.uniform(1e-8, 1e-5, n).astype(np.float32)
    gbits = _rand_bits(rng, n, "f16", 1e-3 * 1024)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    inv = 2.0**-10
    sq, ovf = shard_sqnorm_overflow(gbits, "f16", inv)
    got = shard_step(p, m, v, gbits, "f16", "f16", global_sq=sq, global_overflow=ovf, inv_loss_scale=inv,
                     max_grad_norm=max_norm, step=t, **hp)
    ref = _scalar_step(p.tolist(), m.tolist(), v.tolist(), gbits.tolist(), inv, max_norm, hp["lr"], hp["beta1"],
                       hp["beta2"], hp["eps"], hp["weight_decay"], t)
    for k, name in enumerate(("master", "exp_avg", "exp_avg_sq")):
        r = np.array([e[k] for e in ref], np.float32)
        assert (np.abs(got[k].astype(np.float64) - r.astype(np.float64)) <= np.abs(np.spacing(r))).all(), name
    assert [int(b) for b in got[3]] == [e[3] for e in ref]
