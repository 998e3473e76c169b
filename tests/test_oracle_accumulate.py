"""Pins for the oracle's fp32 gradient-accumulation path (the fp16 gradient
plus fp32 copy of the memory-per-parameter list): accumulation against torch
on the CPU, closed forms, the fp32-gradient norm against math.fsum, AdamW on
fp32 gradients against torch, and equivalence with the 16-bit path for a
single micro-batch."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import adam_update, grad_accumulate, shard_sqnorm_overflow, shard_step

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _lib_vals(bits, fmt):
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def _torch_acc(acc, bits, fmt, inv):
    g = torch.from_numpy(bits.view(np.int16).copy()).view({"f16": torch.float16, "bf16": torch.bfloat16}[fmt])
    a = torch.zeros(bits.size, dtype=torch.float32) if acc is None else torch.from_numpy(acc.copy())
    a.add_(g.float() * inv)              # fp32: exact product (inv a power of two), one rounding in the add
    return a.numpy()


@pytest.mark.parametrize("fmt,inv", [("f16", 2.0**-16), ("bf16", 1.0), ("f16", 2.0**-10)])
def test_accumulate_matches_torch(fmt, inv):
    rng = np.random.default_rng(3)
    n = 200_000
    acc = None
    ref = None
    for k in range(5):
        bits = W.to_bits16((rng.standard_normal(n) * 1e-3 / inv).astype(np.float32), fmt)
        acc, ovf = grad_accumulate(acc, bits, fmt, inv)
        ref = _torch_acc(ref, bits, fmt, inv)
        assert not ovf
        assert (acc == ref).all()


def test_accumulate_closed_forms():
    c = np.float32(0.375)
    bits = W.to_bits16(np.full(64, c, np.float32), "f16")
    acc = None
    for k in range(1, 9):
        acc, _ = grad_accumulate(acc, bits, "f16", 0.5)
        assert (acc == np.float32(k * 0.375 * 0.5)).all()
    # the first micro-batch is just the unscaled gradient
    rng = np.random.default_rng(1)
    b = W.to_bits16(rng.standard_normal(1000).astype(np.float32), "bf16")
    a, _ = grad_accumulate(None, b, "bf16", 2.0**-3)
    assert (a == (_lib_vals(b, "bf16") * 2.0**-3).astype(np.float32)).all()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_accumulate_overflow_flag(fmt):
    b = np.zeros(17, np.uint16)
    assert grad_accumulate(None, b, fmt, 1.0)[1] is False
    for pos in (0, 8, 16):
        c = b.copy()
        c[pos] = W.POS_INF_BITS[fmt]
        acc, ovf = grad_accumulate(np.ones(17, np.float32), c, fmt, 1.0)
        assert ovf and np.isinf(acc[pos])


def test_f32_sqnorm_against_fsum():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(300_001) * 1e-3).astype(np.float32)
    for inv in (1.0, 2.0**-7):
        sq, ovf = shard_sqnorm_overflow(x, "f32", inv)
        ref = math.fsum(((x.astype(np.float64) * inv) ** 2).tolist())
        assert not ovf and abs(sq - ref) <= 1e-14 * ref
    assert shard_sqnorm_overflow(np.full(10, 0.5, np.float32), "f32", 1.0) == (2.5, False)
    y = x.copy(); y[7] = np.inf
    assert shard_sqnorm_overflow(y, "f32", 1.0) == (math.inf, True)
    y[9] = np.nan
    sq, ovf = shard_sqnorm_overflow(y, "f32", 1.0)
    assert ovf and math.isnan(sq)
    assert shard_sqnorm_overflow(np.zeros(0, np.float32), "f32", 1.0) == (0.0, False)


def test_adamw_on_f32_grads_matches_torch():
    rng = np.random.default_rng(12)
    n = 50_000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = rng.uniform(1e-8, 1e-5, n).astype(np.float32)
    g32 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    out = adam_update(p, m, v, g32, "f32", 0.3, step=50, weight_decay=0.1, param_fmt="bf16", **HP)
    param = torch.nn.Parameter(torch.from_numpy(p.astype(np.float64)))
    opt = torch.optim.AdamW([param], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=0.1, foreach=False)
    param.grad = torch.from_numpy(g32.astype(np.float64) * 0.3)
    opt.state[param] = {"step": torch.tensor(49.0, dtype=torch.float64),
                        "exp_avg": torch.from_numpy(m.astype(np.float64)),
                        "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    opt.step()
    ref = param.detach().numpy().astype(np.float32)
    assert (np.abs(out[0].astype(np.float64) - ref) <= np.abs(np.spacing(ref))).all()


def test_single_microbatch_equals_16bit_path():
    """One accumulated micro-batch (inv a power of two: exact) stepped as an
    fp32 gradient gives bit-identical results to stepping the 16-bit gradient."""
    w = W.GPT2_SMALL
    p, m, v, g = W.shard_inputs(w, 0, 100_000)
    inv = 1.0 / w.loss_scale
    acc, _ = grad_accumulate(None, g, "f16", inv)
    kw = dict(max_grad_norm=1.0, weight_decay=0.01, step=7, **HP)
    sq16, _ = shard_sqnorm_overflow(g, "f16", inv)
    sq32, _ = shard_sqnorm_overflow(acc, "f32", 1.0)
    assert abs(sq16 - sq32) <= 1e-14 * sq16
    a = shard_step(p, m, v, g, "f16", "f16", global_sq=sq16, global_overflow=False, inv_loss_scale=inv, **kw)
    b = shard_step(p, m, v, acc, "f32", "f16", global_sq=sq16, global_overflow=False, inv_loss_scale=1.0, **kw)
    for x, y in zip(a[:4], b[:4]):
        assert (x == y).all()
