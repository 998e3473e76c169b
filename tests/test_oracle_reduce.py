"""Pins for the oracle's reduction of the ranks' gradient slices of one
partition (the local half of the gradient reduce-scatter): against torch on
the CPU summing in rank order, closed forms, the recursive-summation error
bound around the exactly rounded sum, and the overflow flag."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import grad_accumulate, grad_reduce

TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _slices(rng, k, n, fmt, inv, scale=1e-3):
    return [W.to_bits16((rng.standard_normal(n) * scale / inv).astype(np.float32), fmt) for _ in range(k)]


def _torch_rank_order(slices, fmt, inv):
    acc = None
    for b in slices:
        g = torch.from_numpy(b.view(np.int16).copy()).view(TDT[fmt]).float() * inv   # exact: inv a power of two
        acc = g.clone() if acc is None else acc + g                                 # one fp32 rounding per add
    return acc.numpy()


@pytest.mark.parametrize("k", [1, 2, 5, 16])
@pytest.mark.parametrize("fmt,inv", [("f16", 2.0**-16), ("bf16", 1.0)])
def test_reduce_matches_torch_rank_order(k, fmt, inv):
    rng = np.random.default_rng(k)
    sl = _slices(rng, k, 100_003, fmt, inv)
    acc, ovf = grad_reduce(sl, fmt, inv)
    assert not ovf and acc.dtype == np.float32
    assert np.array_equal(acc.view(np.uint32), _torch_rank_order(sl, fmt, inv).view(np.uint32))


def test_one_slice_is_the_first_accumulation():
    rng = np.random.default_rng(1)
    (b,) = _slices(rng, 1, 5000, "f16", 2.0**-10)
    acc, _ = grad_reduce([b], "f16", 2.0**-10)
    ref, _ = grad_accumulate(None, b, "f16", 2.0**-10)
    assert np.array_equal(acc.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_closed_forms(fmt):
    n = 257
    c = W.to_bits16(np.full(n, 0.375, np.float32), fmt)          # exact in both formats
    for k in (1, 3, 8, 16):
        acc, _ = grad_reduce([c] * k, fmt, 0.5)
        assert (acc == np.float32(0.375 * 0.5 * k)).all()
    neg = c ^ np.uint16(0x8000)
    acc, _ = grad_reduce([c, neg, c, neg], fmt, 1.0)              # +c - c + c - c = 0 exactly
    assert (acc == 0).all()


@pytest.mark.parametrize("fmt,inv", [("f16", 2.0**-16), ("bf16", 1.0)])
def test_within_recursive_summation_bound_of_exact_sum(fmt, inv):
    """|acc - exact| <= (K-1) u sum_k |partial sums|, u = 2^-24; the partial
    sums are bounded by the running sum of magnitudes."""
    rng = np.random.default_rng(9)
    k, n = 12, 20_000
    sl = _slices(rng, k, n, fmt, inv)
    acc, _ = grad_reduce(sl, fmt, inv)
    vals = [torch.from_numpy(b.view(np.int16).copy()).view(TDT[fmt]).double().numpy() * inv for b in sl]
    mags = np.sum(np.abs(vals), axis=0)
    for i in range(0, n, 97):
        exact = math.fsum(v[i] for v in vals)
        assert abs(float(acc[i]) - exact) <= (k - 1) * 2.0**-24 * mags[i] * 1.0000001 + 1e-45


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("where", [0, 6, 15])
def test_overflow_in_any_slice(fmt, where):
    rng = np.random.default_rng(where)
    sl = _slices(rng, 16, 1000, fmt, 1.0)
    sl[where] = sl[where].copy()
    sl[where][500] = W.POS_INF_BITS[fmt]
    acc, ovf = grad_reduce(sl, fmt, 1.0)
    assert ovf and not np.isfinite(acc[500]) and np.isfinite(np.delete(acc, 500)).all()
    assert not grad_reduce(sl[:where] + sl[where + 1:], fmt, 1.0)[1]


def test_no_slices_is_an_error():
    with pytest.raises(ValueError):
        grad_reduce([], "f16", 1.0)
