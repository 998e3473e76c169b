"""Pins for the oracle's partition plan: invariants and brute force.

The layout reading (contiguous list order, end padding only, N_d equal
partitions of a multiple of `align`) is checked here against an element-by-
element enumeration that shares nothing with oracle.plan.
"""
import itertools
import random

import pytest

import workloads as W
from oracle import partition_plan, rank_fragments, rank_range


def _enumerate_flat(shapes):
    """Brute force: list every element as (tensor, index-in-tensor)."""
    flat = []
    for t, shape in enumerate(shapes):
        count = 1
        for d in shape:
            count *= d
        for j in range(count):
            flat.append((t, j))
    return flat


def _brute_fragments(shapes, n_d, align, rank):
    flat = _enumerate_flat(shapes)
    S = 0
    while n_d * S < len(flat):           # smallest multiple of align that fits
        S += align
    padded = flat + [None] * (n_d * S - len(flat))
    part = padded[rank * S:(rank + 1) * S]
    frags = []
    for pos, item in enumerate(part):
        if item is None:
            continue
        t, j = item
        if frags and frags[-1][0] == t and frags[-1][1] + frags[-1][3] == j:
            frags[-1][3] += 1
        else:
            frags.append([t, j, pos, 1])
    return S, [tuple(f) for f in frags]


def _random_shapes(rng, n):
    shapes = []
    for _ in range(n):
        nd = rng.randint(0, 3)
        shapes.append(tuple(rng.randint(0, 7) for _ in range(nd)))
    return shapes


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_small(seed):
    rng = random.Random(seed)
    shapes = _random_shapes(rng, rng.randint(0, 6))
    for n_d, align in itertools.product([1, 2, 3, 5, 8], [1, 2, 8, 128]):
        offsets, S, padded = partition_plan(shapes, n_d, align)
        for r in range(n_d):
            S_bf, frags_bf = _brute_fragments(shapes, n_d, align, r)
            assert S == S_bf
            assert rank_fragments(shapes, n_d, align, r) == frags_bf


@pytest.mark.parametrize("seed", range(20))
def test_invariants(seed):
    rng = random.Random(1000 + seed)
    shapes = [tuple(rng.randint(1, 3000) for _ in range(rng.randint(1, 2))) for _ in range(rng.randint(1, 30))]
    T = sum(W.numel(s) for s in shapes)
    for n_d in (1, 2, 7, 8, 64, 400):
        for align in (1, 8, 128, 512):
            offsets, S, padded = partition_plan(shapes, n_d, align)
            # contiguous list order
            assert offsets[0] == 0
            for i in range(1, len(shapes)):
                assert offsets[i] == offsets[i - 1] + W.numel(shapes[i - 1])
            assert S % align == 0 and padded == n_d * S
            assert 0 <= padded - T < n_d * align           # minimal padding
            # every real element owned by exactly one rank; fragments tile it
            covered = 0
            for r in range(n_d):
                lo, hi = rank_range(shapes, n_d, align, r)
                assert hi - lo == S and lo == r * S
                frs = rank_fragments(shapes, n_d, align, r)
                pos = 0
                for (t, tb, sb, n) in frs:
                    assert n > 0 and sb >= pos                # ordered, disjoint
                    assert lo + sb == offsets[t] + tb         # same flat position
                    assert tb + n <= W.numel(shapes[t])
                    pos = sb + n
                    covered += n
            assert covered == T


def test_empty_and_zero_sized():
    assert partition_plan([], 4, 128) == ([], 0, 0)
    assert partition_plan([(0,), (3, 0)], 2, 8) == ([0, 0], 0, 0)
    offsets, S, padded = partition_plan([()], 3, 1)        # a scalar is one element
    assert (offsets, S, padded) == ([0], 1, 3)
    assert rank_fragments([()], 3, 1, 0) == [(0, 0, 0, 1)]
    assert rank_fragments([()], 3, 1, 2) == []              # wholly padding rank


def test_errors():
    with pytest.raises(ValueError):
        partition_plan([(4,)], 0, 1)
    with pytest.raises(ValueError):
        partition_plan([(4,)], 1, 0)
    with pytest.raises(ValueError):
        rank_fragments([(4,)], 2, 1, 2)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_plans(name):
    """Full-size plans: the same invariants on the real shape lists (these
    are cheap: O(number of tensors))."""
    w = W.get(name)
    T = W.real_total(w)
    offsets, S, padded = partition_plan(w.shapes, w.n_d, w.align)
    assert S % w.align == 0 and 0 <= padded - T < w.n_d * w.align
    frs = rank_fragments(w.shapes, w.n_d, w.align, w.rank)
    real = sum(f[3] for f in frs)
    lo = w.rank * S
    assert real == max(0, min(T, lo + S) - lo)
