"""The whole-shard comparison helpers (fullshard.py) take the same decisions
as the numpy checks in parity.py, element by element, on planted cases (CPU
tensors; the GPU tests run the same code on device tensors)."""
import numpy as np
import pytest
import torch

import fullshard as F
import parity
import workloads as W


def _planted(rng, n=10_000):
    ref = (rng.standard_normal(n) * np.exp(rng.uniform(-20, 5, n))).astype(np.float32)
    ref[:50] = 0.0
    ref[50:60] = 3e-8                                      # below the absolute floor
    got = ref.copy()
    i = rng.choice(n, 200, replace=False)
    got[i] = (ref[i].astype(np.float64) * (1 + rng.choice([-1, 1], 200) * rng.uniform(0, 3e-5, 200))).astype(np.float32)
    got[:50] = rng.uniform(-2e-7, 2e-7, 50).astype(np.float32)    # around the 1e-7 floor
    got[60] = np.nan
    got[61] = np.inf
    return got, ref


def _numpy_bad_f32(got, ref):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    return ~(err <= np.maximum(parity.REL * np.abs(ref.astype(np.float64)), parity.ABS))


def test_tally_f32_matches_parity_check():
    rng = np.random.default_rng(1)
    got, ref = _planted(rng)
    want = int(_numpy_bad_f32(got, ref).sum())
    assert want > 10
    t = F.Tally("x")
    for lo, hi in ((0, 3000), (3000, 10_000)):
        F.tally_f32(t, torch.from_numpy(got[lo:hi]), torch.from_numpy(ref[lo:hi]), lo)
    assert t.n == got.size and t.bad == want and not t.ok()
    first = int(np.flatnonzero(_numpy_bad_f32(got, ref))[0])
    assert t.examples[0][0] == first
    with pytest.raises(AssertionError):
        parity.check_f32("x", got, ref)
    ok = F.Tally("ok")
    F.tally_f32(ok, torch.from_numpy(ref), torch.from_numpy(ref), 0)
    F.assert_all([ok])
    assert ok.worst == 0.0 and t.worst > 1.0                   # a fraction of the allowed error
    half = F.Tally("half")
    r1 = np.array([1.0, 1e-9], np.float32)
    g1 = np.array([1.0 + 0.5e-5, 1e-9 + 0.25e-7], np.float32)
    F.tally_f32(half, torch.from_numpy(g1), torch.from_numpy(r1), 0)
    assert half.ok() and 0.45 < half.worst < 0.51             # float32 rounding of the planted values
    F.assert_all([half, F.Tally("skipped (report only)")])


def test_tally_strict_v_matches_parity():
    rng = np.random.default_rng(2)
    ref = rng.uniform(1e-12, 1e-5, 5000).astype(np.float32)
    got = (ref.astype(np.float64) * (1 + rng.uniform(-2e-6, 2e-6, 5000))).astype(np.float32)
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    want = int((~(err <= 1e-6 * ref.astype(np.float64) + 1e-40)).sum())
    assert 0 < want < 5000
    t = F.Tally("v")
    F.tally_strict_v(t, torch.from_numpy(got), torch.from_numpy(ref), 0)
    assert t.bad == want
    with pytest.raises(AssertionError):
        parity.strict_v(got, ref)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_tally_param_matches_parity(fmt):
    """Beyond 1 ulp a pair fails unless its values are within the 1e-7
    floor: tiny bf16 parameters (|p| ~ 1e-7) many ulps apart pass, ordinary
    ones 2 ulps apart fail; both helpers decide alike.  (fp16 spaces its
    smallest values 6e-8 apart, so there the floor admits no pair 2 ulps
    apart.)"""
    rng = np.random.default_rng(3)
    x = rng.standard_normal(4000).astype(np.float32)
    x[:40] *= np.float32(1e-7)                                   # near zero: the floor applies
    ref = W.to_bits16(x, fmt)
    got = ref.copy()
    got[::7] = (got[::7].astype(np.int64) + rng.choice([-9, -2, -1, 1, 2, 9], got[::7].size)).astype(np.uint16)
    got[5] = 0x8000                                   # -0 against a +0 reference: equal
    ref[5] = 0x0000
    d = np.abs(parity.ordered16(got) - parity.ordered16(ref))
    far = d > 1
    near = np.abs(parity._value16(got, fmt) - parity._value16(ref, fmt)) <= parity.ABS
    want = int((far & ~near).sum())
    assert want > 0 and (int((far & near).sum()) > 0) == (fmt == "bf16")
    t = F.Tally("p")
    F.tally_param(t, torch.from_numpy(got.view(np.int16)), torch.from_numpy(ref.view(np.int16)), 0, fmt)
    assert t.bad == want and t.worst == float(d.max()) and t.beyond_ulp == int((far & near).sum())
    with pytest.raises(AssertionError):
        parity.check_param("p", got, ref, fmt=fmt)
    keep = ~(far & ~near)
    parity.check_param("p", got[keep], ref[keep], fmt=fmt)
    if fmt == "bf16":
        with pytest.raises(AssertionError):            # without the format: 1 ulp only
            parity.check_param("p", got[keep], ref[keep])
    t1 = F.Tally("p1")
    F.tally_param(t1, torch.from_numpy(got.view(np.int16)), torch.from_numpy(got.view(np.int16)), 0, fmt)
    assert t1.ok()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_tally_writeback(fmt):
    import oracle
    rng = np.random.default_rng(4)
    m = (rng.standard_normal(5000) * np.exp(rng.uniform(-30, 5, 5000))).astype(np.float32)
    bits = oracle.encode16_rne(m, fmt)
    t = F.Tally("w")
    F.tally_writeback(t, torch.from_numpy(m), torch.from_numpy(bits.view(np.int16)), 0, fmt)
    assert t.ok() and t.n == m.size
    bits[17] ^= 1
    t2 = F.Tally("w2")
    F.tally_writeback(t2, torch.from_numpy(m), torch.from_numpy(bits.view(np.int16)), 0, fmt)
    assert t2.bad == 1 and t2.examples[0][0] == 17


def test_tally_ulp_f32():
    ref = np.array([1.0, 1.0, 1.0, -2.0, 0.0, 1e-40], np.float32)
    got = np.array([1.0, np.nextafter(np.float32(1), np.float32(2)), 1.0 + 2 * 2.0**-23, -2.0,
                    np.float32(1e-45), 1e-40], np.float32)
    t = F.Tally("u")
    F.tally_ulp_f32(t, torch.from_numpy(got), torch.from_numpy(ref), 0)
    assert t.bad == 1 and t.examples[0][0] == 2


def test_chunk_blocks_and_pmap():
    for begin, S in ((0, 1), (W.CHUNK - 5, 11), (3 * W.CHUNK + 7, 2 * W.CHUNK + 9), (5, 0)):
        b = F.chunk_blocks(begin, S)
        assert [lo for lo, _ in b] == [0] + [hi for _, hi in b[:-1]] if b else S == 0
        assert (b[-1][1] if b else 0) == S
        for lo, hi in b:
            assert (begin + lo) // W.CHUNK == (begin + hi - 1) // W.CHUNK
    out = list(F.pmap(lambda x: x * x, range(100), ahead=3))
    assert out == [(x, x * x) for x in range(100)]
    assert F.by_sub(0) == [] and F.by_sub(F.SUB + 1) == [(0, F.SUB), (F.SUB, F.SUB + 1)]
