"""CPU: the float32 model of the update (tests/f32model.py) against the
library's coefficient block and against the oracle."""
import struct

import numpy as np
import pytest

import f32model
import oracle
import zero_sharded_mixed_partition_amd as Z


def _block(hp):
    blk = np.zeros(Z.zero_adam_coef_bytes(), np.uint8)
    Z.zero_adam_prepare(Z.AdamHyper(**hp), blk)
    return struct.unpack_from("8f", blk.tobytes(), 0)


def test_model_coefficients_equal_the_library_block():
    """Both form the coefficients from the header's description; the model's
    eight float32 values equal the library's block bit for bit."""
    rng = np.random.default_rng(5)
    for _ in range(300):
        hp = dict(lr=float(10 ** rng.uniform(-6, 0)), beta1=float(rng.choice([0.0, 0.5, 0.9, rng.uniform(0, 0.999)])),
                  beta2=float(rng.choice([0.0, 0.99, 0.999, rng.uniform(0, 0.99999)])),
                  eps=float(10 ** rng.uniform(-12, -3)), weight_decay=float(rng.uniform(0, 0.2)),
                  step=int(10 ** rng.uniform(0, 6)), inv_loss_scale=1.0, max_grad_norm=0.0)
        c = f32model.coefficients(**hp)
        want = np.array(_block(hp), np.float32)
        got = np.array([c[k] for k in ("B1", "O1", "B2", "O2", "SS", "RB", "E", "D")], np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), hp


def test_pow_int_closed_forms():
    assert f32model.pow_int(0.5, 10) == 2.0 ** -10
    assert f32model.pow_int(0.9, 0) == 1.0 and f32model.pow_int(0.0, 3) == 0.0
    assert f32model.pow_int(3.0, 5) == 243.0


@pytest.mark.parametrize("seed", range(8))
def test_model_within_the_bar_of_the_oracle(seed):
    """On ordinary steps the float32 model stays within the parity bar of the
    fp64 oracle (it is float32 arithmetic in the documented order)."""
    rng = np.random.default_rng(seed)
    n = 50_000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = rng.uniform(1e-8, 1e-5, n).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    hp = dict(lr=float(10 ** rng.uniform(-5, -2)), beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
              step=int(rng.integers(1, 10 ** 5)), inv_loss_scale=1.0, max_grad_norm=float(rng.choice([0.0, 0.1])))
    sq, _ = oracle.shard_sqnorm_overflow(g, "f32", 1.0)
    rp, rm, rv, _, _ = oracle.shard_step(p, m, v, g, "f32", None, global_sq=sq, global_overflow=False, **hp)
    mp, mm, mv = f32model.adam_update(p, m, v, g, sq, **hp)
    for got, ref in ((mp, rp), (mm, rm), (mv, rv)):
        err = np.abs(got.astype(np.float64) - ref)
        assert (err <= np.maximum(1e-5 * np.abs(ref), 1e-7)).all()


def test_cancellation_floor_values():
    """4 float32 ulps of the larger subtracted term; below the bar unless
    the two terms cancel."""
    from parity import cancellation_floor
    f = cancellation_floor(np.array([0.7, 0.02, -0.5], np.float32), np.array([0.005, 0.0199, -0.49]), 0.99)
    assert f[0] == 4 * np.spacing(np.float32(0.7 * 0.99))          # |p D| = 0.693 > |p D - ref| = 0.688
    assert f[1] == 4 * np.spacing(np.float32(0.02 * 0.99))
    rng = np.random.default_rng(3)
    p = rng.standard_normal(100_000) * rng.choice([0.02, 1.0, 30.0], 100_000)
    ref = p * 0.999 - rng.standard_normal(100_000) * 1e-3 * np.abs(p)     # no cancellation
    bar = np.maximum(1e-5 * np.abs(ref), 1e-7)
    assert (cancellation_floor(p, ref, 0.999) <= bar).all()


def test_cancelling_case_passes_only_with_the_floor():
    """A random-sweep case where the update's two terms (near 0.7 each)
    cancel: the float32 model, which the GPU equals bit for bit, leaves the
    plain bar on a few masters and stays within the raised floor."""
    import test_gpu_random_sweep as T
    from parity import cancellation_floor, check_f32
    n, gfmt, pfmt, p, m, v, g, hp = T._case(346)
    sq, _ = oracle.shard_sqnorm_overflow(g, gfmt, hp["inv_loss_scale"])
    rp = oracle.shard_step(p, m, v, g, gfmt, None, global_sq=sq, global_overflow=False, **hp)[0]
    mp = f32model.adam_update(p, m, v, T._values(g, gfmt), sq, **hp)[0]
    with pytest.raises(AssertionError):
        check_f32("master", mp, rp)
    check_f32("master", mp, rp, floor=cancellation_floor(p, rp, 1.0 - hp["lr"] * hp["weight_decay"]))
