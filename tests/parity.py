"""Shared helpers for the GPU parity tests: device upload/download of seeded
inputs and the tolerance checks, written out once.

Tolerances (the bar every GPU result must meet against the oracle):
  plan, overflow flags, skip decisions   bit-exact
  fp32 master / exp_avg / exp_avg_sq     |x - ref| <= max(1e-5 * |ref|, 1e-7)
  gradient norm                          |n - ref| <= 1e-5 * ref
  fp16 / bf16 parameter copy             at most 1 ulp apart (distance of the
                                         16-bit patterns on the ordered integer
                                         line, +0 and -0 equal)
Besides the bar, `strict_*` checks bound the float32 arithmetic more tightly
(a mis-rounded coefficient such as 1 - beta2 formed in float32 passes the bar
on tiny values but not these).

Where the master's two terms p*(1 - lr*wd) and lr*m_hat/(sqrt(v_hat)+eps)
nearly cancel, float32 rounding of those terms can exceed the 1e-7 floor;
`cancellation_floor` raises the master's absolute floor to a few float32 ulps
of the larger term there (it changes nothing elsewhere).
"""
import numpy as np

REL, ABS = 1e-5, 1e-7


def to_device(a: np.ndarray, fmt: str = None):
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16).copy()).cuda()
        return t.view({"f16": torch.float16, "bf16": torch.bfloat16}[fmt])
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits_of(t) -> np.ndarray:
    """Raw uint16 bits of a 16-bit device tensor."""
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_f32(name, got, ref, rel=REL, abs_=ABS, floor=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, name
    err = np.abs(got - ref)
    tol = np.maximum(rel * np.abs(ref), abs_)
    if floor is not None:
        tol = np.maximum(tol, floor)
    bad = ~(err <= tol)
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} out of tolerance; e.g. idx {i.tolist()} "
                             f"got {got[i].tolist()} ref {ref[i].tolist()}")
    return float(np.max(err / np.maximum(np.abs(ref), 1e-30))) if err.size else 0.0


def ordered16(bits: np.ndarray) -> np.ndarray:
    """Map 16-bit float patterns to integers ordered like the values
    (+0 and -0 both map to 0)."""
    b = bits.astype(np.int64) & 0xFFFF
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _value16(bits: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def cancellation_floor(master_in, master_ref, decay: float, ulps: int = 4) -> np.ndarray:
    """Per element, `ulps` float32 ulps of the larger of the two terms the
    update subtracts: T = max(|p * decay|, |p * decay - ref|), the second
    being the size of lr * m_hat / (sqrt(v_hat) + eps) recovered from the
    oracle's result.  Float32 evaluation of the update rounds each term to
    within a few ulps of its own size, so where they cancel the result can
    differ from the exact one by that much (at most 3 ulps observed)."""
    pd = np.asarray(master_in, np.float64) * decay
    t = np.maximum(np.abs(pd), np.abs(pd - np.asarray(master_ref, np.float64)))
    return ulps * np.spacing(t.astype(np.float32)).astype(np.float64)


def check_param(name, got_bits, ref_bits, max_ulp=1, fmt=None, abs_=ABS):
    """At most max_ulp apart on the ordered-integer line; with fmt given,
    pairs further apart pass if their values differ by at most abs_ (near
    zero the parameter copy inherits the master's absolute floor)."""
    got_bits = np.asarray(got_bits, np.uint16)
    ref_bits = np.asarray(ref_bits, np.uint16)
    d = np.abs(ordered16(got_bits) - ordered16(ref_bits))
    bad = d > max_ulp
    if fmt is not None and bad.any():
        bad &= ~(np.abs(_value16(got_bits, fmt) - _value16(ref_bits, fmt)) <= abs_)
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{name}: {bad.sum()} params more than {max_ulp} ulp off; idx {i.tolist()} "
                             f"got {got_bits[i].tolist()} ref {ref_bits[i].tolist()}")
    return int(d.max()) if d.size else 0


def check_norm(got_sq: float, ref_sq: float, rel=1e-5):
    if np.isnan(ref_sq) or np.isinf(ref_sq):
        assert (np.isnan(got_sq) and np.isnan(ref_sq)) or got_sq == ref_sq, (got_sq, ref_sq)
        return
    n, r = np.sqrt(got_sq), np.sqrt(ref_sq)
    assert abs(n - r) <= rel * r, f"norm {n!r} vs oracle {r!r}"


def strict_v(got, ref):
    """Second moment: both terms are nonnegative, so float32 keeps a few ulp
    relative error everywhere."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    assert (err <= 1e-6 * np.abs(ref) + 1e-40).all(), float(np.max(err / np.maximum(ref, 1e-38)))


def compare_step(got, ref, what="", pfmt=None, master_floor=None):
    """got/ref: (master, exp_avg, exp_avg_sq, param_bits or None).  With the
    parameter format given, a parameter more than 1 ulp off passes within the
    master's 1e-7 absolute floor (check_param).  master_floor (per element,
    e.g. cancellation_floor) raises the master's absolute floor, and with it
    the parameter copy's."""
    out = {}
    for k, name in enumerate(("master", "exp_avg", "exp_avg_sq")):
        out[name] = check_f32(f"{what}{name}", got[k], ref[k], floor=master_floor if k == 0 else None)
    strict_v(got[2], ref[2])
    if ref[3] is not None:
        # the copy is the rounding of the master: its value floor follows the master's
        abs_ = ABS if master_floor is None else np.maximum(ABS, master_floor)
        out["param_ulp"] = check_param(f"{what}param", got[3], ref[3], fmt=pfmt, abs_=abs_)
    return out
