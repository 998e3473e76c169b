"""Pins for the oracle's 16-bit format code against library routines
(numpy float16, torch bfloat16 on the CPU) over every bit pattern, every
rounding tie and the range edges."""
import numpy as np
import pytest
import torch

from oracle import decode16, encode16_rne, is_nonfinite16

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _lib_decode(bits, fmt):
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _lib_encode(x32, fmt):
    if fmt == "f16":
        return x32.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_decode_exhaustive(fmt):
    ours, lib = decode16(ALL, fmt), _lib_decode(ALL, fmt)
    nan = np.isnan(lib)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == lib[~nan]).all()
    assert (np.signbit(ours[~nan]) == np.signbit(lib[~nan])).all()     # -0 kept


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_nonfinite_exhaustive(fmt):
    assert (is_nonfinite16(ALL, fmt) == ~np.isfinite(_lib_decode(ALL, fmt))).all()
    assert is_nonfinite16(ALL, fmt).sum() == (2 * (1 << 10) if fmt == "f16" else 2 * (1 << 7))


def _neighbours(fmt):
    """Every finite 16-bit value, the midpoints between neighbours (ties), and
    float32 values one ulp either side of each midpoint."""
    vals = _lib_decode(ALL, fmt)
    fin = np.sort(np.unique(vals[np.isfinite(vals)]))
    mids = (fin[:-1] + fin[1:]) / 2            # exact in float64
    mids32 = mids.astype(np.float32)
    assert (mids32.astype(np.float64) == mids).all()   # ties are float32 values
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(-np.inf))
    edge = np.array([65504, 65519.99, 65520, 65536, 1e30, 3.3895314e38, 3.4e38,
                     2.0**-24, 2.0**-25, 2.0**-26, 3 * 2.0**-26, 2.0**-133, 2.0**-134,
                     1e-45, 0.0, -0.0, np.inf, -np.inf], np.float32)
    return np.concatenate([fin.astype(np.float32), mids32, up, dn, edge, -mids32, -up])


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_encode_ties_and_edges(fmt):
    x = _neighbours(fmt)
    assert (encode16_rne(x, fmt) == _lib_encode(x, fmt)).all()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_encode_random(fmt):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    assert (encode16_rne(x, fmt) == _lib_encode(x, fmt)).all()
    y = (rng.standard_normal(1 << 18) * np.exp(rng.uniform(-40, 12, 1 << 18))).astype(np.float32)
    assert (encode16_rne(y, fmt) == _lib_encode(y, fmt)).all()


@pytest.mark.parametrize("fmt,qnan", [("f16", 0x7E00), ("bf16", 0x7FC0)])
def test_encode_nan(fmt, qnan):
    out = encode16_rne(np.array([np.nan, -np.nan], np.float32), fmt)
    assert out[0] == qnan and out[1] == (qnan | 0x8000)
    assert is_nonfinite16(out, fmt).all()


def test_hand_examples():
    # 1 + 2^-11 is the midpoint between 1 and 1+2^-10 in fp16: ties to even (1.0)
    assert encode16_rne(np.float32(1 + 2.0**-11), "f16") == 0x3C00
    # 1 + 3*2^-11 lies between 1+2^-10 (odd) and 1+2^-9 (even): goes up
    assert encode16_rne(np.float32(1 + 3 * 2.0**-11), "f16") == 0x3C02
    # bf16: 1 + 2^-8 is a tie between 1 and 1+2^-7 -> 1.0
    assert encode16_rne(np.float32(1 + 2.0**-8), "bf16") == 0x3F80
    # smallest fp16 subnormal and half of it (tie with zero -> zero)
    assert encode16_rne(np.float32(2.0**-24), "f16") == 0x0001
    assert encode16_rne(np.float32(2.0**-25), "f16") == 0x0000
    assert decode16(np.array([0x0001], np.uint16), "f16")[0] == 2.0**-24
    assert decode16(np.array([0x7BFF], np.uint16), "f16")[0] == 65504.0
