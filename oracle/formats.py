"""16-bit floating-point formats, written out from the IEEE 754 definitions.

[Explainer, Ch.02 "The Three Stages", memory-per-parameter list]: the model
copy of a weight and its gradient are 2-byte floats.  Two 2-byte formats are
handled: IEEE binary16 ('f16': 1 sign, 5 exponent bits, bias 15, 10 fraction
bits) and bfloat16 ('bf16': 1 sign, 8 exponent bits, bias 127, 7 fraction
bits, i.e. the upper half of a binary32).

decode16      raw bits -> exact float64 value
is_nonfinite16  exponent field all ones (inf or NaN)
encode16_rne  float32 value -> raw bits, round to nearest, ties to even,
              overflow to infinity, NaN to a quiet NaN of the same sign.
"""
import numpy as np

# (exponent bits, fraction bits, bias)
FORMATS = {"f16": (5, 10, 15), "bf16": (8, 7, 127)}


def _fields(fmt):
    ebits, mbits, bias = FORMATS[fmt]
    emax_field = (1 << ebits) - 1
    emin = 1 - bias                 # exponent of the smallest normal
    emax = emax_field - 1 - bias    # exponent of the largest finite binade
    return ebits, mbits, bias, emax_field, emin, emax


def _decode16_fields(bits: np.ndarray, fmt: str) -> np.ndarray:
    """Exact float64 value of each 16-bit pattern, from its sign, exponent and
    fraction fields."""
    ebits, mbits, bias, emax_field, emin, _ = _fields(fmt)
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> mbits) & emax_field
    f = b & ((1 << mbits) - 1)
    # subnormal/zero: f * 2^(emin - mbits); normal: (2^mbits + f) * 2^(e - bias - mbits)
    sig = np.where(e == 0, f, f + (1 << mbits)).astype(np.float64)
    exp = np.where(e == 0, emin - mbits, e - bias - mbits)
    val = np.ldexp(sig, exp.astype(np.int32))
    special = e == emax_field
    val = np.where(special, np.where(f == 0, np.inf, np.nan), val)
    return sign * val


_DECODE_TABLE = {}


def decode16(bits: np.ndarray, fmt: str) -> np.ndarray:
    """Exact float64 value of each 16-bit pattern: the field decoding above,
    evaluated once for all 65,536 patterns and then looked up by pattern."""
    if fmt not in _DECODE_TABLE:
        _DECODE_TABLE[fmt] = _decode16_fields(np.arange(1 << 16, dtype=np.int64), fmt)
    return _DECODE_TABLE[fmt][np.asarray(bits).astype(np.uint16)]


def is_nonfinite16(bits: np.ndarray, fmt: str) -> np.ndarray:
    """True where the pattern is +-inf or NaN (exponent field all ones)."""
    ebits, mbits, _, emax_field, _, _ = _fields(fmt)
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    return ((b >> mbits) & emax_field) == emax_field


def _encode_bf16_rne(x: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of a binary32 pattern (same sign and
    exponent fields, the top 7 fraction bits), so rounding a float32 to it is
    rounding its pattern to a multiple of 2^16: keep the upper 16 bits and add
    one when the dropped lower 16 bits exceed half (0x8000), or equal half
    while the kept part is odd.  A carry out of the fraction moves into the
    next binade, and past the largest finite value into the infinity pattern,
    as round-to-nearest requires.  NaN becomes the quiet NaN of its sign."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32, order="C")
    u = x32.view(np.uint32)
    upper, lower = u >> np.uint32(16), u & np.uint32(0xFFFF)
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & np.uint32(1)) == 1))
    out = (upper + up).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        out[nan] = np.uint16(0x7FC0) | (upper[nan] & np.uint32(0x8000)).astype(np.uint16)
    return out


def encode16_rne(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round float values (float32 or exactly float32-representable float64)
    to the nearest 16-bit value, ties to even; return raw uint16 bits."""
    if fmt == "bf16":
        return _encode_bf16_rne(x)
    ebits, mbits, bias, emax_field, emin, emax = _fields(fmt)
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    finite = np.isfinite(a)
    a_f = np.where(finite, a, 0.0)
    # binade exponent e with 2^e <= a < 2^(e+1), clamped below at emin
    _, k = np.frexp(a_f)                      # a = frac * 2^k, frac in [0.5, 1)
    e = np.where(a_f > 0, k - 1, emin)
    e = np.maximum(e, emin)
    # a measured in units of the format's spacing (quantum) in that binade
    n = np.ldexp(a_f, (mbits - e).astype(np.int32))
    fl = np.floor(n)
    frac = n - fl
    odd = np.mod(fl, 2.0) == 1.0
    up = (frac > 0.5) | ((frac == 0.5) & odd)
    r = fl + up
    carry = r == float(1 << (mbits + 1))      # rounded up into the next binade
    e = np.where(carry, e + 1, e)
    r = np.where(carry, float(1 << mbits), r)
    overflow = e > emax
    r_int = r.astype(np.int64)
    normal = r_int >= (1 << mbits)
    exp_field = np.where(normal, e + bias, 0)
    mant = np.where(normal, r_int - (1 << mbits), r_int)
    out = (exp_field << mbits) | mant
    inf_bits = emax_field << mbits
    qnan_bits = inf_bits | (1 << (mbits - 1))
    out = np.where(overflow | np.isinf(x), inf_bits, out)
    out = np.where(np.isnan(x), qnan_bits, out)
    out = out | np.where(neg, 1 << 15, 0)
    return out.astype(np.uint16)
