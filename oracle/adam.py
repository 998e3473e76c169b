"""One rank's mixed-precision Adam/AdamW step over its shard (oracle).

What the pages fix: [Explainer, History, "The mixed-precision era"] and
[Explainer, "The 16 Bytes per Parameter Audit"]: training keeps an fp16
weight, an fp32 master copy and two fp32 Adam moments per parameter;
[Explainer, Ch.02 "The Three Stages", "What each stage shards"]: under
ZeRO-1/2 each rank updates only the optimizer states (and, with P_os+g, holds
only the gradients) of its own partition, so the step below runs on one
shard.  The pages give no update formula.  The steps are read as:

  1. unscale the 16-bit gradient by the loss scale and detect inf/NaN
     (dynamic loss scaling, Micikevicius et al. 2018);
  2. squared L2 norm of the unscaled gradient, for max-norm clipping
     (Pascanu et al. 2013, coefficient min(1, max_norm / (norm + 1e-6)));
  3. Adam with bias correction (Kingma & Ba 2015, eps outside the square
     root) and decoupled weight decay scaled by the learning rate
     (Loshchilov & Hutter 2019 with the schedule multiplier equal to lr);
  4. round the updated fp32 master weight to the 16-bit parameter copy.
With gradient accumulation the step consumes the fp32 gradient copy instead
of the 16-bit gradient (format 'f32', already unscaled).
A step whose gradient holds any inf/NaN is skipped: no state changes, the step
counter does not advance and the loss scale is reduced.

Everything is float64; stored results are rounded once to float32 (master,
momentum, variance) and from that float32 master to fp16/bf16 (parameter).
"""
from dataclasses import dataclass, replace
from fractions import Fraction
import math
from typing import Iterable, Optional, Tuple

import numpy as np

from .formats import FORMATS, decode16, encode16_rne, is_nonfinite16


def _magnitude_counts(bits: np.ndarray, fmt: str) -> np.ndarray:
    """How many elements carry each 16-bit magnitude pattern (sign dropped):
    counts[p] for p in [0, 0x8000)."""
    b = np.asarray(bits, dtype=np.uint16)
    return np.bincount(b & np.uint16(0x7FFF), minlength=0x8000).astype(np.int64)


def _sum_squares_from_counts(counts: np.ndarray, fmt: str) -> Fraction:
    """Exact sum of squares of the finite values given by a magnitude
    histogram: sum over patterns p of counts[p] * value(p)^2.

    A finite pattern with exponent field e and fraction f has value
    M * 2^E with integer M (f for e = 0, 2^mbits + f otherwise) and
    E = max(e, 1) - bias - mbits; its square M^2 * 2^(2E) is summed as an
    integer multiple of 2^(2 Emin), Emin = 1 - bias - mbits.
    """
    ebits, mbits, bias = FORMATS[fmt]
    emax_field = (1 << ebits) - 1
    e_min = 1 - bias - mbits
    total = 0
    for p in np.nonzero(counts)[0]:
        p = int(p)
        e, f = p >> mbits, p & ((1 << mbits) - 1)
        if e == emax_field:
            continue                     # inf / NaN: handled by the caller
        M = f if e == 0 else f + (1 << mbits)
        E = max(e, 1) - bias - mbits
        total += int(counts[p]) * M * M << (2 * (E - e_min))
    return Fraction(total) * Fraction(2) ** (2 * e_min)


def _sum_squares_exact(bits: np.ndarray, fmt: str) -> Fraction:
    """Exact sum of squares of the finite 16-bit values, as a rational."""
    return _sum_squares_from_counts(_magnitude_counts(bits, fmt), fmt)


def _grad_f64(grad, fmt: str) -> np.ndarray:
    """Gradient values as float64: decoded 16-bit patterns, or an fp32
    gradient (fmt 'f32', e.g. an fp32 accumulation buffer) widened exactly."""
    if fmt == "f32":
        return np.asarray(grad, dtype=np.float32).astype(np.float64)
    return decode16(grad, fmt)


def _sqnorm_overflow_f32(g32: np.ndarray, inv_loss_scale: float, chunk: int = 1 << 24) -> Tuple[float, bool]:
    """fp32 gradient: overflow = any non-finite element; sq = sum of
    (g * inv_loss_scale)^2.  Each square of an fp32 value times a power of two
    is exact in float64; each 2^24-element chunk is summed pairwise in float64
    and the chunk sums are combined with math.fsum, so the relative error is
    below 1e-14."""
    x = np.asarray(g32, dtype=np.float32)
    finite = np.isfinite(x)
    if not finite.all():
        return (math.nan if np.isnan(x).any() else math.inf), True
    parts = []
    for s in range(0, x.size, chunk):
        y = x[s:s + chunk].astype(np.float64) * inv_loss_scale
        parts.append(float(np.sum(y * y)))
    return math.fsum(parts), False


def shard_sqnorm_overflow(grad_bits: np.ndarray, fmt: str, inv_loss_scale: float) -> Tuple[float, bool]:
    """(sq, overflow) for one gradient shard.

    overflow: some element is inf or NaN (tested on its exponent bits, never
    inferred from the norm).  sq = sum_i (g_i * inv_loss_scale)^2 over the
    whole shard (padding zeros included), computed exactly and rounded once
    to float64; +inf if the shard holds an inf and no NaN, NaN if it holds a
    NaN.
    """
    if fmt == "f32":
        return _sqnorm_overflow_f32(grad_bits, inv_loss_scale)
    bits = np.asarray(grad_bits)
    bad = is_nonfinite16(bits, fmt)
    overflow = bool(bad.any())
    if overflow:
        vals = decode16(bits[bad], fmt)
        return (math.nan if np.isnan(vals).any() else math.inf), True
    exact = _sum_squares_exact(bits, fmt) * Fraction(inv_loss_scale) ** 2
    return float(exact), False


@dataclass(frozen=True)
class SqnormTerms:
    """What one shard contributes to the global (sum of squares, flag), in a
    form whose contributions add up without rounding: for a 16-bit gradient
    the histogram of its finite magnitudes (counts per pattern, sign dropped);
    for an fp32 gradient the float64 sums of its 2^24-element chunks of
    (g * inv_loss_scale)^2.  overflow / has_nan: the shard holds an inf or
    NaN / a NaN."""
    counts: Optional[np.ndarray]
    chunk_sums: Tuple[float, ...]
    overflow: bool
    has_nan: bool


def sqnorm_terms(grad, fmt: str, inv_loss_scale: float) -> SqnormTerms:
    """One shard's terms of the data-parallel norm reduction (see SqnormTerms)."""
    if fmt == "f32":
        x = np.asarray(grad, dtype=np.float32)
        if not np.isfinite(x).all():
            return SqnormTerms(None, (), True, bool(np.isnan(x).any()))
        sums = []
        for s in range(0, x.size, 1 << 24):
            y = x[s:s + (1 << 24)].astype(np.float64) * inv_loss_scale
            sums.append(float(np.sum(y * y)))
        return SqnormTerms(None, tuple(sums), False, False)
    bits = np.asarray(grad)
    bad = is_nonfinite16(bits, fmt)
    if bad.any():
        return SqnormTerms(None, (), True, bool(np.isnan(decode16(bits[bad], fmt)).any()))
    return SqnormTerms(_magnitude_counts(bits, fmt), (), False, False)


def combine_sqnorm_terms(terms: Iterable[SqnormTerms], fmt: str, inv_loss_scale: float) -> Tuple[float, bool]:
    """The data-parallel reduction: the OR of the shards' flags, and the sum
    of squares over all shards, +inf if some shard holds an inf and none a
    NaN, NaN if any holds a NaN.  16-bit: the histograms are added and the
    sum formed exactly from them, rounded once.  fp32: math.fsum over every
    shard's chunk sums (each chunk summed pairwise in float64, so the result
    is within 1e-14 relative of the exact sum)."""
    counts, sums, overflow, has_nan = np.zeros(0x8000, np.int64), [], False, False
    for t in terms:
        overflow |= t.overflow
        has_nan |= t.has_nan
        if t.counts is not None:
            counts += t.counts
        sums.extend(t.chunk_sums)
    if overflow:
        return (math.nan if has_nan else math.inf), True
    if fmt == "f32":
        return math.fsum(sums), False
    return float(_sum_squares_from_counts(counts, fmt) * Fraction(inv_loss_scale) ** 2), False


def global_sqnorm_overflow(shards: Iterable[np.ndarray], fmt: str,
                           inv_loss_scale: float) -> Tuple[float, bool]:
    """The data-parallel reduction of the per-rank results: the global sum of
    squares over all shards (16-bit: exact, one rounding) and the OR of the
    flags."""
    return combine_sqnorm_terms((sqnorm_terms(g, fmt, inv_loss_scale) for g in shards), fmt, inv_loss_scale)


def clip_coefficient(sq: float, max_grad_norm: float) -> float:
    """Max-norm clipping coefficient from the global squared norm:
    min(1, max_norm / (norm + 1e-6)); 1 when clipping is off (max_norm <= 0)."""
    if max_grad_norm <= 0.0:
        return 1.0
    norm = math.sqrt(sq)
    return min(1.0, max_grad_norm / (norm + 1e-6))


def grad_scale(inv_loss_scale: float, coef: float) -> float:
    """Factor applied to the raw 16-bit gradient: unscale, then clip."""
    return inv_loss_scale * coef


def adam_update(master: np.ndarray, exp_avg: np.ndarray, exp_avg_sq: np.ndarray,
                grad_bits: np.ndarray, grad_fmt: str, gscale: float, *, lr: float,
                beta1: float, beta2: float, eps: float, weight_decay: float, step: int,
                param_fmt: Optional[str] = None):
    """Bias-corrected Adam with decoupled weight decay, elementwise, float64.

    step is the 1-based index t of the step being applied.  Returns float32
    (master, exp_avg, exp_avg_sq) and the uint16 bits of the 16-bit parameter
    copy rounded from the new float32 master (None if param_fmt is None).
    """
    if step < 1:
        raise ValueError("step must be >= 1")
    p = np.asarray(master, dtype=np.float64)
    m = np.asarray(exp_avg, dtype=np.float64)
    v = np.asarray(exp_avg_sq, dtype=np.float64)
    g = _grad_f64(grad_bits, grad_fmt) * gscale
    m_new = beta1 * m + (1.0 - beta1) * g
    v_new = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    p_new = p - lr * (m_hat / (np.sqrt(v_hat) + eps) + weight_decay * p)
    master32 = p_new.astype(np.float32)
    param = encode16_rne(master32, param_fmt) if param_fmt is not None else None
    return master32, m_new.astype(np.float32), v_new.astype(np.float32), param


def grad_accumulate(acc32: Optional[np.ndarray], grad_bits: np.ndarray, fmt: str,
                    inv_loss_scale: float) -> Tuple[np.ndarray, bool]:
    """One micro-batch into the fp32 gradient copy.

    [Explainer, Ch.02 "The Three Stages", memory-per-parameter list: an fp16
    gradient plus its fp32 copy]: the copy accumulates the unscaled 16-bit
    micro-batch gradients,
        acc <- float32(acc + g * inv_loss_scale)      (acc None: start at 0)
    with the sum formed in float64 (exact whenever the two exponents are
    within 29 binades, true for gradients of one model) and rounded once to
    float32.  Returns (new acc, overflow) where overflow flags an inf/NaN in
    this micro-batch's 16-bit input.
    """
    t = decode16(grad_bits, fmt) * inv_loss_scale
    base = 0.0 if acc32 is None else np.asarray(acc32, dtype=np.float32).astype(np.float64)
    return (base + t).astype(np.float32), bool(is_nonfinite16(grad_bits, fmt).any())


def grad_reduce(slices, fmt: str, inv_loss_scale: float) -> Tuple[np.ndarray, bool]:
    """The reduced gradient of this rank's partition over the data-parallel
    ranks, from the ranks' 16-bit gradient slices of it, in rank order.

    Plain data parallelism sums the ranks' gradients [Explainer, History,
    "Data parallelism's reign"]; with gradients partitioned each rank keeps
    only the reduced gradient of its own partition [Explainer, Ch.02 "The
    Three Stages", what each stage shards; Ch.05 stage table: reduce-scatter].
    Reading: the sum is formed slice by slice into the fp32 gradient copy,
        acc <- float32(g_0 * inv),  acc <- float32(acc + g_k * inv),  k = 1..K-1,
    each addition rounded once to float32: the fp32 copy accumulating the
    ranks' slices as it accumulates micro-batches (grad_accumulate).
    Returns (acc, overflow), overflow flagging an inf/NaN in any slice.
    """
    if len(slices) < 1:
        raise ValueError("at least one slice")
    acc, ovf = None, False
    for g in slices:
        acc, o = grad_accumulate(acc, g, fmt, inv_loss_scale)
        ovf = ovf or o
    return acc, ovf


@dataclass(frozen=True)
class LossScalerState:
    """Dynamic loss scale.  On an overflowing step: skip it, multiply the
    scale by `backoff` (floored at `min_scale`) and reset the clean-step count.
    After `growth_interval` clean steps in a row: multiply the scale by
    `growth` and reset the count.  backoff = growth = 1 gives a static scale."""
    scale: float
    good_steps: int = 0
    min_scale: float = 1.0
    backoff: float = 0.5
    growth: float = 2.0
    growth_interval: int = 1000


def loss_scaler_update(s: LossScalerState, overflow: bool) -> Tuple[LossScalerState, bool]:
    """Return (new state, skip)."""
    if overflow:
        return replace(s, scale=max(s.scale * s.backoff, s.min_scale), good_steps=0), True
    good = s.good_steps + 1
    if good >= s.growth_interval:
        return replace(s, scale=s.scale * s.growth, good_steps=0), False
    return replace(s, good_steps=good), False


def shard_step(master, exp_avg, exp_avg_sq, grad_bits, grad_fmt, param_fmt, *, global_sq,
               global_overflow, inv_loss_scale, max_grad_norm, lr, beta1, beta2, eps,
               weight_decay, step):
    """Steps 2-4 on one shard given the data-parallel-reduced (sq, overflow).

    Returns (master, exp_avg, exp_avg_sq, param_bits_or_None, applied).  On
    overflow nothing is computed: the inputs come back unchanged, no parameter
    is written and applied is False.
    """
    if global_overflow:
        return master, exp_avg, exp_avg_sq, None, False
    coef = clip_coefficient(global_sq, max_grad_norm)
    out = adam_update(master, exp_avg, exp_avg_sq, grad_bits, grad_fmt,
                      grad_scale(inv_loss_scale, coef), lr=lr, beta1=beta1, beta2=beta2,
                      eps=eps, weight_decay=weight_decay, step=step, param_fmt=param_fmt)
    return (*out, True)
