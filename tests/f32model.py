"""A float32 model of the fused AdamW pass, written from the per-element
operation order that include/zero_shard.h documents for zero_shard_adam_step
(every operation rounded once to float32; fma with one rounding; the
per-step coefficients formed in double, beta^t by binary exponentiation, and
each rounded once).  Test infrastructure: the oracle (fp64) is the parity
reference; this model shows that where the GPU differs from the oracle it
does exactly what float32 arithmetic in the documented order does.

fma(a, b, c) is taken as the float64 value of a*b (exact for float32
operands) plus c, rounded to float32: this equals the single rounding except
when the float64 sum lands exactly on a float32 rounding tie (the tests that
use the model compare bit for bit, so such an element would show)."""
import math

import numpy as np

F32 = np.float32


def _fma(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(F32)


def pow_int(b: float, e: int) -> float:
    """b**e for e >= 0 by binary exponentiation in IEEE double."""
    r = 1.0
    while e > 0:
        if e & 1:
            r = r * b
        b = b * b
        e >>= 1
    return r


def coefficients(lr, beta1, beta2, eps, weight_decay, step, **_):
    bc1, bc2 = 1.0 - pow_int(beta1, step), 1.0 - pow_int(beta2, step)
    return dict(B1=F32(beta1), O1=F32(1.0 - beta1), B2=F32(beta2), O2=F32(1.0 - beta2), SS=F32(lr / bc1),
                RB=F32(1.0 / math.sqrt(bc2)), E=F32(eps), D=F32(1.0 - lr * weight_decay))


def gradient_factor(inv_loss_scale: float, max_grad_norm: float, global_sq: float) -> np.float32:
    coef = 1.0
    if max_grad_norm > 0.0:
        coef = max_grad_norm / (math.sqrt(global_sq) + 1e-6)
        if not coef < 1.0:
            coef = 1.0
    return F32(inv_loss_scale * coef)


def adam_update(p, m, v, g_values, global_sq: float, **hp):
    """(p, m, v) after one step, float32; g_values are the raw gradient values
    as float32 (16-bit values decoded exactly, or the fp32 copy)."""
    c = coefficients(**hp)
    gscale = gradient_factor(hp["inv_loss_scale"], hp["max_grad_norm"], global_sq)
    g = (np.asarray(g_values, F32) * gscale).astype(F32)
    m2 = _fma(c["B1"], m, (c["O1"] * g).astype(F32))
    v2 = _fma(c["B2"], v, ((c["O2"] * g).astype(F32) * g).astype(F32))
    d = _fma(np.sqrt(v2).astype(F32), c["RB"], c["E"])
    p2 = _fma(p, c["D"], -(((c["SS"] * m2).astype(F32)) / d).astype(F32))
    return p2, m2, v2
