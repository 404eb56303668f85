"""Rotary position encoding (RoPE) as a complex multiplication per pair, float64.

Source of the operation: the InferScale review (arXiv 2607.27090), "What
carries the argument" -- keys are stored before rotary position encoding and
re-rotated to serving-time positions on injection -- and the "Axiom &
Free-Parameter Ledger" axiom R_a^T R_b = R_{b-a} (Theorem 6, section 5.1).
The rotation itself is RoFormer's (reference [20] of that page).

Readings (the pages give no formula):
* Pairing: half split (GPT-NeoX style): element j pairs with j + D/2,
  j = 0 .. D/2-1.  The pair is the complex number z_j = x[j] + i x[j + D/2].
* Frequencies: theta_j = base ** (-2j / D) radians per position.
* Sign: z_j' = z_j * exp(+i * pos * theta_j), i.e.
  x'[j] = x[j] cos - x[j+D/2] sin,  x'[j+D/2] = x[j+D/2] cos + x[j] sin.
* Positions are 0-based integers; position 0 is the identity.
"""

import functools
from decimal import Decimal, localcontext

import numpy as np


def inv_freq(head_dim, base):
    """theta_j = base ** (-2j / D) for j = 0 .. D/2 - 1, rounded once to float64.

    Evaluated in 60-digit decimal arithmetic and then rounded, so the value is
    the float64 nearest the exact power on every machine (a vectorised float64
    power is not correctly rounded on every CPU, and an ulp in theta_j moves
    the angle pos * theta_j by up to ~2e-12 at the positions used here).
    The values depend only on (D, base) and are memoised.
    """
    return _inv_freq(int(head_dim), float(base)).copy()


@functools.lru_cache(maxsize=64)
def _inv_freq(head_dim, base):
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    with localcontext() as ctx:
        ctx.prec = 60
        b = Decimal(repr(float(base)))
        vals = [float(b ** (Decimal(-2 * j) / Decimal(head_dim))) for j in range(head_dim // 2)]
    return np.array(vals, dtype=np.float64)


def rotation_factors(pos, head_dim, base):
    """exp(i * pos * theta_j) as complex128, shape pos.shape + (D/2,)."""
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq(head_dim, base)
    w = np.empty(ang.shape, dtype=np.complex128)
    w.real = np.cos(ang)
    w.imag = np.sin(ang)
    return w


def rotate(x, pos, base):
    """Rotate float64 vectors x[..., D] to positions pos (broadcast to x[..., 0]).

    Returns float64 x' with x'[j] + i x'[j+D/2] = (x[j] + i x[j+D/2]) * exp(i pos theta_j).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    w = rotation_factors(pos, d, base)
    z = np.empty(x.shape[:-1] + (half,), dtype=np.complex128)
    z.real = x[..., :half]
    z.imag = x[..., half:]
    zr = z * w
    out = np.empty_like(x)
    out[..., :half] = zr.real
    out[..., half:] = zr.imag
    return out
