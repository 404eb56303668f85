"""Rotary position encoding (RoPE) as a complex multiplication per pair, float64.

Source of the operation: the InferScale review (arXiv 2607.27090), "What
carries the argument" -- keys are stored before rotary position encoding and
re-rotated to serving-time positions on injection -- and the "Axiom &
Free-Parameter Ledger" axiom R_a^T R_b = R_{b-a} (Theorem 6, section 5.1).
The rotation itself is RoFormer's (reference [20] of that page).

Readings (the pages give no formula):
* Pairing, two conventions of the same rotation:
  - half split (GPT-NeoX style, the default): element j pairs with j + D/2,
    z_j = x[j] + i x[j + D/2];
  - interleaved (GPT-J style, RoFormer's own block-diagonal form): element
    2j pairs with 2j + 1, z_j = x[2j] + i x[2j + 1];
  j = 0 .. D/2-1 in both.
* Frequencies: f_j = base ** (-2j / D) radians per position.  Optionally
  rescaled by the long-context rule published with Llama 3.1 (one of the
  models the review evaluates, "Referee Report" Summary); see scaled_frequency.
* Sign: z_j' = z_j * exp(+i * pos * f_j), i.e. x1' = x1 cos - x2 sin,
  x2' = x2 cos + x1 sin for the pair (x1, x2).
* Positions are 0-based integers; position 0 is the identity.
"""

import functools
from dataclasses import dataclass
from decimal import Decimal, localcontext

import numpy as np

HALF_SPLIT = "half_split"
INTERLEAVED = "interleaved"

# pi to 60 significant digits (a published constant)
_PI = Decimal("3.14159265358979323846264338327950288419716939937510582097494")


@dataclass(frozen=True)
class Llama3Scaling:
    """Long-context frequency rule of Llama 3.1 (factor 8, 1, 4, 8192 there)."""
    factor: float
    low_freq_factor: float
    high_freq_factor: float
    original_max_position: int


LLAMA31 = Llama3Scaling(8.0, 1.0, 4.0, 8192)


def scaled_frequency(f, scaling):
    """One frequency f (radians per position, a Decimal) under the rule.

    With wavelength w = 2 pi / f and W = original_max_position: frequencies
    whose wavelength is shorter than W / high_freq_factor are kept; those
    whose wavelength is longer than W / low_freq_factor are divided by
    factor; in between the two are blended linearly in W / w:
    m = (W / w - low) / (high - low), f' = (1 - m) f / factor + m f.
    """
    w_orig = Decimal(int(scaling.original_max_position))
    lo = Decimal(repr(float(scaling.low_freq_factor)))
    hi = Decimal(repr(float(scaling.high_freq_factor)))
    factor = Decimal(repr(float(scaling.factor)))
    wavelen = 2 * _PI / f
    if wavelen < w_orig / hi:
        return f
    if wavelen > w_orig / lo:
        return f / factor
    m = (w_orig / wavelen - lo) / (hi - lo)
    return (1 - m) * f / factor + m * f


def inv_freq(head_dim, base, scaling=None):
    """f_j = base ** (-2j / D) for j = 0 .. D/2 - 1 (then the optional
    frequency rule), rounded once to float64.

    Evaluated in 60-digit decimal arithmetic and then rounded, so the value is
    the float64 nearest the exact result on every machine (a vectorised
    float64 power is not correctly rounded on every CPU, and an ulp in f_j
    moves the angle pos * f_j by up to ~2e-12 at the positions used here).
    The values depend only on (D, base, scaling) and are memoised.
    """
    return _inv_freq(int(head_dim), float(base), scaling).copy()


@functools.lru_cache(maxsize=64)
def _inv_freq(head_dim, base, scaling):
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    with localcontext() as ctx:
        ctx.prec = 60
        b = Decimal(repr(float(base)))
        vals = []
        for j in range(head_dim // 2):
            f = b ** (Decimal(-2 * j) / Decimal(head_dim))
            if scaling is not None:
                f = scaled_frequency(f, scaling)
            vals.append(float(f))
    return np.array(vals, dtype=np.float64)


def rotation_factors(pos, head_dim, base, scaling=None):
    """exp(i * pos * f_j) as complex128, shape pos.shape + (D/2,)."""
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq(head_dim, base, scaling)
    w = np.empty(ang.shape, dtype=np.complex128)
    w.real = np.cos(ang)
    w.imag = np.sin(ang)
    return w


def pair_indices(head_dim, style=HALF_SPLIT):
    """(first, second) element index of each pair j = 0 .. D/2 - 1."""
    half = head_dim // 2
    j = np.arange(half)
    if style == HALF_SPLIT:
        return j, j + half
    if style == INTERLEAVED:
        return 2 * j, 2 * j + 1
    raise ValueError(f"unknown pairing {style!r}")


def rotate(x, pos, base, style=HALF_SPLIT, scaling=None):
    """Rotate float64 vectors x[..., D] to positions pos (broadcast to x[..., 0]).

    Returns float64 x' with x'[a_j] + i x'[b_j] = (x[a_j] + i x[b_j]) * exp(i pos f_j),
    (a_j, b_j) the pairs of the given style.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    first, second = pair_indices(d, style)
    w = rotation_factors(pos, d, base, scaling)
    z = np.empty(x.shape[:-1] + (d // 2,), dtype=np.complex128)
    z.real = x[..., first]
    z.imag = x[..., second]
    zr = z * w
    out = np.empty_like(x)
    out[..., first] = zr.real
    out[..., second] = zr.imag
    return out
