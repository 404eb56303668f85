"""bfloat16 <-> float64, written from the format's definition.

bfloat16 is the top half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits
(bias 127) and 7 stored fraction bits, i.e. 8 significant bits for normal
numbers and a fixed quantum of 2**-133 below 2**-126 (subnormals).

The pages require nothing beyond "bf16" (the InferScale review's "Significance"
paragraph and "minor comments" item 3 mention bf16 equivalence).  The oracle
therefore rounds each exact (float64) result ONCE to the nearest bfloat16,
ties to even; there is no intermediate float32 rounding.
"""

import numpy as np

# Smallest positive normal bfloat16 and the subnormal quantum.
_MIN_NORMAL = 2.0 ** -126
_SUB_QUANTUM_EXP = -133


def bf16_bits_to_f64(bits):
    """Exact value of bfloat16 bit patterns (any integer dtype holding 16 bits)."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    as32 = (b.astype(np.uint32) << np.uint32(16))
    with np.errstate(invalid="ignore"):
        return as32.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round float64 values to bfloat16 bit patterns, nearest, ties to even.

    Normal range: write x = m * 2**e with 0.5 <= |m| < 1 (frexp); the 8
    significant bits are rint(m * 2**8), where rint rounds half to even.  The
    rounded value rint(m*2**8) * 2**(e-8) is exactly representable, so the
    final conversion to float32 (to read off its top 16 bits) is exact; a
    result of 2**128 becomes +-inf, which is the correct overflow.
    Subnormal range: the quantum is 2**-133, so round x * 2**133 to an integer.
    NaN stays NaN (quiet), +-inf stay +-inf, -0.0 keeps its sign.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        m, e = np.frexp(x)
        r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
        sub = np.abs(x) < _MIN_NORMAL
        r_sub = np.ldexp(np.rint(np.ldexp(x, -_SUB_QUANTUM_EXP)), _SUB_QUANTUM_EXP)
        r = np.where(sub, r_sub, r)
        r = np.where(np.isfinite(x), r, x)
        f = r.astype(np.float32)
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits


def ulp_distance(a_bits, b_bits):
    """Distance in bfloat16 units in the last place between two bit patterns.

    Patterns are mapped to a monotone integer line, ord(x) = -(x & 0x7FFF) if
    the sign bit is set, else x & 0x7FFF, so +0 and -0 coincide and adjacent
    representable values differ by one.
    """
    def _ord(bits):
        b = np.asarray(bits).astype(np.int64) & 0xFFFF
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)

    return np.abs(_ord(a_bits) - _ord(b_bits))
