"""FP8 number formats, bit for bit — oracle (test infrastructure only).

The paper review "Training and inference of large language models using 8-bit
floating point", section "Proposed method", assigns the format with four
exponent bits to weights and activations and the one with five exponent bits
to gradients, without giving either format's bit layout.
The layouts below are those of the OCP 8-bit floating point specification
(OFP8): E4M3 ("FN": no infinities, one NaN mantissa pattern) and E5M2 (IEEE-
like, with infinities).  These are the encodings whose largest finite values
are 448 and 57344.

Everything here works on exact float64 values.  Decoding is the closed form of
the format definition; encoding is written as the rounding rule itself
(find the binade, form the quantum, round the quotient half-to-even), not as a
table lookup, so that a brute-force nearest-neighbour search over the 256
decoded codes can pin it independently.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Fp8Format:
    """Parameters of one OFP8 format.

    ``mbits`` mantissa bits, ``ebias`` exponent bias, ``emin`` the exponent of
    the smallest normal binade, ``emax`` the exponent of the largest finite
    binade, ``max`` the largest finite value, ``has_inf`` whether the all-ones
    exponent field encodes infinities (E5M2) or ordinary values (E4M3).
    """

    name: str
    code: int
    mbits: int
    ebits: int
    ebias: int
    emin: int
    emax: int
    max: float
    has_inf: bool


# OFP8: E4M3 has exponent bias 7; S.1111.111 is its only NaN pattern, so the
# top binade (field 15) still holds 256..448 and the largest finite value is
# 1.75 * 2**8 = 448.
E4M3 = Fp8Format("e4m3", 0, mbits=3, ebits=4, ebias=7, emin=-6, emax=8,
                 max=448.0, has_inf=False)
# OFP8: E5M2 has exponent bias 15; field 31 is Inf (mantissa 0) or NaN, so the
# largest finite value is 1.75 * 2**15 = 57344.
E5M2 = Fp8Format("e5m2", 1, mbits=2, ebits=5, ebias=15, emin=-14, emax=15,
                 max=57344.0, has_inf=True)

FORMATS = {0: E4M3, 1: E5M2, "e4m3": E4M3, "e5m2": E5M2}


def _fmt(fmt) -> Fp8Format:
    if isinstance(fmt, Fp8Format):
        return fmt
    return FORMATS[fmt]


# ---------------------------------------------------------------------------
# Input plumbing: bf16 / fp32 bit patterns to exact float64 values.
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values.

    A bfloat16 is the upper half of a float32, so widening is a 16-bit shift;
    float32 -> float64 is exact.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):        # NaN patterns widen to NaN
        return b.view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits) -> np.ndarray:
    """float32 bit patterns (uint32) -> exact float64 values."""
    with np.errstate(invalid="ignore"):
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """Round float64 values to bfloat16 by round-to-nearest-even (IEEE).

    Works on the exact float64 value (not via float32, which would round
    twice).  Overflow past the largest bf16 goes to +-Inf, as IEEE RNE does;
    NaN maps to a quiet NaN with the input's sign.
    """
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint16) << np.uint16(15)
    nan = np.isnan(v)
    isinf = np.isinf(v)
    a = np.abs(np.where(nan | isinf, 0.0, v))
    # bf16: 8 exponent bits (bias 127), 7 mantissa bits; smallest normal 2**-126.
    mant, exp = np.frexp(a)            # a = mant * 2**exp, mant in [0.5, 1)
    e = np.maximum(exp - 1, -126)      # binade exponent, subnormals share -126
    q = np.ldexp(1.0, e - 7)           # quantum of that binade
    n = np.rint(a / q)                 # exact quotient, RNE to an integer
    carry = n == 256.0
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 128.0, n)
    normal = n >= 128.0
    ef = np.where(normal, e + 127, 0)
    mf = np.where(normal, n - 128.0, n)
    inf = (ef >= 255) | isinf
    code = (ef.astype(np.int64) << 7) | mf.astype(np.int64)
    code = np.where(inf, 0x7F80, code)
    code = np.where(nan, 0x7FC0, code)
    return (code.astype(np.uint16) | sign).astype(np.uint16)


def bf16_ulp(v) -> np.ndarray:
    """Spacing of the bfloat16 grid in the binade of |v|: the distance from the
    largest bf16 value <= |v| to the next larger one.

    bfloat16 has 7 stored mantissa bits and the float32 exponent range, so the
    binade [2**e, 2**(e+1)) has spacing 2**(e - 7) for e >= -126; below 2**-126
    (zero included) the subnormals share the spacing 2**-133.  The largest
    finite binade is e = 127, which also stands for finite values beyond the
    largest bf16 (they round to Inf); NaN and Inf give NaN.
    """
    a = np.abs(np.asarray(v, dtype=np.float64))
    finite = np.isfinite(a)
    _, exp = np.frexp(np.where(finite, a, 1.0))    # a = mant * 2**exp, mant in [0.5, 1)
    e = np.where(a >= np.ldexp(1.0, -126), exp - 1, -126)   # zero and subnormals: -126
    e = np.minimum(e, 127)
    return np.where(finite, np.ldexp(1.0, e - 7), np.nan)


# ---------------------------------------------------------------------------
# FP8 decode: closed form of the OFP8 definition.
# ---------------------------------------------------------------------------

def decode(codes, fmt) -> np.ndarray:
    """FP8 codes (uint8) -> exact float64 values (OFP8 definition).

    For exponent field e and mantissa field m:
      e == 0            : (-1)^s * m * 2**(emin - mbits)          (subnormal)
      otherwise         : (-1)^s * (1 + m / 2**mbits) * 2**(e - ebias)
    E4M3: S.1111.111 is NaN.  E5M2: e == 31 is Inf (m == 0) or NaN.
    """
    f = _fmt(fmt)
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> f.mbits) & ((1 << f.ebits) - 1)
    m = c & ((1 << f.mbits) - 1)
    sub = np.ldexp(m.astype(np.float64), f.emin - f.mbits)
    nor = np.ldexp(1.0 + m.astype(np.float64) / (1 << f.mbits), e - f.ebias)
    mag = np.where(e == 0, sub, nor)
    top = (1 << f.ebits) - 1
    if f.has_inf:
        mag = np.where((e == top) & (m == 0), np.inf, mag)
        mag = np.where((e == top) & (m != 0), np.nan, mag)
    else:
        mag = np.where((e == top) & (m == (1 << f.mbits) - 1), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# ---------------------------------------------------------------------------
# FP8 encode: saturating round-to-nearest-even.
# ---------------------------------------------------------------------------

def encode(v, fmt) -> np.ndarray:
    """Exact float64 values -> FP8 codes by saturating round-to-nearest-even.

    Readings (the pages fix neither rounding nor overflow behaviour):
      * rounding is to nearest, ties to the even mantissa, on the full grid
        including subnormals;
      * the cast saturates: |v| > max (and +-Inf) gives +-max;
      * NaN gives 0x7F with the input's sign bit (a NaN code in both formats);
      * the sign is kept for zero and for values that round to zero.

    Steps, for a finite |v| <= max: take the binade exponent
    E = max(floor(log2|v|), emin); the grid spacing there is 2**(E - mbits);
    n = round_half_even(|v| / spacing) is the number of spacings; n * spacing
    is the result (n may carry into the next binade, which is representable).
    """
    f = _fmt(fmt)
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64)
    nan = np.isnan(v)
    a = np.abs(np.where(nan, 0.0, v))
    a = np.where(a > f.max, f.max, a)              # saturate (also +-Inf)
    _, exp = np.frexp(a)                           # a = mant * 2**exp, mant in [0.5,1)
    E = np.maximum(exp - 1, f.emin)                # floor(log2 a), or emin
    spacing = np.ldexp(1.0, E - f.mbits)
    n = np.rint(a / spacing)                       # division by 2**k is exact
    one = 1 << f.mbits
    carry = n == 2 * one
    E = np.where(carry, E + 1, E)
    n = np.where(carry, one, n).astype(np.int64)
    normal = n >= one
    efield = np.where(normal, E + f.ebias, 0)
    mfield = np.where(normal, n - one, n)
    code = (sign << 7) | (efield << f.mbits) | mfield
    code = np.where(nan, 0x7F | (sign << 7), code)
    return code.astype(np.uint8)
