"""Scaling rules: amax, exponent bias, delayed history, per-tensor and per-block
quantization — oracle (test infrastructure only).

All arithmetic is exact: maxima involve no rounding, the bias is found with
integer exponent arithmetic, and ``x * 2**bias`` is exact in float64 for every
bf16/fp32 input and every bias used here.
"""

from __future__ import annotations

import numpy as np

from .formats import Fp8Format, _fmt, decode, encode

MX_BLOCK = 32           # elements per shared-scale block along the K axis
E8M0_BIAS = 127         # E8M0 code c stands for 2**(c - 127)
E8M0_NAN = 0xFF


def amax(x) -> float:
    """Per-tensor maximum absolute value.

    "Training and inference of large language models using 8-bit floating
    point" (paper review), "Proposed method": the per-tensor scaling bias is
    based on the largest absolute value in the tensor.  Taking a maximum
    rounds nothing.  Any NaN makes the result NaN; an empty tensor gives 0.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return 0.0
    return float(np.max(np.abs(x)))


def compute_bias(amax_value, fmt, margin: int = 0, lo: int = -126,
                 hi: int = 126):
    """Exponent bias from the tensor amax, as an integer (scalar or array).

    "Training and inference of large language models using 8-bit floating
    point" (paper review), "Proposed method": the bias comes from log2 of the
    ratio between the format's largest value and the tensor's amplitude, with
    a configurable margin.  The scale applied before the cast is 2**bias.

    Readings (the page gives words, not a formula):
      * log2 is rounded down: bias = floor(log2(fmax / amax)) - margin.  With
        margin 0 this is the largest power of two that keeps the scaled amax
        at or below the format maximum (no element saturates);
      * the margin is a non-negative integer subtracted from the bias;
      * amax == 0, Inf or NaN gives bias 0 (scale 1);
      * the result is clamped to [lo, hi]; [-126, 126] keeps 2**bias and
        2**-bias normal float32 numbers.

    floor(log2(fmax/amax)) is formed exactly: with amax = ma * 2**Ea and
    fmax = mf * 2**Ef (ma, mf in [1, 2)), log2(fmax/amax) = Ef - Ea +
    log2(mf/ma) and log2(mf/ma) lies in (-1, 1), so the floor is Ef - Ea when
    ma <= mf and Ef - Ea - 1 otherwise.
    """
    f = _fmt(fmt)
    a = np.abs(np.asarray(amax_value, dtype=np.float64))
    special = ~np.isfinite(a) | (a == 0.0)
    a = np.where(special, 1.0, a)
    mant_a, exp_a = np.frexp(a)            # a = mant * 2**exp, mant in [0.5, 1)
    mant_f, exp_f = np.frexp(f.max)
    b = (exp_f - exp_a) - (mant_a > mant_f).astype(np.int64) - int(margin)
    b = np.where(special, 0, b)
    b = np.clip(b, lo, hi).astype(np.int64)
    return int(b) if b.ndim == 0 else b


class DelayedScaling:
    """Amax history for delayed scaling.

    "Per-Tensor and Per-Block Scaling Strategies for Effective FP8 Training"
    (summary), "Key Questions Answered" and "Key Actionable Insights": the
    delayed scale is taken from the largest absolute values seen over a number
    of past iterations, which damps single-step outliers.

    Readings: the history is a ring of the last ``window`` raw per-step amaxes;
    the bias for a step is ``compute_bias`` of the maximum over the valid
    entries, which come from earlier steps only; the first step has no
    history, so the caller first pushes that step's own amax (so step 0 uses
    current scaling).  Before any push the window maximum is 0 (bias 0).
    """

    def __init__(self, window: int = 16):
        if window <= 0:
            raise ValueError("window must be positive")
        self.window = int(window)
        self.hist = [0.0] * self.window
        self.count = 0          # valid entries, saturating at window
        self.head = 0           # next slot to overwrite

    def push(self, a: float) -> None:
        self.hist[self.head] = float(a)
        self.head = (self.head + 1) % self.window
        self.count = min(self.count + 1, self.window)

    def window_max(self) -> float:
        if self.count == 0:
            return 0.0
        vals = self.hist[: self.count] if self.count < self.window else self.hist
        # max that propagates NaN, like the per-tensor amax
        return float(np.max(np.asarray(vals, dtype=np.float64)))

    def bias(self, fmt, margin: int = 0) -> int:
        return compute_bias(self.window_max(), fmt, margin)

    def state(self):
        return list(self.hist), self.count, self.head


def quantize(x, fmt, bias: int) -> np.ndarray:
    """Per-tensor cast: codes = encode(x * 2**bias).

    "Training and inference of large language models using 8-bit floating
    point" (paper review), "Proposed method": inputs are scaled before the
    FP8 cast.  ``x`` holds exact float64 values; ldexp is exact here.
    """
    x = np.asarray(x, dtype=np.float64)
    return encode(np.ldexp(x, int(bias)), fmt)


def dequantize(q, fmt, bias: int) -> np.ndarray:
    """Inverse scaling of a per-tensor cast: decode(q) * 2**-bias."""
    return np.ldexp(decode(q, fmt), -int(bias))


def mx_block_exponent(block_amax, fmt, rule: str = "fmax"):
    """Per-block exponent e_b and its E8M0 code for an array of block maxima.

    "Per-Tensor and Per-Block Scaling Strategies for Effective FP8 Training"
    (summary), "Key Questions Answered": micro-scaling divides a tensor into
    blocks, each with its own scaling factor.  The OCP MX specification stores
    such a factor as an E8M0 power of two, code c meaning 2**(c - 127).

    Readings: each block uses the per-tensor rule of ``compute_bias`` with
    margin 0 on its own maximum, clamped to [-127, 127]; the stored code is
    127 - e_b, so dequantization multiplies by 2**(code - 127) = 2**-e_b.  An
    all-zero (or Inf) block gets e_b = 0, code 127; a block holding a NaN gets
    code 0xFF (the E8M0 NaN) and its elements are cast with e_b = 0.

    The option ``rule="ocp"`` follows the OCP MX shared-exponent rule
    instead: the block's scale exponent is floor(log2 amax) minus the
    exponent of the element format's largest binade, i.e. e_b = emax -
    floor(log2 amax), so the block maximum lands in the largest binade and,
    when its significand exceeds the format maximum's (1.75), saturates.
    The conventions for zero, Inf, NaN and the clamp are the same.
    """
    a = np.asarray(block_amax, dtype=np.float64)
    if rule == "fmax":
        e = np.asarray(compute_bias(a, fmt, 0, lo=-127, hi=127), dtype=np.int64)
    elif rule == "ocp":
        fmt = _fmt(fmt)
        finite = np.isfinite(a) & (a > 0)
        _, ex = np.frexp(np.where(finite, a, 1.0))          # a = m 2^ex, 0.5 <= m < 1
        e = np.where(finite, fmt.emax - (ex.astype(np.int64) - 1), 0)
        e = np.clip(e, -127, 127).astype(np.int64)
    else:
        raise ValueError("rule must be 'fmax' or 'ocp'")
    codes = (E8M0_BIAS - e).astype(np.int64)
    codes = np.where(np.isnan(a), E8M0_NAN, codes).astype(np.uint8)
    return e, codes


def mx_quantize(x, fmt=0, rule: str = "fmax"):
    """Per-block cast with 1 x 32 blocks along the last (K) axis.

    Returns (codes[R, C], scales[R, C/32]) with scales as E8M0 codes; `rule`
    picks the block exponent rule of ``mx_block_exponent``.
    Reading: blocks run along the contiguous K axis, which is the reduction
    axis of both GEMM operands, and C must be a multiple of 32.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] % MX_BLOCK:
        raise ValueError("mx_quantize needs a 2-D array with cols % 32 == 0")
    r, c = x.shape
    blocks = x.reshape(r, c // MX_BLOCK, MX_BLOCK)
    if blocks.size:
        bmax = np.max(np.abs(blocks), axis=2)
    else:
        bmax = np.zeros((r, c // MX_BLOCK))
    e, codes = mx_block_exponent(bmax, fmt, rule)
    q = encode(np.ldexp(blocks, e[:, :, None]), fmt).reshape(r, c)
    return q, codes


def mx_dequantize(q, scales, fmt=0) -> np.ndarray:
    """decode(q) * 2**(code - 127) per block; code 0xFF decodes to NaN."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8).astype(np.int64)
    r, c = q.shape
    vals = decode(q, fmt).reshape(r, c // MX_BLOCK, MX_BLOCK)
    mult = np.ldexp(1.0, s - E8M0_BIAS)
    mult = np.where(s == E8M0_NAN, np.nan, mult)
    return (vals * mult[:, :, None]).reshape(r, c)
