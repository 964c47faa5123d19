"""Reference GEMMs on FP8 operands, computed in float64 — oracle (test
infrastructure only).

"Training and inference of large language models using 8-bit floating point"
(paper review), "Proposed method": the FP8 matrix multiplication runs on the
scaled, cast operands and the result is unscaled afterwards.  The GPU path
accumulates in float32 and stores bf16 or float32; this reference forms the
same sum of products in float64 from the decoded operands.

Exactness: an E4M3 x E4M3 product is an integer (at most 225 * 2**28) times
2**-18, so every partial sum over K < 2**17 terms is an exact float64 and the
reference is exact in any summation order.  With E5M2 operands or per-block
scales the float64 sum can round, by at most about 1e-16 relative to the sum
of absolute products.

Layout convention: ``qa`` is op(A) as [M, K] codes and ``qb`` is op(B) as
[N, K] codes, so Y = op(A) . op(B)^T (K is the last axis of both).  Callers
transpose stored [K, M] / [K, N] operands on the host first.
"""

from __future__ import annotations

import numpy as np

from .formats import decode
from .scaling import mx_dequantize

_PANEL = 512            # rows of Y formed per matmul call (bounds host memory)


def _panels(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    m = a.shape[0]
    out = np.empty((m, b.shape[0]), dtype=np.float64)
    bt = np.ascontiguousarray(b.T)
    for r0 in range(0, m, _PANEL):
        out[r0:r0 + _PANEL] = a[r0:r0 + _PANEL] @ bt
    return out


def scaled_gemm_ref(qa, fmt_a, bias_a: int, qb, fmt_b, bias_b: int) -> np.ndarray:
    """Y[m, n] = 2**-(bias_a + bias_b) * sum_k dec(qa[m, k]) * dec(qb[n, k]).

    The unscale by 2**-(bias_a + bias_b) is a power of two, hence exact.
    """
    a = decode(qa, fmt_a)
    b = decode(qb, fmt_b)
    return np.ldexp(_panels(a, b), -(int(bias_a) + int(bias_b)))


def abs_product_sum(qa, fmt_a, bias_a: int, qb, fmt_b, bias_b: int) -> np.ndarray:
    """S[m, n] = sum_k |a[m, k] * b[n, k]| with a, b the dequantized operands
    (scales included); the GEMM tolerance is stated relative to it."""
    a = np.abs(np.ldexp(decode(qa, fmt_a), -int(bias_a)))
    b = np.abs(np.ldexp(decode(qb, fmt_b), -int(bias_b)))
    return _panels(a, b)


def mx_gemm_ref(qa, sa, fmt_a, qb, sb, fmt_b) -> np.ndarray:
    """Block-scaled GEMM: Y[m, n] = sum_j 2**(sa[m,j]-127) * 2**(sb[n,j]-127)
    * sum_{k in block j} dec(qa[m,k]) * dec(qb[n,k]).

    Written as the product of the two dequantized operands; every term
    dec(qa)*2**(sa-127) * dec(qb)*2**(sb-127) is exact in float64, so this is
    the same sum of the same terms.
    """
    a = mx_dequantize(qa, sa, fmt_a)
    b = mx_dequantize(qb, sb, fmt_b)
    return _panels(a, b)


def mx_abs_product_sum(qa, sa, fmt_a, qb, sb, fmt_b) -> np.ndarray:
    a = np.abs(mx_dequantize(qa, sa, fmt_a))
    b = np.abs(mx_dequantize(qb, sb, fmt_b))
    return _panels(a, b)


def gemm_sample_ref(qa, fmt_a, bias_a, qb, fmt_b, bias_b, rows, cols):
    """Selected outputs Y[rows[i], cols[i]] one by one (for full-size checks).

    Returns (y, s): the reference values and the matching sums of absolute
    products.  Each is a K-long dot product in float64.
    """
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    y = np.empty(rows.size)
    s = np.empty(rows.size)
    scale = np.ldexp(1.0, -(int(bias_a) + int(bias_b)))
    for i, (r, c) in enumerate(zip(rows.tolist(), cols.tolist())):
        prod = decode(qa[r], fmt_a) * decode(qb[c], fmt_b)
        y[i] = np.sum(prod) * scale
        s[i] = np.sum(np.abs(prod)) * scale
    return y, s


def mx_gemm_sample_ref(qa, sa, fmt_a, qb, sb, fmt_b, rows, cols):
    """Selected outputs of the block-scaled GEMM one by one; returns (y, s)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    y = np.empty(rows.size)
    s = np.empty(rows.size)
    for i, (r, c) in enumerate(zip(rows.tolist(), cols.tolist())):
        a = mx_dequantize(qa[r:r + 1], sa[r:r + 1], fmt_a)[0]
        b = mx_dequantize(qb[c:c + 1], sb[c:c + 1], fmt_b)[0]
        prod = a * b
        y[i] = np.sum(prod)
        s[i] = np.sum(np.abs(prod))
    return y, s


def rmse(x, xhat) -> float:
    """Root-mean-square quantization error sqrt(mean((xhat - x)**2)) in float64."""
    x = np.asarray(x, dtype=np.float64)
    xhat = np.asarray(xhat, dtype=np.float64)
    if x.size == 0:
        return 0.0
    return float(np.sqrt(np.mean((xhat - x) ** 2)))
