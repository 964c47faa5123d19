"""Exponent-bias sweep of the per-tensor cast, the harness behind a fixed-
scaling study: "Training and inference of large language models using
8-bit floating point" (paper review page), "Research questions" and "Key
findings", compare one fixed bias for all tensors (FP8-CSCALE, which for the
13B model converges only for biases in [-1, 0]) with the amax-derived one
(FP8-AMAX).  For each bias the GPU casts the tensor; the host then reports,
from the returned codes, how far the dequantized tensor is from the input
(RMSE), how many elements were clipped to the format maximum and how many
nonzero elements were flushed to zero, next to the bias FP8-AMAX would pick.
"""

from __future__ import annotations

import numpy as np
import torch

from . import E4M3, E5M2, fp8_amax, fp8_compute_scale, fp8_quantize

# (exponent bits, mantissa bits, exponent bias, max finite value) per format
_FORMATS = {E4M3: (4, 3, 7, 448.0), E5M2: (5, 2, 15, 57344.0)}


def decode_table(fmt) -> np.ndarray:
    """float64 value of each of the 256 codes of an OCP 8-bit format (NaN
    codes decode to NaN, E5M2's 0x7C / 0xFC to +-Inf)."""
    ebits, mbits, ebias, _ = _FORMATS[fmt]
    codes = np.arange(256)
    sign = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> mbits) & ((1 << ebits) - 1)
    m = codes & ((1 << mbits) - 1)
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), 1 - ebias - mbits),
                   np.ldexp(1.0 + m / float(1 << mbits), e - ebias))
    if fmt == E4M3:
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
    else:
        mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def bias_sweep(x: torch.Tensor, fmt=E4M3, biases=range(-3, 4)):
    """Cast x (2-D bf16 / f32 device tensor) with every bias in `biases`.

    Returns {"amax_bias": the FP8-AMAX bias of x, "rows": [{"bias", "rmse",
    "clipped", "flushed"}, ...]} where rmse = sqrt(mean((dequant(q) - x)^2))
    with dequant(q) = decode(q) * 2^-bias, clipped counts |x * 2^bias| >
    max, flushed counts x != 0 whose code is +-0."""
    _, _, _, fmax = _FORMATS[fmt]
    table = decode_table(fmt)
    xv = x.detach().float().cpu().numpy().astype(np.float64)
    ab, _, _ = fp8_compute_scale(fp8_amax(x), fmt, 0)
    bias_dev = torch.empty(1, dtype=torch.int32, device=x.device)
    rows = []
    for b in biases:
        bias_dev.fill_(int(b))
        q, _, _ = fp8_quantize(x, fmt, bias_dev)
        codes = q.cpu().numpy()
        deq = np.ldexp(table[codes], -int(b))
        rows.append({"bias": int(b),
                     "rmse": float(np.sqrt(np.mean((deq - xv) ** 2))),
                     "clipped": int(np.count_nonzero(np.abs(np.ldexp(xv, int(b))) > fmax)),
                     "flushed": int(np.count_nonzero((xv != 0) & ((codes & 0x7F) == 0)))})
    return {"amax_bias": int(ab.cpu().numpy()[0]), "rows": rows}
