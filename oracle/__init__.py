"""CPU oracle for the scaled FP8 linear layer — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct statement of what the GPU
path computes.  It is written in NumPy with float64 arithmetic and exact integer
exponent handling, and it shares no code, table or constant with the HIP
library under ``scaled_quantize_fp8_amd``.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it;
the product path never does.

Sources it follows (cited per function):

* "Training and inference of large language models using 8-bit floating
  point" (paper review page), section "Proposed method": per-tensor scaling
  biases from each tensor's maximum absolute value; a bias taken from log2 of
  the ratio between the format maximum and the tensor's amplitude, with a
  configurable margin; scaling before the FP8 cast and unscaling after the
  matrix multiplication; FP8_E4 for weights and activations, FP8_E5 for
  gradients.
* "Per-Tensor and Per-Block Scaling Strategies for Effective FP8 Training"
  (summary page), sections "Key Questions Answered" and "Key Actionable
  Insights": delayed scaling from maxima observed over several past
  iterations; per-block (MXFP8) scaling with one scale per block.
* The OCP 8-bit floating point specification (OFP8) for the E4M3 and E5M2 bit
  layouts, and the OCP Microscaling (MX) specification for the E8M0 shared
  block scale.  The pages name the formats but do not define their bits.

Readings of points the pages leave open (rounding, saturation, NaN/Inf/-0
conventions, floor in the bias rule, the history window, block size and axis)
are stated in the docstring of the function that applies them.

Parity status: every function here is pinned by CPU tests to something other
than itself (library casts, brute force, closed forms, exact rational
arithmetic).  The NaN conventions (NaN -> 0x7F|sign, NaN block -> E8M0 0xFF)
are conventions the pages do not fix: parity unpinned for NaN payloads.
"""

from .formats import (
    E4M3, E5M2, FORMATS, Fp8Format,
    bf16_bits_to_f64, f32_bits_to_f64, decode, encode, f64_to_bf16_bits,
    bf16_ulp,
)
from .scaling import (
    amax, compute_bias, DelayedScaling, quantize, mx_block_exponent,
    mx_quantize, mx_dequantize, dequantize,
)
from .gemm import (
    scaled_gemm_ref, mx_gemm_ref, abs_product_sum, mx_abs_product_sum,
    rmse, gemm_sample_ref, mx_gemm_sample_ref,
)

__all__ = [
    "E4M3", "E5M2", "FORMATS", "Fp8Format",
    "bf16_bits_to_f64", "f32_bits_to_f64", "decode", "encode",
    "f64_to_bf16_bits", "bf16_ulp",
    "amax", "compute_bias", "DelayedScaling", "quantize",
    "mx_block_exponent", "mx_quantize", "mx_dequantize", "dequantize",
    "scaled_gemm_ref", "mx_gemm_ref", "abs_product_sum",
    "mx_abs_product_sum", "rmse", "gemm_sample_ref", "mx_gemm_sample_ref",
]
