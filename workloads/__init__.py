"""Seeded synthetic inputs for the scaled FP8 linear layer.

This module only draws random numbers and rounds them to bfloat16 bit
patterns.  It holds none of the method's arithmetic (no amax, no scale, no
FP8 cast) and is the one module that both the CPU oracle's tests and the GPU
path's tests and benchmark use, so that both sides read the same bf16 bits.

Workloads are Llama-2-sized linear layers (7B attention projection, 7B MLP,
13B MLP up-projection, 70B MLP) with the value distributions the layer sees:
Gaussian weights, Gaussian activations with rare large outliers, heavy-tailed
gradients, and activations whose columns (K channels) differ widely in scale.
No dataset is involved; these synthetic tensors stand in for real activations,
weights and gradients.

Random streams: NumPy ``Generator(PCG64)`` seeded with
``SeedSequence([seed, config_id, tensor_id, step])``.  Values are drawn in
float32 (Student-t in float64, then narrowed) and rounded to bf16 by
round-to-nearest-even.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TENSOR_IDS = {"X": 0, "W": 1, "dY": 2}


def rng_for(config_id: int, tensor: str, step: int = 0, seed: int = 0):
    ss = np.random.SeedSequence([seed, config_id, TENSOR_IDS[tensor], step])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns, ties to even.

    Input preparation only: the layer's inputs are bf16 tensors, and the
    generators produce them from float32 draws.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def gaussian(rng, shape, std=1.0) -> np.ndarray:
    """bf16 bits of std * N(0, 1)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def gaussian_outliers(rng, shape, std=1.0, p=0.001, factor=50.0) -> np.ndarray:
    """bf16 bits of std * N(0,1), with a Bernoulli(p) mask of entries
    multiplied by ``factor`` (rare large activations)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    mask = rng.random(size=shape, dtype=np.float32) < np.float32(p)
    x[mask] *= np.float32(factor)
    return f32_to_bf16_bits(x)


def student_t(rng, shape, nu=3.0, scale=1e-4) -> np.ndarray:
    """bf16 bits of scale * StudentT(nu) (heavy-tailed gradients)."""
    x = (rng.standard_t(nu, size=shape) * scale).astype(np.float32)
    return f32_to_bf16_bits(x)


def column_lognormal(rng, shape, sigma=1.5) -> np.ndarray:
    """bf16 bits of s_j * N(0,1) with s_j = exp(sigma * N(0,1)) per column j
    (per-channel activation scales along K)."""
    s = np.exp(sigma * rng.standard_normal(size=(1, shape[1]))).astype(np.float32)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= s
    return f32_to_bf16_bits(x)


def log_uniform_std(rng, lo=0.5, hi=4.0) -> float:
    return float(np.exp(rng.uniform(np.log(lo), np.log(hi))))


@dataclass
class Config:
    """One workload: shapes, value recipe and the steps it exercises."""

    cid: int
    name: str
    description: str
    shapes: dict = field(default_factory=dict)


CONFIGS = {
    "c1": Config(1, "current_scaling_256x768x768",
                 "per-tensor current scaling; X[256x768] ~ N(0,1), "
                 "W[768x768] ~ 0.02 N(0,1); E4M3; Y = X W^T, bf16 out",
                 {"X": (256, 768), "W": (768, 768)}),
    "c2": Config(2, "delayed_scaling_llama2_7b_attn_2048x4096x4096",
                 "delayed scaling over 16 steps, window 16; X_t[2048x4096] ~ "
                 "sigma_t N(0,1), sigma_t log-uniform in [0.5, 4], 0.1% of "
                 "entries x50; W[4096x4096] ~ 0.02 N(0,1); E4M3",
                 {"X": (2048, 4096), "W": (4096, 4096), "steps": 16}),
    "c3": Config(3, "backward_mixed_llama2_7b_mlp",
                 "dY[4096x11008] ~ 1e-4 StudentT(3) -> E5M2; W[11008x4096] ~ "
                 "0.02 N(0,1), X[4096x4096] ~ N(0,1) -> E4M3; dX = dY W, "
                 "dW = dY^T X",
                 {"dY": (4096, 11008), "W": (11008, 4096), "X": (4096, 4096)}),
    "c4": Config(4, "mxfp8_llama2_13b_mlp_up_8192x13824x5120",
                 "X[8192x5120] ~ s_j N(0,1), s_j = exp(1.5 N(0,1)) per column; "
                 "W[13824x5120] ~ 0.02 N(0,1); 1x32 blocks, E8M0, E4M3",
                 {"X": (8192, 5120), "W": (13824, 5120)}),
    "c5": Config(5, "llama2_70b_mlp_16384x28672x8192",
                 "X[16384x8192] ~ N(0,1) with 0.05% of entries x100; "
                 "W[28672x8192] ~ 0.015 N(0,1); per-tensor E4M3 and MXFP8",
                 {"X": (16384, 8192), "W": (28672, 8192)}),
}


def make(config: str, tensor: str, step: int = 0, shape=None, seed: int = 0):
    """bf16 bit patterns (uint16 [rows, cols]) of one workload tensor.

    ``shape`` overrides the workload's full shape (same distribution, smaller
    tensor) for fast parity cases.
    """
    cfg = CONFIGS[config]
    shp = tuple(shape) if shape is not None else cfg.shapes[tensor]
    rng = rng_for(cfg.cid, tensor, step, seed)
    if config == "c1":
        return gaussian(rng, shp, 1.0 if tensor == "X" else 0.02)
    if config == "c2":
        if tensor == "X":
            std = log_uniform_std(rng)
            return gaussian_outliers(rng, shp, std=std, p=0.001, factor=50.0)
        return gaussian(rng, shp, 0.02)
    if config == "c3":
        if tensor == "dY":
            return student_t(rng, shp, nu=3.0, scale=1e-4)
        return gaussian(rng, shp, 0.02 if tensor == "W" else 1.0)
    if config == "c4":
        if tensor == "X":
            return column_lognormal(rng, shp, sigma=1.5)
        return gaussian(rng, shp, 0.02)
    if config == "c5":
        if tensor == "X":
            return gaussian_outliers(rng, shp, std=1.0, p=0.0005, factor=100.0)
        return gaussian(rng, shp, 0.015)
    raise KeyError(config)


def all_bf16_patterns() -> np.ndarray:
    """Every one of the 65,536 bf16 bit patterns, in order."""
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)
