"""The bias-sweep harness: its host decode table against the oracle's decode
(CPU), and its per-bias RMSE / clipped / flushed figures against the
oracle's cast of the same tensor (GPU)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2
from scaled_quantize_fp8_amd.sweep import bias_sweep, decode_table
from workloads import make

from gpu_helpers import bf16_dev, need_gpu, say


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_decode_table_matches_oracle(fmt):
    codes = np.arange(256, dtype=np.uint8)
    ref = oracle.decode(codes, fmt)
    got = decode_table(fmt.code)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_sweep_refuses_cpu_tensors():
    with pytest.raises(ValueError):
        bias_sweep(torch.zeros(4, 4, dtype=torch.bfloat16))


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_bias_sweep_matches_oracle(fmt):
    """N(0,1) x 64 at the 256 x 768 layer shape (amax ~ 300): E4M3 clips from
    bias 1 up, the sweep spans clipping and flushing biases."""
    need_gpu()
    bits = make("c1", "X")
    vals = oracle.bf16_bits_to_f64(bits) * 64.0
    x = bf16_dev(bits) * 64
    biases = range(-12, 5, 4) if fmt is E4M3 else range(-20, 9, 7)
    say(f"bias sweep {fmt.name}")
    res = bias_sweep(x, fmt.code, biases)
    assert res["amax_bias"] == oracle.compute_bias(oracle.amax(vals), fmt)
    for row in res["rows"]:
        b = row["bias"]
        q = oracle.quantize(vals, fmt, b)
        deq = oracle.dequantize(q, fmt, b)
        assert row["rmse"] == pytest.approx(oracle.rmse(vals, deq), rel=1e-12)
        assert row["clipped"] == int(np.count_nonzero(np.abs(np.ldexp(vals, b)) > fmt.max))
        assert row["flushed"] == int(np.count_nonzero((vals != 0) & ((q & 0x7F) == 0)))
    assert any(r["clipped"] for r in res["rows"]) and any(r["flushed"] for r in res["rows"])
