"""fp8_amax_scale_noalloc — the entry point that allocates nothing (its
reduction state is the library's static per-GPU array) — against
fp8_amax_scale with a caller workspace, through the C ABI: two calls in a
row, the second on a smaller input, must give the same amax, bias and scales
bit for bit; so must a third call back on the first input."""

import numpy as np
import pytest
import torch

import scaled_quantize_fp8_amd as sq
from gpu_helpers import DEV, f32_bits_of, host, need_gpu, say

pytestmark = pytest.mark.gpu


def _bits(outs):
    a, b, s, si = outs
    return f32_bits_of(a), int(host(b)[0]), f32_bits_of(s), f32_bits_of(si)


def test_amax_scale_noalloc_matches_workspace_entry_point():
    need_gpu()
    g = torch.Generator(device=DEV).manual_seed(77)
    big = torch.randn(8192, 4096, device=DEV, dtype=torch.bfloat16, generator=g) * 3
    big.view(-1)[123457] = -1234.0
    small = torch.randn(300, 200, device=DEV, dtype=torch.float32, generator=g)[:, 5:197]   # strided, f32
    ws = sq.amax_scale_workspace(DEV)
    for i, (x, fmt, margin) in enumerate(((big, sq.E4M3, 0), (small, sq.E5M2, 1), (big, sq.E4M3, 2))):
        say(f"noalloc amax_scale call {i}: shape {tuple(x.shape)} {x.dtype}")
        got = _bits(sq.fp8_amax_scale_noalloc(x, fmt, margin, want_scales=True))
        want = _bits(sq.fp8_amax_scale(x, fmt, ws, margin, want_scales=True))
        assert got == want, (i, got, want)
        ref_a = float(x.float().abs().max())
        assert np.float32(ref_a).view(np.uint32) == np.uint32(got[0])
