"""GPU parity of delayed scaling (amax history -> window max -> bias -> cast
with fused amax -> push), step by step against the oracle's history, plus
checkpoint / resume of the history state."""

import numpy as np
import pytest
import torch

import oracle
import scaled_quantize_fp8_amd as sq
from oracle import E4M3
from workloads import make

from gpu_helpers import (DEV, bf16_dev, f32_bits_of, host, need_gpu, oracle_amax_chunked,
                         oracle_quantize_chunked, say)

pytestmark = pytest.mark.gpu
H = 16


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


class GpuDelayed:
    """The call sequence a delayed-scaled tensor goes through each step."""

    def __init__(self, window=H):
        self.hist = torch.empty(window, dtype=torch.float32, device=DEV)
        self.state = torch.empty(2, dtype=torch.int32, device=DEV)
        sq.fp8_history_init(self.hist, self.state)
        self.step = 0

    def cast(self, x, count_saturated=False):
        if self.step == 0:                       # bootstrap: own amax first
            sq.fp8_history_push(self.hist, self.state, sq.fp8_amax(x))
        bias, _, _ = sq.fp8_compute_scale_delayed(self.hist, self.state, E4M3.code, 0)
        sat = None
        if count_saturated:
            q, _, a, sat = sq.fp8_quantize_sat(x, E4M3.code, bias, want_amax=True)
        else:
            q, _, a = sq.fp8_quantize(x, E4M3.code, bias, want_amax=True)
        if self.step > 0:
            sq.fp8_history_push(self.hist, self.state, a)
        self.step += 1
        return (q, bias, a, sat) if count_saturated else (q, bias, a)


def _oracle_steps(xs):
    h = oracle.DelayedScaling(H)
    out = []
    for t, x in enumerate(xs):
        a = oracle.amax(x)
        if t == 0:
            h.push(a)
        b = h.bias(E4M3)
        q = oracle.quantize(x, E4M3, b)
        sat = int(np.count_nonzero(np.abs(np.ldexp(x, b)) > E4M3.max))
        if t > 0:
            h.push(a)
        out.append((q, b, a, sat))
    return out, h


def test_delayed_40_steps_with_rollover():
    steps = 40
    xs_bits = [make("c2", "X", step=t, shape=(256, 512)) for t in range(steps)]
    xs = [oracle.bf16_bits_to_f64(b) for b in xs_bits]
    ref, h = _oracle_steps(xs)
    g = GpuDelayed()
    sat_total = 0
    for t in range(steps):
        q, bias, a = g.cast(bf16_dev(xs_bits[t]))
        rq, rb, ra, sat = ref[t]
        assert int(host(bias)[0]) == rb, t
        assert host(a)[0] == ra, t
        assert np.array_equal(host(q), rq), t
        sat_total += sat
    hist, count, head = h.state()
    assert np.array_equal(host(g.hist), np.array(hist, dtype=np.float32))
    assert host(g.state).tolist() == [count, head]
    assert sat_total > 0          # the recipe's outliers and std jumps do saturate some steps


def test_history_checkpoint_resume():
    xs_bits = [make("c2", "X", step=t, shape=(128, 256)) for t in range(16)]
    g = GpuDelayed()
    for t in range(8):
        g.cast(bf16_dev(xs_bits[t]))
    saved = (g.hist.clone(), g.state.clone(), g.step)
    first = [g.cast(bf16_dev(xs_bits[t])) for t in range(8, 16)]
    g.hist.copy_(saved[0])
    g.state.copy_(saved[1])
    g.step = saved[2]
    second = [g.cast(bf16_dev(xs_bits[t])) for t in range(8, 16)]
    for (q1, b1, a1), (q2, b2, a2) in zip(first, second):
        assert torch.equal(q1, q2) and torch.equal(b1, b2) and f32_bits_of(a1) == f32_bits_of(a2)


def test_history_window_sizes():
    for window in (1, 3, 16, 64):
        g = GpuDelayed(window)
        h = oracle.DelayedScaling(window)
        rng = np.random.default_rng(window)
        for t in range(2 * window + 3):
            v = float(np.float32(np.exp(rng.uniform(-5, 5))))
            sq.fp8_history_push(g.hist, g.state, torch.tensor([v], dtype=torch.float32, device=DEV))
            h.push(v)
            b, _, _ = sq.fp8_compute_scale_delayed(g.hist, g.state, E4M3.code, 1)
            assert int(host(b)[0]) == h.bias(E4M3, 1)
    g = GpuDelayed(8)
    b, s, si = sq.fp8_compute_scale_delayed(g.hist, g.state, E4M3.code, 0)
    assert int(host(b)[0]) == 0 and host(s)[0] == 1.0


def test_delayed_full_size_7b_attn_16_steps():
    """X_t[2048 x 4096] over 16 steps, window 16 (the recipe's full size):
    bias and amax every step, every byte against the oracle, and the
    saturation the window's bias causes: the elements the GPU cast to the
    format maximum are exactly those the oracle casts there, and among them
    exactly the ones with |x 2^bias_t| > 448 are saturated.  The per-step
    bias and saturation count are logged."""
    g = GpuDelayed()
    h = oracle.DelayedScaling(H)
    log = []
    for t in range(16):
        bits = make("c2", "X", step=t)
        q, bias, a, gsat = g.cast(bf16_dev(bits), count_saturated=True)
        ra = oracle_amax_chunked(bits)
        if t == 0:
            h.push(ra)
        rb = h.bias(E4M3)
        if t > 0:
            h.push(ra)
        assert int(host(bias)[0]) == rb and host(a)[0] == ra
        gq = host(q)
        rq = oracle_quantize_chunked(bits, E4M3, rb)
        assert np.array_equal(gq, rq)
        at_max = (gq & 0x7F) == 0x7E
        assert np.array_equal(at_max, (rq & 0x7F) == 0x7E)
        scaled = np.abs(np.ldexp(oracle.bf16_bits_to_f64(bits), rb))
        sat = scaled > E4M3.max
        assert np.all(at_max[sat])                          # saturated -> the maximum code
        assert int(host(gsat)[0]) == int(np.count_nonzero(sat))   # the device count, exact
        log.append((t, rb, int(np.count_nonzero(sat))))
        say(f"delayed step {t}: bias {rb}, amax {ra:.4g}, saturated {log[-1][2]}")
    # the window lags a growing amax: some step saturates, step 0 never does
    assert log[0][2] == 0 and any(n > 0 for _, _, n in log)
