"""GPU parity of delayed scaling (amax history -> window max -> bias -> cast
with fused amax -> push), step by step against the oracle's history, plus
checkpoint / resume of the history state, and the same step in one launch
(fp8_quantize_delayed) against the call sequence and the oracle."""

import numpy as np
import pytest
import torch

import oracle
import scaled_quantize_fp8_amd as sq
from oracle import E4M3
from workloads import f32_to_bf16_bits, make

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


def _f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


# (name, dtype, shape, transpose, strided view, fmt code, margin): the fused
# row-wise kernel (vector and element paths), the fused cast-transpose
# (16-byte aligned bf16) and the three-call form for other transposed inputs
FUSED_CASES = [
    ("bf16_rows", "bf16", (256, 512), False, False, 0, 0),
    ("bf16_transpose", "bf16", (384, 320), True, False, 0, 0),
    ("bf16_transpose_ragged_e5m2", "bf16", (200, 136), True, False, 1, 1),
    ("bf16_strided_rows", "bf16", (130, 301), False, True, 0, 0),
    ("f32_rows_e5m2", "f32", (96, 1000), False, False, 1, 2),
    ("f32_transpose", "f32", (160, 96), True, False, 0, 0),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_quantize_delayed_matches_three_calls(case):
    """fp8_quantize_delayed (bias from the window, cast, push in one launch)
    against fp8_compute_scale_delayed + fp8_quantize_sat + fp8_history_push on
    a second copy of the history, 20 steps with window 16 (the ring wraps):
    codes, transposed codes, bias, amax and saturation count bit for bit
    every step, the same window and state after every step, and the
    workspace back to zero; the biases and counts also against the oracle's
    history."""
    name, dt, shape, transpose, strided, fmt_code, margin = case
    fmt = oracle.E4M3 if fmt_code == 0 else oracle.E5M2
    rng = np.random.default_rng(hash(name) % 2**32)
    ha = torch.empty(H, dtype=torch.float32, device=DEV)
    sa = torch.empty(2, dtype=torch.int32, device=DEV)
    sq.fp8_history_init(ha, sa)
    hb, sb = ha.clone(), sa.clone()
    ws = sq.amax_scale_workspace(DEV)
    h = oracle.DelayedScaling(H)
    for t in range(20):
        sigma = float(np.exp(rng.uniform(-3, 3)))
        v = rng.standard_normal(shape) * sigma
        v[rng.random(shape) < 0.002] *= 60.0                       # outliers that jump past the window
        if dt == "bf16":
            bits = f32_to_bf16_bits(v.astype(np.float32))
            vals = oracle.bf16_bits_to_f64(bits)
            x = bf16_dev(bits)
        else:
            vals = v.astype(np.float32).astype(np.float64)
            x = _f32_dev(v)
        if strided:
            x = x[:, 1:]
            vals = vals[:, 1:]
        if t == 0:                                                 # bootstrap both copies and the oracle
            a0 = sq.fp8_amax(x)
            sq.fp8_history_push(ha, sa, a0)
            sq.fp8_history_push(hb, sb, a0)
            h.push(oracle.amax(vals))
        q1, qT1, b1, a1, n1 = sq.fp8_quantize_delayed(x, fmt.code, ha, sa, ws, margin, transpose=transpose,
                                                      want_sat=True)
        b2, _, _ = sq.fp8_compute_scale_delayed(hb, sb, fmt.code, margin)
        q2, qT2, a2, n2 = sq.fp8_quantize_sat(x, fmt.code, b2, transpose=transpose, want_amax=True)
        sq.fp8_history_push(hb, sb, a2)
        rb = h.bias(fmt, margin)
        what = f"{name} step {t}"
        assert int(host(b1)[0]) == int(host(b2)[0]) == rb, what
        assert f32_bits_of(a1) == f32_bits_of(a2), what
        assert host(a1)[0] == oracle.amax(vals), what
        assert int(host(n1)[0]) == int(host(n2)[0]), what
        assert int(host(n1)[0]) == int(np.count_nonzero(np.abs(np.ldexp(vals, rb)) > fmt.max)), what
        assert torch.equal(q1, q2), what
        if transpose:
            assert torch.equal(qT1, qT2), what
        assert torch.equal(ha, hb) and torch.equal(sa, sb), what
        assert not host(ws).any(), what
        h.push(oracle.amax(vals))


def test_quantize_delayed_empty_and_empty_window():
    """An empty tensor still takes the window's bias and pushes amax 0, as
    the three calls do; an empty window gives bias 0 (the cast is then
    current-scaled only after the caller's bootstrap push)."""
    ws = sq.amax_scale_workspace(DEV)
    hist = torch.empty(4, dtype=torch.float32, device=DEV)
    state = torch.empty(2, dtype=torch.int32, device=DEV)
    sq.fp8_history_init(hist, state)
    x = bf16_dev(f32_to_bf16_bits(np.full((64, 96), 3.0, dtype=np.float32)))
    _, _, b, a, _ = sq.fp8_quantize_delayed(x, E4M3.code, hist, state, ws)
    assert int(host(b)[0]) == 0 and host(a)[0] == 3.0               # empty window: bias 0
    assert host(state).tolist() == [1, 1] and host(hist)[0] == 3.0
    empty = torch.zeros((0, 96), dtype=torch.bfloat16, device=DEV)
    _, _, b, a, n = sq.fp8_quantize_delayed(empty, E4M3.code, hist, state, ws, want_sat=True)
    assert int(host(b)[0]) == oracle.compute_bias(3.0, E4M3) and host(a)[0] == 0.0 and int(host(n)[0]) == 0
    assert host(state).tolist() == [2, 2] and host(hist)[1] == 0.0
    assert not host(ws).any()


def test_quantize_delayed_full_size_7b_attn_16_steps():
    """The delayed-scaling workload at full size (X_t [2048 x 4096], window
    16), cast with its transposed copy as the linear layer does, in one
    launch per step: bias, amax, saturation count and every byte of q and qT
    against the oracle."""
    hist = torch.empty(H, dtype=torch.float32, device=DEV)
    state = torch.empty(2, dtype=torch.int32, device=DEV)
    sq.fp8_history_init(hist, state)
    ws = sq.amax_scale_workspace(DEV)
    h = oracle.DelayedScaling(H)
    for t in range(16):
        bits = make("c2", "X", step=t)
        x = bf16_dev(bits)
        ra = oracle_amax_chunked(bits)
        if t == 0:
            sq.fp8_history_push(hist, state, sq.fp8_amax(x))
            h.push(ra)
        rb = h.bias(E4M3)
        q, qT, b, a, n = sq.fp8_quantize_delayed(x, E4M3.code, hist, state, ws, transpose=True, want_sat=True)
        h.push(ra)
        assert int(host(b)[0]) == rb and host(a)[0] == ra, t
        rq = oracle_quantize_chunked(bits, E4M3, rb)
        gq = host(q)
        assert np.array_equal(gq, rq), t
        assert np.array_equal(host(qT), rq.T), t
        sat = int(np.count_nonzero(np.abs(np.ldexp(oracle.bf16_bits_to_f64(bits), rb)) > E4M3.max))
        assert int(host(n)[0]) == sat, t
        say(f"fused delayed step {t}: bias {rb}, saturated {sat}")
    hist_ref, count, head = h.state()
    assert np.array_equal(host(hist), np.array(hist_ref, dtype=np.float32))
    assert host(state).tolist() == [count, head]
