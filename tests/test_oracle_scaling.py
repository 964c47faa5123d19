"""Pins for the oracle's amax, bias rule, delayed history and per-tensor /
per-block quantization (CPU only)."""

import numpy as np
import pytest

import oracle
from oracle import E4M3, E5M2, compute_bias, decode, encode
from oracle.scaling import MX_BLOCK
from workloads import all_bf16_patterns, make

FMTS = [E4M3, E5M2]


def _bruteforce_bias(a, fmax, margin, lo=-126, hi=126):
    """Largest integer e with a * 2**e <= fmax, found by scanning e (exact in
    float64), minus the margin, clamped."""
    e = -400
    while a * 2.0 ** (e + 1) <= fmax:
        e += 1
    return min(max(e - margin, lo), hi)


def _positive_finite_bf16():
    x = oracle.bf16_bits_to_f64(all_bf16_patterns())
    return x[np.isfinite(x) & (x > 0)]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_bias_matches_exponent_scan(fmt):
    vals = _positive_finite_bf16()
    assert vals.size == 255 * 128 - 1
    for margin in range(4):
        got = compute_bias(vals, fmt, margin)
        # the scan per value is slow in Python; every 7th value plus the
        # values whose mantissa sits at the 1.75 boundary cover the rule
        sel = np.unique(np.concatenate([np.arange(0, vals.size, 7),
                                        np.nonzero(np.isin(np.frexp(vals)[0], [0.875, 0.875 + 2**-8, 0.875 - 2**-8]))[0]]))
        for i in sel:
            assert got[i] == _bruteforce_bias(vals[i], fmt.max, margin), (vals[i], margin)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_bias_keeps_scaled_amax_in_top_binade(fmt):
    """Scaled amax never exceeds the format max, and the scale is the largest
    power of two with that property: fmax/2 < amax * 2**bias <= fmax."""
    vals = _positive_finite_bf16()
    b = compute_bias(vals, fmt, 0)
    unclamped = (b > -126) & (b < 126)
    s = np.ldexp(vals, b)
    assert np.all(s[unclamped] <= fmt.max)
    assert np.all(s[unclamped] > fmt.max / 2)
    assert np.all(s <= fmt.max)               # clamped ones are smaller still
    # scales are powers of two: 2**b is exact and its mantissa is 0.5
    m, _ = np.frexp(np.ldexp(1.0, b))
    assert np.all(m == 0.5)


def test_bias_hand_values():
    """Values worked by hand from the reading floor(log2(fmax/amax))."""
    assert compute_bias(4.5, E4M3) == 6          # 4.5*64 = 288 <= 448 < 576
    assert compute_bias(430.0, E4M3) == 0
    assert compute_bias(448.0, E4M3) == 0
    assert compute_bias(449.0, E4M3) == -1
    assert compute_bias(760.0, E4M3) == -1       # 380 <= 448 < 760
    assert compute_bias(1.0, E4M3) == 8          # 256 <= 448 < 512
    assert compute_bias(1.0, E5M2) == 15
    assert compute_bias(1.0, E4M3, margin=2) == 6
    assert compute_bias(0.0, E4M3) == 0
    assert compute_bias(np.inf, E4M3) == 0
    assert compute_bias(np.nan, E5M2) == 0
    assert compute_bias(1e-38, E4M3) == 126      # clamped
    assert compute_bias(3e38, E4M3) == -120
    assert compute_bias(2.0 ** -133, E4M3) == 126
    assert compute_bias(2.0 ** -133, E4M3, lo=-127, hi=127) == 127


def test_amax_matches_numpy_and_specials():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((37, 53))
    assert oracle.amax(x) == np.max(np.abs(x))
    x[3, 4] = -1e6
    assert oracle.amax(x) == 1e6
    x[5, 5] = np.inf
    assert oracle.amax(x) == np.inf
    x[6, 6] = np.nan
    assert np.isnan(oracle.amax(x))
    assert oracle.amax(np.zeros((0, 5))) == 0.0


def test_delayed_window_is_max_of_last_16_earlier_steps():
    """The delayed bias at step t is the bias of max(amax[t-16 .. t-1]) (step 0
    bootstraps with its own amax), recomputed here from the full list."""
    rng = np.random.default_rng(5)
    amaxes = np.exp(rng.uniform(-3, 6, 40))
    amaxes[7] = 1e4                       # an outlier that must age out after 16 steps
    h = oracle.DelayedScaling(16)
    h.push(amaxes[0])                      # bootstrap
    for t in range(40):
        window = amaxes[max(0, t - 16):t] if t > 0 else amaxes[:1]
        assert h.window_max() == np.max(window)
        assert h.bias(E4M3) == compute_bias(np.max(window), E4M3)
        if t > 0:
            h.push(amaxes[t])
    assert h.count == 16


def test_delayed_empty_and_state():
    h = oracle.DelayedScaling(4)
    assert h.window_max() == 0.0 and h.bias(E4M3) == 0
    for a in [1.0, 2.0, 3.0, 4.0, 5.0]:
        h.push(a)
    hist, count, head = h.state()
    assert hist == [5.0, 2.0, 3.0, 4.0] and count == 4 and head == 1
    with pytest.raises(ValueError):
        oracle.DelayedScaling(0)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_quantize_current_scaling_never_saturates(fmt):
    """With the current amax and margin 0, no element exceeds the format max
    after scaling, and the largest element lands in the top binade."""
    x = oracle.bf16_bits_to_f64(make("c1", "X"))
    b = compute_bias(oracle.amax(x), fmt)
    q = oracle.quantize(x, fmt, b)
    back = decode(q, fmt)
    assert np.all(np.abs(np.ldexp(x, b)) <= fmt.max)
    assert np.max(np.abs(back)) > fmt.max / 2
    assert np.all(np.isfinite(back))


def test_quantize_half_ulp_relative_to_scale():
    x = oracle.bf16_bits_to_f64(make("c1", "W"))
    b = compute_bias(oracle.amax(x), E4M3)
    deq = oracle.dequantize(oracle.quantize(x, E4M3, b), E4M3, b)
    v = np.ldexp(x, b)
    _, exp = np.frexp(np.abs(v))
    half = np.ldexp(1.0, np.maximum(exp - 1, E4M3.emin) - E4M3.mbits - 1 - b)
    assert np.all(np.abs(deq - x) <= half)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_mx_blocks_top_binade_and_codes(fmt):
    x = oracle.bf16_bits_to_f64(make("c4", "X", shape=(64, 256)))
    q, s = oracle.mx_quantize(x, fmt)
    assert q.shape == x.shape and s.shape == (64, 256 // MX_BLOCK)
    blocks = x.reshape(64, -1, MX_BLOCK)
    bmax = np.max(np.abs(blocks), axis=2)
    e = 127 - s.astype(np.int64)
    scaled = np.ldexp(bmax, e)
    assert np.all(scaled <= fmt.max) and np.all(scaled > fmt.max / 2)
    # brute force of the block exponent by scanning
    for (i, j) in [(0, 0), (5, 3), (63, 7), (17, 1)]:
        assert e[i, j] == _bruteforce_bias(bmax[i, j], fmt.max, 0, -127, 127)
    # element codes are the per-element cast with the block's exponent
    ref = encode(np.ldexp(blocks, e[:, :, None]), fmt).reshape(x.shape)
    assert np.array_equal(q, ref)


def test_mx_edge_blocks():
    x = np.zeros((2, 96))
    x[0, 32:64] = np.linspace(-3, 3, 32)
    x[1, 5] = np.nan
    x[1, 70] = np.inf
    x[1, 64:70] = 1.0
    q, s = oracle.mx_quantize(x, E4M3)
    assert s[0, 0] == 127 and s[0, 2] == 127          # all-zero blocks
    assert s[0, 1] == 127 - compute_bias(3.0, E4M3, lo=-127, hi=127)
    assert s[1, 0] == 0xFF                             # NaN block
    assert q[1, 5] == 0x7F
    assert s[1, 2] == 127                              # Inf block -> scale 1
    assert q[1, 70] == 0x7E and q[1, 64] == encode(np.array([1.0]), E4M3)[0]
    assert np.all(q[0, :32] == 0)
    with pytest.raises(ValueError):
        oracle.mx_quantize(np.zeros((2, 33)), E4M3)
    # subnormal-only block: exponent clamps at 127 (code 0)
    tiny = np.full((1, 32), 2.0 ** -133)
    _, s2 = oracle.mx_quantize(tiny, E4M3)
    assert s2[0, 0] == 0


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_mx_error_dominates_per_tensor(fmt):
    """Each block's exponent is >= the tensor's, and the FP8 grids are closed
    under doubling below max, so per-block rounding is never farther from x
    than per-tensor rounding (elementwise), hence RMSE_mx <= RMSE_tensor."""
    x = oracle.bf16_bits_to_f64(make("c4", "X", shape=(128, 512)))
    b = compute_bias(oracle.amax(x), fmt)
    pt = oracle.dequantize(oracle.quantize(x, fmt, b), fmt, b)
    q, s = oracle.mx_quantize(x, fmt)
    mx = oracle.mx_dequantize(q, s, fmt)
    assert np.all(np.abs(mx - x) <= np.abs(pt - x))
    assert oracle.rmse(x, mx) <= oracle.rmse(x, pt)
    # FP8 relative error is scale-free within the normal range, so blocks help
    # where the per-tensor scale pushes small channels into subnormals
    tiny = np.abs(np.ldexp(x, b)) < 2.0 ** fmt.emin
    better = np.abs(mx - x) < np.abs(pt - x)
    assert np.all(~better | tiny)
    if fmt is E4M3:
        assert np.count_nonzero(better) > 0


def test_mx_uniform_codes_equal_per_tensor():
    """If every block gets the same code c, the bytes equal the per-tensor cast
    with bias 127 - c."""
    rng = np.random.default_rng(9)
    x = rng.uniform(-1, 1, (8, 128))
    x[:, ::32] = 0.99                    # every block's max in [0.99, 1): same exponent
    q, s = oracle.mx_quantize(x, E4M3)
    assert np.all(s == s[0, 0])
    assert np.array_equal(q, oracle.quantize(x, E4M3, 127 - int(s[0, 0])))


# --- the OCP MX shared-exponent rule ---------------------------------------

def _scan_ocp_exponent(a, emax):
    """Integer e with 2**emax <= a * 2**e < 2**(emax + 1), found by stepping
    e (exact in float64): the block maximum lands in the element format's
    top binade."""
    e = -400
    while a * 2.0 ** e < 2.0 ** emax:
        e += 1
    assert a * 2.0 ** e < 2.0 ** (emax + 1)
    return e


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_mx_ocp_exponent_matches_binade_scan(fmt):
    rng = np.random.default_rng(3)
    a = np.concatenate([np.ldexp(rng.uniform(1, 2, 200), rng.integers(-100, 100, 200)),
                        [1.0, 1.75, 1.7500001, 1.9999999, 448.0, 57344.0, 2.0 ** -120]])
    e, codes = oracle.mx_block_exponent(a, fmt, rule="ocp")
    want = np.array([min(max(_scan_ocp_exponent(v, fmt.emax), -127), 127) for v in a])
    assert np.array_equal(e, want)
    assert np.array_equal(codes.astype(np.int64), 127 - want)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_mx_ocp_rule_against_fmax_rule_all_bf16(fmt):
    """Both formats' largest finite value has significand 1.75 (E4M3 448 =
    1.75 * 2**8, E5M2 57344 = 1.75 * 2**15), so over every positive finite
    bf16 amax the two rules agree when the amax significand is at most 1.75
    and the OCP exponent is one larger above it (both before the clamp)."""
    a = _positive_finite_bf16()
    e_f, _ = oracle.mx_block_exponent(a, fmt)
    e_o, _ = oracle.mx_block_exponent(a, fmt, rule="ocp")
    m, _ = np.frexp(a)
    over = 2 * m > 1.75
    inside = (e_f > -127) & (e_f < 126)
    assert np.array_equal(e_o[inside & ~over], e_f[inside & ~over])
    assert np.array_equal(e_o[inside & over], e_f[inside & over] + 1)
    assert np.count_nonzero(inside & over) > 1000


def test_mx_ocp_worked_block():
    """E4M3 block with max 1.8: the OCP rule scales by 2**8 (1.8 -> 460.8,
    which saturates to 448, code 0x7E), the fmax rule by 2**7 (1.8 -> 230.4,
    nearest E4M3 value 224); 1.0 lands on 256 and 128.  Codes for amax 1 are
    127 - 8 = 119 (E4M3) and 127 - 15 = 112 (E5M2)."""
    x = np.zeros((1, 32))
    x[0, 0], x[0, 1] = 1.8, 1.0
    q_o, s_o = oracle.mx_quantize(x, E4M3, rule="ocp")
    q_f, s_f = oracle.mx_quantize(x, E4M3)
    assert s_o[0, 0] == 119 and s_f[0, 0] == 120
    assert q_o[0, 0] == 0x7E and decode(q_o[:, :1], E4M3)[0, 0] == 448.0
    assert decode(q_f[:, :1], E4M3)[0, 0] == 224.0
    assert decode(q_o[:, 1:2], E4M3)[0, 0] == 256.0 and decode(q_f[:, 1:2], E4M3)[0, 0] == 128.0
    _, s5 = oracle.mx_quantize(np.ones((1, 32)), E5M2, rule="ocp")
    assert s5[0, 0] == 112


def test_mx_ocp_edge_blocks_and_bad_rule():
    x = np.zeros((2, 96))
    x[1, 5] = np.nan
    x[1, 70] = np.inf
    x[1, 64:70] = 1.0
    q, s = oracle.mx_quantize(x, E4M3, rule="ocp")
    assert s[0, 0] == 127 and s[1, 0] == 0xFF and s[1, 2] == 127
    assert q[1, 5] == 0x7F and q[1, 70] == 0x7E
    _, s2 = oracle.mx_quantize(np.full((1, 32), 2.0 ** -133), E4M3, rule="ocp")
    assert s2[0, 0] == 0                               # exponent clamps at 127
    with pytest.raises(ValueError):
        oracle.mx_block_exponent(np.ones(2), E4M3, rule="floor")


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_mx_ocp_clipping_bound(fmt):
    """Under the OCP rule only elements whose scaled magnitude exceeds the
    format maximum clip, to the maximum; the block maximum's relative error
    is then below (2 - 1.75) / 2."""
    x = oracle.bf16_bits_to_f64(make("c4", "X", shape=(64, 256)))
    q, s = oracle.mx_quantize(x, fmt, rule="ocp")
    deq = oracle.mx_dequantize(q, s, fmt)
    e = (127 - s.astype(np.int64))[:, :, None]
    scaled = np.abs(np.ldexp(x.reshape(64, -1, MX_BLOCK), e)).reshape(x.shape)
    clipped = scaled > fmt.max
    assert np.all(np.abs(decode(q, fmt))[clipped] == fmt.max)
    assert np.all(np.abs(deq - x)[clipped] < 0.125 * np.abs(x)[clipped])
    assert np.count_nonzero(clipped) > 0
