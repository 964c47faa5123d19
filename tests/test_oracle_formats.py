"""Pins for the oracle's FP8 decode / encode and bf16 rounding (CPU only).

Each test checks the oracle against something other than itself: the OFP8
constants typed in from the specification, PyTorch's CPU float8 casts (a
library routine), a brute-force nearest-neighbour search over the decoded
codes, and invariants of round-to-nearest-even.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2, decode, encode
from workloads import all_bf16_patterns

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ofp8_constants.json")
FMTS = [E4M3, E5M2]
TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_decode_matches_spec_constants(fmt):
    g = _golden()[fmt.name]
    assert fmt.ebias == g["exponent_bias"]
    assert fmt.max == g["max_normal"]
    assert decode(np.array([int(g["max_normal_code"], 16)]), fmt)[0] == g["max_normal"]
    codes = np.arange(256, dtype=np.uint8)
    vals = decode(codes, fmt)
    pos = vals[(codes < 128) & np.isfinite(vals) & (vals > 0)]
    assert pos.min() == g["min_subnormal"]
    assert pos.max() == g["max_normal"]
    normals = pos[pos >= g["min_normal"]]
    subs = pos[pos < g["min_normal"]]
    assert normals.min() == g["min_normal"]
    assert subs.max() == g["max_subnormal"]
    nan_codes = sorted(int(c, 16) for c in g["nan_codes"])
    assert sorted(np.nonzero(np.isnan(vals))[0].tolist()) == nan_codes
    inf_codes = sorted(int(c, 16) for c in g["inf_codes"])
    assert sorted(np.nonzero(np.isinf(vals))[0].tolist()) == inf_codes
    nz = decode(np.array([int(g["neg_zero_code"], 16)]), fmt)[0]
    assert nz == 0.0 and np.signbit(nz)
    assert decode(np.array([int(g["one_code"], 16)]), fmt)[0] == 1.0


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_decode_all_codes_match_torch(fmt):
    codes = np.arange(256, dtype=np.uint8)
    ours = decode(codes, fmt)
    ref = torch.from_numpy(codes).view(TORCH_DT[fmt.name]).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def _brute_encode(v, fmt):
    """Nearest finite code by exhaustive search over the decoded grid; exact
    ties go to the even code (the even mantissa); NaN -> 0x7F|sign; Inf ->
    the largest finite value (the nearest finite point)."""
    v = np.asarray(v, dtype=np.float64)
    codes = np.arange(128)
    vals = decode(codes.astype(np.uint8), fmt)
    keep = np.isfinite(vals)
    codes, vals = codes[keep], vals[keep]
    assert np.all(np.diff(vals) > 0)
    a = np.abs(v)
    # above the largest finite value the nearest finite point is that value
    a_f = np.where(np.isnan(a) | (a > vals[-1]), vals[-1], a)
    hi = np.clip(np.searchsorted(vals, a_f), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    dlo = np.abs(a_f - vals[lo])
    dhi = np.abs(vals[hi] - a_f)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi,
                    np.where(codes[lo] % 2 == 0, lo, hi)))
    out = codes[pick] | (np.signbit(v).astype(np.int64) << 7)
    out = np.where(np.isnan(v), 0x7F | (np.signbit(v).astype(np.int64) << 7), out)
    return out.astype(np.uint8)


def _sweep_values(biases):
    x = oracle.bf16_bits_to_f64(all_bf16_patterns())
    return np.concatenate([np.ldexp(x, b) for b in biases])


BIASES = list(range(-40, 41)) + [-126, -100, 100, 120, 126]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_encode_matches_bruteforce_nearest(fmt):
    v = _sweep_values(BIASES)
    assert np.array_equal(encode(v, fmt), _brute_encode(v, fmt))


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_encode_matches_torch_clamped_cast(fmt):
    """PyTorch's CPU cast rounds to nearest-even but does not saturate, so the
    input is clamped to +-max first (NaN passes through the clamp)."""
    v = _sweep_values(BIASES)
    t = torch.from_numpy(v)
    ref = torch.clamp(t, -fmt.max, fmt.max).to(TORCH_DT[fmt.name]).view(torch.uint8).numpy()
    ours = encode(v, fmt)
    nan = np.isnan(v)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN: both produce a NaN code with the input's sign
    assert np.all(np.isnan(decode(ours[nan], fmt)))
    assert np.array_equal(ours[nan] >> 7, np.signbit(v[nan]).astype(np.uint8))


def test_encode_worked_cases():
    cases = [
        # (value, fmt, code): ties, saturation, signed zero, specials
        (2.0 ** -10, E4M3, 0x00),        # half the smallest subnormal: tie -> 0
        (1.5 * 2 ** -9, E4M3, 0x02),     # tie between codes 1 and 2 -> even 2
        (2.5 * 2 ** -9, E4M3, 0x02),     # tie between codes 2 and 3 -> even 2
        (464.0, E4M3, 0x7E),             # tie between 448 and (absent) 480
        (465.0, E4M3, 0x7E),             # saturates instead of NaN
        (1e30, E4M3, 0x7E),
        (np.inf, E4M3, 0x7E),
        (-np.inf, E4M3, 0xFE),
        (np.nan, E4M3, 0x7F),
        (-0.0, E4M3, 0x80),
        (-1e-9, E4M3, 0x80),
        (15.5, E4M3, 0x58),              # carry into the next binade: 16
        (61440.0, E5M2, 0x7B),           # saturates instead of Inf
        (np.inf, E5M2, 0x7B),
        (np.nan, E5M2, 0x7F),
        (-0.0, E5M2, 0x80),
        (2.0 ** -17, E5M2, 0x00),        # half the smallest subnormal
        (1.0, E5M2, 0x3C),
    ]
    for v, fmt, code in cases:
        got = int(encode(np.array([v]), fmt)[0])
        assert got == code, (v, fmt.name, hex(got), hex(code))
    assert decode(np.array([0x58]), E4M3)[0] == 16.0


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_encode_half_ulp_and_monotone(fmt):
    """Round trip within half a quantum of the value's binade, and the code
    order follows the value order (for non-negative values)."""
    rng = np.random.default_rng(1)
    mag = np.exp(rng.uniform(np.log(2.0 ** (fmt.emin - fmt.mbits - 2)),
                             np.log(fmt.max), size=200000))
    v = np.concatenate([mag, -mag])
    q = encode(v, fmt)
    back = decode(q, fmt)
    _, exp = np.frexp(np.abs(v))
    E = np.maximum(exp - 1, fmt.emin)
    half_quantum = np.ldexp(1.0, E - fmt.mbits - 1)
    assert np.all(np.abs(back - v) <= half_quantum)
    order = np.argsort(mag)
    assert np.all(np.diff(encode(mag[order], fmt).astype(np.int64)) >= 0)


def test_bf16_rounding_matches_bruteforce():
    """The oracle's float64 -> bf16 rounding picks the nearer of the bf16
    neighbours (ties to the even code), checked by brute force over the
    three candidate codes around each value."""
    rng = np.random.default_rng(2)
    v = np.ldexp(rng.uniform(-2, 2, 100000), rng.integers(-140, 120, 100000))
    bits = oracle.f64_to_bf16_bits(v)
    a = np.abs(v)
    lo = (a.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    cands = np.stack([np.maximum(lo - 1, 0), lo, lo + 1], axis=1)
    vals = oracle.bf16_bits_to_f64(cands.astype(np.uint16))
    d = np.abs(vals - a[:, None])
    dmin = d.min(axis=1, keepdims=True)
    tie_ok = (d == dmin)
    # among the nearest candidates prefer an even code
    score = np.where(tie_ok, np.where(cands % 2 == 0, 0, 1), 2)
    best = cands[np.arange(len(a)), np.argmin(score, axis=1)]
    best = best | (np.signbit(v).astype(np.int64) << 15)
    assert np.array_equal(bits.astype(np.int64), best)


def test_bf16_rounding_matches_torch_from_float32():
    """From float32 inputs (no double rounding possible) torch's bf16 cast is
    a library pin for the oracle's rounding."""
    rng = np.random.default_rng(3)
    v32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16_bits(v32.astype(np.float64)), ref)


def test_bf16_ulp_is_distance_to_next_code():
    """bf16_ulp (which widens every bf16-output GEMM tolerance) against brute
    force over all 65,536 patterns: for each finite non-negative bf16 value x
    the spacing is the decoded distance to the next larger code (the largest
    finite value, which has no finite successor, uses its predecessor: same
    binade), and negative values share the spacing of their magnitude.  Zero
    and the subnormals must give the subnormal step 2**-133."""
    pats = all_bf16_patterns().astype(np.int64)
    vals = oracle.bf16_bits_to_f64(pats.astype(np.uint16))
    pos = pats[(pats < 0x7F80)]                       # +0 .. largest finite
    x = oracle.bf16_bits_to_f64(pos.astype(np.uint16))
    nxt = oracle.bf16_bits_to_f64(np.minimum(pos + 1, 0x7F7F).astype(np.uint16))
    prv = oracle.bf16_bits_to_f64(np.maximum(pos - 1, 0).astype(np.uint16))
    want = np.where(pos == 0x7F7F, x - prv, nxt - x)
    assert np.array_equal(oracle.bf16_ulp(x), want)
    assert oracle.bf16_ulp(0.0) == 2.0 ** -133 and oracle.bf16_ulp(-0.0) == 2.0 ** -133
    assert oracle.bf16_ulp(2.0 ** -130) == 2.0 ** -133       # a subnormal
    assert oracle.bf16_ulp(2.0 ** -126) == 2.0 ** -133       # smallest normal: same step
    assert oracle.bf16_ulp(1.0) == 2.0 ** -7 and oracle.bf16_ulp(1.999) == 2.0 ** -7
    neg = pats[(pats > 0x8000) & (pats < 0xFF80)]
    assert np.array_equal(oracle.bf16_ulp(oracle.bf16_bits_to_f64(neg.astype(np.uint16))),
                          oracle.bf16_ulp(-oracle.bf16_bits_to_f64(neg.astype(np.uint16))))
    assert np.all(np.isnan(oracle.bf16_ulp(vals[np.isnan(vals) | np.isinf(vals)])))


def test_bf16_ulp_between_codes():
    """For values between codes (the float64 GEMM references), the spacing is
    that of the two bf16 neighbours enclosing |v|, found by searching the
    sorted table of every finite non-negative bf16 value."""
    pats = np.arange(0, 0x7F80, dtype=np.int64)
    table = oracle.bf16_bits_to_f64(pats.astype(np.uint16))        # increasing
    rng = np.random.default_rng(4)
    v = np.ldexp(rng.uniform(-1, 1, 200000), rng.integers(-140, 128, 200000))
    v = np.concatenate([v, [0.0, -0.0, 2.0 ** -140, 3.0e38]])
    a = np.abs(v)
    i = np.searchsorted(table, a, side="right") - 1                 # largest code <= |v|
    hi = np.minimum(i + 1, table.size - 1)
    lo = np.where(i + 1 > table.size - 1, i - 1, i)
    want = table[hi] - table[lo]
    assert np.array_equal(oracle.bf16_ulp(v), want)


def test_f32_bits_to_f64_closed_form():
    """float32 bit patterns against the IEEE binary32 definition written out:
    (-1)^s 2^(e-127) (1 + m/2^23) for normal codes, (-1)^s 2^-126 m/2^23 for
    subnormals, infinities and NaN for e = 255; spot values plus 4096 random
    patterns."""
    def ieee(u):
        s, e, m = u >> 31, (u >> 23) & 0xFF, u & 0x7FFFFF
        sign = -1.0 if s else 1.0
        if e == 255:
            return sign * math.inf if m == 0 else math.nan
        if e == 0:
            return sign * math.ldexp(m, -149)
        return sign * math.ldexp(0x800000 + m, e - 150)
    spots = {0x3F800000: 1.0, 0xC0000000: -2.0, 0x00000001: 2.0 ** -149, 0x00800000: 2.0 ** -126,
             0x7F7FFFFF: (2 - 2.0 ** -23) * 2.0 ** 127, 0x80000000: -0.0, 0x7F800000: math.inf}
    got = oracle.f32_bits_to_f64(np.array(list(spots), dtype=np.uint32))
    for g, (u, want) in zip(got, spots.items()):
        assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want), hex(u)
    assert np.isnan(oracle.f32_bits_to_f64(np.array([0x7FC00000, 0xFF800001], dtype=np.uint32))).all()
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=4096, dtype=np.uint64).astype(np.uint32)
    got = oracle.f32_bits_to_f64(u)
    for g, x in zip(got, u.tolist()):
        w = ieee(x)
        assert (math.isnan(g) and math.isnan(w)) or (g == w and math.copysign(1.0, g) == math.copysign(1.0, w)), hex(x)
