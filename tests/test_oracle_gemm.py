"""Pins for the oracle's reference GEMMs (CPU only): exact rational brute
force on tiny shapes, identity and K=1 special cases, and the power-of-two
metamorphic relation between inputs, biases and outputs."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import E4M3, E5M2, decode, encode


def _frac_decode(code, fmt):
    """Exact rational value of one FP8 code, from the bit fields."""
    s = -1 if code & 0x80 else 1
    e = (code >> fmt.mbits) & ((1 << fmt.ebits) - 1)
    m = code & ((1 << fmt.mbits) - 1)
    if e == 0:
        return s * Fraction(m, 1 << fmt.mbits) * Fraction(2) ** fmt.emin
    return s * (1 + Fraction(m, 1 << fmt.mbits)) * Fraction(2) ** (e - fmt.ebias)


def _finite_codes(rng, shape, fmt):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    bad = np.isnan(decode(c, fmt)) | np.isinf(decode(c, fmt))
    c[bad] = 0x30
    return c


@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)],
                         ids=lambda f: f.name)
def test_gemm_matches_fractions(fa, fb):
    rng = np.random.default_rng(11)
    m, n, k = 7, 5, 13
    qa = _finite_codes(rng, (m, k), fa)
    qb = _finite_codes(rng, (n, k), fb)
    ba, bb = 3, -2
    y = oracle.scaled_gemm_ref(qa, fa, ba, qb, fb, bb)
    for i in range(m):
        for j in range(n):
            exact = sum(_frac_decode(int(qa[i, t]), fa) * _frac_decode(int(qb[j, t]), fb)
                        for t in range(k)) * Fraction(2) ** (-(ba + bb))
            assert y[i, j] == float(exact)


def test_gemm_e4m3_exact_at_large_k():
    """E4M3 x E4M3 sums are exact in float64 for K < 2**17, so summation
    order cannot matter: compare against a reversed-order sum."""
    rng = np.random.default_rng(12)
    qa = _finite_codes(rng, (4, 8192), E4M3)
    qb = _finite_codes(rng, (3, 8192), E4M3)
    y = oracle.scaled_gemm_ref(qa, E4M3, 0, qb, E4M3, 0)
    for i in range(4):
        for j in range(3):
            p = decode(qa[i], E4M3) * decode(qb[j], E4M3)
            assert y[i, j] == np.sum(p[::-1])
            assert y[i, j] == float(sum(Fraction(v) for v in p.tolist()))


def test_gemm_identity_and_k1():
    rng = np.random.default_rng(13)
    qa = _finite_codes(rng, (6, 16), E4M3)
    one = encode(np.array([1.0]), E4M3)[0]
    eye = np.where(np.eye(16, dtype=bool), one, 0).astype(np.uint8)
    y = oracle.scaled_gemm_ref(qa, E4M3, 2, eye, E4M3, 0)
    assert np.array_equal(y, np.ldexp(decode(qa, E4M3), -2))
    a1 = _finite_codes(rng, (5, 1), E5M2)
    b1 = _finite_codes(rng, (4, 1), E4M3)
    y1 = oracle.scaled_gemm_ref(a1, E5M2, 0, b1, E4M3, 1)
    assert np.array_equal(y1, np.outer(decode(a1[:, 0], E5M2), decode(b1[:, 0], E4M3)) / 2)


def test_gemm_power_of_two_metamorphic():
    """Scaling an input by 2**k leaves its FP8 bytes unchanged, lowers its
    bias by k, and scales Y by exactly 2**k."""
    rng = np.random.default_rng(14)
    x = rng.standard_normal((9, 64))
    w = 0.02 * rng.standard_normal((11, 64))
    bx = oracle.compute_bias(oracle.amax(x), E4M3)
    bw = oracle.compute_bias(oracle.amax(w), E4M3)
    y = oracle.scaled_gemm_ref(oracle.quantize(x, E4M3, bx), E4M3, bx,
                               oracle.quantize(w, E4M3, bw), E4M3, bw)
    for k in (-5, 3, 7):
        xs = np.ldexp(x, k)
        bxs = oracle.compute_bias(oracle.amax(xs), E4M3)
        assert bxs == bx - k
        assert np.array_equal(oracle.quantize(xs, E4M3, bxs), oracle.quantize(x, E4M3, bx))
        ys = oracle.scaled_gemm_ref(oracle.quantize(xs, E4M3, bxs), E4M3, bxs,
                                    oracle.quantize(w, E4M3, bw), E4M3, bw)
        assert np.array_equal(ys, np.ldexp(y, k))


def test_mx_gemm_matches_fractions():
    rng = np.random.default_rng(15)
    m, n, k = 5, 4, 64
    qa = _finite_codes(rng, (m, k), E4M3)
    qb = _finite_codes(rng, (n, k), E5M2)
    sa = rng.integers(110, 140, size=(m, k // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, size=(n, k // 32)).astype(np.uint8)
    y = oracle.mx_gemm_ref(qa, sa, E4M3, qb, sb, E5M2)
    for i in range(m):
        for j in range(n):
            exact = Fraction(0)
            abs_sum = Fraction(0)
            for blk in range(k // 32):
                terms = [_frac_decode(int(qa[i, t]), E4M3) * _frac_decode(int(qb[j, t]), E5M2)
                         for t in range(32 * blk, 32 * blk + 32)]
                sc = Fraction(2) ** (int(sa[i, blk]) - 127) * Fraction(2) ** (int(sb[j, blk]) - 127)
                exact += sum(terms) * sc
                abs_sum += sum(abs(t) for t in terms) * sc
            # float64 summation error bound: K * 2**-53 * sum |terms|
            assert abs(Fraction(float(y[i, j])) - exact) <= k * Fraction(1, 2 ** 53) * abs_sum


def test_mx_gemm_uniform_scales_equal_per_tensor():
    rng = np.random.default_rng(16)
    qa = _finite_codes(rng, (6, 96), E4M3)
    qb = _finite_codes(rng, (7, 96), E4M3)
    sa = np.full((6, 3), 120, dtype=np.uint8)
    sb = np.full((7, 3), 131, dtype=np.uint8)
    y = oracle.mx_gemm_ref(qa, sa, E4M3, qb, sb, E4M3)
    ref = oracle.scaled_gemm_ref(qa, E4M3, 127 - 120, qb, E4M3, 127 - 131)
    assert np.array_equal(y, ref)


def test_sampled_references_agree_with_full():
    rng = np.random.default_rng(17)
    qa = _finite_codes(rng, (20, 96), E5M2)
    qb = _finite_codes(rng, (30, 96), E4M3)
    y = oracle.scaled_gemm_ref(qa, E5M2, 1, qb, E4M3, 4)
    s = oracle.abs_product_sum(qa, E5M2, 1, qb, E4M3, 4)
    rows = rng.integers(0, 20, 50)
    cols = rng.integers(0, 30, 50)
    ys, ss = oracle.gemm_sample_ref(qa, E5M2, 1, qb, E4M3, 4, rows, cols)
    assert np.allclose(ys, y[rows, cols], rtol=0, atol=1e-12 * np.max(s))
    assert np.allclose(ss, s[rows, cols], rtol=1e-15)
    sa = rng.integers(120, 130, (20, 3)).astype(np.uint8)
    sb = rng.integers(120, 130, (30, 3)).astype(np.uint8)
    ym = oracle.mx_gemm_ref(qa, sa, E5M2, qb, sb, E4M3)
    yms, _ = oracle.mx_gemm_sample_ref(qa, sa, E5M2, qb, sb, E4M3, rows, cols)
    assert np.allclose(yms, ym[rows, cols], rtol=1e-14, atol=1e-300)


def test_bf16_output_rounding_and_rmse():
    y = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -3.0e38, 1e39, np.nan])
    bits = oracle.f64_to_bf16_bits(y)
    assert bits.tolist()[:3] == [0x3F80, 0x3F80, 0x3F82]   # ties to even
    assert bits[4] == 0x7F80                                # overflow -> Inf
    assert oracle.rmse(np.array([1.0, 2.0]), np.array([1.0, 4.0])) == np.sqrt(2.0)


@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2)], ids=lambda f: f.name)
def test_abs_product_sum_matches_fractions(fa, fb):
    """abs_product_sum (the scale of every per-tensor GEMM tolerance) against
    the exact rational sum_k |2**-ba dec(a_k) * 2**-bb dec(b_k)| built from
    the bit fields.  The two biases differ, so dropping or swapping one fails;
    E4M3 x E4M3 sums are exact in float64, the others within K * 2**-53."""
    rng = np.random.default_rng(18)
    m, n, k = 6, 5, 40
    qa = _finite_codes(rng, (m, k), fa)
    qb = _finite_codes(rng, (n, k), fb)
    ba, bb = 5, -3
    s = oracle.abs_product_sum(qa, fa, ba, qb, fb, bb)
    assert s.shape == (m, n)
    for i in range(m):
        for j in range(n):
            exact = sum(abs(_frac_decode(int(qa[i, t]), fa) * _frac_decode(int(qb[j, t]), fb)) for t in range(k))
            exact *= Fraction(2) ** (-(ba + bb))
            if fa is E4M3 and fb is E4M3:
                assert s[i, j] == float(exact)
            else:
                assert abs(Fraction(float(s[i, j])) - exact) <= k * Fraction(1, 2 ** 53) * exact


def test_mx_abs_product_sum_matches_fractions():
    """mx_abs_product_sum (the scale of every MX GEMM tolerance) against the
    exact rational sum_j 2**(sa-127) 2**(sb-127) sum_{k in block j}
    |dec(a_k) dec(b_k)|; per-row, per-block codes differ, so a block scale
    taken from the wrong block, row or operand fails."""
    rng = np.random.default_rng(19)
    m, n, k = 4, 5, 96
    qa = _finite_codes(rng, (m, k), E4M3)
    qb = _finite_codes(rng, (n, k), E5M2)
    sa = rng.integers(100, 150, size=(m, k // 32)).astype(np.uint8)
    sb = rng.integers(100, 150, size=(n, k // 32)).astype(np.uint8)
    s = oracle.mx_abs_product_sum(qa, sa, E4M3, qb, sb, E5M2)
    for i in range(m):
        for j in range(n):
            exact = Fraction(0)
            for blk in range(k // 32):
                sc = Fraction(2) ** (int(sa[i, blk]) - 127) * Fraction(2) ** (int(sb[j, blk]) - 127)
                exact += sc * sum(abs(_frac_decode(int(qa[i, t]), E4M3) * _frac_decode(int(qb[j, t]), E5M2))
                                  for t in range(32 * blk, 32 * blk + 32))
            assert abs(Fraction(float(s[i, j])) - exact) <= k * Fraction(1, 2 ** 53) * exact


def test_rmse_closed_forms():
    """rmse against values fixed by its definition sqrt(mean((xhat - x)**2)):
    an error of +-c everywhere gives c; errors (3, 4, 0, 0) give
    sqrt(25 / 4) = 2.5; an empty input gives 0; and on small integer arrays
    the square of the result equals the exact rational mean of squared errors
    to within a few float64 ulps (a sum instead of a mean, a missing square
    root or a missing square fails)."""
    rng = np.random.default_rng(20)
    x = rng.standard_normal(1000)
    sgn = rng.choice([-1.0, 1.0], 1000)
    assert oracle.rmse(x, x + 0.375 * sgn) == pytest.approx(0.375, rel=1e-15)
    assert oracle.rmse(np.zeros(4), np.array([3.0, 4.0, 0.0, 0.0])) == 2.5
    assert oracle.rmse(np.array([1.0, 2.0, 3.0, 4.0]), np.array([2.0, 3.0, 4.0, 5.0])) == 1.0
    assert oracle.rmse(np.zeros(0), np.zeros(0)) == 0.0
    for _ in range(20):
        n = int(rng.integers(1, 50))
        a = rng.integers(-100, 100, n)
        b = rng.integers(-100, 100, n)
        ms = Fraction(int(np.sum((b - a) ** 2)), n)
        r = oracle.rmse(a.astype(np.float64), b.astype(np.float64))
        assert abs(Fraction(r) ** 2 - ms) <= Fraction(4, 2 ** 52) * max(ms, Fraction(1))
