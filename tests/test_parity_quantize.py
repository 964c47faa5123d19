"""GPU parity of amax, bias, per-tensor and per-block casts against the
oracle: bit-exact bytes, biases, float32 amaxes and E8M0 codes."""

import numpy as np
import pytest
import torch

import oracle
import scaled_quantize_fp8_amd as sq
from oracle import E4M3, E5M2
from workloads import all_bf16_patterns, f32_to_bf16_bits, make

from gpu_helpers import (DEV, bf16_dev, f32_bits_of, f32_dev, host, i32_dev, need_gpu,
                         oracle_amax_chunked, oracle_mx_chunked, oracle_quantize_chunked, pack_scales_host, say,
                         u8_dev)

pytestmark = pytest.mark.gpu
FMTS = [E4M3, E5M2]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_cast_every_bf16_pattern_every_bias(fmt):
    """All 65,536 bf16 bit patterns x every bias in [-126, 126]: the GPU bytes
    equal the oracle's (NaN -> 0x7F|sign, saturation, -0, subnormals)."""
    bits = all_bf16_patterns().reshape(256, 256)
    x = bf16_dev(bits)
    vals = oracle.bf16_bits_to_f64(bits)
    mism = []
    for b in range(-126, 127):
        say(f"cast sweep fmt={fmt.name} bias={b}") if b % 50 == 0 else None
        q, _, _ = sq.fp8_quantize(x, fmt.code, i32_dev(b))
        ref = oracle.quantize(vals, fmt, b)
        got = host(q)
        if not np.array_equal(got, ref):
            d = np.argwhere(got != ref)[:3]
            mism.append((b, [(hex(int(bits[tuple(i)])), hex(int(got[tuple(i)])), hex(int(ref[tuple(i)]))) for i in d]))
    assert not mism, mism[:5]


def test_cast_f32_inputs_bit_exact():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2**32, size=(128, 256), dtype=np.uint64).astype(np.uint32)
    u[0, :8] = [0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x00000001, 0x80000001, 0, 0x80000000]
    vals = oracle.f32_bits_to_f64(u)
    x = f32_dev(u)
    for fmt in FMTS:
        for b in (-100, -20, 0, 7, 40, 126):
            q, _, am = sq.fp8_quantize(x, fmt.code, i32_dev(b), want_amax=True)
            assert np.array_equal(host(q), oracle.quantize(vals, fmt, b)), (fmt.name, b)
    assert np.isnan(host(am)[0])


def test_amax_exact_and_nan():
    bits = all_bf16_patterns()
    finite = bits[np.isfinite(oracle.bf16_bits_to_f64(bits))].reshape(1, -1)
    a = sq.fp8_amax(bf16_dev(finite))
    assert host(a)[0] == oracle.amax(oracle.bf16_bits_to_f64(finite))
    assert np.isnan(host(sq.fp8_amax(bf16_dev(bits.reshape(256, 256))))[0])
    x = make("c1", "X")
    a = sq.fp8_amax(bf16_dev(x))
    assert host(a)[0] == oracle.amax(oracle.bf16_bits_to_f64(x))
    z = torch.zeros((0, 5), dtype=torch.bfloat16, device=DEV)
    assert host(sq.fp8_amax(z))[0] == 0.0


def test_compute_scale_matches_oracle():
    rng = np.random.default_rng(4)
    vals = list(np.exp(rng.uniform(-90, 90, 300)).astype(np.float32))
    vals += [0.0, np.inf, np.nan, 448.0, 449.0, 57344.0, 57345.0, 1.75, 1.7500001, 1e-45, 1e-40,
             3.4e38, 2.0 ** -126, 2.0 ** -149, 0.875, 7.0, 224.0]
    for v in vals:
        a = torch.tensor([v], dtype=torch.float32, device=DEV)
        for fmt in FMTS:
            for margin in (0, 1, 3):
                b, s, si = sq.fp8_compute_scale(a, fmt.code, margin)
                ref = oracle.compute_bias(float(np.float32(v)), fmt, margin)
                assert int(host(b)[0]) == ref, (v, fmt.name, margin)
                assert host(s)[0] == 2.0 ** ref and host(si)[0] == 2.0 ** -ref


def test_current_scaling_config_c1():
    """amax -> bias -> cast of X[256x768] and W[768x768], E4M3, margin 0."""
    for name in ("X", "W"):
        bits = make("c1", name)
        x = bf16_dev(bits)
        a = sq.fp8_amax(x)
        b, _, _ = sq.fp8_compute_scale(a, E4M3.code, 0)
        q, _, fused = sq.fp8_quantize(x, E4M3.code, b, want_amax=True)
        vals = oracle.bf16_bits_to_f64(bits)
        ref_a = oracle.amax(vals)
        ref_b = oracle.compute_bias(ref_a, E4M3)
        assert host(a)[0] == ref_a and f32_bits_of(fused) == f32_bits_of(a)
        assert int(host(b)[0]) == ref_b
        assert np.array_equal(host(q), oracle.quantize(vals, E4M3, ref_b))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cast_strided_ragged_and_unaligned(dtype):
    """Leading dimensions larger than cols, ragged tails and unaligned bases
    take the non-vector paths; results stay bit-exact."""
    rng = np.random.default_rng(5)
    full = (rng.standard_normal((41, 136)) * 3).astype(np.float32)
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits
        fb = f32_to_bf16_bits(full)
        t = bf16_dev(fb)
        vals_full = oracle.bf16_bits_to_f64(fb)
    else:
        t = f32_dev(full)
        vals_full = full.astype(np.float64)
    for (r0, c0, c1) in [(0, 0, 128), (0, 0, 136), (1, 3, 100), (2, 1, 131), (0, 5, 5 + 64), (3, 8, 136)]:
        sub = t[r0:, c0:c1]
        vals = vals_full[r0:, c0:c1]
        say(f"strided cast {dtype} view rows {r0}: cols {c0}:{c1}")
        for fmt in FMTS:
            bias = oracle.compute_bias(oracle.amax(vals), fmt)
            q, _, am = sq.fp8_quantize(sub, fmt.code, i32_dev(bias), want_amax=True)
            assert np.array_equal(host(q), oracle.quantize(vals, fmt, bias))
            assert host(am)[0] == oracle.amax(vals)
            assert host(sq.fp8_amax(sub))[0] == oracle.amax(vals)
            # strided output too
            big = torch.full((sub.shape[0], sub.shape[1] + 9), 0xAA, dtype=torch.uint8, device=DEV)
            q2, _, _ = sq.fp8_quantize(sub, fmt.code, i32_dev(bias), q=big[:, 3:3 + sub.shape[1]])
            hb = host(big)
            assert np.array_equal(hb[:, 3:3 + sub.shape[1]], oracle.quantize(vals, fmt, bias))
            assert np.all(hb[:, :3] == 0xAA) and np.all(hb[:, 3 + sub.shape[1]:] == 0xAA)


@pytest.mark.parametrize("shape", [(256, 768), (130, 200), (1, 77), (64, 64), (300, 17), (384, 200),
                                   (272, 1024)])
def test_cast_transpose(shape):
    """Vector kernel (aligned bf16 rows: whole 128 x 64 tiles, a ragged column
    tile, ragged row tiles, a matrix smaller than one tile) and the generic
    kernel (unaligned strides)."""
    rng = np.random.default_rng(6)
    from workloads import f32_to_bf16_bits
    bits = f32_to_bf16_bits((rng.standard_normal(shape) * 0.02).astype(np.float32))
    vals = oracle.bf16_bits_to_f64(bits)
    x = bf16_dev(bits)
    for fmt in FMTS:
        bias = oracle.compute_bias(oracle.amax(vals), fmt)
        q, qT, am = sq.fp8_quantize(x, fmt.code, i32_dev(bias), transpose=True, want_amax=True)
        ref = oracle.quantize(vals, fmt, bias)
        assert np.array_equal(host(q), ref)
        assert np.array_equal(host(qT), ref.T)
        assert host(am)[0] == oracle.amax(vals)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_cast_transpose_special_values(fmt):
    """NaN, +-Inf, -0, saturating and subnormal inputs through the vector
    cast-transpose (256 x 128, bias 3), with the fused amax (NaN)."""
    rng = np.random.default_rng(8)
    from workloads import f32_to_bf16_bits
    bits = f32_to_bf16_bits((rng.standard_normal((256, 128)) * 30).astype(np.float32))
    bits[0, 0] = 0x7FC0
    bits[5, 9] = 0xFF80
    bits[17, 70] = 0x7F80
    bits[100, 33] = 0x8000
    bits[200, 127] = 0x0003
    bits[255, 64] = 0x7F7F
    vals = oracle.bf16_bits_to_f64(bits)
    q, qT, am = sq.fp8_quantize(bf16_dev(bits), fmt.code, i32_dev(3), transpose=True, want_amax=True)
    ref = oracle.quantize(vals, fmt, 3)
    assert np.array_equal(host(q), ref)
    assert np.array_equal(host(qT), ref.T)
    assert np.isnan(host(am)[0])


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mx_cast_bit_exact(fmt, dtype):
    bits = make("c4", "X", shape=(96, 640))
    bits[0, :32] = 0                                   # all-zero block
    bits[1, 40] = 0x7FC0                               # NaN block
    bits[2, 64:96] = 0x0001                            # subnormal-only block
    bits[3, 100] = 0x7F80                              # Inf block
    bits[4, 128:160] = 0x7F7F                          # bf16 max
    vals = oracle.bf16_bits_to_f64(bits)
    x = bf16_dev(bits) if dtype == "bf16" else f32_dev(vals.astype(np.float32))
    q, s = sq.mx_quantize(x, fmt.code)
    rq, rs = oracle.mx_quantize(vals, fmt)
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(q), rq)
    # a strided view (vector kernel, row by row), a strided view starting at
    # an odd column (element kernel, row by row) and, for bf16, a contiguous
    # copy at an odd address (element kernel over one long row)
    for c0 in (32, 33):
        sub = x[5:, c0:c0 + 512]
        q2, s2 = sq.mx_quantize(sub, fmt.code)
        rq2, rs2 = oracle.mx_quantize(vals[5:, c0:c0 + 512], fmt)
        assert np.array_equal(host(s2), rs2) and np.array_equal(host(q2), rq2), c0
    if dtype == "bf16":
        odd = torch.empty(bits.size + 1, dtype=torch.bfloat16, device=DEV)[1:].view(bits.shape)
        odd.copy_(x)
        q3, s3 = sq.mx_quantize(odd, fmt.code)
        assert np.array_equal(host(s3), rs) and np.array_equal(host(q3), rq)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mx_cast_transposed_bit_exact(fmt, dtype):
    """Blocks of 32 rows, written transposed: equals the oracle's MX cast of
    x^T byte for byte.  96 rows (a half tile at the end), 100 columns (a
    ragged tile), blocks holding zeros, NaN, Inf, subnormals and the bf16
    maximum; then a strided input view and strided outputs."""
    bits = make("c4", "X", shape=(96, 100))
    bits[:32, 0] = 0                                   # all-zero block
    bits[40, 1] = 0x7FC0                               # NaN block
    bits[64:96, 2] = 0x0001                            # subnormal-only block
    bits[5, 3] = 0x7F80                                # Inf block
    bits[32:64, 4] = 0x7F7F                            # bf16 max
    bits[70, 5] = 0xFF80                               # -Inf
    vals = oracle.bf16_bits_to_f64(bits)
    x = bf16_dev(bits) if dtype == "bf16" else f32_dev(vals.astype(np.float32))
    say(f"mx transposed cast {fmt.name} {dtype}")
    qT, sT = sq.mx_quantize_t(x, fmt.code)
    rq, rs = oracle.mx_quantize(np.ascontiguousarray(vals.T), fmt)
    assert qT.shape == (100, 96) and sT.shape == (100, 3)
    assert np.array_equal(host(sT), rs)
    assert np.array_equal(host(qT), rq)
    # strided input (ld = 100 + 28) and padded outputs (ldqT = 96 + 16, ld_scales = 5)
    big = torch.zeros((96, 128), dtype=x.dtype, device=DEV)
    big[:, :100] = x
    qbig = torch.full((100, 112), 0xA5, dtype=torch.uint8, device=DEV)
    sbig = torch.full((100, 5), 0x5A, dtype=torch.uint8, device=DEV)
    sq.mx_quantize_t(big[:, :100], fmt.code, qT=qbig[:, :96], scalesT=sbig[:, :3])
    assert np.array_equal(host(qbig[:, :96]), rq) and np.array_equal(host(sbig[:, :3]), rs)
    assert np.all(host(qbig[:, 96:]) == 0xA5) and np.all(host(sbig[:, 3:]) == 0x5A)
    # a view starting one element into each row (element loads), 288 rows:
    # two whole 128-row tiles and a partial one
    tall = torch.zeros((320, 129), dtype=x.dtype, device=DEV)
    tall[:96, 1:101] = x
    tall[96:192, 1:101] = x
    tall[192:288, 1:101] = x
    rq3, rs3 = oracle.mx_quantize(np.ascontiguousarray(np.concatenate([vals, vals, vals])[:288].T), fmt)
    q3, s3 = sq.mx_quantize_t(tall[:288, 1:101], fmt.code)
    assert np.array_equal(host(q3), rq3) and np.array_equal(host(s3), rs3)


def test_mx_cast_transposed_full_size_sampled():
    """X[16384 x 8192] of the 70B-MLP workload: qT [8192 x 16384] and its
    scales exact on 64 sampled qT rows (columns of X)."""
    bits = make("c5", "X")
    x = bf16_dev(bits)
    say("mx transposed cast c5 X")
    qT, sT = sq.mx_quantize_t(x, E4M3.code)
    rng = np.random.default_rng(11)
    cols = np.unique(np.concatenate([[0, bits.shape[1] - 1], rng.integers(0, bits.shape[1], 62)]))
    rq, rs = oracle.mx_quantize(oracle.bf16_bits_to_f64(np.ascontiguousarray(bits[:, cols].T)), E4M3)
    idx = torch.from_numpy(cols).to(DEV)
    assert np.array_equal(host(sT[idx]), rs)
    assert np.array_equal(host(qT[idx]), rq)


def test_mx_cast_transposed_wide_tiles_ragged():
    """A bf16 tensor above 64M elements takes 128 x 128 tiles: [8192 x 8328]
    (the last tile column holds 8 columns) against the oracle on two columns
    of every tile and every column of the partial tile; the packed-scale
    variant writes the same codes and mx_pack_scales of the same scales."""
    bits = make("c5", "X", shape=(8192, 8328))
    x = bf16_dev(bits)
    say("mx transposed cast, wide tiles, 8192 x 8328")
    qT, sT = sq.mx_quantize_t(x, E4M3.code)
    rng = np.random.default_rng(12)
    t = np.arange(0, 8328, 128)
    cols = np.unique(np.concatenate([t + rng.integers(0, np.minimum(128, 8328 - t)) for _ in range(2)] +
                                    [np.arange(8320, 8328), [0, 127, 128]]))
    rq, rs = oracle.mx_quantize(oracle.bf16_bits_to_f64(np.ascontiguousarray(bits[:, cols].T)), E4M3)
    idx = torch.from_numpy(cols).to(DEV)
    assert np.array_equal(host(sT[idx]), rs)
    assert np.array_equal(host(qT[idx]), rq)
    pq, ps = sq.mx_quantize_t_packed(x, E4M3.code)
    assert torch.equal(pq, qT) and torch.equal(ps, sq.mx_pack_scales(sT))


def _every_bf16_as_block_max(seed=21):
    """[2048 x 1024] bf16 bits: block i (1 x 32) holds bf16 pattern i and 31
    elements of smaller or equal magnitude field (the pattern's field minus
    0..127, floored at 0), each with a random sign, so every one of the
    65,536 patterns is the maximum of its own block."""
    rng = np.random.default_rng(seed)
    p = all_bf16_patterns().astype(np.int64)
    mag = (p & 0x7FFF)[:, None] - rng.integers(0, 128, (p.size, 31))
    rest = np.maximum(mag, 0) | (rng.integers(0, 2, (p.size, 31)) << 15)
    return np.concatenate([p[:, None], rest], axis=1).astype(np.uint16).reshape(2048, 1024)


@pytest.mark.parametrize("rule", ["fmax", "ocp"])
@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_mx_rule_every_bf16_block_max(fmt, rule):
    """Both block-exponent rules on blocks whose maxima run over every bf16
    pattern (zeros, subnormals, the 1.75 significand boundary, Inf, NaN):
    codes and scales equal the oracle's, for the row-block and the
    transposed (column-block) entry points."""
    bits = _every_bf16_as_block_max()
    vals = oracle.bf16_bits_to_f64(bits)
    say(f"mx rule {rule} {fmt.name}: every bf16 pattern as a block max")
    rq, rs = oracle.mx_quantize(vals, fmt, rule=rule)
    x = bf16_dev(bits)
    q, s = sq.mx_quantize_rule(x, fmt.code, rule)
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(q), rq)
    qT, sT = sq.mx_quantize_t_rule(x.T.contiguous(), fmt.code, rule)
    assert np.array_equal(host(sT), rs)
    assert np.array_equal(host(qT), rq)
    if rule == "fmax":
        q0, s0 = sq.mx_quantize(x, fmt.code)
        assert np.array_equal(host(q0), rq) and np.array_equal(host(s0), rs)
    else:
        _, rs_f = oracle.mx_quantize(vals, fmt)
        assert np.count_nonzero(rs != rs_f) > 1000         # the rules differ on many blocks


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_mx_ocp_rule_f32_significand_boundary(fmt):
    """f32 block maxima at and around significand 1.75 (the last ulp below,
    1.75 itself, one ulp above, and just below 2) across binades, plus
    strided and unaligned views, under the OCP rule."""
    rng = np.random.default_rng(5)
    sig = np.array([1.75 - 2.0 ** -23, 1.75, 1.75 + 2.0 ** -23, 2 - 2.0 ** -23, 1.0, 1.5])
    exps = rng.integers(-140, 120, 64)
    bmax = np.ldexp(sig[None, :], exps[:, None]).astype(np.float32).ravel()        # 384 blocks
    blocks = bmax[:, None] * rng.uniform(-1, 1, (bmax.size, 32)).astype(np.float32)
    blocks[:, 7] = bmax
    vals = blocks.astype(np.float32).reshape(96, 128).astype(np.float64)
    say(f"mx ocp rule {fmt.name}: f32 significand boundary")
    rq, rs = oracle.mx_quantize(vals, fmt, rule="ocp")
    x = f32_dev(vals.astype(np.float32))
    q, s = sq.mx_quantize_rule(x, fmt.code, "ocp")
    assert np.array_equal(host(s), rs) and np.array_equal(host(q), rq)
    sub = x[3:, 32:96]                                   # strided: the scalar path
    q2, s2 = sq.mx_quantize_rule(sub, fmt.code, "ocp")
    rq2, rs2 = oracle.mx_quantize(vals[3:, 32:96], fmt, rule="ocp")
    assert np.array_equal(host(s2), rs2) and np.array_equal(host(q2), rq2)
    qT, sT = sq.mx_quantize_t_rule(x[:, 32:96], fmt.code, "ocp")   # strided transposed input
    rqT, rsT = oracle.mx_quantize(np.ascontiguousarray(vals[:, 32:96].T), fmt, rule="ocp")
    assert np.array_equal(host(sT), rsT) and np.array_equal(host(qT), rqT)


def test_mx_rmse_below_per_tensor_c4_shape():
    bits = make("c4", "X", shape=(256, 1024))
    vals = oracle.bf16_bits_to_f64(bits)
    q, s = sq.mx_quantize(bf16_dev(bits), E4M3.code)
    rq, rs = oracle.mx_quantize(vals, E4M3)
    assert np.array_equal(host(q), rq) and np.array_equal(host(s), rs)
    b = oracle.compute_bias(oracle.amax(vals), E4M3)
    pt = oracle.dequantize(oracle.quantize(vals, E4M3, b), E4M3, b)
    mx = oracle.mx_dequantize(host(q), host(s), E4M3)
    assert oracle.rmse(vals, mx) <= oracle.rmse(vals, pt)


@pytest.mark.parametrize("name", ["X", "W"])
def test_full_size_70b_mlp_sampled_rows(name):
    """The 70B-MLP tensors at full size, in the launch configuration the
    benchmark times: amax exact, bias exact, per-tensor and MX bytes exact on
    sampled rows (first, last and 62 random rows)."""
    bits = make("c5", name)
    say(f"full-size c5 {name} {bits.shape}")
    x = bf16_dev(bits)
    a = sq.fp8_amax(x)
    ref_a = oracle_amax_chunked(bits)
    assert host(a)[0] == ref_a
    b, _, _ = sq.fp8_compute_scale(a, E4M3.code, 0)
    ref_b = oracle.compute_bias(ref_a, E4M3)
    assert int(host(b)[0]) == ref_b
    q, _, fused = sq.fp8_quantize(x, E4M3.code, b, want_amax=True)
    assert f32_bits_of(fused) == f32_bits_of(a)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, bits.shape[0] - 1], rng.integers(0, bits.shape[0], 62)]))
    assert np.array_equal(host(q[torch.from_numpy(rows).to(DEV)]),
                          oracle_quantize_chunked(bits, E4M3, ref_b, rows))
    mq, ms = sq.mx_quantize(x, E4M3.code)
    rq, rs = oracle_mx_chunked(bits, E4M3, rows)
    idx = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(host(ms[idx]), rs)
    assert np.array_equal(host(mq[idx]), rq)
    # the cast that writes the GEMM's packed scale layout: same codes, and
    # scales equal to the row-major ones packed
    pq, ps = sq.mx_quantize_packed(x, E4M3.code)
    assert torch.equal(pq, mq)
    assert torch.equal(ps, sq.mx_pack_scales(ms))


@pytest.mark.parametrize("rows,cols,dtype,fmt,rule", [
    (300, 640, "bf16", E4M3, "fmax"), (256, 512, "bf16", E4M3, "fmax"), (513, 1056, "f32", E5M2, "fmax"),
    (70, 2048, "bf16", E4M3, "ocp"), (1, 32, "f32", E4M3, "fmax"), (257, 8192, "bf16", E5M2, "ocp")],
    ids=["300x640", "256x512", "513x1056_f32_e5", "70x2048_ocp", "1x32", "257x8192_e5_ocp"])
def test_mx_quantize_packed(rows, cols, dtype, fmt, rule):
    """mx_quantize_packed: codes equal to the oracle's MX cast, scales equal
    to the oracle's E8M0 codes in the packed layout (its definition in the
    header, 127 padding), for ragged and whole 256-row tiles and 16-block
    groups, bf16 and fp32 inputs, both block-exponent rules; also from a
    strided input (no contiguous collapse)."""
    rng = np.random.default_rng(rows * 7 + cols)
    vals = rng.standard_normal((rows, cols)) * np.exp(rng.normal(0.0, 2.0, (1, cols)))
    bits = f32_to_bf16_bits(vals.astype(np.float32))
    xv = oracle.bf16_bits_to_f64(bits) if dtype == "bf16" else vals.astype(np.float32).astype(np.float64)
    x = bf16_dev(bits) if dtype == "bf16" else f32_dev(vals.astype(np.float32))
    rq, rs = oracle.mx_quantize(xv, fmt, rule=rule)
    q, ps = sq.mx_quantize_packed(x, fmt.code, rule=rule)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(ps), pack_scales_host(rs))
    if cols >= 64:
        for c0 in (32, 1):                                   # strided rows; unaligned (element kernel)
            sub = x[:, c0:c0 + cols - 32]
            q2, ps2 = sq.mx_quantize_packed(sub, fmt.code, rule=rule)
            rq2, rs2 = oracle.mx_quantize(xv[:, c0:c0 + cols - 32], fmt, rule=rule)
            assert np.array_equal(host(q2), rq2), c0
            assert np.array_equal(host(ps2), pack_scales_host(rs2)), c0
    if dtype == "bf16":
        # contiguous at an odd address: the element kernel, collapsed into one
        # long row when a row is not a whole number of workgroup iterations
        odd = torch.empty(rows * cols + 1, dtype=torch.bfloat16, device=DEV)[1:].view(rows, cols)
        odd.copy_(x)
        q3, ps3 = sq.mx_quantize_packed(odd, fmt.code, rule=rule)
        assert np.array_equal(host(q3), rq)
        assert np.array_equal(host(ps3), pack_scales_host(rs))


@pytest.mark.parametrize("rows,cols,dtype,fmt,rule", [
    (320, 300, "bf16", E4M3, "fmax"), (512, 256, "bf16", E4M3, "fmax"), (1056, 70, "f32", E5M2, "fmax"),
    (2048, 130, "bf16", E5M2, "ocp"), (32, 1, "bf16", E4M3, "fmax")],
    ids=["320x300", "512x256", "1056x70_f32_e5", "2048x130_e5_ocp", "32x1"])
def test_mx_quantize_t_packed(rows, cols, dtype, fmt, rule):
    """mx_quantize_t_packed: qT equal to the oracle's MX cast of x^T, and its
    E8M0 codes ([cols x rows/32]) in the packed layout with 127 padding
    (ragged and whole tiles and groups, bf16 / fp32, both rules)."""
    rng = np.random.default_rng(rows * 3 + cols)
    vals = rng.standard_normal((rows, cols)) * np.exp(rng.normal(0.0, 2.0, (rows, 1)))
    bits = f32_to_bf16_bits(vals.astype(np.float32))
    xv = oracle.bf16_bits_to_f64(bits) if dtype == "bf16" else vals.astype(np.float32).astype(np.float64)
    x = bf16_dev(bits) if dtype == "bf16" else f32_dev(vals.astype(np.float32))
    rq, rs = oracle.mx_quantize(np.ascontiguousarray(xv.T), fmt, rule=rule)
    qT, ps = sq.mx_quantize_t_packed(x, fmt.code, rule=rule)
    assert np.array_equal(host(qT), rq)
    assert np.array_equal(host(ps), pack_scales_host(rs))


def _oracle_sat_count(vals, fmt, bias):
    """Elements the cast clamps: |x * 2**bias| > fmax, NaN excluded (the
    oracle's encode saturates exactly these)."""
    s = np.abs(np.ldexp(vals, bias))
    return int(np.count_nonzero(~np.isnan(s) & (s > fmt.max)))


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_saturation_count_every_bf16_pattern(fmt):
    """fp8_quantize_sat over all 65,536 bf16 patterns (NaN, +-Inf, subnormals,
    the largest finite values) at biases from -126 to 126 in steps of 7:
    the device count equals the oracle's count of clamped elements, and the
    bytes and fused amax equal fp8_quantize's."""
    bits = all_bf16_patterns().reshape(256, 256)
    x = bf16_dev(bits)
    vals = oracle.bf16_bits_to_f64(bits)
    for b in range(-126, 127, 7):
        q, _, am, n = sq.fp8_quantize_sat(x, fmt.code, i32_dev(b), want_amax=True)
        q0, _, am0 = sq.fp8_quantize(x, fmt.code, i32_dev(b), want_amax=True)
        assert int(host(n)[0]) == _oracle_sat_count(vals, fmt, b), (fmt.name, b)
        assert torch.equal(q, q0) and f32_bits_of(am) == f32_bits_of(am0)


@pytest.mark.parametrize("path", ["rows_vec", "rows_strided", "f32", "transpose_vec", "transpose_generic"])
def test_saturation_count_every_cast_path(path):
    """The count on each kernel the per-tensor cast can take: aligned rows
    (vector loads), a strided unaligned view (element loads), fp32 input, the
    vector cast-transpose (aligned bf16) and the generic cast-transpose
    (unaligned leading dimension); ragged shapes, Inf and NaN planted, a bias
    that clamps the tail of the distribution."""
    rng = np.random.default_rng(44)
    full = (rng.standard_normal((301, 264)) * 40).astype(np.float32)
    full[3, 7], full[100, 200], full[5, 5] = np.inf, -np.inf, np.nan
    if path == "f32":
        x = f32_dev(full)[:, :257]
        vals = full[:, :257].astype(np.float64)
    else:
        fb = f32_to_bf16_bits(full)
        t = bf16_dev(fb)
        vals_full = oracle.bf16_bits_to_f64(fb)
        if path in ("rows_strided", "transpose_generic"):
            x, vals = t[1:, 3:250], vals_full[1:, 3:250]          # unaligned base, ld 264
        elif path == "transpose_vec":
            x, vals = t[:288, :256], vals_full[:288, :256]        # qT rows of 288 bytes: vector kernel
        else:
            x, vals = t[:, :256], vals_full[:, :256]
    transpose = path.startswith("transpose")
    for fmt in FMTS:
        b = oracle.compute_bias(oracle.amax(vals[np.isfinite(vals)]), fmt) + 2     # clamps the top quarter
        say(f"saturation count {path} {fmt.name} bias {b}")
        q, qT, am, n = sq.fp8_quantize_sat(x, fmt.code, i32_dev(b), transpose=transpose, want_amax=True)
        ref = oracle.quantize(vals, fmt, b)
        assert np.array_equal(host(q), ref)
        if transpose:
            assert np.array_equal(host(qT), ref.T)
        want = _oracle_sat_count(vals, fmt, b)
        assert want > 1000 and int(host(n)[0]) == want
        assert np.isnan(host(am)[0])
        # without the fused amax, at a bias that clamps only the infinities
        _, _, _, n0 = sq.fp8_quantize_sat(x, fmt.code, i32_dev(b - 12), transpose=transpose)
        assert int(host(n0)[0]) == _oracle_sat_count(vals, fmt, b - 12)


@pytest.mark.parametrize("path", ["transpose_vec", "transpose_generic"])
def test_cast_transpose_tile_walk(path):
    """A reducing cast-transpose launches a few workgroups per CU, each
    walking at least four tiles.  A matrix of 2145 (vector kernel) or 4225
    (element kernel) tiles, ragged in both directions, with the largest
    magnitude planted in its last tile: q, qT, the fused amax and the
    saturation count against the oracle."""
    rng = np.random.default_rng(45)
    full = (rng.standard_normal((4113, 4112)) * 3).astype(np.float32)
    if path == "transpose_vec":
        rs, cs = slice(0, 4112), slice(0, 4104)       # aligned: 33 x 65 tiles of 128 x 64
    else:
        rs, cs = slice(1, 4113), slice(3, 4108)       # unaligned view: 65 x 65 tiles of 64 x 64
    full[rs, cs][-1, -1] = -1000.0
    fb = f32_to_bf16_bits(full)
    x = bf16_dev(fb)[rs, cs]
    vals = oracle.bf16_bits_to_f64(fb[rs, cs])
    for fmt in FMTS:
        b = oracle.compute_bias(4.0, fmt)          # clamps |x| > 7, about 2% of the elements
        say(f"cast-transpose tile walk {path} {fmt.name} {tuple(x.shape)}")
        q, qT, am, n = sq.fp8_quantize_sat(x, fmt.code, i32_dev(b), transpose=True, want_amax=True)
        ref = oracle.quantize(vals, fmt, b)
        assert np.array_equal(host(q), ref)
        assert np.array_equal(host(qT), ref.T)
        assert host(am)[0] == 1000.0
        want = _oracle_sat_count(vals, fmt, b)
        assert want > 100000 and int(host(n)[0]) == want


def _two_step(x, fmt, margin):
    a = sq.fp8_amax(x)
    b, s, si = sq.fp8_compute_scale(a, fmt, margin)
    return a, b, s, si


def _same_outputs(one, two, what):
    a1, b1, s1, si1 = one
    a2, b2, s2, si2 = two
    assert f32_bits_of(a1) == f32_bits_of(a2), what
    assert int(host(b1)[0]) == int(host(b2)[0]), what
    assert f32_bits_of(s1) == f32_bits_of(s2) and f32_bits_of(si1) == f32_bits_of(si2), what


def test_amax_scale_one_launch_equals_two_step():
    """fp8_amax_scale (one launch: workgroup maxima folded into a running
    maximum in the workspace, a ticket, bias and scales written by the last
    workgroup) gives exactly fp8_amax + fp8_compute_scale, and the oracle's
    amax and bias, on: every bf16 pattern (NaN: bias 0), every finite one,
    fp32 with Inf, a strided unaligned view (element loads), one ragged row,
    an empty tensor, E5M2 and margins; the whole workspace is back to zero
    after every call."""
    ws = sq.amax_scale_workspace(DEV)
    rng = np.random.default_rng(51)
    bits = all_bf16_patterns()
    finite = bits[np.isfinite(oracle.bf16_bits_to_f64(bits))]
    f32 = (rng.standard_normal((130, 257)) * 1e3).astype(np.float32)
    f32[7, 9] = np.inf
    strided = f32_to_bf16_bits((rng.standard_normal((77, 300)) * 5).astype(np.float32))
    cases = [("all bf16", bf16_dev(bits.reshape(256, 256)), oracle.bf16_bits_to_f64(bits)),
             ("finite bf16", bf16_dev(finite.reshape(1, -1)), oracle.bf16_bits_to_f64(finite)),
             ("f32 with inf", f32_dev(f32), f32.astype(np.float64)),
             ("strided view", bf16_dev(strided)[1:, 3:291], oracle.bf16_bits_to_f64(strided)[1:, 3:291]),
             ("one ragged row", bf16_dev(strided[:1, :77]), oracle.bf16_bits_to_f64(strided[:1, :77])),
             ("empty", torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV), np.zeros((0, 64)))]
    for name, x, vals in cases:
        for fmt in FMTS:
            for margin in (0, 2):
                one = sq.fp8_amax_scale(x, fmt.code, ws, margin, want_scales=True)
                _same_outputs(one, _two_step(x, fmt.code, margin), f"{name} {fmt.name} margin {margin}")
                ra = oracle.amax(vals) if vals.size else 0.0
                got = host(one[0])[0]
                assert (np.isnan(got) and np.isnan(ra)) or got == ra
                assert int(host(one[1])[0]) == oracle.compute_bias(ra, fmt, margin)
                assert not host(ws).any(), f"workspace not cleared after {name}"


@pytest.mark.parametrize("shape", [(16384, 8192), (28672, 8192), (24576, 32768)],
                         ids=["70b_mlp_x", "70b_mlp_w", "805M_elements"])
def test_amax_scale_full_size(shape):
    """The 70B-MLP X and W (1024 and 1792 workgroups) and a tensor of 805M
    elements (6144 workgroups): the one-launch amax and bias equal the
    two-step ones, repeated calls agree, and the workspace is back to zero."""
    g = torch.Generator(device=DEV).manual_seed(shape[0])
    x = torch.randn(shape, device=DEV, dtype=torch.bfloat16, generator=g)
    x.view(-1)[shape[0] * 77] = 99.5                    # one outlier far into the tensor
    ws = sq.amax_scale_workspace(DEV)
    say(f"amax_scale full size {shape}")
    ref = _two_step(x, E4M3.code, 0)
    for _ in range(3):
        _same_outputs(sq.fp8_amax_scale(x, E4M3.code, ws, want_scales=True), ref, f"{shape}")
    assert host(ref[0])[0] == 99.5
    assert not host(ws).any()
