"""GPU parity of the scaled FP8 GEMMs against the oracle's float64 sums.

Operands are FP8 codes, biases and E8M0 scales produced by the ORACLE from
the workload generators' bf16 inputs, so expected values never depend on the
HIP path.  Acceptance: |C - C_ref| <= 1e-5 * sum_k |a_k b_k| (fp32 output),
plus one bf16 ulp of C_ref (bf16 output).  An output beyond that bound passes
only where the bound is out of the FP8 instruction's reach: the GPU returned
the value of the pinned model of the instruction's in-group truncation
(``mfma_model``), up to float32 accumulation, rounded to the output type
(``assert_gemm_close`` with ``mfma_operands_pt`` / ``mfma_operands_mx``);
the workload tests report how many outputs that applies to.  The fused
output amax must equal max |C| over the stored output bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import scaled_quantize_fp8_amd as sq
from oracle import E4M3, E5M2
from workloads import f32_to_bf16_bits, make

from gpu_helpers import (DEV, assert_gemm_close, bf16_dev, f32_bits_of, host, host_f64, i32_dev,
                         mfma_operands_mx, mfma_operands_pt, need_gpu, oracle_mx_chunked, oracle_quantize_chunked, pack_scales_host,
                         oracle_amax_chunked, say, u8_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _operand(rng, shape, std, fmt):
    bits = f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))
    vals = oracle.bf16_bits_to_f64(bits)
    b = oracle.compute_bias(oracle.amax(vals), fmt)
    return oracle.quantize(vals, fmt, b), b


def _check_amax(C, amax_out):
    ref = np.max(np.abs(host_f64(C))) if C.numel() else 0.0
    assert host(amax_out)[0] == ref
    assert f32_bits_of(amax_out) == f32_bits_of(sq.fp8_amax(C))


def _run_pt(qa, fa, ba, qb, fb, bb, ta, tb, out_dtype):
    """qa/qb are op(A) [M,K] / op(B) [N,K]; stored transposed when ta/tb."""
    A = u8_dev(qa.T if ta else qa)
    B = u8_dev(qb.T if tb else qb)
    return sq.fp8_scaled_gemm(A, fa.code, i32_dev(ba), B, fb.code, i32_dev(bb), trans_a=ta, trans_b=tb,
                              out_dtype=out_dtype, want_amax=True)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)],
                         ids=["e4e4", "e5e4", "e4e5", "e5e5"])
def test_gemm_ragged_tiles(fa, fb, out_dtype):
    """M=300, N=520, K=400: 2 x 3 macro tiles with ragged M, N and K tails."""
    rng = np.random.default_rng(21)
    M, N, K = 300, 520, 400
    qa, ba = _operand(rng, (M, K), 1.0, fa)
    qb, bb = _operand(rng, (N, K), 0.02, fb)
    say(f"gemm ragged {fa.name}x{fb.name} {out_dtype}")
    C, am = _run_pt(qa, fa, ba, qb, fb, bb, False, False, out_dtype)
    ref = oracle.scaled_gemm_ref(qa, fa, ba, qb, fb, bb)
    s = oracle.abs_product_sum(qa, fa, ba, qb, fb, bb)
    gt = mfma_operands_pt(qa, fa, ba, qb, fb, bb)
    assert_gemm_close(host_f64(C), ref, s, out_dtype == torch.bfloat16, "ragged", gt)
    _check_amax(C, am)


@pytest.mark.parametrize("K", [128, 384, 1024], ids=["K128", "K384", "K1024"])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)],
                         ids=["e4e4", "e5e4", "e4e5", "e5e5"])
def test_gemm_k_multiple_of_128(fa, fb, K):
    """K a multiple of the 128-byte stage (one stage, an odd count, an even
    count) with ragged M = 300, N = 520, then a 40 x 24 problem far smaller
    than one tile, read from operands whose rows are padded (lda = K + 48)."""
    rng = np.random.default_rng(29 + K)
    qa, ba = _operand(rng, (300, K), 1.0, fa)
    qb, bb = _operand(rng, (520, K), 0.02, fb)
    say(f"gemm K%128 {fa.name}x{fb.name} K={K}")
    for dt in (torch.bfloat16, torch.float32):
        C, am = _run_pt(qa, fa, ba, qb, fb, bb, False, False, dt)
        ref = oracle.scaled_gemm_ref(qa, fa, ba, qb, fb, bb)
        s = oracle.abs_product_sum(qa, fa, ba, qb, fb, bb)
        gt = mfma_operands_pt(qa, fa, ba, qb, fb, bb)
        assert_gemm_close(host_f64(C), ref, s, dt == torch.bfloat16, f"K={K}", gt)
        _check_amax(C, am)
    pa = np.zeros((40, K + 48), dtype=np.uint8)
    pb = np.zeros((24, K + 48), dtype=np.uint8)
    pa[:, :K], pb[:, :K] = qa[:40], qb[:24]
    A, B = u8_dev(pa)[:, :K], u8_dev(pb)[:, :K]
    C, am = sq.fp8_scaled_gemm(A, fa.code, i32_dev(ba), B, fb.code, i32_dev(bb), out_dtype=torch.float32,
                               want_amax=True)
    ref = oracle.scaled_gemm_ref(qa[:40], fa, ba, qb[:24], fb, bb)
    s = oracle.abs_product_sum(qa[:40], fa, ba, qb[:24], fb, bb)
    gt = mfma_operands_pt(qa[:40], fa, ba, qb[:24], fb, bb)
    assert_gemm_close(host_f64(C), ref, s, False, f"small K={K}", gt)
    _check_amax(C, am)


@pytest.mark.parametrize("K", [4096, 4224, 4352], ids=["K4096", "K4224", "K4352"])
def test_gemm_small_grid_three_slot_pipeline(K):
    """Per-tensor products with fewer 256 x 256 tiles than compute units and
    K >= 4096 run 128-row tiles with three LDS stage slots, the epilogue
    staging C in those slots.  K = 4096, 4224, 4352 (32, 33, 34 stages: every
    count mod 3, so 1 or 2 zero stages pad the last loop iteration or none).
    Every output of a ragged 300 x 520 product (bf16 and fp32 out) and of an
    interior 512 x 768 one (bf16, staged stores) against the oracle; and the
    first 512 rows bit-identical to the same rows of an 8192-row product,
    which runs 256-row tiles with two slots."""
    rng = np.random.default_rng(83 + K)
    qa, ba = _operand(rng, (512, K), 1.0, E4M3)
    qb, bb = _operand(rng, (768, K), 0.02, E4M3)
    say(f"gemm three-slot K={K}")
    for (m, n, dt) in ((300, 520, torch.bfloat16), (300, 520, torch.float32), (512, 768, torch.bfloat16)):
        C, am = _run_pt(qa[:m], E4M3, ba, qb[:n], E4M3, bb, False, False, dt)
        ref = oracle.scaled_gemm_ref(qa[:m], E4M3, ba, qb[:n], E4M3, bb)
        s_ = oracle.abs_product_sum(qa[:m], E4M3, ba, qb[:n], E4M3, bb)
        gt = mfma_operands_pt(qa[:m], E4M3, ba, qb[:n], E4M3, bb)
        assert_gemm_close(host_f64(C), ref, s_, dt == torch.bfloat16, f"three-slot {m}x{n} K={K}", gt)
        _check_amax(C, am)
    # the same rows inside a product of 8192 rows x 2048 columns (256 tiles)
    big = np.concatenate([qa, rng.integers(0, 0x78, size=(8192 - 512, K), dtype=np.uint8)])
    qb2 = np.concatenate([qb, rng.integers(0, 0x78, size=(2048 - 768, K), dtype=np.uint8)])
    Cs, _ = _run_pt(qa, E4M3, ba, qb2, E4M3, bb, False, False, torch.bfloat16)     # 4 x 8 tiles: three slots
    Cb, _ = _run_pt(big, E4M3, ba, qb2, E4M3, bb, False, False, torch.bfloat16)    # 32 x 8 tiles: two slots
    assert torch.equal(Cs.view(torch.int16), Cb[:512].view(torch.int16))


@pytest.mark.parametrize("mx", [False, True], ids=["pt", "mx"])
def test_gemm_bf16_padded_outputs(mx):
    """bf16 C written into padded views, 2 x 2 interior tiles: row stride
    N + 8 (rows 16-byte aligned: whole-row staged stores) and an 8-byte
    offset with stride N + 4 (rows only 8-byte aligned: per-element path).
    Results equal the oracle's and the padding is left untouched."""
    rng = np.random.default_rng(41)
    M, N, K = 512, 512, 512                 # K >= 512: MX also takes the forward kernel
    qa, ba = _operand(rng, (M, K), 1.0, E4M3)
    qb, bb = _operand(rng, (N, K), 0.02, E4M3)
    if mx:
        sa = rng.integers(118, 136, (M, K // 32)).astype(np.uint8)
        sb = rng.integers(118, 136, (N, K // 32)).astype(np.uint8)
        ref = oracle.mx_gemm_ref(qa, sa, E4M3, qb, sb, E4M3)
        s = oracle.mx_abs_product_sum(qa, sa, E4M3, qb, sb, E4M3)
        gt = mfma_operands_mx(qa, sa, E4M3, qb, sb, E4M3)
    else:
        ref = oracle.scaled_gemm_ref(qa, E4M3, ba, qb, E4M3, bb)
        s = oracle.abs_product_sum(qa, E4M3, ba, qb, E4M3, bb)
        gt = mfma_operands_pt(qa, E4M3, ba, qb, E4M3, bb)
    for pad, off in ((8, 0), (4, 4)):
        say(f"gemm bf16 padded out mx={mx} stride N+{pad} offset {off}")
        big = torch.full((M, N + pad + off), -7.0, dtype=torch.bfloat16, device=DEV)
        flat = big.view(-1)[off:off + M * (N + pad)].view(M, N + pad)
        out = flat[:, :N]
        if mx:
            _, am = sq.mx_scaled_gemm(u8_dev(qa), E4M3.code, u8_dev(sa), u8_dev(qb), E4M3.code, u8_dev(sb),
                                      out=out, want_amax=True)
        else:
            _, am = sq.fp8_scaled_gemm(u8_dev(qa), E4M3.code, i32_dev(ba), u8_dev(qb), E4M3.code, i32_dev(bb),
                                       out=out, want_amax=True)
        assert_gemm_close(host_f64(out), ref, s, True, f"padded out N+{pad}", gt)
        _check_amax(out, am)
        hb = host_f64(big).ravel()
        written = np.zeros(hb.size, dtype=bool)
        idx = off + np.arange(M)[:, None] * (N + pad) + np.arange(N)[None, :]
        written[idx.ravel()] = True
        assert np.all(hb[~written] == -7.0)


@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)], ids=["NT", "TN", "TT"])
def test_gemm_transposed_operands(ta, tb):
    """Transposed storage for op(A) / op(B) (the backward products): M, N
    multiples of 16, K ragged (K = 272)."""
    rng = np.random.default_rng(22)
    M, N, K = 272, 528, 272
    qa, ba = _operand(rng, (M, K), 1e-4, E5M2)
    qb, bb = _operand(rng, (N, K), 0.02, E4M3)
    say(f"gemm transposed ta={ta} tb={tb}")
    C, am = _run_pt(qa, E5M2, ba, qb, E4M3, bb, ta, tb, torch.float32)
    ref = oracle.scaled_gemm_ref(qa, E5M2, ba, qb, E4M3, bb)
    s = oracle.abs_product_sum(qa, E5M2, ba, qb, E4M3, bb)
    gt = mfma_operands_pt(qa, E5M2, ba, qb, E4M3, bb)
    assert_gemm_close(host_f64(C), ref, s, False, f"trans {ta}{tb}", gt)
    _check_amax(C, am)


@pytest.mark.parametrize("M,N,K", [(4112, 4112, 512), (272, 528, 1024), (272, 528, 4096)],
                         ids=["289tiles_K512", "small_K1024", "small_K4096"])
@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)], ids=["NT", "TN", "TT"])
def test_gemm_mn_major_operands_forward_kernel(ta, tb, M, N, K):
    """MN-major storage ([K x M] / [K x N]) with K % 128 == 0 takes the
    forward kernel, whose stages hold K rows of the operand and whose
    fragments come from LDS transpose reads: ragged M and N tiles, a grid of
    289 256 x 256 tiles, and small grids (128 x 256 tiles, op(A) stages of
    128-byte K rows; two and three LDS slots).  Every output against the
    oracle, and bit for bit equal to the same product from K-contiguous
    copies of the operands."""
    rng = np.random.default_rng(26)
    qa, ba = _operand(rng, (M, K), 1e-4, E5M2)
    qb, bb = _operand(rng, (N, K), 0.02, E4M3)
    say(f"gemm MN-major ta={ta} tb={tb} {M}x{N}x{K}")
    C, am = _run_pt(qa, E5M2, ba, qb, E4M3, bb, ta, tb, torch.bfloat16)
    C0, am0 = _run_pt(qa, E5M2, ba, qb, E4M3, bb, False, False, torch.bfloat16)
    assert torch.equal(C.view(torch.int16), C0.view(torch.int16)) and f32_bits_of(am) == f32_bits_of(am0)
    ref = oracle.scaled_gemm_ref(qa, E5M2, ba, qb, E4M3, bb)
    s = oracle.abs_product_sum(qa, E5M2, ba, qb, E4M3, bb)
    gt = mfma_operands_pt(qa, E5M2, ba, qb, E4M3, bb)
    assert_gemm_close(host_f64(C), ref, s, True, f"MN-major {ta}{tb}", gt)
    _check_amax(C, am)


@pytest.mark.parametrize("M,N,K", [(4112, 4112, 528), (272, 528, 1104), (272, 528, 4208), (48, 80, 16)],
                         ids=["289tiles_K528", "small_K1104", "small_K4208", "one_partial_stage_K16"])
@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)],
                         ids=["TN", "NT", "TN_a", "TT"])
def test_gemm_k_tail_forward_kernel(ta, tb, M, N, K):
    """K % 128 != 0 on the forward kernel: the last stage holds K % 128 =
    16, 80 or 112 bytes (or is the only stage, K = 16), and its copies read
    zeros past K (K-contiguous chunks and MN-major K rows alike), on a grid
    of 289 256 x 256 tiles and on small grids (128 x 256 tiles, two and
    three LDS slots).  Every output against the oracle; bit for bit equal to
    the same product with both operands padded by zero bytes to a multiple
    of 128 in K (which runs without the tail) and across operand layouts."""
    rng = np.random.default_rng(27 + K)
    qa, ba = _operand(rng, (M, K), 1e-4, E5M2)
    qb, bb = _operand(rng, (N, K), 0.02, E4M3)
    say(f"gemm K tail ta={ta} tb={tb} {M}x{N}x{K}")
    C, am = _run_pt(qa, E5M2, ba, qb, E4M3, bb, ta, tb, torch.bfloat16)
    kp = (K + 127) // 128 * 128
    pa = np.zeros((M, kp), dtype=np.uint8)
    pb = np.zeros((N, kp), dtype=np.uint8)
    pa[:, :K], pb[:, :K] = qa, qb
    C0, am0 = _run_pt(pa, E5M2, ba, pb, E4M3, bb, False, False, torch.bfloat16)
    assert torch.equal(C.view(torch.int16), C0.view(torch.int16)) and f32_bits_of(am) == f32_bits_of(am0)
    if M * N <= 272 * 528:
        rs, cs = np.arange(M), np.arange(N)
    else:
        rng2 = np.random.default_rng(K)
        rs, cs = _tile_rows(rng2, M), _tile_rows(rng2, N)
    got = host_f64(C[torch.from_numpy(rs).to(DEV)][:, torch.from_numpy(cs).to(DEV)])
    a, b = qa[rs], qb[cs]
    assert_gemm_close(got, oracle.scaled_gemm_ref(a, E5M2, ba, b, E4M3, bb),
                      oracle.abs_product_sum(a, E5M2, ba, b, E4M3, bb), True, f"K tail {ta}{tb} {M}x{N}x{K}",
                      mfma_operands_pt(a, E5M2, ba, b, E4M3, bb))
    _check_amax(C, am)


def test_gemm_degenerate_shapes():
    rng = np.random.default_rng(23)
    qa, ba = _operand(rng, (64, 32), 1.0, E4M3)
    qb, bb = _operand(rng, (48, 32), 1.0, E4M3)
    # K = 0: C = 0, amax 0
    A0 = torch.zeros((64, 0), dtype=torch.uint8, device=DEV)
    B0 = torch.zeros((48, 0), dtype=torch.uint8, device=DEV)
    C, am = sq.fp8_scaled_gemm(A0, 0, i32_dev(0), B0, 0, i32_dev(0), out_dtype=torch.float32, want_amax=True)
    assert np.all(host(C) == 0) and host(am)[0] == 0.0
    # M = 0
    C, am = sq.fp8_scaled_gemm(torch.zeros((0, 32), dtype=torch.uint8, device=DEV), 0, i32_dev(0),
                               u8_dev(qb), 0, i32_dev(bb), want_amax=True)
    assert C.shape == (0, 48) and host(am)[0] == 0.0
    # K = 16 (one partial MFMA block), tiny M, N
    qa1, ba1 = _operand(rng, (3, 16), 1.0, E4M3)
    qb1, bb1 = _operand(rng, (5, 16), 1.0, E4M3)
    C, am = _run_pt(qa1, E4M3, ba1, qb1, E4M3, bb1, False, False, torch.float32)
    assert_gemm_close(host_f64(C), oracle.scaled_gemm_ref(qa1, E4M3, ba1, qb1, E4M3, bb1),
                      oracle.abs_product_sum(qa1, E4M3, ba1, qb1, E4M3, bb1), False, "K=16",
                      mfma_operands_pt(qa1, E4M3, ba1, qb1, E4M3, bb1))
    # identity B: C = dequantized A exactly (fp32 out)
    one = oracle.encode(np.array([1.0]), E4M3)[0]
    eye = np.where(np.eye(32, dtype=bool), one, 0).astype(np.uint8)
    C, _ = _run_pt(qa, E4M3, ba, eye, E4M3, 0, False, False, torch.float32)
    assert np.array_equal(host_f64(C), oracle.dequantize(qa, E4M3, ba))
    # strided output with padding columns untouched
    big = torch.full((64, 64), -7.0, dtype=torch.float32, device=DEV)
    sq.fp8_scaled_gemm(u8_dev(qa), 0, i32_dev(ba), u8_dev(qb), 0, i32_dev(bb), out=big[:, 8:56])
    hb = host(big)
    assert np.all(hb[:, :8] == -7.0) and np.all(hb[:, 56:] == -7.0)
    assert_gemm_close(hb[:, 8:56].astype(np.float64), oracle.scaled_gemm_ref(qa, E4M3, ba, qb, E4M3, bb),
                      oracle.abs_product_sum(qa, E4M3, ba, qb, E4M3, bb), False, "strided out",
                      mfma_operands_pt(qa, E4M3, ba, qb, E4M3, bb))


def test_gemm_deterministic():
    rng = np.random.default_rng(24)
    qa, ba = _operand(rng, (512, 1024), 1.0, E4M3)
    qb, bb = _operand(rng, (768, 1024), 0.02, E4M3)
    C1, a1 = _run_pt(qa, E4M3, ba, qb, E4M3, bb, False, False, torch.bfloat16)
    C2, a2 = _run_pt(qa, E4M3, ba, qb, E4M3, bb, False, False, torch.bfloat16)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    assert f32_bits_of(a1) == f32_bits_of(a2)


def test_gemm_config_c1_full():
    """X[256x768] W[768x768], current scaling, E4M3, Y = X W^T, bf16 and fp32."""
    xb, wb = make("c1", "X"), make("c1", "W")
    xv, wv = oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(wb)
    bx, bw = oracle.compute_bias(oracle.amax(xv), E4M3), oracle.compute_bias(oracle.amax(wv), E4M3)
    qx, qw = oracle.quantize(xv, E4M3, bx), oracle.quantize(wv, E4M3, bw)
    ref = oracle.scaled_gemm_ref(qx, E4M3, bx, qw, E4M3, bw)
    s = oracle.abs_product_sum(qx, E4M3, bx, qw, E4M3, bw)
    ops = mfma_operands_pt(qx, E4M3, bx, qw, E4M3, bw)
    for dt in (torch.bfloat16, torch.float32):
        C, am = _run_pt(qx, E4M3, bx, qw, E4M3, bw, False, False, dt)
        res = assert_gemm_close(host_f64(C), ref, s, dt == torch.bfloat16, "c1", ops)
        say(f"c1 {dt}: {res}")
        _check_amax(C, am)


@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3)], ids=["e4e4", "e5e4"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_mx_gemm_ragged(fa, fb, out_dtype):
    """M=300, N=260, K=352 (K % 128 = 96: a partial last stage of blocks)."""
    xb = make("c4", "X", shape=(300, 352))
    wb = make("c4", "W", shape=(260, 352))
    qa, sa = oracle.mx_quantize(oracle.bf16_bits_to_f64(xb), fa)
    qb, sb = oracle.mx_quantize(oracle.bf16_bits_to_f64(wb), fb)
    say(f"mx gemm {fa.name}x{fb.name} {out_dtype}")
    C, am = sq.mx_scaled_gemm(u8_dev(qa), fa.code, u8_dev(sa), u8_dev(qb), fb.code, u8_dev(sb),
                              out_dtype=out_dtype, want_amax=True)
    ref = oracle.mx_gemm_ref(qa, sa, fa, qb, sb, fb)
    s = oracle.mx_abs_product_sum(qa, sa, fa, qb, sb, fb)
    gt = mfma_operands_mx(qa, sa, fa, qb, sb, fb)
    assert_gemm_close(host_f64(C), ref, s, out_dtype == torch.bfloat16, "mx ragged", gt)
    _check_amax(C, am)


@pytest.mark.parametrize("K", [384, 640, 1024, 1152], ids=["K384", "K640", "K1024", "K1152"])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)],
                         ids=["e4e4", "e5e4", "e4e5", "e5e5"])
def test_mx_gemm_k_multiple_of_128(fa, fb, K):
    """K a multiple of 128 (stage counts 3, 5, 8, 9) with ragged M = 300,
    N = 260, scales passed twice: packed rows (K/32 bytes each,
    dword-aligned: the 32x32x64 kernel from K = 512 on, a partial last
    4-stage scale group at K = 640 and 1152; K = 384 runs the 16x16x128
    kernel) and rows padded to an odd stride (K/32 + 1 bytes), which only
    the 16x16x128 kernel takes, reading them byte by byte."""
    xb = make("c4", "X", shape=(300, K))
    wb = make("c4", "W", shape=(260, K))
    qa, sa = oracle.mx_quantize(oracle.bf16_bits_to_f64(xb), fa)
    qb, sb = oracle.mx_quantize(oracle.bf16_bits_to_f64(wb), fb)
    ref = oracle.mx_gemm_ref(qa, sa, fa, qb, sb, fb)
    s = oracle.mx_abs_product_sum(qa, sa, fa, qb, sb, fb)
    gt = mfma_operands_mx(qa, sa, fa, qb, sb, fb)
    nb = K // 32
    psa = np.zeros((300, nb + 1), dtype=np.uint8)
    psb = np.zeros((260, nb + 1), dtype=np.uint8)
    psa[:, :nb], psb[:, :nb] = sa, sb
    for what, SA, SB, dt in (("packed", u8_dev(sa), u8_dev(sb), torch.bfloat16),
                             ("odd stride", u8_dev(psa)[:, :nb], u8_dev(psb)[:, :nb], torch.float32)):
        say(f"mx gemm K%128 {fa.name}x{fb.name} K={K} {what}")
        C, am = sq.mx_scaled_gemm(u8_dev(qa), fa.code, SA, u8_dev(qb), fb.code, SB, out_dtype=dt,
                                  want_amax=True)
        assert_gemm_close(host_f64(C), ref, s, dt == torch.bfloat16, f"mx K={K} {what}", gt)
        _check_amax(C, am)


@pytest.mark.parametrize("rows,kb,pad", [(300, 20, 4), (256, 16, 0), (1, 1, 0), (513, 256, 0), (70, 36, 1)],
                         ids=["300x20_ld24", "256x16", "1x1", "513x256", "70x36_ld37"])
def test_mx_pack_scales_layout(rows, kb, pad):
    """mx_pack_scales rewrites row-major E8M0 codes into the tiled layout byte
    for byte, padding included (ragged rows and block groups; leading
    dimensions that allow and that do not allow 16-byte loads)."""
    rng = np.random.default_rng(rows * 1000 + kb)
    full = rng.integers(0, 256, (rows, kb + pad)).astype(np.uint8)
    sc = full[:, :kb]
    got = sq.mx_pack_scales(u8_dev(full)[:, :kb])
    torch.cuda.synchronize()
    assert sq.mx_packed_scales_bytes(rows, kb) == got.numel()
    assert np.array_equal(host(got), pack_scales_host(sc))


@pytest.mark.parametrize("M,N,K", [(300, 260, 640), (256, 256, 512), (512, 768, 1152), (130, 1030, 2048)],
                         ids=["300x260x640", "256x256x512", "512x768x1152", "130x1030x2048"])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3)], ids=["e4e4", "e5e4"])
def test_mx_gemm_packed_scales(fa, fb, M, N, K):
    """The block-scaled GEMM reading packed scales (mx_pack_scales) equals the
    row-major-scale GEMM bit for bit (bf16 and fp32 out, fused amax too) and
    the oracle within tolerance: ragged M / N tiles, a partial last group of
    16 blocks (K = 640, 1152), exactly one group (K = 512)."""
    xb = make("c4", "X", shape=(M, K))
    wb = make("c4", "W", shape=(N, K))
    qa, sa = oracle.mx_quantize(oracle.bf16_bits_to_f64(xb), fa)
    qb, sb = oracle.mx_quantize(oracle.bf16_bits_to_f64(wb), fb)
    ref = oracle.mx_gemm_ref(qa, sa, fa, qb, sb, fb)
    s = oracle.mx_abs_product_sum(qa, sa, fa, qb, sb, fb)
    gt = mfma_operands_mx(qa, sa, fa, qb, sb, fb)
    A, B, SA, SB = u8_dev(qa), u8_dev(qb), u8_dev(sa), u8_dev(sb)
    PA, PB = sq.mx_pack_scales(SA), sq.mx_pack_scales(SB)
    assert np.array_equal(host(PA), pack_scales_host(sa)) and np.array_equal(host(PB), pack_scales_host(sb))
    for dt in (torch.bfloat16, torch.float32):
        say(f"mx gemm packed {fa.name}x{fb.name} {M}x{N}x{K} {dt}")
        Cp, amp = sq.mx_scaled_gemm_packed(A, fa.code, PA, B, fb.code, PB, out_dtype=dt, want_amax=True)
        Cr, amr = sq.mx_scaled_gemm(A, fa.code, SA, B, fb.code, SB, out_dtype=dt, want_amax=True)
        torch.cuda.synchronize()
        assert torch.equal(Cp.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           Cr.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
        assert f32_bits_of(amp) == f32_bits_of(amr)
        assert_gemm_close(host_f64(Cp), ref, s, dt == torch.bfloat16, f"mx packed {M}x{N}x{K}", gt)
        _check_amax(Cp, amp)


@pytest.mark.parametrize("M,N,K,fa,fb", [(300, 260, 640, E4M3, E4M3), (300, 260, 768, E4M3, E4M3),
                                         (300, 260, 896, E4M3, E4M3), (4352, 4096, 896, E4M3, E4M3),
                                         (300, 260, 1152, E5M2, E4M3), (1, 33, 2176, E4M3, E5M2),
                                         (300, 260, 544, E4M3, E4M3), (300, 260, 608, E5M2, E4M3),
                                         (4352, 4096, 992, E4M3, E4M3), (1, 33, 2080, E4M3, E5M2)],
                         ids=["300x260x640", "300x260x768", "300x260x896", "4352x4096x896", "300x260x1152_e5e4",
                              "1x33x2176_e4e5", "300x260x544", "300x260x608_e5e4", "4352x4096x992",
                              "1x33x2080_e4e5"])
def test_mx_gemm_row_major_partial_scale_group(M, N, K, fa, fb):
    """Row-major scales with K % 512 != 0 on the 32x32x64 kernel: the last
    group of 16 scale codes holds 1, 2 or 3 whole stages (K = 640, 768, 896)
    or ends inside a stage (K % 128 != 0: 544, 608, 992, 2080, the last
    stage's copies reading zeros past K), and is copied from 16 codes
    before each row's end.  Each scale row is
    followed by NaN codes (0xFF) up to a dword-aligned stride and 4 more,
    which the kernel must not read.
    The product equals the packed-scale product bit for bit and the oracle
    within tolerance; 128-row tiles (4 tiles) and 256-row tiles (272 tiles,
    every output of two rows and columns per tile checked); also E5M2
    operands and a single-row product."""
    xb = make("c4", "X", shape=(M, K))
    wb = make("c4", "W", shape=(N, K))
    qa, sa = oracle.mx_quantize(oracle.bf16_bits_to_f64(xb), fa)
    qb, sb = oracle.mx_quantize(oracle.bf16_bits_to_f64(wb), fb)
    nb = K // 32
    ldp = (nb + 3) // 4 * 4 + 4                      # dword-aligned rows, at least 4 bytes of NaN codes after
    psa = np.full((M, ldp), 0xFF, dtype=np.uint8)
    psb = np.full((N, ldp), 0xFF, dtype=np.uint8)
    psa[:, :nb], psb[:, :nb] = sa, sb
    A, B = u8_dev(qa), u8_dev(qb)
    SA, SB = u8_dev(psa)[:, :nb], u8_dev(psb)[:, :nb]
    say(f"mx gemm row-major partial scale group {M}x{N}x{K}")
    Cr, amr = sq.mx_scaled_gemm(A, fa.code, SA, B, fb.code, SB, want_amax=True)
    Cp, amp = sq.mx_scaled_gemm_packed(A, fa.code, sq.mx_pack_scales(SA), B, fb.code, sq.mx_pack_scales(SB),
                                       want_amax=True)
    torch.cuda.synchronize()
    assert torch.equal(Cr.view(torch.int16), Cp.view(torch.int16)) and f32_bits_of(amr) == f32_bits_of(amp)
    _check_amax(Cr, amr)
    if M * N <= 300 * 260:
        rs, cs = np.arange(M), np.arange(N)
    else:
        rng = np.random.default_rng(K)
        rs, cs = _tile_rows(rng, M), _tile_rows(rng, N)
    got = host_f64(Cr[torch.from_numpy(rs).to(DEV)][:, torch.from_numpy(cs).to(DEV)])
    a, b, ssa, ssb = qa[rs], qb[cs], sa[rs], sb[cs]
    assert_gemm_close(got, oracle.mx_gemm_ref(a, ssa, fa, b, ssb, fb),
                      oracle.mx_abs_product_sum(a, ssa, fa, b, ssb, fb), True, f"mx rm {M}x{N}x{K}",
                      mfma_operands_mx(a, ssa, fa, b, ssb, fb))


@pytest.mark.parametrize("K", [544, 1120], ids=["K544", "K1120"])
def test_mx_gemm_tight_row_major_scales_k_tail(K):
    """Row-major scales in tight rows of K/32 codes with K % 128 != 0 (rows
    not 4-byte aligned: the 16x16x128 kernel) and the same codes packed (the
    32x32x64 kernel with a K tail): both against the oracle, every output of
    a ragged 300 x 260 product, bf16 and fp32 out."""
    xb = make("c4", "X", shape=(300, K))
    wb = make("c4", "W", shape=(260, K))
    qa, sa = oracle.mx_quantize(oracle.bf16_bits_to_f64(xb), E4M3)
    qb, sb = oracle.mx_quantize(oracle.bf16_bits_to_f64(wb), E4M3)
    ref = oracle.mx_gemm_ref(qa, sa, E4M3, qb, sb, E4M3)
    s_ = oracle.mx_abs_product_sum(qa, sa, E4M3, qb, sb, E4M3)
    gt = mfma_operands_mx(qa, sa, E4M3, qb, sb, E4M3)
    A, B, SA, SB = u8_dev(qa), u8_dev(qb), u8_dev(sa), u8_dev(sb)
    for dt in (torch.bfloat16, torch.float32):
        say(f"mx gemm tight row-major scales K={K} {dt}")
        Cr, amr = sq.mx_scaled_gemm(A, E4M3.code, SA, B, E4M3.code, SB, out_dtype=dt, want_amax=True)
        Cp, amp = sq.mx_scaled_gemm_packed(A, E4M3.code, sq.mx_pack_scales(SA), B, E4M3.code,
                                           sq.mx_pack_scales(SB), out_dtype=dt, want_amax=True)
        for what, C, am in (("row-major", Cr, amr), ("packed", Cp, amp)):
            assert_gemm_close(host_f64(C), ref, s_, dt == torch.bfloat16, f"mx tight {what} K={K}", gt)
            _check_amax(C, am)


@pytest.mark.parametrize("M,N,K", [(300, 260, 672), (300, 260, 416), (130, 1030, 96), (4352, 4096, 736)],
                         ids=["300x260x672", "300x260x416", "130x1030x96", "4352x4096x736"])
def test_mx_gemm_packed_k_tail(M, N, K):
    """Packed scales with K % 128 != 0 (and K < 512) on the 32x32x64 kernel:
    the last stage holds 1 or 3 blocks of 32 (or is the only stage, K = 96),
    its copies read zeros past K and its missing blocks take the layout's
    padding code 127.  Bit for bit equal to the same product with both
    operands padded by zero bytes to a multiple of 128 in K (the same packed
    scales: the padding blocks are 127 either way), and the oracle within
    tolerance (every output, or two rows and columns per tile)."""
    xb = make("c4", "X", shape=(M, K))
    wb = make("c4", "W", shape=(N, K))
    qa, sa = oracle.mx_quantize(oracle.bf16_bits_to_f64(xb), E4M3)
    qb, sb = oracle.mx_quantize(oracle.bf16_bits_to_f64(wb), E4M3)
    PA, PB = sq.mx_pack_scales(u8_dev(sa)), sq.mx_pack_scales(u8_dev(sb))
    say(f"mx gemm packed K tail {M}x{N}x{K}")
    C, am = sq.mx_scaled_gemm_packed(u8_dev(qa), E4M3.code, PA, u8_dev(qb), E4M3.code, PB, want_amax=True)
    kp = (K + 127) // 128 * 128
    pa = np.zeros((M, kp), dtype=np.uint8)
    pb = np.zeros((N, kp), dtype=np.uint8)
    pa[:, :K], pb[:, :K] = qa, qb
    C0, am0 = sq.mx_scaled_gemm_packed(u8_dev(pa), E4M3.code, PA, u8_dev(pb), E4M3.code, PB, want_amax=True)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), C0.view(torch.int16)) and f32_bits_of(am) == f32_bits_of(am0)
    _check_amax(C, am)
    if M * N <= 300 * 260:
        rs, cs = np.arange(M), np.arange(N)
    else:
        rng = np.random.default_rng(K)
        rs, cs = _tile_rows(rng, M), _tile_rows(rng, N)
    got = host_f64(C[torch.from_numpy(rs).to(DEV)][:, torch.from_numpy(cs).to(DEV)])
    a, b, ssa, ssb = qa[rs], qb[cs], sa[rs], sb[cs]
    assert_gemm_close(got, oracle.mx_gemm_ref(a, ssa, E4M3, b, ssb, E4M3),
                      oracle.mx_abs_product_sum(a, ssa, E4M3, b, ssb, E4M3), True, f"mx packed tail {M}x{N}x{K}",
                      mfma_operands_mx(a, ssa, E4M3, b, ssb, E4M3))


def test_mx_gemm_extreme_block_scales():
    """Per-block codes spread over a wide range (2^-40 .. 2^40 per block), so a
    wrong block <-> scale pairing cannot hide inside the tolerance."""
    rng = np.random.default_rng(25)
    M, N, K = 64, 80, 256
    qa = rng.integers(0, 0x7E, (M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    qb = rng.integers(0, 0x7E, (N, K)).astype(np.uint8)
    sa = rng.integers(87, 168, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(87, 168, (N, K // 32)).astype(np.uint8)
    C, _ = sq.mx_scaled_gemm(u8_dev(qa), 0, u8_dev(sa), u8_dev(qb), 0, u8_dev(sb), out_dtype=torch.float32)
    ref = oracle.mx_gemm_ref(qa, sa, E4M3, qb, sb, E4M3)
    s = oracle.mx_abs_product_sum(qa, sa, E4M3, qb, sb, E4M3)
    gt = mfma_operands_mx(qa, sa, E4M3, qb, sb, E4M3)
    assert_gemm_close(host_f64(C), ref, s, False, "mx scales", gt)


def test_mx_gemm_uniform_scales_match_per_tensor():
    rng = np.random.default_rng(26)
    qa, ba = _operand(rng, (130, 256), 1.0, E4M3)
    qb, bb = _operand(rng, (70, 256), 1.0, E4M3)
    sa = np.full((130, 8), 127 - ba, dtype=np.uint8)
    sb = np.full((70, 8), 127 - bb, dtype=np.uint8)
    Cm, _ = sq.mx_scaled_gemm(u8_dev(qa), 0, u8_dev(sa), u8_dev(qb), 0, u8_dev(sb), out_dtype=torch.float32)
    Cp, _ = _run_pt(qa, E4M3, ba, qb, E4M3, bb, False, False, torch.float32)
    ref = oracle.scaled_gemm_ref(qa, E4M3, ba, qb, E4M3, bb)
    s = oracle.abs_product_sum(qa, E4M3, ba, qb, E4M3, bb)
    gt = mfma_operands_pt(qa, E4M3, ba, qb, E4M3, bb)
    assert_gemm_close(host_f64(Cm), ref, s, False, "mx uniform", gt)
    assert_gemm_close(host_f64(Cp), ref, s, False, "pt uniform", gt)
    # same codes, same arithmetic: the two kernels agree bit for bit
    assert torch.equal(Cm, Cp)


def test_mx_weight_gradient_via_transposed_casts():
    """dW = dY^T X with MX operands: both cast with blocks along the token
    axis (mx_quantize_t), then the MX GEMM contracts over tokens (K = 1024).
    dY is E5M2 (a gradient), X is E4M3; the oracle casts dY^T and X^T itself."""
    dyb = make("c3", "dY", shape=(1024, 384))
    xb = make("c3", "X", shape=(1024, 256))
    say("mx dW via transposed casts")
    qdy, sdy = sq.mx_quantize_t(bf16_dev(dyb), E5M2.code)
    qx, sx = sq.mx_quantize_t(bf16_dev(xb), E4M3.code)
    C, am = sq.mx_scaled_gemm(qdy, E5M2.code, sdy, qx, E4M3.code, sx, out_dtype=torch.float32, want_amax=True)
    oqdy, osdy = oracle.mx_quantize(oracle.bf16_bits_to_f64(np.ascontiguousarray(dyb.T)), E5M2)
    oqx, osx = oracle.mx_quantize(oracle.bf16_bits_to_f64(np.ascontiguousarray(xb.T)), E4M3)
    assert np.array_equal(host(qdy), oqdy) and np.array_equal(host(sdy), osdy)
    assert np.array_equal(host(qx), oqx) and np.array_equal(host(sx), osx)
    ref = oracle.mx_gemm_ref(oqdy, osdy, E5M2, oqx, osx, E4M3)
    s = oracle.mx_abs_product_sum(oqdy, osdy, E5M2, oqx, osx, E4M3)
    gt = mfma_operands_mx(oqdy, osdy, E5M2, oqx, osx, E4M3)
    assert_gemm_close(host_f64(C), ref, s, False, "mx dW", gt)
    _check_amax(C, am)


def _tile_rows(rng, n, extra=64):
    """Two random indices inside every 256-wide tile of [0, n), the first and
    last index, and `extra` more at random: sorted, unique."""
    t = np.arange(0, n, 256)
    per = np.concatenate([t + rng.integers(0, np.minimum(256, n - t)) for _ in range(2)])
    return np.unique(np.concatenate([per, [0, n - 1], rng.integers(0, n, extra)]))


def test_full_size_70b_mlp_end_to_end_sampled():
    """X[16384 x 8192], W[28672 x 8192] through the whole hot path on the GPU,
    in the benchmark's launch sequence: amax -> bias -> E4M3 cast -> per-tensor
    GEMM (bf16 out, fused amax), and MX cast to packed scales -> MX GEMM.  The
    oracle recomputes amax and bias from the generator's bf16 tensors, casts
    the sampled operand rows (two in every 256-row tile of X and of W, plus
    64 random ones each) and forms every output of those rows and columns in
    float64: about 190 x 290 outputs per GEMM, at least four in each of the
    7168 output tiles.  The fused output amax must equal a standalone
    reduction over the GPU's own output."""
    xb, wb = make("c5", "X"), make("c5", "W")
    x, w = bf16_dev(xb), bf16_dev(wb)
    rng = np.random.default_rng(27)
    rs, cs = _tile_rows(rng, xb.shape[0]), _tile_rows(rng, wb.shape[0])
    ri, ci = torch.from_numpy(rs).to(DEV), torch.from_numpy(cs).to(DEV)
    say("c5 gpu per-tensor path")
    ax, aw = sq.fp8_amax(x), sq.fp8_amax(w)
    bx, _, _ = sq.fp8_compute_scale(ax, 0, 0)
    bw, _, _ = sq.fp8_compute_scale(aw, 0, 0)
    qx, _, _ = sq.fp8_quantize(x, 0, bx)
    qw, _, _ = sq.fp8_quantize(w, 0, bw)
    C, am = sq.fp8_scaled_gemm(qx, 0, bx, qw, 0, bw, want_amax=True)
    am_ref = sq.fp8_amax(C)
    got = host_f64(C[ri][:, ci])
    assert f32_bits_of(am) == f32_bits_of(am_ref)
    del C, qx, qw
    torch.cuda.empty_cache()
    say(f"c5 oracle (per-tensor), {rs.size} x {cs.size} outputs")
    rbx = oracle.compute_bias(oracle_amax_chunked(xb), E4M3)
    rbw = oracle.compute_bias(oracle_amax_chunked(wb), E4M3)
    assert int(host(bx)[0]) == rbx and int(host(bw)[0]) == rbw
    oqx = oracle_quantize_chunked(xb, E4M3, rbx, rs)
    oqw = oracle_quantize_chunked(wb, E4M3, rbw, cs)
    y = oracle.scaled_gemm_ref(oqx, E4M3, rbx, oqw, E4M3, rbw)
    sabs = oracle.abs_product_sum(oqx, E4M3, rbx, oqw, E4M3, rbw)
    res = assert_gemm_close(got, y, sabs, True, "c5 per-tensor", mfma_operands_pt(oqx, E4M3, rbx, oqw, E4M3, rbw))
    say(f"c5 per-tensor: {res}")
    tiles = {(int(r) // 256, int(c) // 256) for r in rs for c in cs}
    assert len(tiles) == (xb.shape[0] // 256) * (wb.shape[0] // 256)
    say("c5 gpu mx path (cast to packed scales)")
    mqx, psx = sq.mx_quantize_packed(x, 0)
    mqw, psw = sq.mx_quantize_packed(w, 0)
    C, am = sq.mx_scaled_gemm_packed(mqx, 0, psx, mqw, 0, psw, want_amax=True)
    got = host_f64(C[ri][:, ci])
    assert f32_bits_of(am) == f32_bits_of(sq.fp8_amax(C))
    say("c5 gpu mx path, row-major scales: same bits")
    _, msx = sq.mx_quantize(x, 0)
    _, msw = sq.mx_quantize(w, 0)
    Cr, amr = sq.mx_scaled_gemm(mqx, 0, msx, mqw, 0, msw, want_amax=True)
    assert torch.equal(Cr.view(torch.int16), C.view(torch.int16))
    assert f32_bits_of(amr) == f32_bits_of(am)
    del C, Cr
    say("c5 oracle (mx)")
    oqxm, osxm = oracle_mx_chunked(xb, E4M3, rs)
    oqwm, oswm = oracle_mx_chunked(wb, E4M3, cs)
    y = oracle.mx_gemm_ref(oqxm, osxm, E4M3, oqwm, oswm, E4M3)
    sabs = oracle.mx_abs_product_sum(oqxm, osxm, E4M3, oqwm, oswm, E4M3)
    res = assert_gemm_close(got, y, sabs, True, "c5 mx", mfma_operands_mx(oqxm, osxm, E4M3, oqwm, oswm, E4M3))
    say(f"c5 mx: {res}")


def test_full_size_7b_attn_delayed_gemm_sampled():
    """The delayed-scaling workload's forward product at full size (X_t
    [2048 x 4096] against W [4096 x 4096], bf16 out) at every one of its 16
    steps: step 0 with the bootstrap bias, step 1 with the window's bias,
    under which X_1 saturates, then the window's maximum.  Biases come from
    the oracle's history, codes from the GPU casts (equal to the oracle's),
    and every output of two sampled rows and columns per 256-wide tile (every
    output tile) is compared with the oracle's float64 product under the
    plain bound, outputs beyond it only where they are the FP8 instruction's
    own result (counted)."""
    h = oracle.DelayedScaling(16)
    wb = make("c2", "W")
    rbw = oracle.compute_bias(oracle.amax(oracle.bf16_bits_to_f64(wb)), E4M3)
    qw = oracle.quantize(oracle.bf16_bits_to_f64(wb), E4M3, rbw)
    Wq = u8_dev(qw)
    rng = np.random.default_rng(41)
    total = {"outputs": 0, "beyond_plain": 0}
    for t in range(16):
        xb = make("c2", "X", step=t)
        xv = oracle.bf16_bits_to_f64(xb)
        if t == 0:
            h.push(oracle.amax(xv))
        rbx = h.bias(E4M3)
        if t > 0:
            h.push(oracle.amax(xv))
        say(f"delayed gemm step {t}: bias {rbx}")
        qx, _, _ = sq.fp8_quantize(bf16_dev(xb), 0, i32_dev(rbx))
        assert np.array_equal(host(qx), oracle.quantize(xv, E4M3, rbx))
        C, am = sq.fp8_scaled_gemm(qx, 0, i32_dev(rbx), Wq, 0, i32_dev(rbw), want_amax=True)
        rs, cs = _tile_rows(rng, 2048), _tile_rows(rng, 4096)
        got = host_f64(C[torch.from_numpy(rs).to(DEV)][:, torch.from_numpy(cs).to(DEV)])
        oqx = oracle.quantize(xv[rs], E4M3, rbx)
        y = oracle.scaled_gemm_ref(oqx, E4M3, rbx, qw[cs], E4M3, rbw)
        sabs = oracle.abs_product_sum(oqx, E4M3, rbx, qw[cs], E4M3, rbw)
        res = assert_gemm_close(got, y, sabs, True, f"delayed step {t}", mfma_operands_pt(oqx, E4M3, rbx, qw[cs], E4M3, rbw))
        total["outputs"] += res["outputs"]
        total["beyond_plain"] += res["beyond_plain"]
        assert f32_bits_of(am) == f32_bits_of(sq.fp8_amax(C))
    say(f"delayed 16 steps: {total}")


def test_full_size_13b_mlp_up_mx_gemm_every_output():
    """The MXFP8 workload at full size, every output: X [8192 x 5120] with
    log-normal column scales and W [13824 x 5120], MX casts on the GPU (codes
    and scales equal to the oracle's for every row), the block-scaled product
    (bf16 out) on row-major and on packed scales (same bits), and all
    113,246,208 outputs against the oracle's float64 product (512-row
    panels).

    The column scales (sigma 1.5) make the products inside a group of 8 K
    very unequal, and the FP8 instruction truncates every product of a group
    onto the grid of the largest: a small fraction of outputs miss
    1e-5 sum|ab| + 1 bf16 ulp.  Each of those must be instruction-limited
    (the pinned model of the instruction is itself that far from the exact
    sum, and the GPU agrees with the model); the count is reported."""
    xb, wb = make("c4", "X"), make("c4", "W")
    x, w = bf16_dev(xb), bf16_dev(wb)
    say("c4 gpu mx casts and products")
    qx, sx = sq.mx_quantize(x, 0)
    qw, sw = sq.mx_quantize(w, 0)
    C, am = sq.mx_scaled_gemm(qx, 0, sx, qw, 0, sw, want_amax=True)
    pqx, psx = sq.mx_quantize_packed(x, 0)
    pqw, psw = sq.mx_quantize_packed(w, 0)
    assert torch.equal(pqx, qx) and torch.equal(pqw, qw)
    Cp, amp = sq.mx_scaled_gemm_packed(pqx, 0, psx, pqw, 0, psw, want_amax=True)
    assert torch.equal(Cp.view(torch.int16), C.view(torch.int16)) and f32_bits_of(amp) == f32_bits_of(am)
    assert f32_bits_of(am) == f32_bits_of(sq.fp8_amax(C))
    got = host_f64(C)
    hqx, hsx, hqw, hsw = host(qx), host(sx), host(qw), host(sw)
    del x, w, C, Cp, qx, sx, qw, sw, pqx, psx, pqw, psw
    torch.cuda.empty_cache()
    say("c4 oracle casts, every row")
    oqx, osx = oracle_mx_chunked(xb, E4M3)
    oqw, osw = oracle_mx_chunked(wb, E4M3)
    assert np.array_equal(hqx, oqx) and np.array_equal(hsx, osx)
    assert np.array_equal(hqw, oqw) and np.array_equal(hsw, osw)
    say("c4 oracle product, 8192 x 13824 x 5120 in float64")
    y = oracle.mx_gemm_ref(oqx, osx, E4M3, oqw, osw, E4M3)
    sabs = oracle.mx_abs_product_sum(oqx, osx, E4M3, oqw, osw, E4M3)
    res = assert_gemm_close(got, y, sabs, True, "c4 mx",
                            mfma_operands_mx(oqx, osx, E4M3, oqw, osw, E4M3))
    say(f"c4 mx every output: {res['beyond_plain']} of {res['outputs']} beyond 1e-5 sum|ab| + 1 bf16 ulp, "
        f"all instruction-limited; largest error / allowance {res['max_err_over_tol']:.3f}")


def test_backward_shapes_7b_mlp_sampled():
    """dX = dY W (A = dY [4096 x 11008] E5M2, B = W stored [11008 x 4096] ->
    trans_b) and dW = dY^T X (A = dY^T, B = X^T, both stored transposed),
    fp32 out: every output of two sampled rows and columns per 256-wide tile
    (so every output tile) plus 64 random rows and columns, against the
    oracle's float64 product; outputs beyond the plain bound only where they
    are the FP8 instruction's own result (counted)."""
    dyb, wb, xb = make("c3", "dY"), make("c3", "W"), make("c3", "X")
    say("c3 oracle casts")
    bdy = oracle.compute_bias(oracle_amax_chunked(dyb), E5M2)
    bw = oracle.compute_bias(oracle_amax_chunked(wb), E4M3)
    bx = oracle.compute_bias(oracle_amax_chunked(xb), E4M3)
    qdy = oracle_quantize_chunked(dyb, E5M2, bdy)
    qw = oracle_quantize_chunked(wb, E4M3, bw)
    qx = oracle_quantize_chunked(xb, E4M3, bx)
    rng = np.random.default_rng(28)
    say("c3 dX")
    dX, _ = sq.fp8_scaled_gemm(u8_dev(qdy), 1, i32_dev(bdy), u8_dev(qw), 0, i32_dev(bw), trans_b=True,
                               out_dtype=torch.float32)
    rs, cs = _tile_rows(rng, 4096), _tile_rows(rng, 4096)
    got = host_f64(dX[torch.from_numpy(rs).to(DEV)][:, torch.from_numpy(cs).to(DEV)])
    a, b = qdy[rs], np.ascontiguousarray(qw[:, cs].T)
    res = assert_gemm_close(got, oracle.scaled_gemm_ref(a, E5M2, bdy, b, E4M3, bw),
                            oracle.abs_product_sum(a, E5M2, bdy, b, E4M3, bw), False, "dX",
                            mfma_operands_pt(a, E5M2, bdy, b, E4M3, bw))
    say(f"c3 dX: {res}")
    del dX
    say("c3 dW")
    dW, _ = sq.fp8_scaled_gemm(u8_dev(qdy), 1, i32_dev(bdy), u8_dev(qx), 0, i32_dev(bx), trans_a=True,
                               trans_b=True, out_dtype=torch.float32)
    rs, cs = _tile_rows(rng, 11008), _tile_rows(rng, 4096)
    got = host_f64(dW[torch.from_numpy(rs).to(DEV)][:, torch.from_numpy(cs).to(DEV)])
    a, b = np.ascontiguousarray(qdy[:, rs].T), np.ascontiguousarray(qx[:, cs].T)
    res = assert_gemm_close(got, oracle.scaled_gemm_ref(a, E5M2, bdy, b, E4M3, bx),
                            oracle.abs_product_sum(a, E5M2, bdy, b, E4M3, bx), False, "dW",
                            mfma_operands_pt(a, E5M2, bdy, b, E4M3, bx))
    say(f"c3 dW: {res}")
    tiles = {(int(r) // 256, int(c) // 256) for r in rs for c in cs}
    assert len(tiles) == 43 * 16


def _repeat_identical(fn, reps, what):
    """Run fn(out) `reps` times into NaN-filled outputs; every run must give
    the first run's output and fused amax bit for bit."""
    ref, ref_am = None, None
    for r in range(reps):
        out = ref if ref is None else torch.empty_like(ref)
        out = fn(out)
        C, am = out
        torch.cuda.synchronize()
        if ref is None:
            ref, ref_am = C, f32_bits_of(am)
            continue
        nd = int((C.view(torch.int16) != ref.view(torch.int16)).sum())
        assert nd == 0, f"{what}: repeat {r} differs from the first run in {nd} outputs"
        assert f32_bits_of(am) == ref_am, f"{what}: repeat {r} fused amax differs"
        del C


@pytest.mark.parametrize("mx", [False, True, "packed"], ids=["pt", "mx", "mx_packed"])
def test_full_size_70b_mlp_gemm_repeat_bit_identical(mx):
    """Run-to-run determinism of the 70B-MLP GEMMs (16384 x 28672 x 8192,
    bf16 out) over every output element: eight launches on the same operands
    must agree bit for bit.  Each launch writes into a NaN-filled buffer, so an
    output the kernel failed to write also shows.  (A missing copy wait once
    left one 8-row block of a stage unpublished in rare tiles: ~1e-5 of the
    outputs changed from run to run, which sampled parity could not see.)"""
    g = torch.Generator(device=DEV).manual_seed(5)
    x = torch.randn(16384, 8192, device=DEV, dtype=torch.bfloat16, generator=g)
    w = torch.randn(28672, 8192, device=DEV, dtype=torch.bfloat16, generator=g) * 0.015
    if mx:
        qx, sx = sq.mx_quantize(x, 0)
        qw, sw = sq.mx_quantize(w, 0)
        if mx == "packed":
            sx, sw = sq.mx_pack_scales(sx), sq.mx_pack_scales(sw)
    else:
        bx, _, _ = sq.fp8_compute_scale(sq.fp8_amax(x), 0, 0)
        bw, _, _ = sq.fp8_compute_scale(sq.fp8_amax(w), 0, 0)
        qx, _, _ = sq.fp8_quantize(x, 0, bx)
        qw, _, _ = sq.fp8_quantize(w, 0, bw)
    del x, w
    torch.cuda.empty_cache()

    def launch(out):
        if out is None:
            out = torch.empty(16384, 28672, device=DEV, dtype=torch.bfloat16)
        out.fill_(float("nan"))
        if mx == "packed":
            return sq.mx_scaled_gemm_packed(qx, 0, sx, qw, 0, sw, out=out, want_amax=True)
        if mx:
            return sq.mx_scaled_gemm(qx, 0, sx, qw, 0, sw, out=out, want_amax=True)
        return sq.fp8_scaled_gemm(qx, 0, bx, qw, 0, bw, out=out, want_amax=True)

    what = {False: "per-tensor", True: "mx", "packed": "mx packed scales"}[mx]
    say(f"70b-mlp {what} gemm x8 determinism")
    _repeat_identical(launch, 8, what)


@pytest.mark.parametrize("mx", [False, True], ids=["pt", "mx"])
def test_backward_7b_mlp_gemms_repeat_bit_identical(mx):
    """Run-to-run determinism of the transposed-operand products of the 7B-MLP
    backward (dX = dY W: 4096 x 4096 x 11008 with op(B) stored transposed;
    dW = dY^T X: 11008 x 4096 x 4096 with both stored transposed), and of the
    MX products over the transposed casts, four launches each."""
    g = torch.Generator(device=DEV).manual_seed(6)
    dy = torch.randn(4096, 11008, device=DEV, dtype=torch.bfloat16, generator=g) * 1e-4
    w = torch.randn(11008, 4096, device=DEV, dtype=torch.bfloat16, generator=g) * 0.02
    x = torch.randn(4096, 4096, device=DEV, dtype=torch.bfloat16, generator=g)
    if mx:
        qdy, sdy = sq.mx_quantize(dy, 1)
        qwt, swt = sq.mx_quantize_t(w, 0)           # W^T [4096 x 11008]: blocks along 11008
        qdyt, sdyt = sq.mx_quantize_t(dy, 1)        # dY^T [11008 x 4096]
        qxt, sxt = sq.mx_quantize_t(x, 0)           # X^T [4096 x 4096]
        cases = [
            ("mx dX", lambda out: sq.mx_scaled_gemm(qdy, 1, sdy, qwt, 0, swt, out=out, want_amax=True),
             (4096, 4096)),
            ("mx dW", lambda out: sq.mx_scaled_gemm(qdyt, 1, sdyt, qxt, 0, sxt, out=out, want_amax=True),
             (11008, 4096)),
        ]
    else:
        bdy, _, _ = sq.fp8_compute_scale(sq.fp8_amax(dy), 1, 0)
        bw, _, _ = sq.fp8_compute_scale(sq.fp8_amax(w), 0, 0)
        bx, _, _ = sq.fp8_compute_scale(sq.fp8_amax(x), 0, 0)
        qdy, _, _ = sq.fp8_quantize(dy, 1, bdy)
        qw, _, _ = sq.fp8_quantize(w, 0, bw)
        qx, _, _ = sq.fp8_quantize(x, 0, bx)
        cases = [
            ("dX", lambda out: sq.fp8_scaled_gemm(qdy, 1, bdy, qw, 0, bw, trans_b=True, out=out, want_amax=True),
             (4096, 4096)),
            ("dW", lambda out: sq.fp8_scaled_gemm(qdy, 1, bdy, qx, 0, bx, trans_a=True, trans_b=True, out=out,
                                                  want_amax=True), (11008, 4096)),
        ]
    for name, fn, shape in cases:
        def launch(out, fn=fn, shape=shape):
            if out is None:
                out = torch.empty(shape, device=DEV, dtype=torch.bfloat16)
            out.fill_(float("nan"))
            return fn(out)
        say(f"7b-mlp backward {name} x4 determinism")
        _repeat_identical(launch, 4, name)
