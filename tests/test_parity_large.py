"""Maximum sizes: tensors whose element offsets pass 2**31 and whose byte
offsets pass 4 GiB, on every kernel of the path.

A [49152 x 49152] bf16 tensor (2,415,919,104 elements, 4.8 GB) goes through
the amax passes, the per-tensor cast with its transposed copy and saturation
count, the MX casts (row blocks and column blocks, row-major and packed
scales) and the one-launch delayed step; a view of it starting one element
into each row goes through the element kernels.  A [589824 x 8192] code matrix
(4.8 GB; row 524288 starts at byte 2**32) goes through the per-tensor and
block-scaled GEMMs.  Inputs are drawn on the device by torch (uniform in
(-1, 1), with the largest magnitude planted past the 2**31-th element), so
the amax is known exactly without a host scan.  Rows and columns sampled on
both sides of the 2**31-element and 4 GiB boundaries are compared with the
oracle; whole outputs are compared between entry points on the device."""

import numpy as np
import pytest
import torch

import oracle
import scaled_quantize_fp8_amd as sq
from oracle import E4M3
from gpu_helpers import (DEV, assert_gemm_close, f32_bits_of, host, host_f64, i32_dev, mfma_operands_mx,
                         mfma_operands_pt, need_gpu, say)

pytestmark = pytest.mark.gpu

R = C = 49152                              # R * C > 2**31
PLANT = (48000, 48123)                     # element 2,359,344,123 > 2**31
ROWS = [0, 21845, 43690, 43691, PLANT[0], R - 1]   # row 43691 starts past 2**31 elements
COLS = [0, 31, PLANT[1], C - 1]


@pytest.fixture(scope="module")
def big():
    need_gpu()
    say(f"large: drawing x [{R} x {C}] bf16 on the device")
    g = torch.Generator(device=DEV).manual_seed(31)
    x = torch.empty(R, C, dtype=torch.bfloat16, device=DEV)
    for r in range(0, R, 4096):
        n = min(4096, R - r)
        x[r:r + n] = (torch.rand(n, C, device=DEV, generator=g) * 2 - 1).to(torch.bfloat16)
    x[PLANT] = -1000.0
    torch.cuda.synchronize()
    yield x
    del x
    torch.cuda.empty_cache()


def _row_vals(x, r):
    return oracle.bf16_bits_to_f64(host(x[r].view(torch.int16)).view(np.uint16))


def _col_vals(x, c):
    return oracle.bf16_bits_to_f64(host(x[:, c].contiguous().view(torch.int16)).view(np.uint16))


def test_large_per_tensor_cast_transpose_and_amax(big):
    x = big
    say("large: amax passes")
    assert host(sq.fp8_amax(x))[0] == 1000.0
    ws = sq.amax_scale_workspace(DEV)
    a, b, _, _ = sq.fp8_amax_scale(x, E4M3.code, ws)
    rb = oracle.compute_bias(1000.0, E4M3)
    assert host(a)[0] == 1000.0 and int(host(b)[0]) == rb
    # a bias 3 above the amax's: only the planted element saturates
    bs = rb + 3
    say(f"large: cast-transpose with amax and saturation count, bias {bs}")
    q, qT, am, n = sq.fp8_quantize_sat(x, E4M3.code, i32_dev(bs), transpose=True, want_amax=True)
    assert host(am)[0] == 1000.0 and int(host(n)[0]) == 1
    for r in ROWS:
        assert np.array_equal(host(q[r]), oracle.quantize(_row_vals(x, r), E4M3, bs)), r
    for c in COLS:
        assert np.array_equal(host(qT[c]), oracle.quantize(_col_vals(x, c), E4M3, bs)), c
    # the row-wise cast alone (one long row of 2.4e9 elements) writes the same codes
    q2, _, _ = sq.fp8_quantize(x, E4M3.code, i32_dev(bs))
    assert torch.equal(q2, q)


def test_large_mx_casts(big):
    x = big
    say("large: MX casts, row blocks")
    q, s = sq.mx_quantize(x, E4M3.code)
    for r in ROWS:
        rq, rs = oracle.mx_quantize(_row_vals(x, r)[None, :], E4M3)
        assert np.array_equal(host(q[r]), rq[0]) and np.array_equal(host(s[r]), rs[0]), r
    pq, ps = sq.mx_quantize_packed(x, E4M3.code)
    assert torch.equal(pq, q) and torch.equal(ps, sq.mx_pack_scales(s))
    del q, s, pq, ps
    torch.cuda.empty_cache()
    say("large: MX casts, column blocks (transposed)")
    qT, sT = sq.mx_quantize_t(x, E4M3.code)
    for c in COLS:
        rq, rs = oracle.mx_quantize(_col_vals(x, c)[None, :], E4M3)
        assert np.array_equal(host(qT[c]), rq[0]) and np.array_equal(host(sT[c]), rs[0]), c
    pqT, psT = sq.mx_quantize_t_packed(x, E4M3.code)
    assert torch.equal(pqT, qT) and torch.equal(psT, sq.mx_pack_scales(sT))


def test_large_delayed_step(big):
    x = big
    hist = torch.empty(16, dtype=torch.float32, device=DEV)
    state = torch.empty(2, dtype=torch.int32, device=DEV)
    sq.fp8_history_init(hist, state)
    sq.fp8_history_push(hist, state, sq.fp8_amax(x))
    ws = sq.amax_scale_workspace(DEV)
    say("large: one-launch delayed step with the transposed copy")
    q, qT, b, a, n = sq.fp8_quantize_delayed(x, E4M3.code, hist, state, ws, transpose=True, want_sat=True)
    rb = oracle.compute_bias(1000.0, E4M3)
    assert int(host(b)[0]) == rb and host(a)[0] == 1000.0 and int(host(n)[0]) == 0
    assert host(state).tolist() == [2, 2] and host(hist)[:2].tolist() == [1000.0, 1000.0]
    for r in ROWS:
        assert np.array_equal(host(q[r]), oracle.quantize(_row_vals(x, r), E4M3, rb)), r
    for c in COLS:
        assert np.array_equal(host(qT[c]), oracle.quantize(_col_vals(x, c), E4M3, rb)), c


def test_large_unaligned_view(big):
    """The element kernels at the same size: a view starting one element
    into each row (no 16-byte loads), 49120 columns (a multiple of 32)."""
    v = big[:, 1:C - 31]
    cols = [0, 30, PLANT[1] - 1, v.shape[1] - 1]
    say("large: unaligned view, element amax, cast-transpose and row-wise cast")
    assert host(sq.fp8_amax(v))[0] == 1000.0
    bs = oracle.compute_bias(1000.0, E4M3) + 3
    q, qT, am, n = sq.fp8_quantize_sat(v, E4M3.code, i32_dev(bs), transpose=True, want_amax=True)
    assert host(am)[0] == 1000.0 and int(host(n)[0]) == 1
    for r in ROWS:
        assert np.array_equal(host(q[r]), oracle.quantize(_row_vals(big, r)[1:C - 31], E4M3, bs)), r
    for c in cols:
        assert np.array_equal(host(qT[c]), oracle.quantize(_col_vals(big, c + 1), E4M3, bs)), c
    q2, _, am2, n2 = sq.fp8_quantize_sat(v, E4M3.code, i32_dev(bs), want_amax=True)
    assert torch.equal(q2, q) and host(am2)[0] == 1000.0 and int(host(n2)[0]) == 1
    del q, qT, q2
    torch.cuda.empty_cache()
    say("large: unaligned view, MX element kernel")
    mq, ms = sq.mx_quantize(v, E4M3.code)
    for r in ROWS:
        rq, rs = oracle.mx_quantize(_row_vals(big, r)[None, 1:C - 31], E4M3)
        assert np.array_equal(host(mq[r]), rq[0]) and np.array_equal(host(ms[r]), rs[0]), r


GM, GN, GK = 589824, 256, 8192            # A: 4.83 GB; row 524288 starts at byte 2**32
GROWS = [0, 1, 262144, 524287, 524288, 524289, GM - 256, GM - 1]


def _codes(rows, cols, g):
    """E4M3 codes, every finite value (0x00-0x7E, either sign), no NaN."""
    c = torch.randint(0, 0x7F, (rows, cols), device=DEV, dtype=torch.uint8, generator=g)
    s = torch.randint(0, 2, (rows, cols), device=DEV, dtype=torch.uint8, generator=g)
    return c | (s << 7)


def test_large_gemms_past_4gib():
    need_gpu()
    say(f"large: GEMM operands A [{GM} x {GK}], B [{GN} x {GK}] codes")
    g = torch.Generator(device=DEV).manual_seed(32)
    A = torch.empty(GM, GK, dtype=torch.uint8, device=DEV)
    for r in range(0, GM, 65536):
        A[r:r + 65536] = _codes(min(65536, GM - r), GK, g)
    B = _codes(GN, GK, g)
    ba, bb = 9, 8                            # products up to 448^2 * 8192, scaled down by 2^-17
    rows = np.array(GROWS)
    hA, hB = host(A[torch.from_numpy(rows).to(DEV)]), host(B)
    say("large: per-tensor GEMM")
    Cp, am = sq.fp8_scaled_gemm(A, E4M3.code, i32_dev(ba), B, E4M3.code, i32_dev(bb), want_amax=True)
    y = oracle.scaled_gemm_ref(hA, E4M3, ba, hB, E4M3, bb)
    sabs = oracle.abs_product_sum(hA, E4M3, ba, hB, E4M3, bb)
    assert_gemm_close(host_f64(Cp[torch.from_numpy(rows).to(DEV)]), y, sabs, True, "large pt",
                      mfma_operands_pt(hA, E4M3, ba, hB, E4M3, bb))
    assert f32_bits_of(am) == f32_bits_of(sq.fp8_amax(Cp))
    del Cp
    say("large: block-scaled GEMM, row-major and packed scales")
    sa = torch.randint(120, 135, (GM, GK // 32), device=DEV, dtype=torch.uint8, generator=g)
    sb = torch.randint(120, 135, (GN, GK // 32), device=DEV, dtype=torch.uint8, generator=g)
    Cm, amm = sq.mx_scaled_gemm(A, E4M3.code, sa, B, E4M3.code, sb, want_amax=True)
    Ck, amk = sq.mx_scaled_gemm_packed(A, E4M3.code, sq.mx_pack_scales(sa), B, E4M3.code, sq.mx_pack_scales(sb),
                                       want_amax=True)
    assert torch.equal(Ck.view(torch.int16), Cm.view(torch.int16)) and f32_bits_of(amk) == f32_bits_of(amm)
    hsa, hsb = host(sa[torch.from_numpy(rows).to(DEV)]), host(sb)
    y = oracle.mx_gemm_ref(hA, hsa, E4M3, hB, hsb, E4M3)
    sabs = oracle.mx_abs_product_sum(hA, hsa, E4M3, hB, hsb, E4M3)
    assert_gemm_close(host_f64(Cm[torch.from_numpy(rows).to(DEV)]), y, sabs, True, "large mx",
                      mfma_operands_mx(hA, hsa, E4M3, hB, hsb, E4M3))
    assert f32_bits_of(amm) == f32_bits_of(sq.fp8_amax(Cm))
