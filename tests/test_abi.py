"""C-ABI checks that run without a GPU: the library loads, exports every
function ``include/scaled_fp8.h`` declares, and rejects bad arguments with
the documented status codes before making any HIP call (so no call here
touches a device: every one of them fails host-side validation)."""

import ctypes
import os
import re

import pytest

import scaled_quantize_fp8_amd as sq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "scaled_fp8.h")

OK, NULL, SHAPE, ALIGN, DTYPE, FORMAT, LAUNCH, UNSUP = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = 0x10000          # 16-byte aligned, never dereferenced (validation fails first)
S = None                # default stream


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sq.library_path()):
        pytest.skip("libscaled_fp8.so not built")
    return sq.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(fp8_\w+|mx_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for want in ["fp8_amax", "fp8_compute_scale", "fp8_history_init", "fp8_history_push",
                 "fp8_compute_scale_delayed", "fp8_quantize", "mx_quantize", "mx_quantize_t",
                 "mx_quantize_rule", "mx_quantize_t_rule", "fp8_scaled_gemm", "mx_scaled_gemm", "fp8_status_string",
                 "fp8_abi_version", "mx_packed_scales_bytes", "mx_pack_scales", "mx_quantize_packed",
                 "mx_quantize_t_packed", "mx_scaled_gemm_packed", "fp8_quantize_sat", "fp8_amax_scale",
                 "fp8_amax_scale_noalloc", "fp8_quantize_delayed"]:
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert sq.fp8_status_string(OK) == "ok"
    for code in (NULL, SHAPE, ALIGN, DTYPE, FORMAT, LAUNCH, UNSUP):
        assert sq.fp8_status_string(code) not in ("ok", "unknown status")
    assert sq.fp8_status_string(-99) == "unknown status"
    assert sq.fp8_abi_version() >= 6


def test_amax_validation(lib):
    assert lib.fp8_amax(FAKE, 0, 4, 4, 4, None, S) == NULL
    assert lib.fp8_amax(FAKE, 7, 4, 4, 4, FAKE, S) == DTYPE
    assert lib.fp8_amax(FAKE, 0, 4, 8, 4, FAKE, S) == SHAPE          # ld < cols
    assert lib.fp8_amax(FAKE, 0, -1, 8, 8, FAKE, S) == SHAPE
    assert lib.fp8_amax(None, 0, 4, 4, 4, FAKE, S) == NULL


def test_amax_scale_validation(lib):
    a = lib.fp8_amax_scale
    # x, dtype, rows, cols, ld, fmt, margin, amax, bias, scale, scale_inv, workspace, stream
    assert a(FAKE, 0, 4, 4, 4, 0, 0, FAKE, FAKE, None, None, None, S) == NULL       # workspace
    assert a(FAKE, 0, 4, 4, 4, 0, 0, None, FAKE, None, None, FAKE, S) == NULL       # amax
    assert a(FAKE, 0, 4, 4, 4, 0, 0, FAKE, None, None, None, FAKE, S) == NULL       # bias
    assert a(FAKE, 0, 4, 4, 4, 0, 0, FAKE, FAKE, None, None, FAKE + 2, S) == ALIGN
    assert a(FAKE, 9, 4, 4, 4, 0, 0, FAKE, FAKE, None, None, FAKE, S) == DTYPE
    assert a(FAKE, 0, 4, 4, 4, 3, 0, FAKE, FAKE, None, None, FAKE, S) == FORMAT
    assert a(FAKE, 0, 4, 8, 4, 0, 0, FAKE, FAKE, None, None, FAKE, S) == SHAPE
    assert a(None, 0, 4, 4, 4, 0, 0, FAKE, FAKE, None, None, FAKE, S) == NULL
    n = lib.fp8_amax_scale_noalloc          # rejected before the scratch lookup (no HIP call)
    assert n(FAKE, 0, 4, 4, 4, 0, 0, None, FAKE, None, None, S) == NULL
    assert n(FAKE, 0, 4, 4, 4, 0, 0, FAKE, None, None, None, S) == NULL
    assert n(FAKE, 9, 4, 4, 4, 0, 0, FAKE, FAKE, None, None, S) == DTYPE
    assert n(FAKE, 0, 4, 4, 4, 3, 0, FAKE, FAKE, None, None, S) == FORMAT
    assert n(FAKE, 0, 4, 8, 4, 0, 0, FAKE, FAKE, None, None, S) == SHAPE
    assert n(None, 0, 4, 4, 4, 0, 0, FAKE, FAKE, None, None, S) == NULL


def test_scale_and_history_validation(lib):
    assert lib.fp8_compute_scale(None, 0, 0, FAKE, None, None, S) == NULL
    assert lib.fp8_compute_scale(FAKE, 0, 0, None, None, None, S) == NULL
    assert lib.fp8_compute_scale(FAKE, 2, 0, FAKE, None, None, S) == FORMAT
    assert lib.fp8_history_init(None, FAKE, 16, S) == NULL
    assert lib.fp8_history_init(FAKE, FAKE, 0, S) == SHAPE
    assert lib.fp8_history_init(FAKE, FAKE, 4097, S) == SHAPE
    assert lib.fp8_history_push(FAKE, FAKE, 16, None, S) == NULL
    assert lib.fp8_history_push(FAKE, FAKE, -3, FAKE, S) == SHAPE
    assert lib.fp8_compute_scale_delayed(FAKE, FAKE, 16, 9, 0, FAKE, None, None, S) == FORMAT
    assert lib.fp8_compute_scale_delayed(FAKE, None, 16, 0, 0, FAKE, None, None, S) == NULL
    assert lib.fp8_compute_scale_delayed(FAKE, FAKE, 0, 0, 0, FAKE, None, None, S) == SHAPE


def test_quantize_delayed_validation(lib):
    d = lib.fp8_quantize_delayed
    # x, dtype, rows, cols, ld, fmt, margin, hist, state, window, q, ldq, qT, ldqT, bias, amax, sat, ws, stream
    ok = [FAKE, 0, 4, 4, 4, 0, 0, FAKE, FAKE, 16, FAKE, 4, None, 0, FAKE, FAKE, None, FAKE, S]

    def call(**kw):
        args = list(ok)
        names = ["x", "dtype", "rows", "cols", "ld", "fmt", "margin", "hist", "state", "window", "q", "ldq", "qT",
                 "ldqT", "bias", "amax", "sat", "ws", "stream"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return d(*args)
    for k in ("hist", "state", "q", "bias", "amax", "ws"):
        assert call(**{k: None}) == NULL, k
    assert call(window=0) == SHAPE
    assert call(window=4097) == SHAPE
    assert call(dtype=5) == DTYPE
    assert call(fmt=2) == FORMAT
    assert call(ld=2) == SHAPE
    assert call(ldq=3) == SHAPE
    assert call(qT=FAKE, ldqT=2) == SHAPE
    assert call(x=None) == NULL
    assert call(ws=FAKE + 4) == ALIGN              # 4-byte aligned, the 64-bit count needs 8


def test_quantize_validation(lib):
    q = lib.fp8_quantize
    assert q(FAKE, 0, 4, 4, 4, 0, None, FAKE, 4, None, 0, None, S) == NULL      # bias
    assert q(FAKE, 0, 4, 4, 4, 0, FAKE, None, 4, None, 0, None, S) == NULL      # q
    assert q(FAKE, 3, 4, 4, 4, 0, FAKE, FAKE, 4, None, 0, None, S) == DTYPE
    assert q(FAKE, 0, 4, 4, 4, 5, FAKE, FAKE, 4, None, 0, None, S) == FORMAT
    assert q(FAKE, 0, 4, 4, 2, 0, FAKE, FAKE, 4, None, 0, None, S) == SHAPE     # ld
    assert q(FAKE, 0, 4, 4, 4, 0, FAKE, FAKE, 3, None, 0, None, S) == SHAPE     # ldq
    assert q(FAKE, 0, 4, 8, 8, 0, FAKE, FAKE, 8, FAKE, 2, None, S) == SHAPE     # ldqT < rows
    assert q(None, 0, 4, 4, 4, 0, FAKE, FAKE, 4, None, 0, None, S) == NULL
    qs = lib.fp8_quantize_sat
    assert qs(FAKE, 0, 4, 4, 4, 0, FAKE, FAKE, 4, None, 0, None, None, S) == NULL  # sat_out required
    assert qs(FAKE, 0, 4, 4, 4, 0, None, FAKE, 4, None, 0, None, FAKE, S) == NULL  # bias
    assert qs(FAKE, 3, 4, 4, 4, 0, FAKE, FAKE, 4, None, 0, None, FAKE, S) == DTYPE
    assert qs(FAKE, 0, 4, 4, 4, 5, FAKE, FAKE, 4, None, 0, None, FAKE, S) == FORMAT
    assert qs(FAKE, 0, 4, 4, 2, 0, FAKE, FAKE, 4, None, 0, None, FAKE, S) == SHAPE
    assert qs(FAKE, 0, 4, 8, 8, 0, FAKE, FAKE, 8, FAKE, 2, None, FAKE, S) == SHAPE
    m = lib.mx_quantize
    assert m(FAKE, 0, 4, 48, 48, 0, FAKE, 48, FAKE, 2, S) == SHAPE              # cols % 32
    assert m(FAKE, 0, 4, 64, 64, 0, None, 64, FAKE, 2, S) == NULL
    assert m(FAKE, 0, 4, 64, 64, 0, FAKE, 64, None, 2, S) == NULL
    assert m(FAKE, 0, 4, 64, 64, 0, FAKE, 64, FAKE, 1, S) == SHAPE              # ld_scales
    assert m(FAKE, 2, 4, 64, 64, 0, FAKE, 64, FAKE, 2, S) == DTYPE
    assert m(FAKE, 0, 4, 64, 64, 2, FAKE, 64, FAKE, 2, S) == FORMAT
    t = lib.mx_quantize_t
    # x, dtype, rows, cols, ld, fmt, qT, ldqT, scalesT, ld_scales, s
    assert t(FAKE, 0, 48, 8, 8, 0, FAKE, 48, FAKE, 2, S) == SHAPE                # rows % 32
    assert t(FAKE, 0, 64, 8, 8, 0, None, 64, FAKE, 2, S) == NULL
    assert t(FAKE, 0, 64, 8, 8, 0, FAKE, 64, None, 2, S) == NULL
    assert t(FAKE, 0, 64, 8, 8, 0, FAKE, 32, FAKE, 2, S) == SHAPE                # ldqT < rows
    assert t(FAKE, 0, 64, 8, 8, 0, FAKE, 64, FAKE, 1, S) == SHAPE                # ld_scales
    assert t(FAKE, 0, 64, 8, 4, 0, FAKE, 64, FAKE, 2, S) == SHAPE                # ld < cols
    assert t(FAKE, 5, 64, 8, 8, 0, FAKE, 64, FAKE, 2, S) == DTYPE
    assert t(FAKE, 0, 64, 8, 8, 3, FAKE, 64, FAKE, 2, S) == FORMAT
    assert t(None, 0, 64, 8, 8, 0, FAKE, 64, FAKE, 2, S) == NULL


def test_mx_rule_validation(lib):
    m = lib.mx_quantize_rule
    # x, dtype, rows, cols, ld, fmt, rule, q, ldq, scales, ld_scales, s
    assert m(FAKE, 0, 4, 64, 64, 0, 2, FAKE, 64, FAKE, 2, S) == FORMAT          # unknown rule
    assert m(FAKE, 0, 4, 64, 64, 0, -1, FAKE, 64, FAKE, 2, S) == FORMAT
    assert m(FAKE, 0, 4, 64, 64, 2, 1, FAKE, 64, FAKE, 2, S) == FORMAT
    assert m(FAKE, 0, 4, 48, 48, 0, 1, FAKE, 48, FAKE, 2, S) == SHAPE           # cols % 32
    assert m(FAKE, 0, 4, 64, 64, 0, 1, None, 64, FAKE, 2, S) == NULL
    assert m(FAKE, 2, 4, 64, 64, 0, 1, FAKE, 64, FAKE, 2, S) == DTYPE
    assert m(FAKE, 0, 4, 64, 64, 0, 1, FAKE, 64, FAKE, 1, S) == SHAPE           # ld_scales
    assert m(None, 0, 4, 64, 64, 0, 1, FAKE, 64, FAKE, 2, S) == NULL
    assert m(None, 0, 0, 64, 64, 0, 1, FAKE, 64, FAKE, 2, S) == OK              # empty: no launch
    t = lib.mx_quantize_t_rule
    assert t(FAKE, 0, 64, 8, 8, 0, 7, FAKE, 64, FAKE, 2, S) == FORMAT
    assert t(FAKE, 0, 48, 8, 8, 0, 1, FAKE, 48, FAKE, 2, S) == SHAPE            # rows % 32
    assert t(FAKE, 0, 64, 8, 8, 0, 1, FAKE, 64, None, 2, S) == NULL
    assert t(FAKE, 0, 64, 8, 8, 0, 1, FAKE, 32, FAKE, 2, S) == SHAPE            # ldqT < rows
    assert t(None, 0, 64, 8, 8, 0, 1, FAKE, 64, FAKE, 2, S) == NULL


def test_gemm_validation(lib):
    g = lib.fp8_scaled_gemm
    # M, N, K, A, fa, ta, lda, ba, B, fb, tb, ldb, bb, C, dt, ldc, amax, s
    assert g(64, 64, 64, FAKE, 0, 0, 64, None, FAKE, 0, 0, 64, FAKE, FAKE, 0, 64, None, S) == NULL
    assert g(64, 64, 64, FAKE, 4, 0, 64, FAKE, FAKE, 0, 0, 64, FAKE, FAKE, 0, 64, None, S) == FORMAT
    assert g(64, 64, 64, FAKE, 0, 0, 64, FAKE, FAKE, 0, 0, 64, FAKE, FAKE, 9, 64, None, S) == DTYPE
    assert g(64, 64, 40, FAKE, 0, 0, 48, FAKE, FAKE, 0, 0, 48, FAKE, FAKE, 0, 64, None, S) == SHAPE
    assert g(64, 64, 64, FAKE, 0, 0, 32, FAKE, FAKE, 0, 0, 64, FAKE, FAKE, 0, 64, None, S) == SHAPE
    assert g(64, 64, 64, FAKE, 0, 0, 64, FAKE, FAKE, 0, 0, 64, FAKE, FAKE, 0, 32, None, S) == SHAPE
    assert g(40, 64, 64, FAKE, 0, 1, 48, FAKE, FAKE, 0, 0, 64, FAKE, FAKE, 0, 64, None, S) == SHAPE
    assert g(64, 64, 64, FAKE + 8, 0, 0, 64, FAKE, FAKE, 0, 0, 64, FAKE, FAKE, 0, 64, None, S) == ALIGN
    assert g(64, 64, 64, FAKE, 0, 0, 72, FAKE, FAKE, 0, 0, 64, FAKE, FAKE, 0, 64, None, S) == ALIGN
    assert g(64, 64, 64, None, 0, 0, 64, FAKE, FAKE, 0, 0, 64, FAKE, FAKE, 0, 64, None, S) == NULL
    assert g(64, 64, 64, FAKE, 0, 0, 64, FAKE, FAKE, 0, 0, 64, FAKE, None, 0, 64, None, S) == NULL
    assert g(64, 64, 64, FAKE, 0, 0, 1 << 23, FAKE, FAKE, 0, 0, 64, FAKE, FAKE, 0, 64, None, S) == UNSUP
    mg = lib.mx_scaled_gemm
    # M, N, K, A, fa, lda, As, ldsa, B, fb, ldb, Bs, ldsb, C, dt, ldc, amax, s
    assert mg(64, 64, 48, FAKE, 0, 48, FAKE, 4, FAKE, 0, 48, FAKE, 4, FAKE, 0, 64, None, S) == SHAPE
    assert mg(64, 64, 64, FAKE, 0, 64, None, 4, FAKE, 0, 64, FAKE, 4, FAKE, 0, 64, None, S) == NULL
    assert mg(64, 64, 64, FAKE, 0, 64, FAKE, 1, FAKE, 0, 64, FAKE, 4, FAKE, 0, 64, None, S) == SHAPE
    assert mg(64, 64, 64, FAKE + 4, 0, 64, FAKE, 4, FAKE, 0, 64, FAKE, 4, FAKE, 0, 64, None, S) == ALIGN
    assert mg(64, 64, 64, FAKE, 0, 64, FAKE, 2, FAKE, 0, 72, FAKE, 4, FAKE, 0, 64, None, S) == ALIGN
    assert mg(64, 64, 64, FAKE, 3, 64, FAKE, 4, FAKE, 0, 64, FAKE, 4, FAKE, 0, 64, None, S) == FORMAT


def test_packed_scales_size_and_validation(lib):
    """Size formula of the packed E8M0 layout (256-row tiles x 16-block groups
    x 4 KiB) and the host-side checks of the two packed entry points."""
    assert sq.mx_packed_scales_bytes(0, 0) == 0
    assert sq.mx_packed_scales_bytes(1, 1) == 4096
    assert sq.mx_packed_scales_bytes(256, 16) == 4096
    assert sq.mx_packed_scales_bytes(257, 16) == 8192
    assert sq.mx_packed_scales_bytes(256, 17) == 8192
    assert sq.mx_packed_scales_bytes(16384, 256) == 64 * 16 * 4096
    assert sq.mx_packed_scales_bytes(300, 20) == 2 * 2 * 4096
    assert lib.mx_packed_scales_bytes(-1, 4) == SHAPE
    p = lib.mx_pack_scales
    # scales, rows, kblocks, ld, packed, s
    assert p(FAKE, 4, 8, 4, FAKE, S) == SHAPE
    assert p(FAKE, -1, 8, 8, FAKE, S) == SHAPE
    assert p(None, 4, 8, 8, FAKE, S) == NULL
    assert p(FAKE, 4, 8, 8, None, S) == NULL
    assert p(FAKE, 4, 8, 8, FAKE + 4, S) == ALIGN
    assert p(None, 0, 0, 0, None, S) == OK
    c = lib.mx_quantize_packed
    # x, dt, rows, cols, ld, fmt, rule, q, ldq, packed, s
    assert c(FAKE, 0, 4, 64, 64, 0, 0, None, 64, FAKE, S) == NULL
    assert c(FAKE, 0, 4, 64, 64, 0, 0, FAKE, 64, None, S) == NULL
    assert c(FAKE, 0, 4, 48, 48, 0, 0, FAKE, 48, FAKE, S) == SHAPE
    assert c(FAKE, 0, 4, 64, 32, 0, 0, FAKE, 64, FAKE, S) == SHAPE
    assert c(FAKE, 0, 4, 64, 64, 0, 0, FAKE, 64, FAKE + 8, S) == ALIGN
    assert c(FAKE, 5, 4, 64, 64, 0, 0, FAKE, 64, FAKE, S) == DTYPE
    assert c(FAKE, 0, 4, 64, 64, 3, 0, FAKE, 64, FAKE, S) == FORMAT
    assert c(FAKE, 0, 4, 64, 64, 0, 9, FAKE, 64, FAKE, S) == FORMAT
    assert c(None, 0, 4, 64, 64, 0, 0, FAKE, 64, FAKE, S) == NULL
    t = lib.mx_quantize_t_packed
    # x, dt, rows, cols, ld, fmt, rule, qT, ldqT, packed, s
    assert t(FAKE, 0, 64, 16, 16, 0, 0, None, 64, FAKE, S) == NULL
    assert t(FAKE, 0, 48, 16, 16, 0, 0, FAKE, 48, FAKE, S) == SHAPE
    assert t(FAKE, 0, 64, 16, 16, 0, 0, FAKE, 32, FAKE, S) == SHAPE
    assert t(FAKE, 0, 64, 16, 16, 0, 0, FAKE, 64, FAKE + 4, S) == ALIGN
    assert t(FAKE, 0, 64, 16, 16, 0, 7, FAKE, 64, FAKE, S) == FORMAT
    g = lib.mx_scaled_gemm_packed
    # M, N, K, A, fa, lda, Ap, B, fb, ldb, Bp, C, dt, ldc, amax, s
    assert g(64, 64, 0, FAKE, 0, 16, FAKE, FAKE, 0, 16, FAKE, FAKE, 0, 64, None, S) == UNSUP
    assert g(64, 64, 48, FAKE, 0, 48, FAKE, FAKE, 0, 48, FAKE, FAKE, 0, 64, None, S) == SHAPE
    assert g(64, 64, 512, FAKE, 0, 512, None, FAKE, 0, 512, FAKE, FAKE, 0, 64, None, S) == NULL
    assert g(64, 64, 512, FAKE, 0, 512, FAKE, FAKE, 0, 512, FAKE + 4, FAKE, 0, 64, None, S) == ALIGN
    assert g(64, 64, 512, FAKE + 4, 0, 512, FAKE, FAKE, 0, 512, FAKE, FAKE, 0, 64, None, S) == ALIGN
    assert g(64, 64, 512, FAKE, 2, 512, FAKE, FAKE, 0, 512, FAKE, FAKE, 0, 64, None, S) == FORMAT
    assert g(64, 64, 512, FAKE, 0, 512, FAKE, FAKE, 0, 512, FAKE, FAKE, 7, 64, None, S) == DTYPE
    assert g(64, 64, 512, FAKE, 0, 512, FAKE, FAKE, 0, 512, FAKE, FAKE, 0, 32, None, S) == SHAPE
    assert g(64, 64, 512, FAKE, 0, 512, FAKE, FAKE, 0, 512, FAKE, None, 0, 64, None, S) == NULL


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sq.fp8_amax(x)
    with pytest.raises(ValueError):
        sq.mx_quantize(torch.zeros(4, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        sq.mx_quantize_t(torch.zeros(32, 4, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        sq.mx_quantize_rule(torch.zeros(4, 32, dtype=torch.bfloat16), rule="ocp")
    with pytest.raises(ValueError):
        sq.mx_quantize_rule(torch.zeros(4, 32, dtype=torch.bfloat16), rule="nearest")
    with pytest.raises(ValueError):
        sq.mx_quantize_t_rule(torch.zeros(32, 4, dtype=torch.bfloat16), rule="ocp")
