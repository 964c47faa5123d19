"""scaled_quantize_fp8_amd — scaled FP8 linear-layer kernels for MI355X (gfx950).

A thin ctypes binding over ``libscaled_fp8.so`` (C ABI declared in
``include/scaled_fp8.h``).  Each function here has the name of the C entry
point it marshals arguments for; every step of the computation runs in the
library's HIP kernels on the tensors' device and on the current HIP stream.
PyTorch only supplies device memory and the stream.  There is no CPU
implementation behind this module: a missing library or a CPU tensor raises.

FP8 tensors are ``torch.uint8`` holding OCP E4M3 / E5M2 codes; E8M0 block
scales are ``torch.uint8`` codes; biases are ``torch.int32`` device scalars.
Matrices are 2-D row-major (``stride(1) == 1``); the leading dimension is
``stride(0)``.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "E4M3", "E5M2", "load_library", "library_path", "Fp8Error",
    "fp8_amax", "fp8_amax_scale", "fp8_amax_scale_noalloc", "amax_scale_workspace", "AMAX_SCALE_WORKSPACE_BYTES",
    "fp8_compute_scale", "fp8_history_init", "fp8_history_push",
    "fp8_compute_scale_delayed", "fp8_quantize", "fp8_quantize_sat", "fp8_quantize_delayed", "mx_quantize",
    "mx_quantize_t",
    "mx_quantize_rule", "mx_quantize_t_rule", "MX_RULE_FMAX", "MX_RULE_OCP",
    "fp8_scaled_gemm", "mx_scaled_gemm", "fp8_status_string", "fp8_abi_version",
    "mx_packed_scales_bytes", "mx_pack_scales", "mx_quantize_packed", "mx_quantize_t_packed",
    "mx_scaled_gemm_packed",
]

E4M3 = 0
E5M2 = 1
_DT_BF16 = 0
_DT_F32 = 1
_FMT_NAMES = {"e4m3": E4M3, "e5m2": E5M2, E4M3: E4M3, E5M2: E5M2}
MX_RULE_FMAX = 0
MX_RULE_OCP = 1
AMAX_SCALE_WORKSPACE_BYTES = 256       # FP8_AMAX_SCALE_WORKSPACE_BYTES
_RULE_NAMES = {"fmax": MX_RULE_FMAX, "ocp": MX_RULE_OCP, MX_RULE_FMAX: MX_RULE_FMAX,
               MX_RULE_OCP: MX_RULE_OCP}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64

_SIGNATURES = {
    "fp8_status_string": ([_i], ctypes.c_char_p),
    "fp8_abi_version": ([], _i),
    "fp8_amax": ([_p, _i, _i64, _i64, _i64, _p, _p], _i),
    "fp8_amax_scale": ([_p, _i, _i64, _i64, _i64, _i, _i, _p, _p, _p, _p, _p, _p], _i),
    "fp8_amax_scale_noalloc": ([_p, _i, _i64, _i64, _i64, _i, _i, _p, _p, _p, _p, _p], _i),
    "fp8_compute_scale": ([_p, _i, _i, _p, _p, _p, _p], _i),
    "fp8_history_init": ([_p, _p, _i, _p], _i),
    "fp8_history_push": ([_p, _p, _i, _p, _p], _i),
    "fp8_compute_scale_delayed": ([_p, _p, _i, _i, _i, _p, _p, _p, _p], _i),
    "fp8_quantize": ([_p, _i, _i64, _i64, _i64, _i, _p, _p, _i64, _p, _i64, _p, _p], _i),
    "fp8_quantize_sat": ([_p, _i, _i64, _i64, _i64, _i, _p, _p, _i64, _p, _i64, _p, _p, _p], _i),
    "fp8_quantize_delayed": ([_p, _i, _i64, _i64, _i64, _i, _i, _p, _p, _i, _p, _i64, _p, _i64, _p, _p, _p, _p,
                              _p], _i),
    "mx_quantize": ([_p, _i, _i64, _i64, _i64, _i, _p, _i64, _p, _i64, _p], _i),
    "mx_quantize_t": ([_p, _i, _i64, _i64, _i64, _i, _p, _i64, _p, _i64, _p], _i),
    "mx_quantize_rule": ([_p, _i, _i64, _i64, _i64, _i, _i, _p, _i64, _p, _i64, _p], _i),
    "mx_quantize_t_rule": ([_p, _i, _i64, _i64, _i64, _i, _i, _p, _i64, _p, _i64, _p], _i),
    "fp8_scaled_gemm": ([_i64, _i64, _i64, _p, _i, _i, _i64, _p, _p, _i, _i, _i64, _p,
                         _p, _i, _i64, _p, _p], _i),
    "mx_scaled_gemm": ([_i64, _i64, _i64, _p, _i, _i64, _p, _i64, _p, _i, _i64, _p, _i64,
                        _p, _i, _i64, _p, _p], _i),
    "mx_packed_scales_bytes": ([_i64, _i64], _i64),
    "mx_pack_scales": ([_p, _i64, _i64, _i64, _p, _p], _i),
    "mx_quantize_packed": ([_p, _i, _i64, _i64, _i64, _i, _i, _p, _i64, _p, _p], _i),
    "mx_quantize_t_packed": ([_p, _i, _i64, _i64, _i64, _i, _i, _p, _i64, _p, _p], _i),
    "mx_scaled_gemm_packed": ([_i64, _i64, _i64, _p, _i, _i64, _p, _p, _i, _i64, _p,
                               _p, _i, _i64, _p, _p], _i),
}


class Fp8Error(RuntimeError):
    """A library call returned a negative status."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status} ({fp8_status_string(status)})")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libscaled_fp8.so")


def load_library() -> ctypes.CDLL:
    """Load libscaled_fp8.so (built in-tree); raise if it has not been built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m scaled_quantize_fp8_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = lib
    return _LIB


def fp8_status_string(status: int) -> str:
    return load_library().fp8_status_string(int(status)).decode()


def fp8_abi_version() -> int:
    return int(load_library().fp8_abi_version())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Fp8Error(fn, status)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device}); there is no CPU path")
    return t


def _mat(t: torch.Tensor, name: str):
    _dev(t, name)
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.shape[0] > 0 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must be row-major (stride(1) == 1)")
    ld = t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)
    return t.shape[0], t.shape[1], ld


def _dtype_code(t: torch.Tensor, name: str) -> int:
    if t.dtype == torch.bfloat16:
        return _DT_BF16
    if t.dtype == torch.float32:
        return _DT_F32
    raise ValueError(f"{name} must be bfloat16 or float32, got {t.dtype}")


def _fmt(fmt) -> int:
    if fmt not in _FMT_NAMES:
        raise ValueError(f"unknown FP8 format {fmt!r}")
    return _FMT_NAMES[fmt]


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _u8(t: torch.Tensor, name: str) -> torch.Tensor:
    _dev(t, name)
    if t.dtype != torch.uint8:
        raise ValueError(f"{name} must be uint8 (FP8 / E8M0 codes), got {t.dtype}")
    return t


def _scalar(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    _dev(t, name)
    if t.dtype != dtype or t.numel() < 1:
        raise ValueError(f"{name} must be a {dtype} device tensor with at least one element")
    return t


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def fp8_amax(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """max |x| of a 2-D bf16/f32 tensor, as a float32 device tensor of shape [1]."""
    rows, cols, ld = _mat(x, "x")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _scalar(out, torch.float32, "out")
    _check("fp8_amax", load_library().fp8_amax(
        _ptr(x), _dtype_code(x, "x"), rows, cols, ld, _ptr(out), _stream(x)))
    return out


def amax_scale_workspace(device) -> torch.Tensor:
    """A zeroed workspace for fp8_amax_scale (FP8_AMAX_SCALE_WORKSPACE_BYTES);
    each call leaves it zero again, so one per stream of calls suffices."""
    return torch.zeros(AMAX_SCALE_WORKSPACE_BYTES // 4, dtype=torch.int32, device=device)


def _amax_scale_outputs(x, amax_out, bias_out, scale_out, scale_inv_out, want_scales):
    if amax_out is None:
        amax_out = torch.empty(1, dtype=torch.float32, device=x.device)
    if bias_out is None:
        bias_out = torch.empty(1, dtype=torch.int32, device=x.device)
    _scalar(amax_out, torch.float32, "amax_out")
    _scalar(bias_out, torch.int32, "bias_out")
    if want_scales:
        if scale_out is None:
            scale_out = torch.empty(1, dtype=torch.float32, device=x.device)
        if scale_inv_out is None:
            scale_inv_out = torch.empty(1, dtype=torch.float32, device=x.device)
    for t, n in ((scale_out, "scale_out"), (scale_inv_out, "scale_inv_out")):
        if t is not None:
            _scalar(t, torch.float32, n)
    return amax_out, bias_out, scale_out, scale_inv_out


def fp8_amax_scale(x: torch.Tensor, fmt, workspace: torch.Tensor, margin: int = 0, amax_out=None, bias_out=None,
                   scale_out=None, scale_inv_out=None, want_scales: bool = False):
    """Current scaling in one launch: amax of x and its bias (and optionally
    2**bias, 2**-bias).  ``workspace``: a device tensor of at least
    AMAX_SCALE_WORKSPACE_BYTES, zero before the first use
    (amax_scale_workspace); each call leaves it zero.  Returns
    (amax, bias, scale or None, scale_inv or None)."""
    rows, cols, ld = _mat(x, "x")
    _dev(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < AMAX_SCALE_WORKSPACE_BYTES or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor of AMAX_SCALE_WORKSPACE_BYTES")
    amax_out, bias_out, scale_out, scale_inv_out = _amax_scale_outputs(x, amax_out, bias_out, scale_out,
                                                                       scale_inv_out, want_scales)
    _check("fp8_amax_scale", load_library().fp8_amax_scale(
        _ptr(x), _dtype_code(x, "x"), rows, cols, ld, _fmt(fmt), int(margin), _ptr(amax_out), _ptr(bias_out),
        _ptr(scale_out), _ptr(scale_inv_out), _ptr(workspace), _stream(x)))
    return amax_out, bias_out, scale_out, scale_inv_out


def fp8_amax_scale_noalloc(x: torch.Tensor, fmt, margin: int = 0, amax_out=None, bias_out=None, scale_out=None,
                           scale_inv_out=None, want_scales: bool = False):
    """fp8_amax_scale with the reduction state in the library's own per-GPU
    array (the C entry point allocates nothing; calls that overlap on one GPU
    race).  Returns (amax, bias, scale or None, scale_inv or None)."""
    rows, cols, ld = _mat(x, "x")
    amax_out, bias_out, scale_out, scale_inv_out = _amax_scale_outputs(x, amax_out, bias_out, scale_out,
                                                                       scale_inv_out, want_scales)
    _check("fp8_amax_scale_noalloc", load_library().fp8_amax_scale_noalloc(
        _ptr(x), _dtype_code(x, "x"), rows, cols, ld, _fmt(fmt), int(margin), _ptr(amax_out), _ptr(bias_out),
        _ptr(scale_out), _ptr(scale_inv_out), _stream(x)))
    return amax_out, bias_out, scale_out, scale_inv_out


def fp8_compute_scale(amax: torch.Tensor, fmt, margin: int = 0, bias_out=None,
                      scale_out=None, scale_inv_out=None):
    """Bias floor(log2(fmax/amax)) - margin; returns (bias int32[1],
    scale float32[1], scale_inv float32[1])."""
    _scalar(amax, torch.float32, "amax")
    dev = amax.device
    bias_out = torch.empty(1, dtype=torch.int32, device=dev) if bias_out is None else bias_out
    scale_out = torch.empty(1, dtype=torch.float32, device=dev) if scale_out is None else scale_out
    scale_inv_out = torch.empty(1, dtype=torch.float32, device=dev) if scale_inv_out is None else scale_inv_out
    _check("fp8_compute_scale", load_library().fp8_compute_scale(
        _ptr(amax), _fmt(fmt), int(margin), _ptr(bias_out), _ptr(scale_out),
        _ptr(scale_inv_out), _stream(amax)))
    return bias_out, scale_out, scale_inv_out


def fp8_history_init(hist: torch.Tensor, state: torch.Tensor) -> None:
    """Zero a delayed-scaling history (float32[window]) and its state (int32[2])."""
    _scalar(hist, torch.float32, "hist")
    _scalar(state, torch.int32, "state")
    _check("fp8_history_init", load_library().fp8_history_init(
        _ptr(hist), _ptr(state), hist.numel(), _stream(hist)))


def fp8_history_push(hist: torch.Tensor, state: torch.Tensor, amax: torch.Tensor) -> None:
    """Append one step's amax to the history ring."""
    _scalar(hist, torch.float32, "hist")
    _scalar(state, torch.int32, "state")
    _scalar(amax, torch.float32, "amax")
    _check("fp8_history_push", load_library().fp8_history_push(
        _ptr(hist), _ptr(state), hist.numel(), _ptr(amax), _stream(hist)))


def fp8_compute_scale_delayed(hist: torch.Tensor, state: torch.Tensor, fmt, margin: int = 0,
                              bias_out=None, scale_out=None, scale_inv_out=None):
    """Bias from the maximum over the history window; returns (bias, scale, scale_inv)."""
    _scalar(hist, torch.float32, "hist")
    _scalar(state, torch.int32, "state")
    dev = hist.device
    bias_out = torch.empty(1, dtype=torch.int32, device=dev) if bias_out is None else bias_out
    scale_out = torch.empty(1, dtype=torch.float32, device=dev) if scale_out is None else scale_out
    scale_inv_out = torch.empty(1, dtype=torch.float32, device=dev) if scale_inv_out is None else scale_inv_out
    _check("fp8_compute_scale_delayed", load_library().fp8_compute_scale_delayed(
        _ptr(hist), _ptr(state), hist.numel(), _fmt(fmt), int(margin), _ptr(bias_out),
        _ptr(scale_out), _ptr(scale_inv_out), _stream(hist)))
    return bias_out, scale_out, scale_inv_out


def _quantize_outputs(x, bias, q, transpose, qT, want_amax, amax_out):
    rows, cols, ld = _mat(x, "x")
    _scalar(bias, torch.int32, "bias")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    _u8(q, "q")
    qr, qc, ldq = _mat(q, "q")
    if (qr, qc) != (rows, cols):
        raise ValueError("q must have the shape of x")
    ldqT = 0
    if transpose or qT is not None:
        if qT is None:
            qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
        _u8(qT, "qT")
        tr, tc, ldqT = _mat(qT, "qT")
        if (tr, tc) != (cols, rows):
            raise ValueError("qT must have the transposed shape of x")
    if want_amax or amax_out is not None:
        if amax_out is None:
            amax_out = torch.empty(1, dtype=torch.float32, device=x.device)
        _scalar(amax_out, torch.float32, "amax_out")
    return rows, cols, ld, q, ldq, qT, ldqT, amax_out


def fp8_quantize(x: torch.Tensor, fmt, bias: torch.Tensor, q: torch.Tensor | None = None,
                 transpose: bool = False, qT: torch.Tensor | None = None,
                 want_amax: bool = False, amax_out: torch.Tensor | None = None):
    """Per-tensor cast q = sat_RNE(x * 2**bias).  Returns (q, qT or None,
    amax of x or None); ``transpose`` also writes qT = q^T, ``want_amax`` fuses
    the input amax into the same pass."""
    rows, cols, ld, q, ldq, qT, ldqT, amax_out = _quantize_outputs(x, bias, q, transpose, qT, want_amax, amax_out)
    _check("fp8_quantize", load_library().fp8_quantize(
        _ptr(x), _dtype_code(x, "x"), rows, cols, ld, _fmt(fmt), _ptr(bias), _ptr(q), ldq,
        _ptr(qT), ldqT, _ptr(amax_out), _stream(x)))
    return q, qT, amax_out


def fp8_quantize_sat(x: torch.Tensor, fmt, bias: torch.Tensor, q: torch.Tensor | None = None,
                     transpose: bool = False, qT: torch.Tensor | None = None,
                     want_amax: bool = False, amax_out: torch.Tensor | None = None,
                     sat_out: torch.Tensor | None = None):
    """fp8_quantize plus the number of elements the cast saturates
    (|x * 2**bias| > fmax, NaN excluded), counted on the device into a
    one-element int64 tensor (the C call's uint64).  Returns (q, qT or None,
    amax or None, sat)."""
    rows, cols, ld, q, ldq, qT, ldqT, amax_out = _quantize_outputs(x, bias, q, transpose, qT, want_amax, amax_out)
    if sat_out is None:
        sat_out = torch.empty(1, dtype=torch.int64, device=x.device)
    _scalar(sat_out, torch.int64, "sat_out")
    _check("fp8_quantize_sat", load_library().fp8_quantize_sat(
        _ptr(x), _dtype_code(x, "x"), rows, cols, ld, _fmt(fmt), _ptr(bias), _ptr(q), ldq,
        _ptr(qT), ldqT, _ptr(amax_out), _ptr(sat_out), _stream(x)))
    return q, qT, amax_out, sat_out


def fp8_quantize_delayed(x: torch.Tensor, fmt, hist: torch.Tensor, state: torch.Tensor, workspace: torch.Tensor,
                         margin: int = 0, q: torch.Tensor | None = None, transpose: bool = False,
                         qT: torch.Tensor | None = None, want_sat: bool = False, bias_out=None, amax_out=None,
                         sat_out=None):
    """One step of delayed scaling in one launch: the bias from the history
    window, the cast of x with it, and the push of x's amax into the window
    (bit for bit fp8_compute_scale_delayed + fp8_quantize_sat + fp8_history_push).
    ``workspace``: as for fp8_amax_scale (amax_scale_workspace), left zero.
    Returns (q, qT or None, bias, amax, saturated count or None)."""
    _scalar(hist, torch.float32, "hist")
    _scalar(state, torch.int32, "state")
    _dev(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < AMAX_SCALE_WORKSPACE_BYTES or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor of AMAX_SCALE_WORKSPACE_BYTES")
    dev = x.device
    if bias_out is None:
        bias_out = torch.empty(1, dtype=torch.int32, device=dev)
    _scalar(bias_out, torch.int32, "bias_out")
    rows, cols, ld, q, ldq, qT, ldqT, amax_out = _quantize_outputs(x, bias_out, q, transpose, qT, True, amax_out)
    if want_sat or sat_out is not None:
        if sat_out is None:
            sat_out = torch.empty(1, dtype=torch.int64, device=dev)
        _scalar(sat_out, torch.int64, "sat_out")
    _check("fp8_quantize_delayed", load_library().fp8_quantize_delayed(
        _ptr(x), _dtype_code(x, "x"), rows, cols, ld, _fmt(fmt), int(margin), _ptr(hist), _ptr(state), hist.numel(),
        _ptr(q), ldq, _ptr(qT), ldqT, _ptr(bias_out), _ptr(amax_out), _ptr(sat_out), _ptr(workspace), _stream(x)))
    return q, qT, bias_out, amax_out, sat_out


def _rule(rule) -> int:
    if rule not in _RULE_NAMES:
        raise ValueError(f"unknown MX rule {rule!r} (use 'fmax' or 'ocp')")
    return _RULE_NAMES[rule]


def mx_quantize(x: torch.Tensor, fmt=E4M3, q: torch.Tensor | None = None,
                scales: torch.Tensor | None = None):
    """Per-block (1 x 32 along cols) cast; returns (q [R x C] codes, scales
    [R x C/32] E8M0 codes)."""
    return _mx_cast("mx_quantize", x, fmt, None, q, scales)


def mx_quantize_rule(x: torch.Tensor, fmt=E4M3, rule="fmax", q: torch.Tensor | None = None,
                     scales: torch.Tensor | None = None):
    """mx_quantize with a choice of block-exponent rule: "fmax" (block max
    at or below the format maximum) or "ocp" (the OCP MX rule: block max in
    the format's top binade, saturating above the format maximum)."""
    return _mx_cast("mx_quantize_rule", x, fmt, _rule(rule), q, scales)


def _mx_cast(name, x, fmt, rule, q, scales):
    rows, cols, ld = _mat(x, "x")
    if cols % 32:
        raise ValueError(f"{name} needs cols % 32 == 0")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _u8(q, "q")
    _u8(scales, "scales")
    _, _, ldq = _mat(q, "q")
    _, _, lds = _mat(scales, "scales")
    fmt_rule = (_fmt(fmt),) if rule is None else (_fmt(fmt), rule)
    _check(name, getattr(load_library(), name)(
        _ptr(x), _dtype_code(x, "x"), rows, cols, ld, *fmt_rule, _ptr(q), ldq, _ptr(scales),
        lds, _stream(x)))
    return q, scales


def mx_quantize_t(x: torch.Tensor, fmt=E4M3, qT: torch.Tensor | None = None,
                  scalesT: torch.Tensor | None = None):
    """Per-block cast with 32 x 1 blocks along rows, written transposed;
    returns (qT [C x R] codes, scalesT [C x R/32] E8M0 codes), the MX cast of
    x^T."""
    return _mx_cast_t("mx_quantize_t", x, fmt, None, qT, scalesT)


def mx_quantize_t_rule(x: torch.Tensor, fmt=E4M3, rule="fmax", qT: torch.Tensor | None = None,
                       scalesT: torch.Tensor | None = None):
    """mx_quantize_t with a choice of block-exponent rule ("fmax" or "ocp",
    as in mx_quantize_rule)."""
    return _mx_cast_t("mx_quantize_t_rule", x, fmt, _rule(rule), qT, scalesT)


def _mx_cast_t(name, x, fmt, rule, qT, scalesT):
    rows, cols, ld = _mat(x, "x")
    if rows % 32:
        raise ValueError(f"{name} needs rows % 32 == 0")
    if qT is None:
        qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if scalesT is None:
        scalesT = torch.empty((cols, rows // 32), dtype=torch.uint8, device=x.device)
    _u8(qT, "qT")
    _u8(scalesT, "scalesT")
    _, _, ldq = _mat(qT, "qT")
    _, _, lds = _mat(scalesT, "scalesT")
    fmt_rule = (_fmt(fmt),) if rule is None else (_fmt(fmt), rule)
    _check(name, getattr(load_library(), name)(
        _ptr(x), _dtype_code(x, "x"), rows, cols, ld, *fmt_rule, _ptr(qT), ldq, _ptr(scalesT),
        lds, _stream(x)))
    return qT, scalesT


def _out_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return _DT_BF16
    if dtype == torch.float32:
        return _DT_F32
    raise ValueError("out dtype must be bfloat16 or float32")


def fp8_scaled_gemm(A: torch.Tensor, fmt_a, bias_a: torch.Tensor, B: torch.Tensor, fmt_b,
                    bias_b: torch.Tensor, trans_a: bool = False, trans_b: bool = False,
                    out_dtype: torch.dtype = torch.bfloat16, want_amax: bool = False,
                    out: torch.Tensor | None = None, amax_out: torch.Tensor | None = None):
    """C = 2**-(bias_a + bias_b) * op(A) @ op(B)^T with op(A) [M x K], op(B)
    [N x K]; A is stored [M x K] (or [K x M] with trans_a), B [N x K] (or
    [K x N] with trans_b).  Returns (C, amax of C or None)."""
    _u8(A, "A")
    _u8(B, "B")
    _scalar(bias_a, torch.int32, "bias_a")
    _scalar(bias_b, torch.int32, "bias_b")
    ar, ac, lda = _mat(A, "A")
    br, bc, ldb = _mat(B, "B")
    M, K = (ac, ar) if trans_a else (ar, ac)
    N, Kb = (bc, br) if trans_b else (br, bc)
    if K != Kb:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    _dev(out, "out")
    orow, ocol, ldc = _mat(out, "out")
    if (orow, ocol) != (M, N):
        raise ValueError("out must be [M x N]")
    if want_amax or amax_out is not None:
        if amax_out is None:
            amax_out = torch.empty(1, dtype=torch.float32, device=A.device)
        _scalar(amax_out, torch.float32, "amax_out")
    _check("fp8_scaled_gemm", load_library().fp8_scaled_gemm(
        M, N, K, _ptr(A), _fmt(fmt_a), int(bool(trans_a)), lda, _ptr(bias_a),
        _ptr(B), _fmt(fmt_b), int(bool(trans_b)), ldb, _ptr(bias_b),
        _ptr(out), _out_code(out.dtype), ldc, _ptr(amax_out), _stream(A)))
    return out, amax_out


def mx_scaled_gemm(A: torch.Tensor, fmt_a, A_scales: torch.Tensor, B: torch.Tensor, fmt_b,
                   B_scales: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                   want_amax: bool = False, out: torch.Tensor | None = None,
                   amax_out: torch.Tensor | None = None):
    """Block-scaled C = A @ B^T with A [M x K], B [N x K] and E8M0 scales
    [M x K/32], [N x K/32].  Returns (C, amax of C or None)."""
    _u8(A, "A")
    _u8(B, "B")
    _u8(A_scales, "A_scales")
    _u8(B_scales, "B_scales")
    M, K, lda = _mat(A, "A")
    N, Kb, ldb = _mat(B, "B")
    if K != Kb:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    _, _, lds_a = _mat(A_scales, "A_scales")
    _, _, lds_b = _mat(B_scales, "B_scales")
    if tuple(A_scales.shape) != (M, K // 32) or tuple(B_scales.shape) != (N, K // 32):
        raise ValueError("scales must be [rows x K/32]")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    _dev(out, "out")
    orow, ocol, ldc = _mat(out, "out")
    if (orow, ocol) != (M, N):
        raise ValueError("out must be [M x N]")
    if want_amax or amax_out is not None:
        if amax_out is None:
            amax_out = torch.empty(1, dtype=torch.float32, device=A.device)
        _scalar(amax_out, torch.float32, "amax_out")
    _check("mx_scaled_gemm", load_library().mx_scaled_gemm(
        M, N, K, _ptr(A), _fmt(fmt_a), lda, _ptr(A_scales), lds_a, _ptr(B), _fmt(fmt_b), ldb,
        _ptr(B_scales), lds_b, _ptr(out), _out_code(out.dtype), ldc, _ptr(amax_out), _stream(A)))
    return out, amax_out


def mx_packed_scales_bytes(rows: int, kblocks: int) -> int:
    """Bytes of the packed E8M0 layout of a [rows x kblocks] scale matrix:
    ceil(rows / 256) * ceil(kblocks / 16) * 4096."""
    n = load_library().mx_packed_scales_bytes(int(rows), int(kblocks))
    if n < 0:
        raise Fp8Error("mx_packed_scales_bytes", n)
    return n


def mx_pack_scales(scales: torch.Tensor, packed: torch.Tensor | None = None) -> torch.Tensor:
    """E8M0 codes [rows x kblocks] (row-major, as mx_quantize writes them) in
    the packed layout mx_scaled_gemm_packed reads: a 1-D uint8 tensor of
    mx_packed_scales_bytes(rows, kblocks) bytes."""
    _u8(scales, "scales")
    rows, kb, ld = _mat(scales, "scales")
    n = mx_packed_scales_bytes(rows, kb)
    if packed is None:
        packed = torch.empty(n, dtype=torch.uint8, device=scales.device)
    _u8(packed, "packed")
    if packed.dim() != 1 or packed.numel() != n or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous 1-D uint8 tensor of {n} bytes")
    _check("mx_pack_scales", load_library().mx_pack_scales(_ptr(scales), rows, kb, ld, _ptr(packed),
                                                           _stream(scales)))
    return packed


def mx_scaled_gemm_packed(A: torch.Tensor, fmt_a, A_packed: torch.Tensor, B: torch.Tensor, fmt_b,
                          B_packed: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                          want_amax: bool = False, out: torch.Tensor | None = None,
                          amax_out: torch.Tensor | None = None):
    """mx_scaled_gemm with both scale operands in the packed layout
    (mx_pack_scales of A's [M x K/32] and B's [N x K/32] codes); needs
    K > 0 (K % 32 == 0 as for mx_scaled_gemm).  Returns (C, amax of C or
    None)."""
    _u8(A, "A")
    _u8(B, "B")
    _u8(A_packed, "A_packed")
    _u8(B_packed, "B_packed")
    M, K, lda = _mat(A, "A")
    N, Kb, ldb = _mat(B, "B")
    if K != Kb:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    for t, rows, name in ((A_packed, M, "A_packed"), (B_packed, N, "B_packed")):
        if t.numel() != mx_packed_scales_bytes(rows, K // 32) or not t.is_contiguous():
            raise ValueError(f"{name} must be the packed scales of a [{rows} x {K // 32}] matrix")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    _dev(out, "out")
    orow, ocol, ldc = _mat(out, "out")
    if (orow, ocol) != (M, N):
        raise ValueError("out must be [M x N]")
    if want_amax or amax_out is not None:
        if amax_out is None:
            amax_out = torch.empty(1, dtype=torch.float32, device=A.device)
        _scalar(amax_out, torch.float32, "amax_out")
    _check("mx_scaled_gemm_packed", load_library().mx_scaled_gemm_packed(
        M, N, K, _ptr(A), _fmt(fmt_a), lda, _ptr(A_packed), _ptr(B), _fmt(fmt_b), ldb, _ptr(B_packed),
        _ptr(out), _out_code(out.dtype), ldc, _ptr(amax_out), _stream(A)))
    return out, amax_out


def mx_quantize_packed(x: torch.Tensor, fmt=E4M3, rule="fmax", q: torch.Tensor | None = None,
                       packed: torch.Tensor | None = None):
    """Per-block cast (1 x 32 blocks along the rows, E8M0 codes) writing the
    codes in the packed layout mx_scaled_gemm_packed reads; returns (q codes
    [R x C], packed codes as a 1-D uint8 tensor of
    mx_packed_scales_bytes(R, C / 32) bytes)."""
    rows, cols, ld = _mat(x, "x")
    dt = _dtype_code(x, "x")
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    _u8(q, "q")
    qr, qc, ldq = _mat(q, "q")
    if (qr, qc) != (rows, cols):
        raise ValueError("q must have the shape of x")
    n = mx_packed_scales_bytes(rows, cols // 32)
    if packed is None:
        packed = torch.empty(n, dtype=torch.uint8, device=x.device)
    _u8(packed, "packed")
    if packed.dim() != 1 or packed.numel() != n or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous 1-D uint8 tensor of {n} bytes")
    _check("mx_quantize_packed", load_library().mx_quantize_packed(
        _ptr(x), dt, rows, cols, ld, _fmt(fmt), _rule(rule), _ptr(q), ldq, _ptr(packed), _stream(x)))
    return q, packed


def mx_quantize_t_packed(x: torch.Tensor, fmt=E4M3, rule="fmax", qT: torch.Tensor | None = None,
                         packed: torch.Tensor | None = None):
    """MX cast of x^T (blocks of 32 rows of x, qT [C x R]) with the E8M0 codes
    of qT in the packed layout; returns (qT, packed codes as a 1-D uint8
    tensor of mx_packed_scales_bytes(C, R / 32) bytes)."""
    rows, cols, ld = _mat(x, "x")
    dt = _dtype_code(x, "x")
    if rows % 32:
        raise ValueError("rows must be a multiple of 32")
    if qT is None:
        qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    _u8(qT, "qT")
    qr, qc, ldqT = _mat(qT, "qT")
    if (qr, qc) != (cols, rows):
        raise ValueError("qT must have the transposed shape of x")
    n = mx_packed_scales_bytes(cols, rows // 32)
    if packed is None:
        packed = torch.empty(n, dtype=torch.uint8, device=x.device)
    _u8(packed, "packed")
    if packed.dim() != 1 or packed.numel() != n or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous 1-D uint8 tensor of {n} bytes")
    _check("mx_quantize_t_packed", load_library().mx_quantize_t_packed(
        _ptr(x), dt, rows, cols, ld, _fmt(fmt), _rule(rule), _ptr(qT), ldqT, _ptr(packed), _stream(x)))
    return qT, packed
