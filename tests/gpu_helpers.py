"""Helpers shared by the GPU parity tests: moving the generators' bf16 bits
to the device and back, the GEMM acceptance bound, and a chunked oracle cast
for full-size tensors.  Expected values always come from ``oracle``."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle

import mfma_model

DEV = "cuda:0"


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    """Progress line that names the case before the GPU work starts."""
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_dev(bits_or_vals: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits_or_vals)
    if a.dtype == np.uint32:
        a = a.view(np.float32)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(DEV)


def u8_dev(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(DEV)


def i32_dev(v: int) -> torch.Tensor:
    return torch.tensor([int(v)], dtype=torch.int32, device=DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def f32_bits_of(t: torch.Tensor) -> int:
    return int(t.detach().cpu().view(torch.int32).numpy()[0]) & 0xFFFFFFFF


def _chunks(n, chunk):
    return [(i, min(i + chunk, n)) for i in range(0, n, chunk)]


def _pool():
    import concurrent.futures as cf
    import os
    return cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1))


def oracle_quantize_chunked(bits: np.ndarray, fmt, bias: int, rows=None, chunk=1024):
    """Oracle per-tensor cast of (selected rows of) a bf16 tensor, row chunks
    on a few threads (NumPy releases the GIL in its array operations)."""
    rows = np.arange(bits.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((rows.size, bits.shape[1]), dtype=np.uint8)

    def one(se):
        r = rows[se[0]:se[1]]
        out[se[0]:se[1]] = oracle.quantize(oracle.bf16_bits_to_f64(bits[r]), fmt, bias)

    with _pool() as ex:
        list(ex.map(one, _chunks(rows.size, chunk)))
    return out


def oracle_amax_chunked(bits: np.ndarray, chunk=4096) -> float:
    with _pool() as ex:
        parts = list(ex.map(lambda se: oracle.amax(oracle.bf16_bits_to_f64(bits[se[0]:se[1]])),
                            _chunks(bits.shape[0], chunk)))
    return max(parts) if parts else 0.0


def oracle_mx_chunked(bits: np.ndarray, fmt, rows=None, chunk=1024):
    rows = np.arange(bits.shape[0]) if rows is None else np.asarray(rows)
    q = np.empty((rows.size, bits.shape[1]), dtype=np.uint8)
    s = np.empty((rows.size, bits.shape[1] // 32), dtype=np.uint8)

    def one(se):
        r = rows[se[0]:se[1]]
        q[se[0]:se[1]], s[se[0]:se[1]] = oracle.mx_quantize(oracle.bf16_bits_to_f64(bits[r]), fmt)

    with _pool() as ex:
        list(ex.map(one, _chunks(rows.size, chunk)))
    return q, s


def _fmt(fmt):
    return oracle.FORMATS[fmt] if not isinstance(fmt, oracle.Fp8Format) else fmt


def mfma_operands_pt(qa, fa, ba, qb, fb, bb):
    """The operands behind C = op(A) op(B)^T of a per-tensor product, as the
    FP8 instruction model needs them (``mfma_model``): dequantized values
    2**-bias dec(q) and alignment exponents (binade exponent - bias)."""
    fa, fb = _fmt(fa), _fmt(fb)
    return (oracle.dequantize(qa, fa, ba), oracle.dequantize(qb, fb, bb),
            mfma_model.code_exponents(qa, fa) - int(ba), mfma_model.code_exponents(qb, fb) - int(bb))


def mfma_operands_mx(qa, sa, fa, qb, sb, fb):
    """As mfma_operands_pt for a block-scaled product: dec(q) 2**(code - 127)
    and binade exponent + (code - 127) per 32-element block."""
    fa, fb = _fmt(fa), _fmt(fb)

    def ex(q, s, f):
        return mfma_model.code_exponents(q, f) + np.repeat(np.asarray(s, dtype=np.int64) - 127, 32, axis=1)

    return (oracle.mx_dequantize(qa, sa, fa), oracle.mx_dequantize(qb, sb, fb), ex(qa, sa, fa), ex(qb, sb, fb))


# Float32 accumulation allowance of the instruction-limited test, relative to
# sum |a b|: the model sums its groups exactly, the GPU in float32 (K / 64
# roundings of at most 2**-24 |partial sum| each for the K of these tests).
ACC_MARGIN = 2.0 ** -18


def _bf16_round(v: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(v))


def assert_gemm_close(y_gpu: np.ndarray, y_ref: np.ndarray, s_ref: np.ndarray, bf16_out: bool,
                      what: str = "", operands=None) -> dict:
    """Acceptance bound: |y - y_ref| <= 1e-5 * sum_k |a_k b_k| (fp32 output),
    plus one bf16 ulp of y_ref for bf16 output.

    Without ``operands`` every output must meet it.  With ``operands``
    (mfma_operands_pt / mfma_operands_mx of the rows behind y), an output
    beyond it still passes when the GPU returned the instruction's own
    result: the value of the pinned model of the FP8 instruction's in-group
    truncation (``mfma_model``), up to float32 accumulation (2**-18 sum |a b|),
    rounded to the output type.  The plain bound is then out of the
    instruction's reach for that output: its correctly rounded result misses
    it.  Returns the counts: outputs, outputs beyond the plain bound (all
    instruction-limited when the call returns) and the largest ratio of
    error to the plain allowance."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    tol = 1e-5 * s_ref
    if bf16_out:
        tol = tol + oracle.bf16_ulp(y_ref)
    err = np.abs(y_gpu - y_ref)
    bad = ~(err <= tol)
    out = {"outputs": int(err.size), "beyond_plain": int(bad.sum()), "max_err_over_tol": 0.0}
    if not bad.any():
        return out
    idx = np.argwhere(bad)
    first = [(tuple(i), y_gpu[tuple(i)], y_ref[tuple(i)], tol[tuple(i)]) for i in idx[:5]]
    if operands is None:
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first {first}")
    r, c = idx[:, 0], idx[:, 1]
    ym = mfma_model.outputs(operands, r, c)
    d = ACC_MARGIN * s_ref[r, c]
    lo, hi = ym - d, ym + d
    if bf16_out:
        lo, hi = _bf16_round(lo), _bf16_round(hi)
    g = y_gpu[r, c]
    ok = (g >= lo) & (g <= hi)
    if not ok.all():
        j = np.flatnonzero(~ok)[:5]
        raise AssertionError(
            f"{what}: {int((~ok).sum())} of {bad.sum()} outputs beyond 1e-5 sum|ab| are not the FP8 "
            f"instruction model's result; first (row, col, gpu, model, ref, tol): "
            f"{[(int(r[i]), int(c[i]), g[i], ym[i], y_ref[r[i], c[i]], tol[r[i], c[i]]) for i in j]}")
    out["max_err_over_tol"] = float(np.max(err[bad] / tol[bad]))
    return out


def pack_scales_host(sc):
    """The packed E8M0 layout, straight from its definition in the header:
    code (r, j) at ((r // 256) * G + j // 16) * 4096 + (r % 256) * 16 + j % 16,
    G = ceil(kb / 16), 127 wherever the matrix has no code."""
    rows, kb = sc.shape
    T, G = -(-rows // 256), -(-kb // 16)
    out = np.full(T * G * 4096, 127, dtype=np.uint8)
    r = np.arange(rows)[:, None]
    j = np.arange(kb)[None, :]
    out[((r // 256) * G + j // 16) * 4096 + (r % 256) * 16 + j % 16] = sc
    return out
