"""FP8 linear layer, forward and backward, over the library's entry points.

"Training and inference of large language models using 8-bit floating
point" (paper review page), "Proposed method": every tensor of a linear
layer gets a power-of-two scale from its amax, weights and activations are
cast to E4M3 and gradients to E5M2, and the matrix products run on the FP8
operands and are unscaled afterwards.  "Per-Tensor and Per-Block Scaling
Strategies for Effective FP8 Training" (summary page), "Key Questions
Answered": the scale may come from the amaxes of past iterations (delayed
scaling) or from each block of the tensor (per-block, MX).

Every step runs in the HIP library; this module only routes tensors between
entry points.  The products:

    forward   Y  = X W^T      A = X   [T x in],   B = W   [out x in]
    backward  dX = dY W       op(A) = dY [T x out],  op(B) = W^T [in x out]
              dW = dY^T X     op(A) = dY^T [out x T], op(B) = X^T [in x T]

Per-tensor recipes pass the backward products the codes as they are stored:
W and X from the forward casts and dY as op(B) / op(A) stored MN-major
(`trans_a` / `trans_b`), which the forward GEMM kernel reads with LDS
transposes as fast as K-contiguous operands, so no transposed copy is cast.
Only an MN-major operand of 2 GiB or more does not qualify; then the casts
also write the transposed copy (one pass) and that product reads
K-contiguous operands.  The MX recipe casts W^T, X^T and dY^T
with blocks along their new contiguous axis, the products' K.

Recipes:
    "current"  per-tensor, bias from the tensor's own amax (two passes:
               amax and bias in one launch, then the cast);
    "delayed"  per-tensor, bias from the largest amax of the last `history`
               steps; one launch per tensor and step takes the bias from the
               window, casts, reduces the tensor's amax and pushes it into
               the history.  The first step has no history and pushes its
               own amax first (current scaling);
    "mx"       per-block: 1 x 32 blocks along each product's K axis, E8M0
               block scales; `mx_rule` picks the block-exponent rule
               ("fmax": block max at or below the format maximum; "ocp": the
               OCP MX rule, block max in the format's top binade);
    "constant" one fixed bias for every tensor (the fixed-scaling baseline
               the pages compare FP8-AMAX against, FP8-CSCALE; "Research
               questions" / "Key findings" of the paper review page).
"""

from __future__ import annotations

import math

import torch

from . import (E4M3, E5M2, _rule, amax_scale_workspace, fp8_amax_scale, fp8_history_init, fp8_history_push,
               fp8_quantize, fp8_quantize_delayed, fp8_quantize_sat, fp8_scaled_gemm, mx_quantize_packed,
               mx_quantize_rule, mx_quantize_t_packed, mx_quantize_t_rule, mx_scaled_gemm,
               mx_scaled_gemm_packed)

RECIPES = ("current", "delayed", "mx", "constant")


def _mn_major_ok(k: int, lda_k: int, ldb_k: int) -> bool:
    """Whether a per-tensor product can read its operands MN-major: K % 16
    == 0 (any K tail runs on the fast kernel) and each MN-major operand
    spans < 2 GiB (K x its leading dimension)."""
    return k > 0 and k % 16 == 0 and lda_k < (1 << 31) - 4096 and ldb_k < (1 << 31) - 4096


def _packable(m: int, n: int, k: int) -> bool:
    """Whether an MX product of these sizes runs on packed scales: the casts
    then write the layout the GEMM copies whole cache lines of (the fast
    kernel for every K; same result, bit for bit, as row-major scales where
    both run it)."""
    return k > 0 and k % 32 == 0 and m > 0 and n > 0


class _History:
    """Delayed-scaling state of one tensor: `window` past amaxes and
    {count, head}, in device memory (checkpointing copies these buffers)."""

    def __init__(self, window: int, device):
        self.window = window
        self.hist = torch.empty(window, dtype=torch.float32, device=device)
        self.state = torch.empty(2, dtype=torch.int32, device=device)
        fp8_history_init(self.hist, self.state)
        self.steps = 0


def _cast(x2, fmt, bias, transpose, want_amax, log):
    """The cast; with a scale log it also counts saturated elements on the
    device (fp8_quantize_sat: same bytes)."""
    if log is None:
        q, qT, amax = fp8_quantize(x2, fmt, bias, transpose=transpose, want_amax=want_amax)
        return q, qT, amax, None
    return fp8_quantize_sat(x2, fmt, bias, transpose=transpose, want_amax=want_amax)


def _per_tensor_cast(x2: torch.Tensor, fmt, recipe: str, margin: int, hist: _History | None,
                     transpose: bool, const_bias: torch.Tensor | None = None, log=None, name: str = "",
                     ws: torch.Tensor | None = None):
    """Bias and FP8 codes (plus the transposed copy) of one tensor; with a
    `log` list, appends (name, bias, amax, saturated) as device scalars (amax
    None for the constant recipe; saturated = elements the cast clamped)."""
    amax = None
    if recipe == "constant":
        bias = const_bias
        q, qT, _, sat = _cast(x2, fmt, bias, transpose, False, log)
    elif recipe == "current":
        amax, bias, _, _ = fp8_amax_scale(x2, fmt, ws, margin)       # amax and bias in one launch
        q, qT, _, sat = _cast(x2, fmt, bias, transpose, False, log)
    elif hist.steps == 0:
        # delayed, first step: the history bootstraps with this step's own
        # amax (pushed once), so the step is current-scaled
        amax, bias, _, _ = fp8_amax_scale(x2, fmt, ws, margin)
        fp8_history_push(hist.hist, hist.state, amax)
        q, qT, _, sat = _cast(x2, fmt, bias, transpose, False, log)
        hist.steps += 1
    else:
        # delayed: bias from the window, cast, push of this step's amax, in
        # one launch
        q, qT, bias, amax, sat = fp8_quantize_delayed(x2, fmt, hist.hist, hist.state, ws, margin,
                                                      transpose=transpose, want_sat=log is not None)
        hist.steps += 1
    if log is not None:
        log.append((name, bias.clone(), None if amax is None else amax.clone(), sat))
    return bias, q, qT


class Fp8LinearFunction(torch.autograd.Function):
    """Y = X W^T with FP8 operands (no additive bias)."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, layer: "Fp8Linear"):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1])
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        recipe = layer.recipe
        if recipe == "mx":
            rule = layer.mx_rule
            if _packable(x2.shape[0], w.shape[0], x2.shape[1]):
                qx, px = mx_quantize_packed(x2, E4M3, rule)
                qw, pw = mx_quantize_packed(w, E4M3, rule)
                y, amax = mx_scaled_gemm_packed(qx, E4M3, px, qw, E4M3, pw, out_dtype=x.dtype, want_amax=True)
            else:
                qx, sx = mx_quantize_rule(x2, E4M3, rule)
                qw, sw = mx_quantize_rule(w, E4M3, rule)
                y, amax = mx_scaled_gemm(qx, E4M3, sx, qw, E4M3, sw, out_dtype=x.dtype, want_amax=True)
            if ctx.needs_input_grad[0] or ctx.needs_input_grad[1]:
                # backward operands: blocks along out (W^T, the K of dX) and
                # along tokens (X^T, the K of dW)
                T, N = x2.shape[0], w.shape[0]
                ctx.pk_dx = _packable(T, w.shape[1], N)
                ctx.pk_dw = _packable(N, w.shape[1], T)
                qwT, swT = (mx_quantize_t_packed if ctx.pk_dx else mx_quantize_t_rule)(w, E4M3, rule)
                qxT, sxT = (mx_quantize_t_packed if ctx.pk_dw else mx_quantize_t_rule)(x2, E4M3, rule)
                ctx.save_for_backward(qwT, swT, qxT, sxT)
        else:
            # backward products on the stored codes where the fast kernel
            # takes them MN-major: dX = dY W with W [out x in] as op(B)
            # (K = out), dW = dY^T X with dY [T x out] and X [T x in] (K = T)
            T, N, D = x2.shape[0], w.shape[0], w.shape[1]
            ctx.mn_dx = _mn_major_ok(N, 0, N * D)
            ctx.mn_dw = _mn_major_ok(T, T * N, T * D)
            bx, qx, qxT = _per_tensor_cast(x2, E4M3, recipe, layer.margin, layer._hx, not ctx.mn_dw,
                                           layer._bias, layer._log, "x", layer._ws)
            bw, qw, qwT = _per_tensor_cast(w, E4M3, recipe, layer.margin, layer._hw, not ctx.mn_dx,
                                           layer._bias, layer._log, "w", layer._ws)
            y, amax = fp8_scaled_gemm(qx, E4M3, bx, qw, E4M3, bw, out_dtype=x.dtype, want_amax=True)
            ctx.save_for_backward(qw if ctx.mn_dx else qwT, bw, qx if ctx.mn_dw else qxT, bx)
        layer.last_output_amax = amax
        ctx.layer = layer
        ctx.lead = lead
        ctx.dtype = x.dtype
        return y.reshape(*lead, w.shape[0])

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        layer = ctx.layer
        dy2 = dy.reshape(-1, dy.shape[-1])
        if not dy2.is_contiguous():
            dy2 = dy2.contiguous()
        if dy2.dtype != ctx.dtype:
            raise TypeError(f"gradient dtype {dy2.dtype} differs from the forward's {ctx.dtype}")
        dx = dw = None
        if layer.recipe == "mx":
            qwT, swT, qxT, sxT = ctx.saved_tensors
            if ctx.needs_input_grad[0]:
                if ctx.pk_dx:
                    qdy, pdy = mx_quantize_packed(dy2, E5M2, layer.mx_rule)
                    dx, _ = mx_scaled_gemm_packed(qdy, E5M2, pdy, qwT, E4M3, swT, out_dtype=ctx.dtype)
                else:
                    qdy, sdy = mx_quantize_rule(dy2, E5M2, layer.mx_rule)
                    dx, _ = mx_scaled_gemm(qdy, E5M2, sdy, qwT, E4M3, swT, out_dtype=ctx.dtype)
            if ctx.needs_input_grad[1]:
                if ctx.pk_dw:
                    qdyT, pdyT = mx_quantize_t_packed(dy2, E5M2, layer.mx_rule)
                    dw, _ = mx_scaled_gemm_packed(qdyT, E5M2, pdyT, qxT, E4M3, sxT, out_dtype=ctx.dtype)
                else:
                    qdyT, sdyT = mx_quantize_t_rule(dy2, E5M2, layer.mx_rule)
                    dw, _ = mx_scaled_gemm(qdyT, E5M2, sdyT, qxT, E4M3, sxT, out_dtype=ctx.dtype)
        else:
            qw_, bw, qx_, bx = ctx.saved_tensors           # W, X codes (MN-major use) or W^T, X^T
            bdy, qdy, qdyT = _per_tensor_cast(dy2, E5M2, layer.recipe, layer.margin, layer._hdy,
                                              ctx.needs_input_grad[1] and not ctx.mn_dw, layer._bias,
                                              layer._log, "dy", layer._ws)
            if ctx.needs_input_grad[0]:
                dx, _ = fp8_scaled_gemm(qdy, E5M2, bdy, qw_, E4M3, bw, trans_b=ctx.mn_dx, out_dtype=ctx.dtype)
            if ctx.needs_input_grad[1]:
                if ctx.mn_dw:
                    dw, _ = fp8_scaled_gemm(qdy, E5M2, bdy, qx_, E4M3, bx, trans_a=True, trans_b=True,
                                            out_dtype=ctx.dtype)
                else:
                    dw, _ = fp8_scaled_gemm(qdyT, E5M2, bdy, qx_, E4M3, bx, out_dtype=ctx.dtype)
        if dx is not None:
            dx = dx.reshape(*ctx.lead, dx.shape[-1])
        return dx, dw, None


class Fp8Linear(torch.nn.Module):
    """Linear layer y = x W^T whose three products run in FP8 on the GPU.
    `bias` is the fixed exponent bias of the "constant" recipe (scale 2^bias
    for every tensor); the layer has no additive bias.

    in_features, out_features and the token count must be multiples of 32
    (the MX block; the per-tensor products would take any multiple of 16).
    `last_output_amax` holds max |y| of the latest forward,
    reduced in the GEMM's epilogue, for a next layer's scale."""

    def __init__(self, in_features: int, out_features: int, recipe: str = "current",
                 margin: int = 0, history: int = 16, bias: int = 0, log_scales: bool = False,
                 mx_rule: str = "fmax", device=None, dtype=torch.bfloat16):
        super().__init__()
        if recipe not in RECIPES:
            raise ValueError(f"recipe must be one of {RECIPES}")
        if in_features % 32 or out_features % 32:
            raise ValueError("in_features and out_features must be multiples of 32")
        if dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("dtype must be bfloat16 or float32")
        self.in_features, self.out_features = in_features, out_features
        self.recipe, self.margin = recipe, int(margin)
        _rule(mx_rule)                                   # validates the name
        self.mx_rule = mx_rule
        self.weight = torch.nn.Parameter(torch.empty(out_features, in_features, device=device, dtype=dtype))
        torch.nn.init.kaiming_uniform_(self.weight, a=math.sqrt(5))
        self.last_output_amax = None
        self._hx = self._hw = self._hdy = None
        # current and delayed scaling: one reduction workspace for the
        # layer's one-launch scales and delayed steps (x, w, dy are cast one
        # after another on the stream); a buffer, so that it follows the
        # layer to its device
        if recipe in ("current", "delayed"):
            self.register_buffer("_ws", amax_scale_workspace(self.weight.device), persistent=False)
        else:
            self._ws = None
        if log_scales and recipe == "mx":
            raise ValueError("scale logging covers the per-tensor recipes")
        self._log = [] if log_scales else None
        if recipe == "constant":
            if not -126 <= int(bias) <= 126:
                raise ValueError("bias must lie in [-126, 126]")
            self.register_buffer("_bias", torch.tensor([int(bias)], dtype=torch.int32, device=self.weight.device))
        else:
            self._bias = None
        if recipe == "delayed":
            dev = self.weight.device
            self._hx, self._hw, self._hdy = (_History(history, dev), _History(history, dev),
                                             _History(history, dev))

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected {self.in_features} input features, got {x.shape[-1]}")
        tokens = x.numel() // self.in_features
        if tokens % 32:
            raise ValueError("the number of tokens must be a multiple of 32")
        if x.dtype != self.weight.dtype:
            raise TypeError("input and weight dtypes differ")
        return Fp8LinearFunction.apply(x, self.weight, self)

    def scale_history(self) -> dict:
        """Per-step (bias, amax, saturated) of each tensor ("x", "w", "dy")
        since the layer was built or the log cleared, in step order:
        saturated is the number of elements the cast clamped to +-max (a
        delayed scale lagging a growing amax).  Copies the logged device
        scalars to the host."""
        if self._log is None:
            raise RuntimeError("the layer was built without log_scales=True")
        out = {"x": [], "w": [], "dy": []}
        for name, b, a, n in self._log:
            out[name].append((int(b.cpu()[0]), None if a is None else float(a.cpu()[0]), int(n.cpu()[0])))
        return out

    def bias_histogram(self) -> dict:
        """Count of steps per bias value, for each tensor: the per-tensor scale
        distribution over the logged steps."""
        hist = {}
        for name, rows in self.scale_history().items():
            h = {}
            for b, *_ in rows:
                h[b] = h.get(b, 0) + 1
            hist[name] = dict(sorted(h.items()))
        return hist

    def clear_scale_log(self) -> None:
        if self._log is not None:
            self._log.clear()

    def extra_repr(self) -> str:
        extra = f", mx_rule={self.mx_rule}" if self.recipe == "mx" else ""
        return f"in_features={self.in_features}, out_features={self.out_features}, recipe={self.recipe}{extra}"
