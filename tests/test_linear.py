"""The FP8 linear layer (forward Y = X W^T, backward dX = dY W and
dW = dY^T X) against the oracle's emulation of the same recipe: the oracle
computes every amax, bias, per-tensor or MX cast itself from the bf16 inputs
and forms the three products in float64; the GPU results must meet the GEMM
acceptance bound of the parity tests.  CPU tests cover argument checks."""

import numpy as np
import pytest
import torch

import oracle
import scaled_quantize_fp8_amd as sq
from oracle import E4M3, E5M2
from scaled_quantize_fp8_amd.linear import Fp8Linear
from workloads import make

from gpu_helpers import DEV, assert_gemm_close, bf16_dev, host, host_f64, mfma_operands_mx, mfma_operands_pt, need_gpu, say

T, IN, OUT = 256, 512, 384


def _tensors(step=0, x_scale=1.0, shape=(T, IN, OUT)):
    t, i, o = shape
    xb = make("c1", "X", step=step, shape=(t, i))
    x = oracle.bf16_bits_to_f64(xb) * x_scale                 # exact: power-of-two scales only
    wb = make("c1", "W", shape=(o, i))
    dyb = make("c3", "dY", step=step, shape=(t, o))
    return x, oracle.bf16_bits_to_f64(wb), oracle.bf16_bits_to_f64(dyb)


def _dev(v):
    return torch.from_numpy(v.astype(np.float32)).to(DEV).to(torch.bfloat16)


def _run(layer, x, dy):
    xt = _dev(x).requires_grad_(True)
    y = layer(xt)
    y.backward(_dev(dy))
    return host_f64(y), host_f64(xt.grad), host_f64(layer.weight.grad), layer.last_output_amax


def _check(what, got, ref, s, gt):
    assert_gemm_close(got, ref, s, True, what, gt)


def _check_pt(y, dx, dw, x, w, dy, bx, bw, bdy):
    qx, qw, qdy = oracle.quantize(x, E4M3, bx), oracle.quantize(w, E4M3, bw), oracle.quantize(dy, E5M2, bdy)
    qwT, qxT, qdyT = (np.ascontiguousarray(a.T) for a in (qw, qx, qdy))
    for what, got, a, fa, ba, b, fb, bb in (("y", y, qx, E4M3, bx, qw, E4M3, bw),
                                            ("dx", dx, qdy, E5M2, bdy, qwT, E4M3, bw),
                                            ("dw", dw, qdyT, E5M2, bdy, qxT, E4M3, bx)):
        ref = oracle.scaled_gemm_ref(a, fa, ba, b, fb, bb)
        s = oracle.abs_product_sum(a, fa, ba, b, fb, bb)
        gt = mfma_operands_pt(a, fa, ba, b, fb, bb)
        _check(what, got, ref, s, gt)


@pytest.mark.gpu
def test_linear_current_scaling_matches_oracle():
    need_gpu()
    x, w, dy = _tensors()
    layer = Fp8Linear(IN, OUT, recipe="current", device=DEV)
    with torch.no_grad():
        layer.weight.copy_(_dev(w))
    say("fp8 linear, current scaling")
    y, dx, dw, amax = _run(layer, x, dy)
    bx, bw = oracle.compute_bias(oracle.amax(x), E4M3), oracle.compute_bias(oracle.amax(w), E4M3)
    bdy = oracle.compute_bias(oracle.amax(dy), E5M2)
    _check_pt(y, dx, dw, x, w, dy, bx, bw, bdy)
    assert host(amax)[0] == np.max(np.abs(y))


@pytest.mark.gpu
def test_linear_backward_k_tails_on_stored_codes():
    """T = 288 tokens and 416 outputs: the backward products' K (T for dW,
    out for dX) are not multiples of 128, and they still read the stored
    codes MN-major (K tails on the fast kernel); Y, dX and dW against the
    oracle."""
    from scaled_quantize_fp8_amd.linear import _mn_major_ok
    need_gpu()
    t, i, o = 288, 512, 416
    assert _mn_major_ok(o, 0, o * i) and _mn_major_ok(t, t * o, t * i)
    x, w, dy = _tensors(shape=(t, i, o))
    layer = Fp8Linear(i, o, recipe="current", device=DEV)
    with torch.no_grad():
        layer.weight.copy_(_dev(w))
    say("fp8 linear, current scaling, K tails in the backward")
    y, dx, dw, amax = _run(layer, x, dy)
    bx, bw = oracle.compute_bias(oracle.amax(x), E4M3), oracle.compute_bias(oracle.amax(w), E4M3)
    bdy = oracle.compute_bias(oracle.amax(dy), E5M2)
    _check_pt(y, dx, dw, x, w, dy, bx, bw, bdy)
    assert host(amax)[0] == np.max(np.abs(y))


@pytest.mark.gpu
def test_linear_delayed_scaling_three_steps():
    """Activations whose scale jumps (x1, x16, x1/8): the layer's biases follow
    the oracle's delayed-scaling history (step 0 current, later steps the
    window maximum of earlier steps), forward and backward."""
    need_gpu()
    layer = Fp8Linear(IN, OUT, recipe="delayed", history=16, device=DEV)
    hx, hw, hdy = oracle.DelayedScaling(16), oracle.DelayedScaling(16), oracle.DelayedScaling(16)
    for step, xs in enumerate((1.0, 16.0, 0.125)):
        x, w, dy = _tensors(step, xs)
        if step == 0:
            with torch.no_grad():
                layer.weight.copy_(_dev(w))
        layer.weight.grad = None
        say(f"fp8 linear, delayed scaling step {step}")
        y, dx, dw, _ = _run(layer, x, dy)
        biases = []
        for h, v, fmt in ((hx, x, E4M3), (hw, w, E4M3), (hdy, dy, E5M2)):
            if step == 0:
                h.push(oracle.amax(v))
            biases.append(h.bias(fmt))
            if step > 0:
                h.push(oracle.amax(v))
        _check_pt(y, dx, dw, x, w, dy, *biases)


@pytest.mark.gpu
def test_linear_constant_bias_matches_oracle():
    """The fixed-scaling recipe: bias -1 for every tensor, no amax pass."""
    need_gpu()
    x, w, dy = _tensors()
    layer = Fp8Linear(IN, OUT, recipe="constant", bias=-1, device=DEV)
    with torch.no_grad():
        layer.weight.copy_(_dev(w))
    say("fp8 linear, constant bias -1")
    y, dx, dw, _ = _run(layer, x, dy)
    _check_pt(y, dx, dw, x, w, dy, -1, -1, -1)


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [(T, IN, OUT), (512, 512, 640)], ids=["256x512x384", "512x512x640"])
@pytest.mark.parametrize("rule", ["fmax", "ocp"])
def test_linear_mx_matches_oracle(rule, shape):
    """The MX recipe's three products against the oracle's.  At 256 x 512 x 384
    only the forward product (K = 512) runs on packed scales; at 512 x 512 x
    640 all three do (K = 512, 640, 512)."""
    need_gpu()
    x, w, dy = _tensors(shape=shape)
    layer = Fp8Linear(shape[1], shape[2], recipe="mx", mx_rule=rule, device=DEV)
    with torch.no_grad():
        layer.weight.copy_(_dev(w))
    say(f"fp8 linear, MX, rule {rule}, T x in x out {shape}")
    y, dx, dw, amax = _run(layer, x, dy)
    qx, sx = oracle.mx_quantize(x, E4M3, rule)
    qw, sw = oracle.mx_quantize(w, E4M3, rule)
    qdy, sdy = oracle.mx_quantize(dy, E5M2, rule)
    qwT, swT = oracle.mx_quantize(np.ascontiguousarray(w.T), E4M3, rule)
    qdyT, sdyT = oracle.mx_quantize(np.ascontiguousarray(dy.T), E5M2, rule)
    qxT, sxT = oracle.mx_quantize(np.ascontiguousarray(x.T), E4M3, rule)
    for what, got, a, sa, fa, b, sb, fb in (("y", y, qx, sx, E4M3, qw, sw, E4M3),
                                            ("dx", dx, qdy, sdy, E5M2, qwT, swT, E4M3),
                                            ("dw", dw, qdyT, sdyT, E5M2, qxT, sxT, E4M3)):
        ref = oracle.mx_gemm_ref(a, sa, fa, b, sb, fb)
        s = oracle.mx_abs_product_sum(a, sa, fa, b, sb, fb)
        gt = mfma_operands_mx(a, sa, fa, b, sb, fb)
        _check(what, got, ref, s, gt)
    assert host(amax)[0] == np.max(np.abs(y))


@pytest.mark.gpu
def test_linear_scale_log_16_delayed_steps():
    """The delayed-scaling workload of the 7B attention projection (activation
    scales drawn per step, 0.1% outliers x50), 16 steps at 256 tokens: the
    logged per-step biases, amaxes and device-counted saturated elements of
    x, w and dy equal the oracle's history and counts, and the histogram
    counts every step once."""
    need_gpu()
    layer = Fp8Linear(IN, OUT, recipe="delayed", history=16, log_scales=True, device=DEV)
    wv = oracle.bf16_bits_to_f64(make("c2", "W", shape=(OUT, IN)))
    with torch.no_grad():
        layer.weight.copy_(_dev(wv))
    hx, hw, hdy = oracle.DelayedScaling(16), oracle.DelayedScaling(16), oracle.DelayedScaling(16)
    want = {"x": [], "w": [], "dy": []}
    for step in range(16):
        xv = oracle.bf16_bits_to_f64(make("c2", "X", step=step, shape=(T, IN)))
        dyv = oracle.bf16_bits_to_f64(make("c3", "dY", step=step, shape=(T, OUT)))
        layer.weight.grad = None
        say(f"scale log step {step}")
        _run(layer, xv, dyv)
        for name, h, v, fmt in (("x", hx, xv, E4M3), ("w", hw, wv, E4M3), ("dy", hdy, dyv, E5M2)):
            if step == 0:
                h.push(oracle.amax(v))
            b = h.bias(fmt)
            want[name].append((b, oracle.amax(v), int(np.count_nonzero(np.abs(np.ldexp(v, b)) > fmt.max))))
            if step > 0:
                h.push(oracle.amax(v))
    got = layer.scale_history()
    for name in ("x", "w", "dy"):
        assert got[name] == want[name], name
    say(f"saturated per step: x {[n for *_, n in got['x']]}, dy {[n for *_, n in got['dy']]}")
    hist = layer.bias_histogram()
    assert all(sum(h.values()) == 16 for h in hist.values())
    assert len(hist["x"]) > 1                      # the activation scale moved


@pytest.mark.gpu
@pytest.mark.parametrize("recipe", ["current", "delayed"])
def test_linear_backward_on_stored_codes(recipe):
    """A full-size layer whose backward products read the stored codes
    MN-major (dX = dY W with W [out x in] as op(B); dW = dY^T X with
    dY [T x out] and X [T x in], 272 output tiles), so no cast writes a
    transposed copy: Y, dX and dW on sampled rows and columns (two per
    256-wide tile, so every output tile) against the oracle's products, two
    steps for the delayed recipe.  (The smaller layers of the other tests
    take the same path on 128 x 256 tiles.)"""
    from scaled_quantize_fp8_amd.linear import _mn_major_ok
    need_gpu()
    t, i, o = 2048, 4352, 4096
    assert _mn_major_ok(o, 0, o * i) and _mn_major_ok(t, t * o, t * i)
    layer = Fp8Linear(i, o, recipe=recipe, device=DEV)
    rng = np.random.default_rng(61)

    def rows(n):
        return np.unique(np.concatenate([np.minimum(np.arange(0, n, 256)[:, None] + rng.integers(0, 256, (1, 2)),
                                                    n - 1).ravel(), [0, n - 1]]))
    hs = [oracle.DelayedScaling(16) for _ in range(3)]
    for step in range(2 if recipe == "delayed" else 1):
        x, w, dy = _tensors(step=step, shape=(t, i, o))
        with torch.no_grad():
            layer.weight.copy_(_dev(w))
        layer.weight.grad = None
        say(f"fp8 linear {recipe} step {step}, backward on stored codes, {t} x {i} -> {o}")
        y, dx, dw, _ = _run(layer, x, dy)
        if recipe == "current":
            bx, bw, bdy = (oracle.compute_bias(oracle.amax(x), E4M3), oracle.compute_bias(oracle.amax(w), E4M3),
                           oracle.compute_bias(oracle.amax(dy), E5M2))
        else:
            # step 0 pushes its own amax first; later steps take the window's bias, then push
            biases = []
            for h, v, fmt in zip(hs, (x, w, dy), (E4M3, E4M3, E5M2)):
                if step == 0:
                    h.push(oracle.amax(v))
                biases.append(h.bias(fmt))
                if step > 0:
                    h.push(oracle.amax(v))
            bx, bw, bdy = biases
        qx, qw, qdy = oracle.quantize(x, E4M3, bx), oracle.quantize(w, E4M3, bw), oracle.quantize(dy, E5M2, bdy)
        rt, ri, ro = rows(t), rows(i), rows(o)
        for what, got, a, fa, ba, b, fb, bb in (
                ("y", y[np.ix_(rt, ro)], qx[rt], E4M3, bx, qw[ro], E4M3, bw),
                ("dx", dx[np.ix_(rt, ri)], qdy[rt], E5M2, bdy, np.ascontiguousarray(qw.T[ri]), E4M3, bw),
                ("dw", dw[np.ix_(ro, ri)], np.ascontiguousarray(qdy.T[ro]), E5M2, bdy,
                 np.ascontiguousarray(qx.T[ri]), E4M3, bx)):
            ref = oracle.scaled_gemm_ref(a, fa, ba, b, fb, bb)
            s = oracle.abs_product_sum(a, fa, ba, b, fb, bb)
            _check(f"{recipe} step {step} {what}", got, ref, s, mfma_operands_pt(a, fa, ba, b, fb, bb))


@pytest.mark.gpu
def test_linear_batched_input_shape():
    need_gpu()
    layer = Fp8Linear(IN, OUT, device=DEV)
    x = bf16_dev(make("c1", "X", shape=(T, IN))).view(2, T // 2, IN).requires_grad_(True)
    y = layer(x)
    assert y.shape == (2, T // 2, OUT)
    y.sum().backward()
    assert x.grad.shape == x.shape and layer.weight.grad.shape == layer.weight.shape


def test_linear_argument_checks():
    with pytest.raises(ValueError):
        Fp8Linear(IN, OUT, recipe="fp16")
    with pytest.raises(ValueError):
        Fp8Linear(IN, OUT, recipe="constant", bias=200)
    with pytest.raises(ValueError):
        Fp8Linear(IN, OUT, recipe="mx", log_scales=True)
    with pytest.raises(ValueError):
        Fp8Linear(IN, OUT, recipe="mx", mx_rule="round")
    with pytest.raises(RuntimeError):
        Fp8Linear(IN, OUT).scale_history()
    with pytest.raises(ValueError):
        Fp8Linear(100, OUT)
    layer = Fp8Linear(IN, OUT)                       # CPU parameters: the product path refuses them
    with pytest.raises(ValueError):
        layer(torch.zeros(T, IN, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        layer(torch.zeros(T, IN + 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        layer(torch.zeros(T + 16, IN, dtype=torch.bfloat16))
