"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every call keeps its scalars (biases, amaxes, the delayed-scaling window and
its state, the one-launch reductions' workspace) in device memory and only
launches kernels on the caller's stream: no host round trip, no allocation
and no memset.  So the whole step can be captured once and replayed.  Each
replay runs on new inputs, copied in eagerly between replays, and must equal
the same calls run eagerly on the same inputs, bit for bit.  The window and
state that the graph's pushes advance must also match the eager copy's.  On
the first replay the codes and the current-scaling bias are also checked
against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import scaled_quantize_fp8_amd as sq
from gpu_helpers import DEV, f32_bits_of, host, need_gpu, say
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

M, N, K = 512, 768, 1024


class _Buffers:
    """Outputs and state of one run of the step (graph or eager)."""

    def __init__(self):
        u8 = dict(dtype=torch.uint8, device=DEV)
        f32 = dict(dtype=torch.float32, device=DEV)
        i32 = dict(dtype=torch.int32, device=DEV)
        self.ax, self.aw, self.ay, self.aym, self.ad = (torch.empty(1, **f32) for _ in range(5))
        self.ax_na = torch.empty(1, **f32)
        self.bx, self.bw, self.bd, self.bx_na = (torch.empty(1, **i32) for _ in range(4))
        self.sat = torch.empty(1, dtype=torch.int64, device=DEV)
        self.qx, self.qd = torch.empty(M, K, **u8), torch.empty(M, K, **u8)
        self.qw = torch.empty(N, K, **u8)
        self.qdT = torch.empty(K, M, **u8)
        self.mqx, self.mqw = torch.empty(M, K, **u8), torch.empty(N, K, **u8)
        self.psx = torch.empty(sq.mx_packed_scales_bytes(M, K // 32), **u8)
        self.psw = torch.empty(sq.mx_packed_scales_bytes(N, K // 32), **u8)
        self.y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        self.ym = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        self.ws_x, self.ws_w, self.ws_d = (sq.amax_scale_workspace(DEV) for _ in range(3))
        self.hist = torch.empty(16, **f32)
        self.state = torch.empty(2, **i32)

    def reset_history(self):
        sq.fp8_history_init(self.hist, self.state)

    def run(self, x, w):
        """One step: current scaling of x and w in one launch each, their
        E4M3 casts and the per-tensor GEMM with its output amax; the
        delayed-scaling step of x with its transposed copy and saturation
        count; the MX casts into packed scales and the MX GEMM; the
        no-allocation one-launch scale of x."""
        sq.fp8_amax_scale(x, sq.E4M3, self.ws_x, amax_out=self.ax, bias_out=self.bx)
        sq.fp8_amax_scale(w, sq.E4M3, self.ws_w, amax_out=self.aw, bias_out=self.bw)
        sq.fp8_quantize(x, sq.E4M3, self.bx, q=self.qx)
        sq.fp8_quantize(w, sq.E4M3, self.bw, q=self.qw)
        sq.fp8_scaled_gemm(self.qx, sq.E4M3, self.bx, self.qw, sq.E4M3, self.bw, out=self.y, amax_out=self.ay)
        sq.fp8_quantize_delayed(x, sq.E4M3, self.hist, self.state, self.ws_d, q=self.qd, transpose=True,
                                qT=self.qdT, want_sat=True, bias_out=self.bd, amax_out=self.ad, sat_out=self.sat)
        sq.mx_quantize_packed(x, sq.E4M3, q=self.mqx, packed=self.psx)
        sq.mx_quantize_packed(w, sq.E4M3, q=self.mqw, packed=self.psw)
        sq.mx_scaled_gemm_packed(self.mqx, sq.E4M3, self.psx, self.mqw, sq.E4M3, self.psw, out=self.ym,
                                 amax_out=self.aym)
        sq.fp8_amax_scale_noalloc(x, sq.E4M3, amax_out=self.ax_na, bias_out=self.bx_na)

    def tensors(self):
        return {k: v for k, v in vars(self).items() if isinstance(v, torch.Tensor) and not k.startswith("ws_")}


def _bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits, so that NaN and -0 compare exactly."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    elif t.dtype == torch.float32:
        t = t.view(torch.int32)
    return host(t)


def test_step_captured_in_graph_replays_like_eager():
    need_gpu()
    gen = torch.Generator(device=DEV).manual_seed(2024)
    x = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    w = torch.empty(N, K, dtype=torch.bfloat16, device=DEV)

    def new_inputs(step):
        # the amplitude changes from step to step, so biases, window and
        # saturation counts move; a NaN planted in one step
        x.copy_(torch.randn(M, K, device=DEV, generator=gen) * (0.5 + 3.0 * (step % 3)))
        w.copy_(torch.randn(N, K, device=DEV, generator=gen) * 0.02)
        if step == 3:
            x[7, 9] = float("nan")

    G, E = _Buffers(), _Buffers()
    new_inputs(0)
    G.reset_history()
    G.run(x, w)                          # eager warm-up on the graph's buffers
    torch.cuda.synchronize()
    G.reset_history()
    E.reset_history()
    torch.cuda.synchronize()
    say("graph capture: the step (current, delayed and MX paths)")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        G.run(x, w)
    torch.cuda.synchronize()
    for step in range(6):
        new_inputs(step)
        graph.replay()
        E.run(x, w)                      # same stream: runs after the replay, on the same inputs
        torch.cuda.synchronize()
        say(f"graph replay {step}: bias x {int(host(E.bx)[0])}, delayed bias {int(host(E.bd)[0])}, "
            f"saturated {int(host(E.sat)[0])}")
        gt, et = G.tensors(), E.tensors()
        for k in et:
            assert np.array_equal(_bits(gt[k]), _bits(et[k])), (step, k)
        if step == 0:
            xb = f32_to_bf16_bits(host(x.float()))
            xv = oracle.bf16_bits_to_f64(xb)
            rb = oracle.compute_bias(oracle.amax(xv), oracle.E4M3)
            assert int(host(G.bx)[0]) == rb
            assert f32_bits_of(G.ax) == f32_bits_of(torch.tensor([oracle.amax(xv)], dtype=torch.float32))
            assert np.array_equal(host(G.qx), oracle.quantize(xv, oracle.E4M3, rb))
            rq, rs = oracle.mx_quantize(xv, oracle.E4M3)
            assert np.array_equal(host(G.mqx), rq)
