"""One MoE layer's expert computation on one GPU, forward and backward, as a
chain of libmxmoe calls.  MoELayer takes token rows already grouped by
expert; RoutedMoELayer (at the end) adds the route plan, the dispatch and the
combine around it for top-k routed tokens (no router: the expert choices and
weights are inputs).  This is the layer-level view of the public
write-ups on Cursor's MXFP8 MoE kernels (aigc.bar "被忽视的量化税": the
quantization passes next to the grouped GEMMs of a layer; lpnh.cn 2479732
section 1: the forward and backward passes and the transposed quantization
the backward needs; kucoin.com MoK page, section 02: MXFP8 built into the
grouped-GEMM and SwiGLU data path).

Shapes: X [M, H] token rows, group offsets [G+1] (rows of expert g are
[o_g, o_{g+1})); W1 [G, 2I, H] gate+up weights in the interleaved row order
of ``swiglu_interleave``; W2 [G, H, I] down weights.

  forward    F1  X -> row-wise Xq (gate+up operand) and column-wise X^T
                 (gate+up weight gradient)            mx_quantize_dual
             F2  hq = MXFP8(silu(X W1g^T) * X W1u^T), and the bf16 gate/up
                 values for the backward pass         mx_grouped_gemm_swiglu
             F3  Y = hq W2^T                          mx_grouped_gemm
  backward   B1  dY -> row-wise (down dgrad) and column-wise (down wgrad)
                                                      mx_quantize_dual
             B2  dH = dY W2                           mx_grouped_gemm_dgrad
             B3  d(gate, up) and h from dH and the saved gate/up, quantized
                 as they are made: d(gate, up) row-wise and column-wise, h
                 column-wise                          mx_swiglu_backward_quant
             B4  dW2 = dY^T h per expert              mx_grouped_gemm_wgrad
             B5  dX = d(gate, up) W1                  mx_grouped_gemm_dgrad
             B6  dW1 = d(gate, up)^T X per expert     mx_grouped_gemm_wgrad
             With fuse_swiglu_backward=False, B3 is the unfused chain instead:
             mx_swiglu_backward writes d(gate, up) and h in bf16, then
             mx_quantize_cols(h) and mx_quantize_dual(d(gate, up)) read them
             back (the same bytes come out; the fused call saves the bf16
             round trip through HBM).
  weights    W1, W2 -> row-wise (forward operands) and column-wise (dgrad
             operands, one group per expert)          mx_quantize_dual

Every step runs in the library's kernels; this module only allocates the
buffers once and issues the calls in order on the current stream
(step_overlapped: the independent ones on two streams).
"""
import torch

from . import (mx_cols_capacity, mx_combine, mx_gather_quantize, mx_grouped_gemm, mx_grouped_gemm_dgrad,
               mx_grouped_gemm_swiglu, mx_grouped_gemm_wgrad, mx_quantize_cols, mx_quantize_dual, mx_route_plan,
               mx_scale_bytes, mx_swiglu_backward, mx_swiglu_backward_quant)

FORWARD = ("F1 quantize X", "F2 gate+up GEMM + SwiGLU + quantize", "F3 down GEMM")
BACKWARD = ("B1 quantize dY", "B2 down dgrad", "B3 SwiGLU backward + quantize", "B4 down wgrad",
            "B5 gate+up dgrad", "B6 gate+up wgrad")
BACKWARD_UNFUSED = ("B1 quantize dY", "B2 down dgrad", "B3a SwiGLU backward", "B3b quantize h (cols)",
                    "B3c quantize d(gate,up)", "B4 down wgrad", "B5 gate+up dgrad", "B6 gate+up wgrad")
WEIGHTS = ("W1 quantize", "W2 quantize")
ROUTED_FORWARD = ("R route plan", "D dispatch + quantize X", FORWARD[1], FORWARD[2], "C combine")
ROUTED_BACKWARD = ("C' reverse combine + quantize dOut",) + BACKWARD[1:] + ("D' reverse dispatch",)
KIND = {
    "R route plan": "routing", "D dispatch + quantize X": "quant", "C combine": "routing",
    "C' reverse combine + quantize dOut": "quant", "D' reverse dispatch": "routing",
    "F1 quantize X": "quant", "F2 gate+up GEMM + SwiGLU + quantize": "gemm", "F3 down GEMM": "gemm",
    "B1 quantize dY": "quant", "B2 down dgrad": "gemm", "B3 SwiGLU backward + quantize": "quant",
    "B3a SwiGLU backward": "elementwise", "B3b quantize h (cols)": "quant", "B3c quantize d(gate,up)": "quant",
    "B4 down wgrad": "gemm", "B5 gate+up dgrad": "gemm", "B6 gate+up wgrad": "gemm",
    "W1 quantize": "quant", "W2 quantize": "quant",
}


def _u8(*shape, device):
    return torch.empty(shape, dtype=torch.uint8, device=device)


def _bf16(*shape, device):
    return torch.empty(shape, dtype=torch.bfloat16, device=device)


class QuantPair:
    """Row-wise and column-wise MXFP8 buffers of a bf16 [R, C] tensor whose
    rows form G groups."""

    def __init__(self, R, C, G, device):
        self.Mcap = mx_cols_capacity(R, G)
        self.q = _u8(R, C, device=device)
        self.s = _u8(mx_scale_bytes(R, C), device=device)
        self.qT = _u8(C, self.Mcap, device=device)
        self.sT = _u8(mx_scale_bytes(C, self.Mcap), device=device)
        self.P = torch.empty(G + 1, dtype=torch.int32, device=device)

    def fill(self, x, offsets):
        mx_quantize_dual(x, offsets, self.Mcap, self.q, self.s, self.qT, self.sT, self.P)


class MoELayer:
    """Buffers and calls of one layer for fixed M, H, I and routing."""

    def __init__(self, offsets, M, H, I, device="cuda", fuse_swiglu_backward=True):
        self.M, self.H, self.I = M, H, I
        self.fused = fuse_swiglu_backward
        self.stages = WEIGHTS + FORWARD + (BACKWARD if self.fused else BACKWARD_UNFUSED)
        self.offsets = offsets
        G = self.G = offsets.numel() - 1
        self.woff1 = torch.arange(G + 1, dtype=torch.int32, device=device) * (2 * I)
        self.woff2 = torch.arange(G + 1, dtype=torch.int32, device=device) * H
        self.w1 = QuantPair(G * 2 * I, H, G, device)
        self.w2 = QuantPair(G * H, I, G, device)
        self.x = QuantPair(M, H, G, device)
        self.hq = _u8(M, I, device=device)
        self.hs = _u8(mx_scale_bytes(M, I), device=device)
        self.preact = _bf16(M, 2 * I, device=device)
        self.y = _bf16(M, H, device=device)
        self.dy = QuantPair(M, H, G, device)
        self.dh = _bf16(M, I, device=device)
        if not self.fused:  # bf16 d(gate, up) and h exist only in the unfused chain
            self.dpre = _bf16(M, 2 * I, device=device)
            self.h = _bf16(M, I, device=device)
            self.hP = torch.empty(G + 1, dtype=torch.int32, device=device)
        self.hT = _u8(I, self.x.Mcap, device=device)
        self.hTs = _u8(mx_scale_bytes(I, self.x.Mcap), device=device)
        self.dW2 = _bf16(G, H, I, device=device)
        self.dgu = QuantPair(M, 2 * I, G, device)
        self.dx = _bf16(M, H, device=device)
        self.dW1 = _bf16(G, 2 * I, H, device=device)

    def flops(self):
        """Matrix flops of one forward + backward over the routed rows."""
        fwd = 2 * self.M * (2 * self.I) * self.H + 2 * self.M * self.H * self.I
        return 3 * fwd

    # -- the steps; mark(name) is called after each one is issued --
    def quantize_weights(self, W1, W2, mark=None):
        G = self.G
        self.w1.fill(W1.reshape(G * 2 * self.I, self.H), self.woff1)
        _mark(mark, "W1 quantize")
        self.w2.fill(W2.reshape(G * self.H, self.I), self.woff2)
        _mark(mark, "W2 quantize")

    def forward(self, X, mark=None):
        self.x.fill(X, self.offsets)
        _mark(mark, FORWARD[0])
        return self.forward_experts(mark)

    def forward_experts(self, mark=None):
        """F2 and F3 on the quantized rows already in self.x."""
        G, H, I = self.G, self.H, self.I
        mx_grouped_gemm_swiglu(self.x.q, self.x.s, self.w1.q.view(G, 2 * I, H), self.w1.s, self.offsets,
                               hq=self.hq, hs=self.hs, preact=self.preact)
        _mark(mark, FORWARD[1])
        mx_grouped_gemm(self.hq, self.hs, self.w2.q.view(G, H, I), self.w2.s, self.offsets, out=self.y)
        _mark(mark, FORWARD[2])
        return self.y

    def backward(self, dY, mark=None):
        names = BACKWARD if self.fused else BACKWARD_UNFUSED
        self.dy.fill(dY, self.offsets)
        _mark(mark, names[0])
        return self.backward_experts(mark)

    def backward_experts(self, mark=None):
        """B2 to the end on the quantized output gradient already in self.dy."""
        G = self.G
        names = BACKWARD if self.fused else BACKWARD_UNFUSED
        mx_grouped_gemm_dgrad(self.dy.q, self.dy.s, self.w2.qT, self.w2.sT, self.offsets, G, out=self.dh)
        _mark(mark, names[1])
        if self.fused:
            dgu = self.dgu
            mx_swiglu_backward_quant(self.preact, self.dh, self.offsets, self.x.Mcap, dgu.q, dgu.s, dgu.qT, dgu.sT,
                                     self.hT, self.hTs, dgu.P)
            _mark(mark, names[2])
        else:
            mx_swiglu_backward(self.preact, self.dh, dpre=self.dpre, h=self.h)
            _mark(mark, names[2])
            mx_quantize_cols(self.h, self.offsets, self.x.Mcap, self.hT, self.hTs, self.hP)
            _mark(mark, names[3])
            self.dgu.fill(self.dpre, self.offsets)
            _mark(mark, names[4])
        mx_grouped_gemm_wgrad(self.dy.qT, self.dy.sT, self.hT, self.hTs, self.dy.P, dW=self.dW2)
        _mark(mark, names[-3])
        mx_grouped_gemm_dgrad(self.dgu.q, self.dgu.s, self.w1.qT, self.w1.sT, self.offsets, G, out=self.dx)
        _mark(mark, names[-2])
        mx_grouped_gemm_wgrad(self.dgu.qT, self.dgu.sT, self.x.qT, self.x.sT, self.x.P, dW=self.dW1)
        _mark(mark, names[-1])
        return self.dx, self.dW1, self.dW2

    def step(self, X, dY, W1, W2, mark=None):
        self.quantize_weights(W1, W2, mark)
        self.forward(X, mark)
        return self.backward(dY, mark)

    def step_overlapped(self, X, dY, W1, W2):
        """The same step with its independent calls on two streams (the
        current one and a second one of default priority), so that a call
        can start on the workgroup slots another call's last round leaves
        idle.  Same calls, same buffers, same results bit for bit:
          current  W1 quantize, quantize X, F2 | F3 (after W2) | B3 (after
                   B2) | B5, B6
          second   W2 quantize, B1, B2 | B4 (after B3)
        The second stream starts after all earlier work on the current one
        and the current one waits for all of the second's before returning,
        so consecutive steps never overlap on a buffer."""
        if not self.fused:
            raise ValueError("the overlapped step runs the fused SwiGLU backward")
        G, H, I = self.G, self.H, self.I
        main = torch.cuda.current_stream()
        if getattr(self, "_side", None) is None or self._side.device != main.device:
            self._side = torch.cuda.Stream(device=main.device)
        side = self._side
        w2_done = torch.cuda.Event()
        b2_done = torch.cuda.Event()
        b3_done = torch.cuda.Event()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            self.w2.fill(W2.reshape(G * H, I), self.woff2)
            w2_done.record(side)
            self.dy.fill(dY, self.offsets)
            mx_grouped_gemm_dgrad(self.dy.q, self.dy.s, self.w2.qT, self.w2.sT, self.offsets, G, out=self.dh)
            b2_done.record(side)
        self.w1.fill(W1.reshape(G * 2 * I, H), self.woff1)
        self.x.fill(X, self.offsets)
        mx_grouped_gemm_swiglu(self.x.q, self.x.s, self.w1.q.view(G, 2 * I, H), self.w1.s, self.offsets,
                               hq=self.hq, hs=self.hs, preact=self.preact)
        main.wait_event(w2_done)
        mx_grouped_gemm(self.hq, self.hs, self.w2.q.view(G, H, I), self.w2.s, self.offsets, out=self.y)
        main.wait_event(b2_done)
        dgu = self.dgu
        mx_swiglu_backward_quant(self.preact, self.dh, self.offsets, self.x.Mcap, dgu.q, dgu.s, dgu.qT, dgu.sT,
                                 self.hT, self.hTs, dgu.P)
        b3_done.record(main)
        with torch.cuda.stream(side):
            side.wait_event(b3_done)
            mx_grouped_gemm_wgrad(self.dy.qT, self.dy.sT, self.hT, self.hTs, self.dy.P, dW=self.dW2)
        mx_grouped_gemm_dgrad(dgu.q, dgu.s, self.w1.qT, self.w1.sT, self.offsets, G, out=self.dx)
        mx_grouped_gemm_wgrad(dgu.qT, dgu.sT, self.x.qT, self.x.sT, self.x.P, dW=self.dW1)
        main.wait_stream(side)
        return self.dx, self.dW1, self.dW2


def _mark(mark, name):
    if mark is not None:
        mark(name)


class RoutedMoELayer:
    """One GPU's share of an expert-parallel MoE layer: T tokens routed top-k
    to G local experts (experts int32 [T, k], routing weights float32
    [T, k]), dispatched, run through MoELayer's expert computation, and
    combined (kucoin.com MoK page, section 02: pull dispatch into local expert
    order, MXFP8 on the dispatch path, results pushed back to their tokens;
    here the source is local memory and the exchange a gather).

      R   route plan: offsets, slots, per-slot weights     mx_route_plan
      D   dispatch: gather X rows by slot, quantize both ways (in place of
          F1)                                              mx_gather_quantize
      F2, F3 as MoELayer
      C   combine: out[t] = sum_j w[t, j] y[slot(t, j)]     mx_combine
      C'  reverse combine: gather dOut rows by slot, times the slot's
          weight, quantize both ways (in place of B1)      mx_gather_quantize
      B2 .. B6 as MoELayer
      D'  reverse dispatch: dX[t] = sum_j dx[slot(t, j)]   mx_combine
    The routing weights' own gradient (the router's) is not computed.
    Every row of the layer's buffers is a slot (M = T k); entries routed to
    an expert outside [0, G) are dropped."""

    def __init__(self, T, k, G, H, I, device="cuda"):
        self.T, self.k, self.G, self.H, self.I = T, k, G, H, I
        self.offsets = torch.zeros(G + 1, dtype=torch.int32, device=device)
        self.src = torch.empty(T * k, dtype=torch.int32, device=device)
        self.slot_of = torch.empty((T, k), dtype=torch.int32, device=device)
        self.slot_weight = torch.empty(T * k, dtype=torch.float32, device=device)
        self.layer = MoELayer(self.offsets, T * k, H, I, device)
        self.out = _bf16(T, H, device=device)
        self.dX = _bf16(T, H, device=device)
        self.stages = WEIGHTS + ROUTED_FORWARD + ROUTED_BACKWARD

    def flops(self):
        return self.layer.flops()

    def forward(self, X, experts, weights, mark=None):
        L = self.layer
        mx_route_plan(experts, self.G, weights, self.offsets, self.src, self.slot_of, self.slot_weight)
        _mark(mark, ROUTED_FORWARD[0])
        x = L.x
        mx_gather_quantize(X, self.src, L.M, self.offsets, x.Mcap, None, x.q, x.s, x.qT, x.sT, x.P)
        _mark(mark, ROUTED_FORWARD[1])
        L.forward_experts(mark)
        mx_combine(L.y, self.slot_of, weights, out=self.out)
        _mark(mark, ROUTED_FORWARD[4])
        return self.out

    def backward(self, dOut, mark=None):
        L = self.layer
        dy = L.dy
        mx_gather_quantize(dOut, self.src, L.M, self.offsets, dy.Mcap, self.slot_weight, dy.q, dy.s, dy.qT, dy.sT,
                           dy.P)
        _mark(mark, ROUTED_BACKWARD[0])
        L.backward_experts(mark)
        mx_combine(L.dx, self.slot_of, None, out=self.dX)
        _mark(mark, ROUTED_BACKWARD[-1])
        return self.dX, L.dW1, L.dW2

    def step(self, X, dOut, experts, weights, W1, W2, mark=None):
        self.layer.quantize_weights(W1, W2, mark)
        self.forward(X, experts, weights, mark)
        return self.backward(dOut, mark)
