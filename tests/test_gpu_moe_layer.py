"""The MoE-layer chain (mxfp8_block_scaled_04_amd.moe_layer) on a small layer:
each stage's output against the fp64 oracle computed from that stage's own
GPU inputs, so a wrong buffer or operand anywhere in the chain shows up at
its stage.  The kernels themselves have their own parity tests; tolerances
here are theirs (GEMMs: 8e-3 |ref| + 1e-3 rms; quantization: bit-exact).
The layer's fused SwiGLU backward + quantization stage is checked against the
unfused calls (bf16 d(gate, up) and h, then the quantizers) and those against
the oracle's quantization; the whole step with and without the fusion must
agree bit for bit."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_04_amd as mx
import oracle
from mxfp8_block_scaled_04_amd import workloads as W
from mxfp8_block_scaled_04_amd.moe_layer import BACKWARD, BACKWARD_UNFUSED, FORWARD, WEIGHTS, MoELayer, RoutedMoELayer
from tests.mxtest import bf16_to_f64, bits, canonical_scales, combine_ok, gemm_tolerance_ok, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mx.load()


def wT_operands(qT, sT, G, Nout, Kin):
    """Expert g's W^T [Kin, Nout] from a column-wise quantized [G*Nout, Kin]
    weight (columns [g Nout, (g+1) Nout)) as oracle GEMM operands."""
    Wcap = qT.shape[1]
    q = u8(qT)
    s = canonical_scales(sT, Kin, Wcap)
    Bq = np.stack([q[:, g * Nout:(g + 1) * Nout] for g in range(G)])
    Bs = np.stack([s[:, g * Nout // 32:(g + 1) * Nout // 32] for g in range(G)])
    return Bq, Bs


def check_points(got, ref):
    ok, ratio = gemm_tolerance_ok(got, ref)
    assert ok, ratio


SIZES = [300, 0, 150, 250]


def small_layer(fuse):
    G, H, I = len(SIZES), 512, 256
    M = sum(SIZES)
    off_h = W.offsets_from_sizes(SIZES)
    off = torch.from_numpy(off_h).to(DEV)
    X = W.normal_bf16((M, H), 1.0, 1, DEV)
    W1 = mx.swiglu_interleave(W.normal_bf16((G, 2 * I, H), 1.2 / np.sqrt(H), 2, DEV))
    W2 = W.normal_bf16((G, H, I), 0.05, 3, DEV)
    dY = W.normal_bf16((M, H), 1.0, 4, DEV)
    layer = MoELayer(off, M, H, I, fuse_swiglu_backward=fuse)
    seen = []
    layer.step(X, dY, W1, W2, mark=seen.append)
    torch.cuda.synchronize()
    assert seen == list(layer.stages)
    return layer, (X, dY, W1, W2, off, off_h, G, H, I, M)


def test_moe_layer_chain_stages():
    layer, (X, dY, W1, W2, off, off_h, G, H, I, M) = small_layer(True)
    assert layer.stages == WEIGHTS + FORWARD + BACKWARD
    rng = np.random.default_rng(0)

    # weights and F1: bit-exact quantizations
    q, s = oracle.quantize_rows(bits(W1.reshape(G * 2 * I, H)))
    assert np.array_equal(u8(layer.w1.q), q) and np.array_equal(canonical_scales(layer.w1.s, G * 2 * I, H), s)
    qT, sT, P = oracle.quantize_cols(bits(W2.reshape(G * H, I)), (np.arange(G + 1) * H).astype(np.int32),
                                     layer.w2.Mcap)
    assert np.array_equal(u8(layer.w2.qT), qT)
    q, s = oracle.quantize_rows(bits(X))
    assert np.array_equal(u8(layer.x.q), q)
    qT, sT, P = oracle.quantize_cols(bits(X), off_h, layer.x.Mcap)
    assert np.array_equal(u8(layer.x.qT), qT) and np.array_equal(layer.x.P.cpu().numpy(), P)

    # F2: the fused kernel on the chain's operands, called on its own
    hq, hs, pre = mx.mx_grouped_gemm_swiglu(layer.x.q, layer.x.s, layer.w1.q.view(G, 2 * I, H), layer.w1.s, off,
                                            preact=True)
    torch.cuda.synchronize()
    assert torch.equal(hq, layer.hq)
    assert np.array_equal(canonical_scales(hs, M, I), canonical_scales(layer.hs, M, I))
    assert torch.equal(pre.view(torch.int16), layer.preact.view(torch.int16))

    # F3: Y = hq W2^T
    rows = rng.integers(0, M, 1500)
    cols = rng.integers(0, H, 1500)
    W2q = u8(layer.w2.q).reshape(G, H, I)
    W2s = canonical_scales(layer.w2.s, G * H, I).reshape(G, H, I // 32)
    ref = oracle.grouped_gemm_points(u8(layer.hq), canonical_scales(layer.hs, M, I), W2q, W2s, off_h, rows, cols)
    check_points(bf16_to_f64(layer.y)[rows, cols], ref)

    # B1 + B2: dH = dY W2
    q, s = oracle.quantize_rows(bits(dY))
    assert np.array_equal(u8(layer.dy.q), q)
    Bq, Bs = wT_operands(layer.w2.qT, layer.w2.sT, G, H, I)
    cols = rng.integers(0, I, 1500)
    ref = oracle.grouped_gemm_points(q, s, Bq, Bs, off_h, rows, cols)
    check_points(bf16_to_f64(layer.dh)[rows, cols], ref)

    # B3: the fused SwiGLU backward + quantization against the unfused calls
    # on the saved gate/up and dH (bf16 d(gate, up) and h, then quantized)
    dpre, h = mx.mx_swiglu_backward(layer.preact, layer.dh, h=True)
    dq, ds, dqT, dsT, P = mx.mx_quantize_dual(dpre, off, layer.x.Mcap)
    hT, hTs, hP = mx.mx_quantize_cols(h, off, layer.x.Mcap)
    torch.cuda.synchronize()
    assert torch.equal(dq, layer.dgu.q) and torch.equal(dqT, layer.dgu.qT) and torch.equal(hT, layer.hT)
    assert torch.equal(P, layer.dgu.P) and torch.equal(hP, layer.dgu.P)
    assert np.array_equal(canonical_scales(ds, M, 2 * I), canonical_scales(layer.dgu.s, M, 2 * I))
    Mcap = layer.x.Mcap
    assert np.array_equal(canonical_scales(dsT, 2 * I, Mcap), canonical_scales(layer.dgu.sT, 2 * I, Mcap))
    assert np.array_equal(canonical_scales(hTs, I, Mcap), canonical_scales(layer.hTs, I, Mcap))

    # B3 (h part) + B4: dW2 = dY^T h per expert
    qT, sT, P = oracle.quantize_cols(bits(h), off_h, layer.x.Mcap)
    assert np.array_equal(u8(layer.hT), qT) and np.array_equal(layer.dgu.P.cpu().numpy(), P)
    Aq, As = u8(layer.dy.qT), canonical_scales(layer.dy.sT, H, layer.x.Mcap)
    gs = rng.integers(0, G, 1500)
    ns = rng.integers(0, H, 1500)
    ks = rng.integers(0, I, 1500)
    ref = oracle.wgrad_points(Aq, As, qT, sT, P, gs, ns, ks)
    check_points(bf16_to_f64(layer.dW2)[gs, ns, ks], ref)

    # B3 (d(gate, up) row-wise) + B5: dX = d(gate, up) W1
    q, s = oracle.quantize_rows(bits(dpre))
    assert np.array_equal(u8(layer.dgu.q), q)
    assert np.array_equal(canonical_scales(layer.dgu.s, M, 2 * I), s)
    Bq, Bs = wT_operands(layer.w1.qT, layer.w1.sT, G, 2 * I, H)
    cols = rng.integers(0, H, 1500)
    ref = oracle.grouped_gemm_points(q, s, Bq, Bs, off_h, rows, cols)
    check_points(bf16_to_f64(layer.dx)[rows, cols], ref)

    # B3 (d(gate, up) column-wise) + B6: dW1 = d(gate, up)^T X per expert
    qT, sT, P = oracle.quantize_cols(bits(dpre), off_h, layer.x.Mcap)
    assert np.array_equal(u8(layer.dgu.qT), qT)
    ns = rng.integers(0, 2 * I, 1500)
    ks = rng.integers(0, H, 1500)
    ref = oracle.wgrad_points(qT, sT, u8(layer.x.qT), canonical_scales(layer.x.sT, H, layer.x.Mcap), P, gs, ns, ks)
    check_points(bf16_to_f64(layer.dW1)[gs, ns, ks], ref)


def test_moe_layer_fused_and_unfused_steps_agree():
    """The same step with the SwiGLU backward fused and unfused: every
    quantized buffer and every result bit for bit, and the unfused chain's
    bf16 intermediates as mx_swiglu_backward makes them."""
    fused, _ = small_layer(True)
    plain, (X, dY, W1, W2, off, off_h, G, H, I, M) = small_layer(False)
    assert plain.stages == WEIGHTS + FORWARD + BACKWARD_UNFUSED
    for name in ("y", "dh", "dx", "dW1", "dW2", "preact"):
        a, b = getattr(fused, name), getattr(plain, name)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
    for name in ("hq", "hT"):
        assert torch.equal(getattr(fused, name), getattr(plain, name)), name
    assert torch.equal(fused.dgu.q, plain.dgu.q) and torch.equal(fused.dgu.qT, plain.dgu.qT)
    assert torch.equal(fused.dgu.P, plain.dgu.P)
    Mcap = plain.x.Mcap
    assert np.array_equal(canonical_scales(fused.dgu.s, M, 2 * I), canonical_scales(plain.dgu.s, M, 2 * I))
    assert np.array_equal(canonical_scales(fused.dgu.sT, 2 * I, Mcap), canonical_scales(plain.dgu.sT, 2 * I, Mcap))
    assert np.array_equal(canonical_scales(fused.hTs, I, Mcap), canonical_scales(plain.hTs, I, Mcap))
    dpre, h = mx.mx_swiglu_backward(plain.preact, plain.dh, h=True)
    torch.cuda.synchronize()
    assert torch.equal(dpre.view(torch.int16), plain.dpre.view(torch.int16))
    assert torch.equal(h.view(torch.int16), plain.h.view(torch.int16))


def test_moe_layer_overlapped_step_matches_the_sequential_one():
    """The two-stream step: the same results bit for bit as the one-stream
    step, on two consecutive steps with the outputs cleared in between (a
    missing wait between the streams, or between steps, would read a buffer
    before it is written)."""
    seq, (X, dY, W1, W2, off, off_h, G, H, I, M) = small_layer(True)
    ovl = MoELayer(off, M, H, I)
    for rep in range(2):
        for t in (ovl.y, ovl.dx, ovl.dW1, ovl.dW2, ovl.dh, ovl.hT, ovl.dgu.q, ovl.dgu.qT):
            t.zero_()
        ovl.step_overlapped(X, dY, W1, W2)
        torch.cuda.synchronize()
        for name in ("y", "dh", "dx", "dW1", "dW2", "preact"):
            a, b = getattr(seq, name), getattr(ovl, name)
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (rep, name)
        for name in ("hq", "hT"):
            assert torch.equal(getattr(seq, name), getattr(ovl, name)), (rep, name)
        assert torch.equal(seq.dgu.q, ovl.dgu.q) and torch.equal(seq.dgu.qT, ovl.dgu.qT), rep


def test_routed_layer_is_dispatch_experts_and_combine():
    """The routed layer (600 tokens, top-4 of 8 experts): its plan against the
    oracle; its expert side bit for bit equal to a plain MoELayer step on the
    gathered token rows and the gathered, weight-scaled output gradient
    (formed here with torch: an fp32 product rounded to bf16); its combined
    output and token gradient against the oracle's combine."""
    T, k, G, H, I = 600, 4, 8, 512, 256
    e, w = W.topk_routing(T, k, G, 0.5, 41)
    ed, wd = torch.from_numpy(e).to(DEV), torch.from_numpy(w).to(DEV)
    X = W.normal_bf16((T, H), 1.0, 42, DEV)
    dOut = W.normal_bf16((T, H), 1.0, 43, DEV)
    W1 = mx.swiglu_interleave(W.normal_bf16((G, 2 * I, H), 1.2 / np.sqrt(H), 44, DEV))
    W2 = W.normal_bf16((G, H, I), 0.05, 45, DEV)
    R = RoutedMoELayer(T, k, G, H, I)
    seen = []
    R.step(X, dOut, ed, wd, W1, W2, mark=seen.append)
    torch.cuda.synchronize()
    assert seen == list(R.stages)
    o_ref, s_ref, so_ref = oracle.route_plan(e, G)
    assert np.array_equal(R.offsets.cpu().numpy(), o_ref) and np.array_equal(R.src.cpu().numpy(), s_ref)
    assert np.array_equal(R.slot_of.cpu().numpy(), so_ref)

    src = R.src.long()
    Xg = X.index_select(0, src)
    dYg = (dOut.index_select(0, src).float() * R.slot_weight[:, None]).to(torch.bfloat16)
    plain = MoELayer(R.offsets.clone(), T * k, H, I)
    plain.step(Xg, dYg, W1, W2)
    torch.cuda.synchronize()
    L = R.layer
    for name in ("y", "dh", "dx", "dW1", "dW2", "preact"):
        assert torch.equal(getattr(L, name).view(torch.int16), getattr(plain, name).view(torch.int16)), name
    for name in ("q", "qT"):
        assert torch.equal(getattr(L.x, name), getattr(plain.x, name)), name
        assert torch.equal(getattr(L.dy, name), getattr(plain.dy, name)), name

    ok, equal = combine_ok(bits(R.out), bits(L.y), so_ref, w)
    assert ok, equal
    ok, equal = combine_ok(bits(R.dX), bits(L.dx), so_ref, None)
    assert ok, equal


def test_routed_layer_with_dropped_entries_and_empty_experts():
    """Routing where experts 1, 4 and 6 get no token and about 10 % of the
    entries name no expert (-1): the routed rows are the first offsets[G]
    slots; their expert side equals a plain MoELayer over just those rows,
    the weight gradients of the empty experts are zero, and the combines skip
    the dropped entries."""
    T, k, G, H, I = 500, 4, 8, 512, 256
    rng = np.random.default_rng(51)
    e = rng.choice([0, 2, 3, 5, 7], (T, k)).astype(np.int32)
    e[rng.random((T, k)) < 0.1] = -1
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    ed, wd = torch.from_numpy(e).to(DEV), torch.from_numpy(w).to(DEV)
    X = W.normal_bf16((T, H), 1.0, 52, DEV)
    dOut = W.normal_bf16((T, H), 1.0, 53, DEV)
    W1 = mx.swiglu_interleave(W.normal_bf16((G, 2 * I, H), 1.2 / np.sqrt(H), 54, DEV))
    W2 = W.normal_bf16((G, H, I), 0.05, 55, DEV)
    R = RoutedMoELayer(T, k, G, H, I)
    R.step(X, dOut, ed, wd, W1, W2)
    torch.cuda.synchronize()
    o_ref, s_ref, so_ref = oracle.route_plan(e, G)
    Mr = int(o_ref[-1])
    assert Mr < T * k and np.array_equal(R.offsets.cpu().numpy(), o_ref)
    assert np.array_equal(R.slot_of.cpu().numpy(), so_ref)

    src = R.src[:Mr].long()
    plain = MoELayer(R.offsets.clone(), Mr, H, I)
    plain.step(X.index_select(0, src),
               (dOut.index_select(0, src).float() * R.slot_weight[:Mr, None]).to(torch.bfloat16), W1, W2)
    torch.cuda.synchronize()
    L = R.layer
    for name in ("y", "dh", "dx", "preact"):
        assert torch.equal(getattr(L, name)[:Mr].view(torch.int16), getattr(plain, name).view(torch.int16)), name
    for name in ("dW1", "dW2"):
        assert torch.equal(getattr(L, name).view(torch.int16), getattr(plain, name).view(torch.int16)), name
    for g in (1, 4, 6):
        assert not L.dW1[g].abs().sum() and not L.dW2[g].abs().sum(), g
    ok, equal = combine_ok(bits(R.out), bits(L.y[:Mr]), so_ref, w)
    assert ok, equal
    ok, equal = combine_ok(bits(R.dX), bits(L.dx[:Mr]), so_ref, None)
    assert ok, equal


def test_routed_layer_at_full_size_equals_the_plain_layer():
    """The routed layer at the benchmark's shape (4096 tokens top-8 of 16
    experts, H 7168, I 2048): its expert side, bit for bit, equals a plain
    MoELayer step on the gathered rows and the gathered, weight-scaled output
    gradient."""
    T, k, G, H, I = 4096, 8, 16, 7168, 2048
    e, w = W.topk_routing(T, k, G, 0.5, 61)
    ed, wd = torch.from_numpy(e).to(DEV), torch.from_numpy(w).to(DEV)
    X = W.normal_bf16((T, H), 1.0, 62, DEV)
    dOut = W.normal_bf16((T, H), 1.0, 63, DEV)
    W1 = mx.swiglu_interleave(W.normal_bf16((G, 2 * I, H), 0.02, 64, DEV))
    W2 = W.normal_bf16((G, H, I), 0.02, 65, DEV)
    R = RoutedMoELayer(T, k, G, H, I)
    R.step(X, dOut, ed, wd, W1, W2)
    torch.cuda.synchronize()
    src = R.src.long()
    plain = MoELayer(R.offsets.clone(), T * k, H, I)
    plain.step(X.index_select(0, src),
               (dOut.index_select(0, src).float() * R.slot_weight[:, None]).to(torch.bfloat16), W1, W2)
    torch.cuda.synchronize()
    L = R.layer
    for name in ("y", "dh", "dx", "dW1", "dW2", "preact"):
        assert torch.equal(getattr(L, name).view(torch.int16), getattr(plain, name).view(torch.int16)), name
    for name in ("q", "s", "qT", "sT"):
        assert torch.equal(getattr(L.x, name), getattr(plain.x, name)), name
        assert torch.equal(getattr(L.dy, name), getattr(plain.dy, name)), name
