"""The MoE-layer step captured as a HIP graph (torch.cuda.CUDAGraph): every
entry point it calls only launches kernels on the given stream and
allocates nothing, so the whole forward + backward chain can be recorded
once and replayed (the two-stream step too: its fork and join become graph
dependencies).  Each replay, with eager work and synchronizations
between replays (the outputs are cleared by eager kernels first, so a
replay that skipped a write would show), must reproduce the eager step bit
for bit."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_04_amd as mx
from mxfp8_block_scaled_04_amd import workloads as W
from mxfp8_block_scaled_04_amd.moe_layer import MoELayer, RoutedMoELayer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mx.load()


def outputs(layer):
    """The step's results that every step writes in full."""
    out = {"y": layer.y, "dx": layer.dx, "dW1": layer.dW1, "dW2": layer.dW2, "hq": layer.hq,
           "preact": layer.preact, "dh": layer.dh, "dgu.q": layer.dgu.q, "dgu.qT": layer.dgu.qT, "hT": layer.hT}
    if not layer.fused:
        out.update(dpre=layer.dpre, h=layer.h)
    return out


def bits_of(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("fuse,overlap", [(True, False), (False, False), (True, True)])
def test_layer_step_graph_replays_match_eager(fuse, overlap):
    M, H, I, G = 4096, 512, 256, 8
    sizes = W.dirichlet_sizes(M, G, 0.5, 21)
    off = torch.from_numpy(W.offsets_from_sizes(sizes)).to(DEV)
    X = W.normal_bf16((M, H), 1.0, 22, DEV)
    dY = W.normal_bf16((M, H), 1.0, 23, DEV)
    W1 = mx.swiglu_interleave(W.normal_bf16((G, 2 * I, H), 1.2 / np.sqrt(H), 24, DEV))
    W2 = W.normal_bf16((G, H, I), 1.2 / np.sqrt(I), 25, DEV)
    layer = MoELayer(off, M, H, I, fuse_swiglu_backward=fuse)
    run = layer.step_overlapped if overlap else layer.step

    run(X, dY, W1, W2)
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in outputs(layer).items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(X, dY, W1, W2)  # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(X, dY, W1, W2)
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outputs(layer).values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outputs(layer).items():
            assert torch.equal(bits_of(v), bits_of(want[k])), f"replay {rep}: {k} differs from the eager step"


def test_routed_layer_step_graph_replays_match_eager():
    """The routed step (route plan, dispatch, experts, combine and their
    backward) recorded once and replayed."""
    T, k, G, H, I = 1024, 4, 8, 512, 256
    e, w = W.topk_routing(T, k, G, 0.5, 26)
    ed, wd = torch.from_numpy(e).to(DEV), torch.from_numpy(w).to(DEV)
    X = W.normal_bf16((T, H), 1.0, 27, DEV)
    dOut = W.normal_bf16((T, H), 1.0, 28, DEV)
    W1 = mx.swiglu_interleave(W.normal_bf16((G, 2 * I, H), 1.2 / np.sqrt(H), 29, DEV))
    W2 = W.normal_bf16((G, H, I), 1.2 / np.sqrt(I), 30, DEV)
    R = RoutedMoELayer(T, k, G, H, I)
    run = lambda: R.step(X, dOut, ed, wd, W1, W2)
    res = lambda: {"out": R.out, "dX": R.dX, "dW1": R.layer.dW1, "dW2": R.layer.dW2, "src": R.src,
                   "slot_of": R.slot_of, "offsets": R.offsets}
    run()
    torch.cuda.synchronize()
    want = {n: v.clone() for n, v in res().items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in res().values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, v in res().items():
            assert torch.equal(bits_of(v), bits_of(want[n])), f"replay {rep}: {n} differs from the eager step"


def test_routed_layer_graph_follows_new_routing():
    """One capture serves every routing of the same shape: the plan, the
    group offsets and the slots are computed on the device from the expert
    ids the graph reads, so rewriting the ids and weights in place between
    replays must give the eager step on the new routing, bit for bit."""
    T, k, G, H, I = 1024, 4, 8, 512, 256
    routings = [W.topk_routing(T, k, G, a, s) for a, s in ((0.5, 40), (0.1, 41), (5.0, 42))]
    X = W.normal_bf16((T, H), 1.0, 43, DEV)
    dOut = W.normal_bf16((T, H), 1.0, 44, DEV)
    W1 = mx.swiglu_interleave(W.normal_bf16((G, 2 * I, H), 1.2 / np.sqrt(H), 45, DEV))
    W2 = W.normal_bf16((G, H, I), 1.2 / np.sqrt(I), 46, DEV)
    ed = torch.from_numpy(routings[0][0]).to(DEV)
    wd = torch.from_numpy(routings[0][1]).to(DEV)
    R = RoutedMoELayer(T, k, G, H, I)
    ref = RoutedMoELayer(T, k, G, H, I)
    run = lambda: R.step(X, dOut, ed, wd, W1, W2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for e, w in routings[1:] + routings[:1]:
        ed.copy_(torch.from_numpy(e))
        wd.copy_(torch.from_numpy(w))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref.step(X, dOut, ed, wd, W1, W2)
        torch.cuda.synchronize()
        assert torch.equal(R.offsets, ref.offsets) and torch.equal(R.slot_of, ref.slot_of)
        for name in ("out", "dX"):
            assert torch.equal(bits_of(getattr(R, name)), bits_of(getattr(ref, name))), name
        for name in ("dW1", "dW2"):
            assert torch.equal(bits_of(getattr(R.layer, name)), bits_of(getattr(ref.layer, name))), name


def test_layer_graph_follows_new_group_sizes():
    """The plain layer's capture reads the group offsets from device memory:
    new group sizes written in place between replays (an empty group, a
    one-row group, a single group) must give the eager step on them, bit for
    bit, in every output that the step writes in full."""
    M, H, I, G = 4096, 512, 256, 8
    size_sets = [W.dirichlet_sizes(M, G, 0.5, 31), [0, 1, 2047, 0, 1000, 31, 33, 984],
                 [0, 0, 0, M, 0, 0, 0, 0], W.dirichlet_sizes(M, G, 5.0, 32)]
    off = torch.from_numpy(W.offsets_from_sizes(size_sets[0])).to(DEV)
    X = W.normal_bf16((M, H), 1.0, 33, DEV)
    dY = W.normal_bf16((M, H), 1.0, 34, DEV)
    W1 = mx.swiglu_interleave(W.normal_bf16((G, 2 * I, H), 1.2 / np.sqrt(H), 35, DEV))
    W2 = W.normal_bf16((G, H, I), 1.2 / np.sqrt(I), 36, DEV)
    layer = MoELayer(off, M, H, I)
    ref = MoELayer(off, M, H, I)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.step(X, dY, W1, W2)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.step(X, dY, W1, W2)
    torch.cuda.synchronize()
    full = ("y", "dx", "dW1", "dW2", "hq", "preact", "dh")
    for sizes in size_sets[1:] + size_sets[:1]:
        assert sum(sizes) == M
        off.copy_(torch.from_numpy(W.offsets_from_sizes(sizes)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref.step(X, dY, W1, W2)
        torch.cuda.synchronize()
        for name in full:
            assert torch.equal(bits_of(getattr(layer, name)), bits_of(getattr(ref, name))), (sizes, name)
        assert torch.equal(layer.dgu.q, ref.dgu.q), sizes
