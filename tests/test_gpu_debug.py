"""The debug build (libmxmoe_debug.so: the same kernels with MXMOE_DEBUG,
whose device-side contract checks are read by mx_debug_flags): silent on
valid inputs, with every output bit-identical to the release build's, and
recording malformed group offsets and padded offsets (the SwiGLU backward
with its quantizations fused included).  Malformed offsets are
safe to run: the kernels clamp them (wrong results, no access out of
bounds), and the debug checks only record."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_04_amd as mx
import oracle
from mxfp8_block_scaled_04_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def libs():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    saved = mx._lib
    yield mx.open_library(mx.RELEASE_LIB_PATH), mx.open_library(mx.DEBUG_LIB_PATH)
    mx._lib = saved


def under(lib, fn):
    saved = mx._lib
    mx._lib = lib
    try:
        out = fn()
        torch.cuda.synchronize()
        return out
    finally:
        mx._lib = saved


def flat(out):
    if isinstance(out, torch.Tensor):
        return [out]
    return [t for o in out if o is not None for t in flat(o)]


def same(a, b):
    return all(torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y) for x, y in zip(flat(a), flat(b)))


def pipeline(d, off):
    """Every entry point that takes offsets, on the tiny MoE workload."""
    x, w, G = d["x"], d["w"], d["G"]
    N, K = w.shape[1], w.shape[2]
    Xq, Xs = mx.mx_quantize_rows(x)
    Wq, Ws = mx.mx_quantize_rows(w.reshape(G * N, K))
    Wq = Wq.reshape(G, N, K)
    out = {"cols": mx.mx_quantize_cols(x, off), "dual": mx.mx_quantize_dual(x, off),
           "fwd": mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, off)}
    wi = mx.swiglu_interleave(torch.cat([w, w.flip(1)], dim=1))
    Wi, Wis = mx.mx_quantize_rows(wi.reshape(G * 2 * N, K))
    hq, hs, pre = mx.mx_grouped_gemm_swiglu(Xq, Xs, Wi.reshape(G, 2 * N, K), Wis, off, preact=True)
    # hs: the scale bytes the contract defines (I = 128: the padding blocks
    # 4-7 of each row are left untouched)
    out["swiglu"] = (hq, pre, torch.from_numpy(oracle.unpack_scales(hs.cpu().numpy(), x.shape[0], N)))
    # its backward, plain and with the quantizations fused (scales compared
    # in their canonical form)
    M = x.shape[0]
    dh = W.normal_bf16((M, N), 1.0, 7, DEV)
    out["swiglu_bwd"] = mx.mx_swiglu_backward(pre, dh, h=True)
    q, s, qT, sT, hT, hTs, P2 = mx.mx_swiglu_backward_quant(pre, dh, off)
    Mcap = qT.shape[1]
    canon = lambda t, R, C: torch.from_numpy(oracle.unpack_scales(t.cpu().numpy(), R, C))
    out["swiglu_bwd_quant"] = (q, qT, hT, P2, canon(s, M, 2 * N), canon(sT, 2 * N, Mcap), canon(hTs, N, Mcap))
    # dispatch and combine: 128 tokens routed top-2 to the 4 experts
    e, wts = W.topk_routing(128, 2, G, 0.5, 8)
    ed, wd = torch.from_numpy(e).to(DEV), torch.from_numpy(wts).to(DEV)
    offs, src, slot_of, slot_w = mx.mx_route_plan(ed, G, wd)
    Mr = 256
    gq = mx.mx_gather_quantize(x[:128], src, Mr, offs, None, slot_w)
    McapR = gq[2].shape[1]
    out["routing"] = (offs, src, slot_of, slot_w, gq[0], gq[2], gq[4], canon(gq[1], Mr, K), canon(gq[3], K, McapR),
                      mx.mx_combine(x[:Mr], slot_of, wd))
    # backward of a projection with 256 outputs (dgrad contracts over them)
    N2 = 256
    w2 = W.normal_bf16((G, N2, K), 0.05, 6, DEV)
    dy = W.normal_bf16((x.shape[0], N2), 1.0, 5, DEV)
    dyq, dys = mx.mx_quantize_rows(dy)
    woff = torch.arange(0, G + 1, dtype=torch.int32, device=DEV) * N2
    wT, wTs, _ = mx.mx_quantize_cols(w2.reshape(G * N2, K), woff)
    out["dgrad"] = mx.mx_grouped_gemm_dgrad(dyq, dys, wT, wTs, off, G)
    A, As, P = mx.mx_quantize_cols(dy, off)
    B, Bs, _ = mx.mx_quantize_cols(x, off)
    out["wgrad"] = mx.mx_grouped_gemm_wgrad(A, As, B, Bs, P)
    return out


def test_release_build_has_no_checks(libs):
    rel, _ = libs
    with pytest.raises(mx.MxError) as e:
        under(rel, mx.mx_debug_flags)
    assert e.value.status == 5


def test_valid_inputs_silent_and_identical(libs):
    rel, dbg = libs
    d = W.tiny_moe(seed=0, device=DEV)
    off = torch.from_numpy(d["offsets"]).to(DEV)
    under(dbg, mx.mx_debug_flags)  # start from a clear word
    got = under(dbg, lambda: pipeline(d, off))
    assert under(dbg, mx.mx_debug_flags) == 0
    want = under(rel, lambda: pipeline(d, off))
    for k in want:
        assert same(got[k], want[k]), k


def test_malformed_offsets_recorded(libs):
    _, dbg = libs
    d = W.tiny_moe(seed=0, device=DEV)
    x, w = d["x"], d["w"][:3]
    bad = torch.tensor([0, 300, 200, 512], dtype=torch.int32, device=DEV)  # a decreasing step
    under(dbg, mx.mx_debug_flags)
    under(dbg, lambda: mx.mx_quantize_cols(x, bad))
    assert under(dbg, mx.mx_debug_flags) & 1
    Xq, Xs = under(dbg, lambda: mx.mx_quantize_rows(x))
    Wq, Ws = under(dbg, lambda: mx.mx_quantize_rows(w.reshape(3 * 128, 256)))
    under(dbg, lambda: mx.mx_grouped_gemm(Xq, Xs, Wq.reshape(3, 128, 256), Ws, bad))
    assert under(dbg, mx.mx_debug_flags) & 1
    over = torch.tensor([0, 160, 600], dtype=torch.int32, device=DEV)  # o[G] past M = 512
    under(dbg, lambda: mx.mx_quantize_cols(x, over))
    assert under(dbg, mx.mx_debug_flags) & 1
    valid = torch.tensor([0, 160, 512], dtype=torch.int32, device=DEV)
    under(dbg, lambda: mx.mx_quantize_cols(x, valid))
    assert under(dbg, mx.mx_debug_flags) == 0
    pre = W.normal_bf16((512, 256), 1.0, 8, DEV)
    dh = W.normal_bf16((512, 128), 1.0, 9, DEV)
    under(dbg, lambda: mx.mx_swiglu_backward_quant(pre, dh, bad))
    assert under(dbg, mx.mx_debug_flags) & 1
    under(dbg, lambda: mx.mx_swiglu_backward_quant(pre, dh, valid))
    assert under(dbg, mx.mx_debug_flags) == 0


def test_malformed_padded_offsets_recorded(libs):
    _, dbg = libs
    d = W.tiny_moe(seed=0, device=DEV)
    x = d["x"]
    off = torch.from_numpy(d["offsets"]).to(DEV)
    A, As, P = under(dbg, lambda: mx.mx_quantize_cols(x, off))
    under(dbg, mx.mx_debug_flags)
    badP = torch.tensor([0, 256, 100, 512, 768], dtype=torch.int32, device=DEV)  # not a multiple of 256, decreasing
    under(dbg, lambda: mx.mx_grouped_gemm_wgrad(A, As, A, As, badP))
    assert under(dbg, mx.mx_debug_flags) & 2
