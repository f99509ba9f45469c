"""GPU parity of mx_swiglu_backward against the fp64 oracle.

The kernel computes in fp32 with hardware exp2 and reciprocal and rounds to
bf16; the oracle computes in double and rounds once.  Per element (u = 2^-24):
  |dg - dg_ref| <= 2^-8 |dg_ref| + 2^-18 |dh up| (1 + |g|)
  |du - du_ref| <= 2^-8 |du_ref| + 2^-20 |dh g|
  |h - h_ref|   <= 2^-8 |h_ref|  + 2^-20 |g up|
(half a bf16 step of the result, plus the fp32 error of sigma and of the
cancelling 1 + g (1 - sigma) near silu's minimum), and at least 99 % of the
results must equal the oracle's bf16 bit patterns exactly.
"""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_04_amd as mx
import oracle
from mxfp8_block_scaled_04_amd import workloads as W
from tests.mxtest import bits

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAN = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mx.load()


def f64(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def deinterleave(a, I):
    """[M, 2I] in the interleaved order -> (gate [M, I], up [M, I])."""
    M = a.shape[0]
    a4 = a.reshape(M, I // 32, 2, 32)
    return a4[:, :, 0].reshape(M, I), a4[:, :, 1].reshape(M, I)


def check(pre, dh, rows=None, min_exact=0.99):
    M, N2 = pre.shape
    I = N2 // 2
    dpre = torch.full((M, N2), NAN, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    h = torch.full((M, I), NAN, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    dpre, h = mx.mx_swiglu_backward(pre, dh, dpre=dpre, h=h)
    dpre2, none = mx.mx_swiglu_backward(pre, dh)
    torch.cuda.synchronize()
    assert none is None and torch.equal(dpre.view(torch.int16), dpre2.view(torch.int16))
    pb, db, gb, hb = bits(pre), bits(dh), bits(dpre), bits(h)
    if rows is not None:
        pb, db, gb, hb = pb[rows], db[rows], gb[rows], hb[rows]
    g, u = (f64(t) for t in deinterleave(pb, I))
    d = f64(db)
    dg_b, du_b = deinterleave(gb, I)
    dg_ref, du_ref, h_ref = oracle.swiglu_backward(g, u, d)
    exact = []
    for got_b, ref, slack in ((dg_b, dg_ref, 2.0 ** -18 * np.abs(d * u) * (1 + np.abs(g))),
                              (du_b, du_ref, 2.0 ** -20 * np.abs(d * g)),
                              (hb, h_ref, 2.0 ** -20 * np.abs(g * u))):
        got = f64(got_b)
        assert np.all(np.isfinite(got))
        bound = 2.0 ** -8 * np.abs(ref) + slack + 1e-38
        bad = np.argwhere(np.abs(got - ref) > bound)
        assert bad.size == 0, f"element {bad[0]}: {got[tuple(bad[0])]!r} vs {ref[tuple(bad[0])]!r}"
        exact.append(float(np.mean(got_b == oracle.bf16_round(ref))))
    print("bit-exact fractions (dg, du, h):", exact)
    assert min(exact) >= min_exact, exact


@pytest.mark.parametrize("M,I", [(513, 256), (1, 32), (64, 2048), (300, 96)])
def test_swiglu_backward_full(M, I):
    pre = W.normal_bf16((M, 2 * I), 1.7, 500 + M, DEV)
    dh = W.normal_bf16((M, I), 1.0, 600 + M, DEV)
    check(pre, dh)


def test_swiglu_backward_special_values():
    """Saturated gates (+-20, +-90, +-300), zeros, silu's minimum, bf16
    subnormals and large magnitudes (products stay below the bf16 maximum).
    Where fp32's exp overflows (gate <= -89) the kernel's results are zero and
    the oracle's tiny: only the per-element bounds apply."""
    M, I = 8, 64
    rng = np.random.default_rng(7)
    g = rng.choice([0.0, -0.0, 20.0, -20.0, 90.0, -90.0, 300.0, -300.0, -1.2784645, 1e-39, -3e-39, 1e10, -1e10,
                    2.5], (M, I))
    u = rng.choice([0.0, 1.0, -3.0, 1e-38, 7e10, -2.0 ** -130], (M, I))
    d = rng.choice([0.0, 1.0, -0.5, 1e-20, 3e15], (M, I))
    pre = np.stack([g.reshape(M, I // 32, 32), u.reshape(M, I // 32, 32)], axis=2).reshape(M, 2 * I)
    to_dev = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(DEV)
    check(to_dev(pre), to_dev(d), min_exact=0.0)


def test_swiglu_backward_gate_up_shape_sampled():
    """The gate+up workload's activation shape, [32768, 2048]: full run,
    256 sampled rows checked."""
    M, I = 32768, 2048
    pre = W.normal_bf16((M, 2 * I), 1.7, 11, DEV)
    dh = W.normal_bf16((M, I), 1.0, 12, DEV)
    rows = np.sort(np.random.default_rng(13).choice(M, 256, replace=False))
    check(pre, dh, rows=rows)


FILL = 0xEE


def fused_against_chain(preact, dh, sizes):
    """mx_swiglu_backward_quant against mx_swiglu_backward followed by
    mx_quantize_dual of d(gate, up) and mx_quantize_cols of h (each of those
    checked against the oracle by its own tests), every output prefilled with
    FILL: every byte, written or left alone, must be the same."""
    M, I = dh.shape
    off = None if sizes is None else torch.from_numpy(W.offsets_from_sizes(sizes)).to(DEV)
    G = 1 if sizes is None else len(sizes)
    Mcap = mx.mx_cols_capacity(M, G)
    fill = lambda *shape: torch.full(shape, FILL, dtype=torch.uint8, device=DEV)
    bufs = lambda: (fill(M, 2 * I), fill(mx.mx_scale_bytes(M, 2 * I)), fill(2 * I, Mcap),
                    fill(mx.mx_scale_bytes(2 * I, Mcap)), fill(I, Mcap), fill(mx.mx_scale_bytes(I, Mcap)))
    q, s, qT, sT, hT, hTs = bufs()
    dpre, h = mx.mx_swiglu_backward(preact, dh, h=True)
    _, _, _, _, P = mx.mx_quantize_dual(dpre, off, Mcap, q, s, qT, sT)
    mx.mx_quantize_cols(h, off, Mcap, hT, hTs)
    f = bufs()
    got = mx.mx_swiglu_backward_quant(preact, dh, off, Mcap, *f)
    torch.cuda.synchronize()
    for name, a, b in zip(("q", "s", "qT", "sT", "hT", "hTs"), (q, s, qT, sT, hT, hTs), got[:6]):
        assert torch.equal(a, b), f"{name}: {int((a != b).sum())} bytes differ"
    if P is not None:
        assert torch.equal(P, got[6])


@pytest.mark.parametrize("sizes,I", [([100, 0, 37, 300, 163], 128), ([1, 31, 33, 0, 257, 5], 256), ([513], 384),
                                     ([0, 0, 64], 128), (None, 128)])
def test_swiglu_backward_quant_matches_the_chain(sizes, I):
    M = 300 if sizes is None else sum(sizes)
    preact = (W.normal_bf16((M, 2 * I), 1.0, 60 + M, DEV).float() * 3).to(torch.bfloat16)
    dh = W.normal_bf16((M, I), 1.0, 61 + M, DEV)
    fused_against_chain(preact, dh, sizes)


def test_swiglu_backward_quant_layer_shape():
    """The MoE layer's shape (32768 rows, I = 2048, the 16 Dirichlet groups)."""
    d = W.moe_gate_up(seed=0, device=DEV)
    M, I = d["M"], d["N"] // 2
    preact = (W.normal_bf16((M, 2 * I), 1.0, 70, DEV).float() * 3).to(torch.bfloat16)
    dh = W.normal_bf16((M, I), 1.0, 71, DEV)
    fused_against_chain(preact, dh, list(d["sizes"]))
