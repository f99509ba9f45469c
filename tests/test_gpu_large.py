"""Inputs past 2^31 elements and 4 GiB.

Every kernel addresses its operands with 64-bit arithmetic, or with 32-bit
offsets from a 64-bit base set per tile; only inputs this large exercise the
upper halves of those addresses.  X is bf16 [600000, 7424]: 4.45e9 elements,
8.9 GB in, 4.45 GB of row-wise codes, and a column-wise result [7424, Mcap]
of 4.46 GB.  It is drawn on the device from a seeded generator.  The outputs
are checked on rows and columns sampled around the 2^31-element and 2^32-byte
boundaries and at both ends, against the oracle on the same input bits
(quantization: bit for bit; GEMMs: the grouped-GEMM tolerance).
"""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_04_amd as mx
import oracle
from mxfp8_block_scaled_04_amd import workloads as W
from tests.mxtest import bf16_to_f64, bits, gemm_tolerance_ok, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"
M, K = 600000, 7424
SIZES = [350001, 249999]


def boundary_rows():
    """Rows at the ends and around the rows holding element 2^31 of X and
    byte 2^32 of its fp8 codes."""
    rows = {0, 1, 31, 32, M - 33, M - 32, M - 1, SIZES[0] - 1, SIZES[0]}
    for b in (2 ** 31 // K, 2 ** 32 // K):
        rows |= {b - 1, b, b + 1}
    rng = np.random.default_rng(5)
    rows |= set(rng.integers(0, M, 24).tolist())
    return np.array(sorted(rows), np.int64)


@pytest.fixture(scope="module")
def big():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mx.load()
    x = W.normal_bf16((M, K), 1.0, 91, DEV)
    off_h = W.offsets_from_sizes(SIZES)
    off = torch.from_numpy(off_h).to(DEV)
    Mcap = mx.mx_cols_capacity(M, len(SIZES))
    assert K * Mcap > 2 ** 32 and M * K > 2 ** 32
    q, s = mx.mx_quantize_rows(x)
    qT, sT, P = mx.mx_quantize_cols(x, off, Mcap)
    torch.cuda.synchronize()
    data = dict(x=x, off=off, off_h=off_h, Mcap=Mcap, q=q, s=s, qT=qT, sT=sT, P=P)
    del x, q, s, qT, sT
    yield data
    data.clear()
    torch.cuda.empty_cache()


def unit_scales(packed, r, R_total, C):
    """Canonical scales [C / 32] of row r of a packed [R_total, C] scale array:
    its 32-row unit is a contiguous slice, unpacked by the oracle."""
    KB = 8 * ((C + 255) // 256)
    u = r // 32
    piece = u8(packed[u * 32 * KB:(u + 1) * 32 * KB])
    return oracle.unpack_scales(piece, 32, C)[r % 32]


def test_rows_past_4gib(big):
    rows = boundary_rows()
    idx = torch.from_numpy(rows).to(DEV)
    q_ref, s_ref = oracle.quantize_rows(bits(big["x"].index_select(0, idx)))
    assert np.array_equal(u8(big["q"].index_select(0, idx)), q_ref)
    for i, r in enumerate(rows):
        assert np.array_equal(unit_scales(big["s"], int(r), M, K), s_ref[i]), r


def test_cols_past_4gib(big):
    Mcap = big["Mcap"]
    cols = np.array(sorted({0, 1, 31, 32, 2 ** 32 // Mcap - 1, 2 ** 32 // Mcap, 2 ** 32 // Mcap + 1, K - 33,
                            K - 1}), np.int64)
    assert cols[-1] * Mcap > 2 ** 32
    idx = torch.from_numpy(cols).to(DEV)
    qT_ref, sT_ref, P_ref = oracle.quantize_cols(bits(big["x"].index_select(1, idx)), big["off_h"], Mcap)
    assert np.array_equal(big["P"].cpu().numpy(), P_ref)
    assert np.array_equal(u8(big["qT"].index_select(0, idx)), qT_ref)
    for i, c in enumerate(cols):
        assert np.array_equal(unit_scales(big["sT"], int(c), K, Mcap), sT_ref[i]), c


def test_dual_past_4gib_equals_the_single_layouts(big):
    q, s, qT, sT, P = mx.mx_quantize_dual(big["x"], big["off"], big["Mcap"])
    torch.cuda.synchronize()
    # every byte: M, K and the padded groups fill the layouts exactly (no
    # pad rows, blocks or columns)
    assert M % 32 == 0 and K % 256 == 0 and int(big["P"][-1]) == big["Mcap"]
    assert torch.equal(q, big["q"]) and torch.equal(s, big["s"])
    assert torch.equal(qT, big["qT"]) and torch.equal(sT, big["sT"]) and torch.equal(P, big["P"])


def test_grouped_gemm_with_a_4gib_operand(big):
    """Forward over the 4.45 GB row-wise codes (two experts, N = 256): all
    256 outputs of the sampled rows against the oracle, each row's group
    rebuilt on the host from the sampled rows alone."""
    G, N = len(SIZES), 256
    w = W.normal_bf16((G, N, K), 0.02, 92, DEV)
    Wq, Ws = mx.mx_quantize_rows(w.reshape(G * N, K))
    out = mx.mx_grouped_gemm(big["q"], big["s"], Wq.reshape(G, N, K), Ws, big["off"])
    torch.cuda.synchronize()
    rows = boundary_rows()
    groups = np.searchsorted(big["off_h"], rows, side="right") - 1
    order = np.argsort(groups, kind="stable")
    rows, groups = rows[order], groups[order]
    sub_off = np.searchsorted(groups, np.arange(G + 1), side="left").astype(np.int32)
    idx = torch.from_numpy(rows).to(DEV)
    Xq = u8(big["q"].index_select(0, idx))
    Xs = np.stack([unit_scales(big["s"], int(r), M, K) for r in rows])
    Wq_h = u8(Wq).reshape(G, N, K)
    Ws_h = oracle.unpack_scales(u8(Ws), G * N, K).reshape(G, N, K // 32)
    lr = np.repeat(np.arange(rows.size), N)
    lc = np.tile(np.arange(N), rows.size)
    ref = oracle.grouped_gemm_points(Xq, Xs, Wq_h, Ws_h, sub_off, lr, lc)
    got = bf16_to_f64(out.index_select(0, idx)).reshape(-1)
    ok, ratio = gemm_tolerance_ok(got, ref)
    assert ok, ratio


def test_wgrad_with_a_4gib_operand(big):
    """dW[g] = A_g^T B_g with A the 4.46 GB column-wise codes [7424, Mcap]
    and B those of a second [M, 256] input: sampled (g, n, k) against the
    oracle on the sampled rows of A."""
    Mcap = big["Mcap"]
    x2 = W.normal_bf16((M, 256), 1.0, 93, DEV)
    B, Bs, _ = mx.mx_quantize_cols(x2, big["off"], Mcap)
    dW = mx.mx_grouped_gemm_wgrad(big["qT"], big["sT"], B, Bs, big["P"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    ns = np.array(sorted({0, K - 1, 2 ** 32 // Mcap, 2 ** 32 // Mcap + 1} | set(rng.integers(0, K, 12).tolist())),
                  np.int64)
    Aq = u8(big["qT"].index_select(0, torch.from_numpy(ns).to(DEV)))
    As = np.stack([unit_scales(big["sT"], int(n), K, Mcap) for n in ns])
    Bq_h = u8(B)
    Bs_h = oracle.unpack_scales(u8(Bs), 256, Mcap)
    gs = np.repeat([0, 1], ns.size * 8)
    ln = np.tile(np.repeat(np.arange(ns.size), 8), 2)
    ks = rng.integers(0, 256, gs.size)
    ref = oracle.wgrad_points(Aq, As, Bq_h, Bs_h, big["P"].cpu().numpy(), gs, ln, ks)
    got = bf16_to_f64(dW)[gs, ns[ln], ks]
    ok, ratio = gemm_tolerance_ok(got, ref)
    assert ok, ratio
