"""GPU parity of the dual-layout quantize (one read, row-wise and column-wise
results) against the CPU oracle's row-wise and column-wise quantization:
codes, packed scales (padding bytes included) and padded group offsets must
match bit for bit (lpnh.cn 2479732 section 1: the backward pass quantizes
the same gradient along both axes)."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_04_amd as mx
import oracle
from mxfp8_block_scaled_04_amd import workloads as W
from tests.mxtest import bits, canonical_scales, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mx.load()


FILL = 0xEE  # every output byte is prefilled: the kernel must write all of them


def check_dual(x_dev, sizes):
    M, N = x_dev.shape
    off = None if sizes is None else W.offsets_from_sizes(sizes)
    off_dev = None if off is None else torch.from_numpy(off).to(DEV)
    G = 1 if off is None else len(off) - 1
    Mcap = mx.mx_cols_capacity(M, G)
    fill = lambda *shape: torch.full(shape, FILL, dtype=torch.uint8, device=DEV)
    q, s, qT, sT, P = mx.mx_quantize_dual(x_dev, off_dev, Mcap, fill(M, N), fill(mx.mx_scale_bytes(M, N)),
                                          fill(N, Mcap), fill(mx.mx_scale_bytes(N, Mcap)))
    torch.cuda.synchronize()
    xb = bits(x_dev)
    q_ref, s_ref = oracle.quantize_rows(xb)
    assert np.array_equal(u8(q), q_ref), np.argwhere(u8(q) != q_ref)[:5]
    assert np.array_equal(u8(s), oracle.pack_scales(s_ref, N))  # pads included
    Mcap = qT.shape[1]
    qT_ref, sT_ref, P_ref = oracle.quantize_cols(xb, off, Mcap)
    if P is not None:
        assert np.array_equal(P.cpu().numpy(), P_ref)
    assert np.array_equal(u8(qT), qT_ref), np.argwhere(u8(qT) != qT_ref)[:5]
    assert np.array_equal(canonical_scales(sT, N, Mcap), sT_ref)
    assert np.count_nonzero(u8(sT)) == np.count_nonzero(sT_ref)  # pad bytes are zero


@pytest.mark.parametrize("sizes,N", [([160, 0, 96, 256], 64), ([1, 31, 33, 0, 257, 5], 96), ([300], 288),
                                     ([0, 0, 64], 32), ([512], 512), ([45], 256), ([7, 250, 700], 160),
                                     # the last group's last row tile ends before the packed array's pad
                                     # rows [M, 32 ceil(M / 32)): they are still written as zeros
                                     ([5, 256], 64), ([10, 250], 96)])
def test_dual_groups(sizes, N):
    g = torch.Generator(device=DEV)
    g.manual_seed(sum(sizes) * 7 + N)
    M = sum(sizes)
    x = (torch.randn((M, N), generator=g, device=DEV) * 3).to(torch.bfloat16)
    check_dual(x, sizes)


def test_dual_tiny_moe_and_null_offsets():
    # special blocks of the tiny workload: all-zero, bf16 denormals, a 1e4 outlier
    d = W.tiny_moe(seed=0, device=DEV)
    check_dual(d["x"], d["sizes"])
    check_dual(d["x"], None)
    check_dual(d["x"][:300, :224], None)


def test_dual_empty_rows():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    check_dual(x, [0, 0, 0])


def test_dual_down_backward_sampled():
    # the down projection's gradient dY [32768, 7168] with its 16 groups
    d = W.moe_down_backward(seed=0, device=DEV)
    off = d["offsets"]
    x = d["dy"]
    M, N = x.shape
    q, s, qT, sT, P = mx.mx_quantize_dual(x, torch.from_numpy(off).to(DEV))
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, M - 1], off[1:-1], off[1:-1] - 1, rng.integers(0, M, 64)]))
    rows = rows[(rows >= 0) & (rows < M)]
    q_ref, s_ref = oracle.quantize_rows(bits(x[torch.from_numpy(rows).to(DEV)]))
    assert np.array_equal(u8(q[torch.from_numpy(rows).to(DEV)]), q_ref)
    assert np.array_equal(canonical_scales(s, M, N)[rows], s_ref)
    Mcap = qT.shape[1]
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 24)]))
    qT_ref, sT_ref, P_ref = oracle.quantize_cols(bits(x[:, torch.from_numpy(cols).to(DEV)]), off, Mcap)
    assert np.array_equal(P.cpu().numpy(), P_ref)
    assert np.array_equal(u8(qT[torch.from_numpy(cols).to(DEV)]), qT_ref)
    assert np.array_equal(canonical_scales(sT, N, Mcap)[cols], sT_ref)


def test_dual_quant_bandwidth_sampled():
    """The quantize-bandwidth workload [131072, 7168] with no groups, as the
    benchmark runs it: sampled rows of the row-wise result (every 64-column
    sub-tile pair of each, so both halves of the jointly stored 128-byte
    pieces) and sampled columns of the column-wise result."""
    x = W.quant_bandwidth(seed=0, device=DEV)
    M, N = x.shape
    q, s, qT, sT, P = mx.mx_quantize_dual(x)
    torch.cuda.synchronize()
    assert P is None
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M - 1], rng.integers(0, M, 128)]))
    ridx = torch.from_numpy(rows).to(DEV)
    q_ref, s_ref = oracle.quantize_rows(bits(x[ridx]))
    assert np.array_equal(u8(q[ridx]), q_ref)
    assert np.array_equal(canonical_scales(s, M, N)[rows], s_ref)
    Mcap = qT.shape[1]
    cols = np.unique(np.concatenate([[0, 63, 64, 255, 256, N - 1], rng.integers(0, N, 16)]))
    cidx = torch.from_numpy(cols).to(DEV)
    qT_ref, sT_ref, _ = oracle.quantize_cols(bits(x[:, cidx]), None, Mcap)
    assert np.array_equal(u8(qT[cidx]), qT_ref)
    assert np.array_equal(canonical_scales(sT, N, Mcap)[cols], sT_ref)
