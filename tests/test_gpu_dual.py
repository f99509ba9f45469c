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
from tests.parity import assert_cols_are_oracle, assert_rows_are_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mx.load()


FILL = 0xEE  # every output byte is prefilled: the kernel must write all of them


def prefilled_dual(x_dev, off):
    """mx_quantize_dual into outputs whose every byte starts as FILL."""
    M, N = x_dev.shape
    off_dev = None if off is None else torch.from_numpy(off).to(DEV)
    G = 1 if off is None else len(off) - 1
    Mcap = mx.mx_cols_capacity(M, G)
    fill = lambda *shape: torch.full(shape, FILL, dtype=torch.uint8, device=DEV)
    out = mx.mx_quantize_dual(x_dev, off_dev, Mcap, fill(M, N), fill(mx.mx_scale_bytes(M, N)),
                              fill(N, Mcap), fill(mx.mx_scale_bytes(N, Mcap)))
    torch.cuda.synchronize()
    return out


def check_dual(x_dev, sizes):
    M, N = x_dev.shape
    off = None if sizes is None else W.offsets_from_sizes(sizes)
    q, s, qT, sT, P = prefilled_dual(x_dev, off)
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


def test_dual_down_backward_full():
    """The down projection's gradient dY [32768, 7168] with its 16 groups:
    every row-wise and column-wise code, packed scale byte and padded offset
    against the oracle."""
    d = W.moe_down_backward(seed=0, device=DEV)
    x = d["dy"]
    q, s, qT, sT, P = prefilled_dual(x, d["offsets"])
    torch.cuda.synchronize()
    assert_rows_are_oracle(x, q, s)
    assert_cols_are_oracle(x, d["offsets"], qT, sT, P)


def test_dual_quant_bandwidth_full():
    """The quantize-bandwidth workload [131072, 7168] with no groups, as the
    benchmark runs it: both results in full against the oracle."""
    x = W.quant_bandwidth(seed=0, device=DEV)
    q, s, qT, sT, P = prefilled_dual(x, None)
    assert P is None
    assert_rows_are_oracle(x, q, s)
    assert_cols_are_oracle(x, None, qT, sT)


def test_dual_element_map_exhaustive():
    """The exhaustive (bf16 pattern, scale) blocks through the dual kernel in
    both orientations: its row-wise result of X and its column-wise result of
    X^T must both be exactly the oracle's row-wise result of X."""
    from tests.test_gpu_quantize import _exhaustive_blocks, transposed_padded

    xb = _exhaustive_blocks()
    R, K = xb.shape
    q_ref, s_ref = oracle.quantize_rows(xb)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(DEV)
    q, s, _, _, _ = prefilled_dual(x, None)
    assert np.array_equal(u8(q), q_ref), np.argwhere(u8(q) != q_ref)[:5]
    assert np.array_equal(u8(s), oracle.pack_scales(s_ref, K))
    xT = transposed_padded(xb, 32)
    _, _, qT, sT, _ = prefilled_dual(xT, None)
    assert qT.shape[1] == K
    assert np.array_equal(u8(qT)[:R], q_ref), np.argwhere(u8(qT)[:R] != q_ref)[:5]
    assert np.array_equal(canonical_scales(sT, qT.shape[0], K)[:R], s_ref)
