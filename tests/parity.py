"""Harness of the GEMM parity tests (no method arithmetic here): the output
sample the measurement recipe fixes, oracle calls spread over host threads,
and the check that every GPU-quantized operand is the oracle's own
quantization of the same bf16 tensor, so that each GEMM check runs end to end
from the bf16 inputs.

The sample of a large grouped GEMM output is workloads.gemm_sample (a
128 x 128 tile per non-empty group, 4096 uniform points, every element of
the groups below 32 rows).  The oracle threads release the GIL (ctypes), so
the points run in parallel.
"""
import concurrent.futures
import os

import numpy as np
import torch

import oracle
from mxfp8_block_scaled_04_amd.workloads import gemm_sample  # noqa: F401  (re-exported for the tests)
from tests.mxtest import bits, canonical_scales, u8


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    # at most 16: the host CPU share that goes with one GPU of an 8-GPU node
    return max(1, min(n, 16))


THREADS = host_threads()


def _pool_map(fn, items):
    with concurrent.futures.ThreadPoolExecutor(THREADS) as ex:
        return list(ex.map(fn, items))


def _chunks(n):
    return [c for c in np.array_split(np.arange(n), THREADS) if c.size]


def oracle_points(Xq, Xs, Wq, Ws, offsets, rows, cols):
    """oracle.grouped_gemm_points over host threads."""
    parts = _pool_map(lambda c: oracle.grouped_gemm_points(Xq, Xs, Wq, Ws, offsets, rows[c], cols[c]),
                      _chunks(rows.size))
    return np.concatenate(parts) if parts else np.zeros(0)


def oracle_by_rows(fn, X, Xs, weights, offsets):
    """fn(X[rows], Xs[rows], *weights, offsets of the slice) over row slices
    on host threads, outputs joined along rows: for the row-grouped oracles
    (grouped_gemm, grouped_gemm_swiglu), whose rows are independent.  A slice
    [r0, r1) keeps each row's group: its offsets are clip(offsets - r0)."""
    offsets = np.asarray(offsets, np.int64)

    def run(c):
        r0, r1 = int(c[0]), int(c[-1]) + 1
        off = np.clip(offsets - r0, 0, r1 - r0).astype(np.int32)
        return fn(X[r0:r1], Xs[r0:r1], *weights, off)

    parts = _pool_map(run, _chunks(X.shape[0]))
    if isinstance(parts[0], tuple):
        return tuple(np.concatenate([p[i] for p in parts]) for i in range(len(parts[0])))
    return np.concatenate(parts)


def oracle_swiglu_blocks(Xq, Xs, Wgq, Wgs, Wuq, Wus, offsets, rows, blocks):
    """oracle.grouped_gemm_swiglu_blocks over host threads (blocks split into
    contiguous chunks, outputs joined in order)."""
    parts = _pool_map(lambda c: oracle.grouped_gemm_swiglu_blocks(Xq, Xs, Wgq, Wgs, Wuq, Wus, offsets, rows[c],
                                                                   blocks[c]), _chunks(rows.size))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(len(parts[0])))


def oracle_full(Xq, Xs, Wq, Ws, offsets):
    """The whole fp64 grouped-GEMM reference [M, N], rows over host threads."""
    return oracle_by_rows(oracle.grouped_gemm, Xq, Xs, (Wq, Ws), offsets)


def oracle_wgrad_full(Aq, As, Bq, Bs, padded):
    """The whole fp64 wgrad reference [G, N, K], groups over host threads."""
    G = len(padded) - 1
    N, K = Aq.shape[0], Bq.shape[0]
    out = np.zeros((G, N, K), np.float64)
    gg, nn, kk = np.meshgrid(np.arange(G), np.arange(N), np.arange(K), indexing="ij")
    gg, nn, kk = gg.ravel(), nn.ravel(), kk.ravel()
    out.reshape(-1)[:] = oracle_wgrad_points(Aq, As, Bq, Bs, padded, gg, nn, kk)
    return out


def oracle_wgrad_points(Aq, As, Bq, Bs, padded, gs, ns, ks):
    parts = _pool_map(lambda c: oracle.wgrad_points(Aq, As, Bq, Bs, padded, gs[c], ns[c], ks[c]),
                      _chunks(gs.size))
    return np.concatenate(parts) if parts else np.zeros(0)


def oracle_quantize_rows(xbits):
    """oracle.quantize_rows of uint16 [R, K] over host threads."""
    parts = _pool_map(lambda c: oracle.quantize_rows(xbits[c[0]:c[-1] + 1]), _chunks(xbits.shape[0]))
    return np.concatenate([q for q, _ in parts]), np.concatenate([s for _, s in parts])


def oracle_quantize_cols(xbits, offsets, Mcap):
    """oracle.quantize_cols of uint16 [M, N] over host threads (columns are
    independent: each thread takes a range of them)."""
    N = xbits.shape[1]
    cuts = [c for c in np.array_split(np.arange(N // 8), THREADS) if c.size]

    def run(c):
        n0, n1 = 8 * int(c[0]), 8 * (int(c[-1]) + 1)
        return oracle.quantize_cols(np.ascontiguousarray(xbits[:, n0:n1]), offsets, Mcap)

    parts = _pool_map(run, cuts)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]), parts[0][2]


def assert_rows_are_oracle(x_dev, q_dev, s_dev):
    """The GPU's row-wise codes and packed scales of bf16 x are exactly the
    oracle's (packed pad bytes included).  Returns the oracle's codes and
    canonical scales."""
    xb = bits(x_dev)
    R, K = xb.shape
    q_ref, s_ref = oracle_quantize_rows(xb)
    q = u8(q_dev).reshape(R, K)
    assert np.array_equal(q, q_ref), f"row-wise codes differ at {np.argwhere(q != q_ref)[:3].tolist()}"
    assert np.array_equal(u8(s_dev), oracle.pack_scales(s_ref, K)), "packed row-wise scales differ"
    return q_ref, s_ref


def assert_cols_are_oracle(x_dev, offsets, qT_dev, sT_dev, P_dev=None):
    """The GPU's column-wise codes, packed scales and padded offsets of bf16
    x are exactly the oracle's.  Returns the oracle's qT, canonical sT, P."""
    xb = bits(x_dev)
    N = xb.shape[1]
    Mcap = qT_dev.shape[1]
    qT_ref, sT_ref, P_ref = oracle_quantize_cols(xb, offsets, Mcap)
    assert np.array_equal(u8(qT_dev), qT_ref), "column-wise codes differ"
    assert np.array_equal(canonical_scales(sT_dev, N, Mcap), sT_ref), "column-wise scales differ"
    assert np.count_nonzero(u8(sT_dev)) == np.count_nonzero(sT_ref), "column-wise scale pad bytes are not zero"
    if P_dev is not None:
        assert np.array_equal(P_dev.cpu().numpy(), P_ref), "padded offsets differ"
    return qT_ref, sT_ref, P_ref


def gathered(out_dev, rows, cols):
    """bf16 elements out[rows[i], cols[i]] as float64 (gathered on the GPU)."""
    r = torch.from_numpy(rows).to(out_dev.device)
    c = torch.from_numpy(cols).to(out_dev.device)
    return out_dev[r, c].float().cpu().numpy().astype(np.float64)
