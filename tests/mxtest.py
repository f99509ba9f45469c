"""Shared helpers of the GPU parity tests (no method arithmetic: conversions
between torch tensors and numpy bit patterns, the tolerance check, sampling)."""
import numpy as np
import torch

import oracle


def bits(x):
    """torch bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u8(x):
    return x.detach().cpu().contiguous().numpy().view(np.uint8)


def bf16_to_f64(t):
    return t.detach().cpu().float().numpy().astype(np.float64)


def gemm_tolerance_ok(gpu, ref, rms=None):
    """|gpu - ref| <= 8e-3 |ref| + 1e-3 rms(ref) elementwise; returns (ok, worst ratio)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = 8e-3 * np.abs(ref) + 1e-3 * rms
    err = np.abs(gpu - ref)
    finite = np.all(np.isfinite(gpu))
    ratio = float(np.max(err / np.maximum(bound, 1e-300))) if ref.size else 0.0
    return bool(finite and np.all(err <= bound)), ratio


def canonical_scales(packed, R, K):
    """Kernel's packed scale array -> canonical [R, K/32] via the oracle's unpack."""
    return oracle.unpack_scales(u8(packed), R, K)


def sample_points(rng, M, N, offsets, n_random=4096, block=8):
    """Deterministic sample of output points: n_random uniform points, a
    block x block patch at the start of every non-empty group, and every row
    (first 8 columns, last column) of groups with fewer than 32 rows."""
    rows = list(rng.integers(0, M, n_random))
    cols = list(rng.integers(0, N, n_random))
    G = len(offsets) - 1
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi <= lo:
            continue
        for r in range(lo, min(lo + block, hi)):
            for c in range(min(block, N)):
                rows.append(r)
                cols.append(c)
        if hi - lo < 32:
            for r in range(lo, hi):
                for c in list(range(min(8, N))) + [N - 1]:
                    rows.append(r)
                    cols.append(c)
        rows.append(hi - 1)
        cols.append(N - 1)
    return np.array(rows, np.int64), np.array(cols, np.int64)
