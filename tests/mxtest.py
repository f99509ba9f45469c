"""Shared helpers of the GPU parity tests (no method arithmetic: conversions
between torch tensors and numpy bit patterns, the tolerance check)."""
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
