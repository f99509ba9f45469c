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


def combine_ok(out_bits, y_bits, slot_of, w=None):
    """A combine's bf16 result (bit patterns [T, N]) against the oracle's exact
    sum of the same y rows (y_bits [M, N], slot_of [T, k], w [T, k] or
    None): within the bf16 rounding (2^-8 of the value) plus the fp32
    rounding of the k steps (k 2^-24 of the magnitude sum), and at least 99 %
    equal to the oracle's bf16 rounding.  Returns (ok, fraction equal)."""
    exact = oracle.combine(y_bits, slot_of, w)
    got = (np.asarray(out_bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    yv = (np.asarray(y_bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    k = slot_of.shape[1]
    mag = np.zeros_like(exact)
    for j in range(k):
        valid = slot_of[:, j] >= 0
        wj = np.ones(slot_of.shape[0]) if w is None else np.abs(w[:, j]).astype(np.float64)
        mag[valid] += wj[valid, None] * np.abs(yv[slot_of[valid, j]])
    bound = 2.0 ** -8 * np.abs(exact) + k * 2.0 ** -24 * mag + 2.0 ** -133
    equal = float(np.mean(np.asarray(out_bits) == oracle.bf16_round(exact))) if exact.size else 1.0
    return bool(np.all(np.abs(got - exact) <= bound)) and equal >= 0.99, equal
