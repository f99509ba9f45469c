"""Python binding of libmxmoe (MXFP8 quantization + block-scaled grouped GEMM
for MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libmxmoe.so``; PyTorch supplies device memory and the stream.  The
functions carry the names of the C entry points (see include/libmxmoe.h for
the contract of each).  If the library has not been built, importing works
but every call raises ``RuntimeError`` -- there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MXMOE_DEBUG=1 loads the debug build (device-side contract checks, read with
# debug_flags()); otherwise the release build
RELEASE_LIB_PATH = os.path.join(_HERE, "libmxmoe.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libmxmoe_debug.so")
LIB_PATH = DEBUG_LIB_PATH if os.environ.get("MXMOE_DEBUG") == "1" else RELEASE_LIB_PATH

MX_OK = 0
_lib = None


class MxError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


def load():
    """Load libmxmoe.so (built by ``python -m mxfp8_block_scaled_04_amd.build``)."""
    global _lib
    if _lib is None:
        _lib = open_library(LIB_PATH)
    return _lib


def open_library(path):
    """ctypes handle of a libmxmoe build at `path`, with the C signatures set."""
    if not os.path.exists(path):
        raise RuntimeError(f"{os.path.basename(path)} not built ({path}); run python -m mxfp8_block_scaled_04_amd.build")
    lib = ctypes.CDLL(path)
    P, I64, I32, ST = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    lib.mx_status_str.argtypes = [ctypes.c_int]
    lib.mx_status_str.restype = ctypes.c_char_p
    lib.mx_version.restype = ctypes.c_int
    lib.mx_scale_bytes.argtypes = [I64, I64]
    lib.mx_scale_bytes.restype = I64
    lib.mx_cols_capacity.argtypes = [I64, I32]
    lib.mx_cols_capacity.restype = I64
    lib.mx_quantize_rows.argtypes = [P, I64, I64, I64, P, P, P]
    lib.mx_quantize_rows.restype = ST
    lib.mx_quantize_cols.argtypes = [P, I64, I64, I64, P, I32, P, P, I64, P, P]
    lib.mx_quantize_cols.restype = ST
    lib.mx_quantize_dual.argtypes = [P, I64, I64, I64, P, I32, P, P, P, P, I64, P, P]
    lib.mx_quantize_dual.restype = ST
    lib.mx_grouped_gemm.argtypes = [P, P, P, P, P, I32, I64, I64, I64, P, P]
    lib.mx_grouped_gemm.restype = ST
    lib.mx_grouped_gemm_swiglu.argtypes = [P, P, P, P, P, I32, I64, I64, I64, P, P, P, P]
    lib.mx_grouped_gemm_swiglu.restype = ST
    lib.mx_swiglu_backward.argtypes = [P, P, I64, I64, P, P, P]
    lib.mx_swiglu_backward.restype = ST
    lib.mx_validate_offsets.argtypes = [P, I32, I64, P, P]
    lib.mx_validate_offsets.restype = ST
    lib.mx_stream21.argtypes = [P, P, I64, P]
    lib.mx_stream21.restype = ST
    lib.mx_probe_mfma_scale.argtypes = [P, P, P, P, P, P, I32, P]
    lib.mx_probe_mfma_scale.restype = ST
    lib.mx_swiglu_backward_quant.argtypes = [P, P, I64, I64, P, I32, P, P, P, P, P, P, I64, P, P]
    lib.mx_swiglu_backward_quant.restype = ST
    lib.mx_route_plan.argtypes = [P, P, I64, I32, I32, P, P, P, P, P]
    lib.mx_route_plan.restype = ST
    lib.mx_gather_quantize.argtypes = [P, I64, I64, I64, P, P, I64, P, I32, P, P, P, P, I64, P, P]
    lib.mx_gather_quantize.restype = ST
    lib.mx_combine.argtypes = [P, I64, I64, I64, P, P, I64, I32, P, P]
    lib.mx_combine.restype = ST
    lib.mx_debug_flags.argtypes = [P, P]
    lib.mx_debug_flags.restype = ST
    lib.mx_grouped_gemm_dgrad.argtypes = [P, P, P, P, P, I32, I64, I64, I64, I64, P, P]
    lib.mx_grouped_gemm_dgrad.restype = ST
    lib.mx_grouped_gemm_wgrad.argtypes = [P, P, P, P, P, I32, I64, I64, I64, P, P]
    lib.mx_grouped_gemm_wgrad.restype = ST
    return lib


# Exported C symbols, in header order.
SYMBOLS = (
    "mx_status_str", "mx_version", "mx_scale_bytes", "mx_cols_capacity", "mx_quantize_rows",
    "mx_quantize_cols", "mx_quantize_dual", "mx_grouped_gemm", "mx_grouped_gemm_swiglu", "mx_grouped_gemm_dgrad", "mx_grouped_gemm_wgrad",
    "mx_swiglu_backward", "mx_swiglu_backward_quant", "mx_route_plan", "mx_gather_quantize", "mx_combine",
    "mx_validate_offsets", "mx_stream21", "mx_probe_mfma_scale", "mx_debug_flags",
)


def status_str(status):
    try:
        return load().mx_status_str(int(status)).decode()
    except RuntimeError:
        return str(status)


def mx_scale_bytes(R, K):
    return int(load().mx_scale_bytes(int(R), int(K)))


def mx_cols_capacity(M, G=1):
    return int(load().mx_cols_capacity(int(M), int(G)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc, where):
    if rc != MX_OK:
        raise MxError(rc, where)


def _bits16(x):
    if x.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return x
    raise TypeError(f"expected bf16 (or its 16-bit pattern), got {x.dtype}")


def mx_quantize_rows(x, q=None, s=None, stream=None):
    """Row-wise MXFP8 of bf16 x [M, K] (row stride may exceed K).
    Returns (q uint8 [M, K], s uint8 packed scales [mx_scale_bytes(M, K)])."""
    x = _bits16(x)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(mx_scale_bytes(M, K), dtype=torch.uint8, device=x.device)
    rc = load().mx_quantize_rows(_ptr(x), M, K, x.stride(0), _ptr(q), _ptr(s), _stream(stream))
    _check(rc, "mx_quantize_rows")
    return q, s


def mx_quantize_cols(x, group_offsets=None, Mcap=None, qT=None, sT=None, padded_offsets=None, stream=None):
    """Column-wise (transposed) MXFP8 of bf16 x [M, N] with optional row groups.
    Returns (qT uint8 [N, Mcap], sT packed scales, padded_offsets int32 [G+1] or None)."""
    x = _bits16(x)
    M, N = x.shape
    G = 1 if group_offsets is None else group_offsets.numel() - 1
    if Mcap is None:
        Mcap = mx_cols_capacity(M, G)
    if qT is None:
        qT = torch.empty((N, Mcap), dtype=torch.uint8, device=x.device)
    if sT is None:
        sT = torch.empty(mx_scale_bytes(N, Mcap), dtype=torch.uint8, device=x.device)
    if group_offsets is not None and padded_offsets is None:
        padded_offsets = torch.empty(G + 1, dtype=torch.int32, device=x.device)
    rc = load().mx_quantize_cols(_ptr(x), M, N, x.stride(0), _ptr(group_offsets), G, _ptr(qT), _ptr(sT), Mcap,
                                 _ptr(padded_offsets), _stream(stream))
    _check(rc, "mx_quantize_cols")
    return qT, sT, padded_offsets


def mx_quantize_dual(x, group_offsets=None, Mcap=None, q=None, s=None, qT=None, sT=None, padded_offsets=None,
                     stream=None):
    """Row-wise and column-wise MXFP8 of bf16 x [M, N] from one read.
    Returns (q, s, qT, sT, padded_offsets): the results of mx_quantize_rows and
    mx_quantize_cols."""
    x = _bits16(x)
    M, N = x.shape
    G = 1 if group_offsets is None else group_offsets.numel() - 1
    if Mcap is None:
        Mcap = mx_cols_capacity(M, G)
    if q is None:
        q = torch.empty((M, N), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(mx_scale_bytes(M, N), dtype=torch.uint8, device=x.device)
    if qT is None:
        qT = torch.empty((N, Mcap), dtype=torch.uint8, device=x.device)
    if sT is None:
        sT = torch.empty(mx_scale_bytes(N, Mcap), dtype=torch.uint8, device=x.device)
    if group_offsets is not None and padded_offsets is None:
        padded_offsets = torch.empty(G + 1, dtype=torch.int32, device=x.device)
    rc = load().mx_quantize_dual(_ptr(x), M, N, x.stride(0), _ptr(group_offsets), G, _ptr(q), _ptr(s), _ptr(qT),
                                 _ptr(sT), Mcap, _ptr(padded_offsets), _stream(stream))
    _check(rc, "mx_quantize_dual")
    return q, s, qT, sT, padded_offsets


def mx_grouped_gemm(Xq, Xs, Wq, Ws, group_offsets, out=None, stream=None):
    """out[m, n] = sum_k deq(Xq[m, k]) deq(Wq[g(m), n, k]) in bf16.
    Xq uint8 [M, K]; Wq uint8 [G, N, K]; scales packed; group_offsets int32 [G+1]."""
    M, K = Xq.shape
    G, N, K2 = Wq.shape
    if K2 != K:
        raise ValueError("K mismatch")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=Xq.device)
    rc = load().mx_grouped_gemm(_ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws), _ptr(group_offsets), G, M, N, K, _ptr(out),
                                _stream(stream))
    _check(rc, "mx_grouped_gemm")
    return out


def swiglu_interleave(w):
    """Row order of the gate+up weights for mx_grouped_gemm_swiglu: w [G, 2I, K]
    with gate rows [0, I) and up rows [I, 2I) -> rows alternating 32-row gate
    and up blocks (a view-free reordering; works on bf16 or fp8 code rows)."""
    G, N2, K = w.shape
    I = N2 // 2
    gate = w[:, :I].reshape(G, I // 32, 32, K)
    up = w[:, I:].reshape(G, I // 32, 32, K)
    return torch.stack([gate, up], dim=2).reshape(G, N2, K)


def mx_grouped_gemm_swiglu(Xq, Xs, Wq, Ws, group_offsets, hq=None, hs=None, preact=None, stream=None):
    """Gate+up grouped GEMM + SwiGLU + MXFP8 quantization of the result.
    Wq uint8 [G, 2I, K] in swiglu_interleave order.  preact: None, True (allocate)
    or a bf16 [M, 2I] tensor that also receives the gate/up values.
    Returns (hq uint8 [M, I], hs packed, preact or None)."""
    M, K = Xq.shape
    G, N2, K2 = Wq.shape
    if K2 != K or N2 % 2:
        raise ValueError("shape mismatch")
    I = N2 // 2
    if hq is None:
        hq = torch.empty((M, I), dtype=torch.uint8, device=Xq.device)
    if hs is None:
        hs = torch.empty(mx_scale_bytes(M, I), dtype=torch.uint8, device=Xq.device)
    if preact is True:
        preact = torch.empty((M, N2), dtype=torch.bfloat16, device=Xq.device)
    if preact is not None and tuple(preact.shape) != (M, N2):
        raise ValueError("preact shape")
    rc = load().mx_grouped_gemm_swiglu(_ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws), _ptr(group_offsets), G, M, I, K,
                                       _ptr(hq), _ptr(hs), _ptr(preact), _stream(stream))
    _check(rc, "mx_grouped_gemm_swiglu")
    return hq, hs, preact


def mx_swiglu_backward(preact, dh, dpre=None, h=None, stream=None):
    """SwiGLU backward: preact bf16 [M, 2I] (interleaved gate/up, as saved by
    mx_grouped_gemm_swiglu), dh bf16 [M, I] -> (dpre bf16 [M, 2I], h or None).
    h: None, True (allocate) or a bf16 [M, I] tensor to receive silu(g) u."""
    M, N2 = preact.shape
    I = N2 // 2
    if tuple(dh.shape) != (M, I):
        raise ValueError("shape mismatch")
    if not (preact.is_contiguous() and dh.is_contiguous()) or (
            h is not None and h is not True and not h.is_contiguous()):
        raise ValueError("contiguous tensors required")
    if dpre is None:
        dpre = torch.empty((M, N2), dtype=torch.bfloat16, device=preact.device)
    if h is True:
        h = torch.empty((M, I), dtype=torch.bfloat16, device=preact.device)
    rc = load().mx_swiglu_backward(_ptr(_bits16(preact)), _ptr(_bits16(dh)), M, I, _ptr(dpre), _ptr(h),
                                   _stream(stream))
    _check(rc, "mx_swiglu_backward")
    return dpre, h


def mx_swiglu_backward_quant(preact, dh, group_offsets=None, Mcap=None, q=None, s=None, qT=None, sT=None, hT=None,
                             hTs=None, padded_offsets=None, stream=None):
    """SwiGLU backward with its quantizations fused: the results of
    mx_swiglu_backward (dpre, h) quantized as mx_quantize_dual(dpre) and
    mx_quantize_cols(h), without dpre or h.  Returns (q, s, qT, sT, hT, hTs,
    padded_offsets)."""
    preact, dh = _bits16(preact), _bits16(dh)
    M, I = dh.shape
    if preact.shape != (M, 2 * I):
        raise ValueError("preact must be [M, 2I] for dh [M, I]")
    if not (preact.is_contiguous() and dh.is_contiguous()):
        raise ValueError("contiguous tensors required")
    G = 1 if group_offsets is None else group_offsets.numel() - 1
    if Mcap is None:
        Mcap = mx_cols_capacity(M, G)
    dev = dh.device
    if q is None:
        q = torch.empty((M, 2 * I), dtype=torch.uint8, device=dev)
    if s is None:
        s = torch.empty(mx_scale_bytes(M, 2 * I), dtype=torch.uint8, device=dev)
    if qT is None:
        qT = torch.empty((2 * I, Mcap), dtype=torch.uint8, device=dev)
    if sT is None:
        sT = torch.empty(mx_scale_bytes(2 * I, Mcap), dtype=torch.uint8, device=dev)
    if hT is None:
        hT = torch.empty((I, Mcap), dtype=torch.uint8, device=dev)
    if hTs is None:
        hTs = torch.empty(mx_scale_bytes(I, Mcap), dtype=torch.uint8, device=dev)
    if group_offsets is not None and padded_offsets is None:
        padded_offsets = torch.empty(G + 1, dtype=torch.int32, device=dev)
    rc = load().mx_swiglu_backward_quant(_ptr(preact), _ptr(dh), M, I, _ptr(group_offsets), G, _ptr(q), _ptr(s),
                                         _ptr(qT), _ptr(sT), _ptr(hT), _ptr(hTs), Mcap, _ptr(padded_offsets),
                                         _stream(stream))
    _check(rc, "mx_swiglu_backward_quant")
    return q, s, qT, sT, hT, hTs, padded_offsets


def mx_route_plan(experts, G, weights=None, offsets=None, src=None, slot_of=None, slot_weight=None, stream=None):
    """experts int32 [T, k] (device), G experts (, float32 weights [T, k]) ->
    (offsets int32 [G+1], src int32 [T k], slot_of int32 [T, k],
    slot_weight float32 [T k] or None): the stable sort of the routed entries
    by expert (entries outside [0, G) dropped, slot -1)."""
    if experts.dtype != torch.int32 or experts.dim() != 2 or not experts.is_contiguous():
        raise ValueError("experts must be a contiguous int32 [T, k] tensor")
    T, k = experts.shape
    dev = experts.device
    if weights is not None and (weights.dtype != torch.float32 or tuple(weights.shape) != (T, k)
                                or not weights.is_contiguous()):
        raise ValueError("weights must be a contiguous float32 [T, k] tensor")
    if offsets is None:
        offsets = torch.empty(G + 1, dtype=torch.int32, device=dev)
    if src is None:
        src = torch.empty(T * k, dtype=torch.int32, device=dev)
    if slot_of is None:
        slot_of = torch.empty((T, k), dtype=torch.int32, device=dev)
    if weights is not None and slot_weight is None:
        slot_weight = torch.empty(T * k, dtype=torch.float32, device=dev)
    rc = load().mx_route_plan(_ptr(experts), _ptr(weights), T, k, G, _ptr(offsets), _ptr(src), _ptr(slot_of),
                              _ptr(slot_weight), _stream(stream))
    _check(rc, "mx_route_plan")
    return offsets, src, slot_of, slot_weight


def mx_gather_quantize(x, src, M, group_offsets=None, Mcap=None, row_scale=None, q=None, s=None, qT=None, sT=None,
                       padded_offsets=None, stream=None):
    """mx_quantize_dual of the matrix whose row r is x[src[r]] (x bf16 [T, N],
    src int32 [>= M]), each row optionally scaled by row_scale[r] (float32)
    in fp32 and rounded to bf16 first.  Returns (q, s, qT, sT, padded_offsets)."""
    x = _bits16(x)
    T, N = x.shape
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    G = 1 if group_offsets is None else group_offsets.numel() - 1
    if Mcap is None:
        Mcap = mx_cols_capacity(M, G)
    if src.dtype != torch.int32 or src.numel() < M:
        raise ValueError("src must be an int32 tensor of at least M entries")
    if row_scale is not None and (row_scale.dtype != torch.float32 or row_scale.numel() < M):
        raise ValueError("row_scale must be a float32 tensor of at least M entries")
    dev = x.device
    if q is None:
        q = torch.empty((M, N), dtype=torch.uint8, device=dev)
    if s is None:
        s = torch.empty(mx_scale_bytes(M, N), dtype=torch.uint8, device=dev)
    if qT is None:
        qT = torch.empty((N, Mcap), dtype=torch.uint8, device=dev)
    if sT is None:
        sT = torch.empty(mx_scale_bytes(N, Mcap), dtype=torch.uint8, device=dev)
    if group_offsets is not None and padded_offsets is None:
        padded_offsets = torch.empty(G + 1, dtype=torch.int32, device=dev)
    rc = load().mx_gather_quantize(_ptr(x), T, N, x.stride(0), _ptr(src), _ptr(row_scale), M, _ptr(group_offsets), G,
                                   _ptr(q), _ptr(s), _ptr(qT), _ptr(sT), Mcap, _ptr(padded_offsets), _stream(stream))
    _check(rc, "mx_gather_quantize")
    return q, s, qT, sT, padded_offsets


def mx_combine(y, slot_of, weights=None, out=None, stream=None):
    """y bf16 [M, N] expert-ordered rows, slot_of int32 [T, k] (, float32
    weights [T, k]) -> bf16 [T, N]: the weighted (or plain) sum of each
    token's expert rows."""
    y = _bits16(y)
    M, N = y.shape
    if y.stride(1) != 1:
        raise ValueError("y rows must be contiguous")
    if slot_of.dtype != torch.int32 or slot_of.dim() != 2 or not slot_of.is_contiguous():
        raise ValueError("slot_of must be a contiguous int32 [T, k] tensor")
    T, k = slot_of.shape
    if weights is not None and (weights.dtype != torch.float32 or tuple(weights.shape) != (T, k)
                                or not weights.is_contiguous()):
        raise ValueError("weights must be a contiguous float32 [T, k] tensor")
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=y.device)
    rc = load().mx_combine(_ptr(y), M, N, y.stride(0), _ptr(slot_of), _ptr(weights), T, k, _ptr(_bits16(out)),
                           _stream(stream))
    _check(rc, "mx_combine")
    return out


def mx_validate_offsets(group_offsets, M, result=None, stream=None):
    """Device check of group offsets: returns an int32 device tensor [1] holding
    0 if 0 <= o[0] <= ... <= o[G] <= M, else 1 + the first bad index."""
    if result is None:
        result = torch.empty(1, dtype=torch.int32, device=group_offsets.device)
    rc = load().mx_validate_offsets(_ptr(group_offsets), group_offsets.numel() - 1, M, _ptr(result),
                                    _stream(stream))
    _check(rc, "mx_validate_offsets")
    return result


def mx_stream21(src, dst, stream=None):
    """Calibration stream: reads all of src (2x dst's bytes), writes dst."""
    if src.numel() * src.element_size() != 2 * dst.numel() * dst.element_size():
        raise ValueError("src must hold twice dst's bytes")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("contiguous tensors required")
    rc = load().mx_stream21(_ptr(src), _ptr(dst), dst.numel() * dst.element_size(), _stream(stream))
    _check(rc, "mx_stream21")
    return dst


def mx_probe_mfma_scale(A, B, SA, SB, C, out=None, stream=None):
    """Diagnostic: D[t] = C[t] + the scaled fp8 product of A[t] [32, 64] and
    B[t] [32, 64] (row n of B = column n of the product), one matrix
    instruction per t, as the hardware rounds it.  A, B uint8 [T, 32, 64];
    SA, SB uint8 [T, 32, 2]; C float32 [T, 32, 32]."""
    T = A.shape[0]
    if (A.shape != (T, 32, 64) or B.shape != (T, 32, 64) or SA.shape != (T, 32, 2) or SB.shape != (T, 32, 2)
            or C.shape != (T, 32, 32) or C.dtype != torch.float32):
        raise ValueError("shapes: A, B [T, 32, 64] uint8; SA, SB [T, 32, 2] uint8; C [T, 32, 32] float32")
    if not all(t.is_contiguous() for t in (A, B, SA, SB, C)):
        raise ValueError("contiguous tensors required")
    if out is None:
        out = torch.empty_like(C)
    rc = load().mx_probe_mfma_scale(_ptr(A), _ptr(B), _ptr(SA), _ptr(SB), _ptr(C), _ptr(out), T, _stream(stream))
    _check(rc, "mx_probe_mfma_scale")
    return out


def mx_debug_flags(stream=None):
    """Debug build only: synchronizes the stream and returns (and clears) the
    contract violations the kernels recorded (bit 1 group offsets, 2 padded
    offsets, 4 empty work tile); raises MxError(MX_ERR_UNSUPPORTED) on the
    release build."""
    flags = ctypes.c_uint32(0)
    rc = load().mx_debug_flags(ctypes.byref(flags), _stream(stream))
    _check(rc, "mx_debug_flags")
    return int(flags.value)


def mx_grouped_gemm_dgrad(dYq, dYs, WTq, WTs, group_offsets, G, out=None, stream=None):
    """dX[m, n] = sum_k deq(dY[m, k]) deq(W[g(m), k, n]) in bf16, with W^T read in
    place from mx_quantize_cols of W.view(G*K, N) (offsets g*K): WTq [N, Wcap]."""
    M, K = dYq.shape
    N, Wcap = WTq.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dYq.device)
    rc = load().mx_grouped_gemm_dgrad(_ptr(dYq), _ptr(dYs), _ptr(WTq), _ptr(WTs), _ptr(group_offsets), int(G), M, N,
                                      K, Wcap, _ptr(out), _stream(stream))
    _check(rc, "mx_grouped_gemm_dgrad")
    return out


def mx_grouped_gemm_wgrad(A, As, B, Bs, padded_offsets, dW=None, stream=None):
    """dW[g, n, k] = sum over group g's padded span of deq(A[n, t]) deq(B[k, t]).
    A uint8 [N, Mcap] (dY^T), B uint8 [K, Mcap] (X^T); padded_offsets int32 [G+1]."""
    N, Mcap = A.shape
    K, Mcap2 = B.shape
    if Mcap2 != Mcap:
        raise ValueError("Mcap mismatch")
    G = padded_offsets.numel() - 1
    if dW is None:
        dW = torch.empty((G, N, K), dtype=torch.bfloat16, device=A.device)
    rc = load().mx_grouped_gemm_wgrad(_ptr(A), _ptr(As), _ptr(B), _ptr(Bs), _ptr(padded_offsets), G, N, K, Mcap,
                                      _ptr(dW), _stream(stream))
    _check(rc, "mx_grouped_gemm_wgrad")
    return dW
