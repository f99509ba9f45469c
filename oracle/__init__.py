"""CPU oracle for MXFP8 quantization and the block-scaled grouped GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library ``libmxmoe`` and its Python binding) never imports it, and the
two share no code.

The arithmetic lives in ``mxref.c`` (plain C, double precision, exact steps);
this module only builds it with gcc and marshals numpy arrays through ctypes.
The definitions follow the public write-ups on Cursor's Blackwell MoE kernels
(aigc.bar "被忽视的量化税"/"秘密武器"; lpnh.cn 2479732 section 1); the readings
of what the pages leave open are stated in ``mxref.c``.

Parity status of each function (what pins it in ``tests/test_oracle.py``):
  e4m3_encode / quantize_with_scale  exhaustive vs an independent table-search
                                     encoder over every finite bf16 x every S
  block_scale                        exhaustive closed form over every amax
  quantize_rows / quantize_cols      hand-worked blocks (tests/golden), invariants,
                                     cols == rows of the transposed group slices
  pack / unpack_scales               hand-computed offsets (tests/golden)
  grouped_gemm(_points)              exact rational brute force on small shapes,
                                     one-hot closed form
  wgrad(_points)                     exact rational brute force on small shapes
  silu                               closed forms (0, ln 3, large |x|), odd-part
                                     identity silu(x) - silu(-x) = x
  block_scale_f64 / quantize_f64_*   closed-form scale sweep; equal to the bf16
                                     path on bf16 values; independent
                                     table-search encoder on off-grid values
  swiglu_quantize                    saturated-gate reduction to quantize_rows,
                                     zero gate, quantization-error invariants
  grouped_gemm_swiglu(_blocks)       one-hot routing closed form (expert and
                                     gate/up roles), full vs sampled agreement
  dsilu                              closed forms (0, ln 3, large |x|), central
                                     differences of silu
  bf16_round                         torch's float32 -> bf16 conversion on
                                     float32 values, hand-worked ties, values
                                     past float32 precision (no double rounding)
  swiglu_backward                    zero and saturated gates in closed form
  route_plan                         brute force (a sort of (expert, entry)
                                     pairs), histogram offsets, inverse maps
  f32_round / gather_rows            identity gathers, exact power-of-two
                                     scales, hand-worked double-rounding cases
  combine                            one-hot weights reduce to the gather,
                                     hand-worked sums, linearity in the weights
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxref.c")
_LIB_PATH = os.path.join(_HERE, "libmxref.so")
_lib = None


def build(force=False):
    """Compile mxref.c into oracle/libmxref.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "mxref.h"))
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-fPIC",
             "-shared", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("MXREF_LIB")  # a test may point at a deliberately broken build
    if not path:
        path = build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.mxref_bf16_value.argtypes = [ctypes.c_uint16]
    lib.mxref_bf16_value.restype = ctypes.c_double
    lib.mxref_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.mxref_e4m3_value.restype = ctypes.c_double
    lib.mxref_e4m3_encode.argtypes = [ctypes.c_double]
    lib.mxref_e4m3_encode.restype = ctypes.c_uint8
    lib.mxref_block_scale.argtypes = [P, I64, I64]
    lib.mxref_block_scale.restype = ctypes.c_uint8
    lib.mxref_quantize_with_scale.argtypes = [P, I64, ctypes.c_uint8, P]
    lib.mxref_dequant.argtypes = [ctypes.c_uint8, ctypes.c_uint8]
    lib.mxref_dequant.restype = ctypes.c_double
    lib.mxref_quantize_rows.argtypes = [P, I64, I64, P, P]
    lib.mxref_quantize_cols.argtypes = [P, I64, I64, P, ctypes.c_int32, I64, P, P, P]
    lib.mxref_quantize_cols.restype = ctypes.c_int
    lib.mxref_packed_scale_bytes.argtypes = [I64, I64]
    lib.mxref_packed_scale_bytes.restype = I64
    lib.mxref_pack_scales.argtypes = [P, I64, I64, P]
    lib.mxref_unpack_scales.argtypes = [P, I64, I64, P]
    lib.mxref_grouped_gemm.argtypes = [P, P, P, P, P, ctypes.c_int32, I64, I64, I64, P]
    lib.mxref_grouped_gemm_points.argtypes = [P, P, P, P, P, ctypes.c_int32, I64, I64, I64, P, P, I64, P]
    lib.mxref_wgrad.argtypes = [P, P, P, P, P, ctypes.c_int32, I64, I64, I64, P]
    lib.mxref_wgrad_points.argtypes = [P, P, P, P, P, ctypes.c_int32, I64, I64, I64, P, P, P, I64, P]
    lib.mxref_silu.argtypes = [ctypes.c_double]
    lib.mxref_silu.restype = ctypes.c_double
    lib.mxref_block_scale_f64.argtypes = [P, I64]
    lib.mxref_block_scale_f64.restype = ctypes.c_uint8
    lib.mxref_quantize_f64_with_scale.argtypes = [P, I64, ctypes.c_uint8, P]
    lib.mxref_quantize_rows_f64.argtypes = [P, I64, I64, P, P]
    lib.mxref_swiglu_quantize.argtypes = [P, P, I64, I64, P, P, P]
    lib.mxref_dsilu.argtypes = [ctypes.c_double]
    lib.mxref_dsilu.restype = ctypes.c_double
    lib.mxref_bf16_round.argtypes = [ctypes.c_double]
    lib.mxref_bf16_round.restype = ctypes.c_uint16
    lib.mxref_bf16_round_n.argtypes = [P, I64, P]
    lib.mxref_swiglu_backward.argtypes = [P, P, P, I64, P, P, P]
    lib.mxref_route_plan.argtypes = [P, I64, ctypes.c_int32, ctypes.c_int32, P, P, P]
    lib.mxref_f32_round.argtypes = [ctypes.c_double]
    lib.mxref_f32_round.restype = ctypes.c_double
    lib.mxref_gather_rows.argtypes = [P, I64, I64, P, P, I64, P]
    lib.mxref_combine.argtypes = [P, I64, I64, P, P, I64, ctypes.c_int32, P]
    _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def bf16_value(bits):
    return _load().mxref_bf16_value(int(bits))


def e4m3_value(code):
    return _load().mxref_e4m3_value(int(code))


def e4m3_encode(y):
    return int(_load().mxref_e4m3_encode(float(y)))


def block_scale(block_bits):
    a, p = _c(block_bits, np.uint16)
    return int(_load().mxref_block_scale(p, a.size, 1))


def quantize_with_scale(x_bits, S):
    a, p = _c(x_bits, np.uint16)
    q = np.empty(a.size, np.uint8)
    _load().mxref_quantize_with_scale(p, a.size, int(S), q.ctypes.data_as(ctypes.c_void_p))
    return q.reshape(np.shape(x_bits))


def dequant(q, S):
    return _load().mxref_dequant(int(q), int(S))


def quantize_rows(x_bits):
    """bf16 bits [M, K] -> (codes uint8 [M, K], canonical scales uint8 [M, K/32])."""
    x, p = _c(x_bits, np.uint16)
    M, K = x.shape
    assert K % 32 == 0
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 32), np.uint8)
    _load().mxref_quantize_rows(p, M, K, q.ctypes.data_as(ctypes.c_void_p), s.ctypes.data_as(ctypes.c_void_p))
    return q, s


def cols_capacity(M, G):
    return 256 * ((M + 255) // 256 + max(G, 1) - 1)


def quantize_cols(x_bits, offsets=None, Mcap=None):
    """bf16 bits [M, N] -> (qT [N, Mcap], canonical sT [N, Mcap/32], padded offsets [G+1])."""
    x, p = _c(x_bits, np.uint16)
    M, N = x.shape
    if offsets is None:
        G = 1
        op = None
    else:
        off, op = _c(offsets, np.int32)
        G = off.size - 1
    if Mcap is None:
        Mcap = cols_capacity(M, G)
    qT = np.empty((N, Mcap), np.uint8)
    sT = np.empty((N, Mcap // 32), np.uint8)
    padded = np.empty(G + 1, np.int32)
    rc = _load().mxref_quantize_cols(p, M, N, op, G, Mcap, qT.ctypes.data_as(ctypes.c_void_p),
                                     sT.ctypes.data_as(ctypes.c_void_p), padded.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("Mcap too small")
    return qT, sT, padded


def packed_scale_bytes(R, K):
    return int(_load().mxref_packed_scale_bytes(R, K))


def pack_scales(s, K):
    s, p = _c(s, np.uint8)
    R = s.shape[0]
    out = np.empty(packed_scale_bytes(R, K), np.uint8)
    _load().mxref_pack_scales(p, R, K, out.ctypes.data_as(ctypes.c_void_p))
    return out


def unpack_scales(packed, R, K):
    pk, p = _c(packed, np.uint8)
    s = np.empty((R, K // 32), np.uint8)
    _load().mxref_unpack_scales(p, R, K, s.ctypes.data_as(ctypes.c_void_p))
    return s


def grouped_gemm(Xq, Xs, Wq, Ws, offsets):
    """fp64 reference out [M, N]; Wq [G, N, K], Ws [G, N, K/32] canonical."""
    Xq, px = _c(Xq, np.uint8)
    Xs, pxs = _c(Xs, np.uint8)
    Wq, pw = _c(Wq, np.uint8)
    Ws, pws = _c(Ws, np.uint8)
    off, po = _c(offsets, np.int32)
    M, K = Xq.shape
    G, N, _ = Wq.shape
    out = np.empty((M, N), np.float64)
    _load().mxref_grouped_gemm(px, pxs, pw, pws, po, G, M, N, K, out.ctypes.data_as(ctypes.c_void_p))
    return out


def grouped_gemm_points(Xq, Xs, Wq, Ws, offsets, rows, cols):
    Xq, px = _c(Xq, np.uint8)
    Xs, pxs = _c(Xs, np.uint8)
    Wq, pw = _c(Wq, np.uint8)
    Ws, pws = _c(Ws, np.uint8)
    off, po = _c(offsets, np.int32)
    r, pr = _c(rows, np.int64)
    c, pc = _c(cols, np.int64)
    M, K = Xq.shape
    G, N, _ = Wq.shape
    out = np.empty(r.size, np.float64)
    _load().mxref_grouped_gemm_points(px, pxs, pw, pws, po, G, M, N, K, pr, pc, r.size,
                                      out.ctypes.data_as(ctypes.c_void_p))
    return out


def wgrad(Aq, As, Bq, Bs, padded):
    Aq, pa = _c(Aq, np.uint8)
    As, pas = _c(As, np.uint8)
    Bq, pb = _c(Bq, np.uint8)
    Bs, pbs = _c(Bs, np.uint8)
    P, pp = _c(padded, np.int32)
    N, Mcap = Aq.shape
    K = Bq.shape[0]
    G = P.size - 1
    dW = np.empty((G, N, K), np.float64)
    _load().mxref_wgrad(pa, pas, pb, pbs, pp, G, N, K, Mcap, dW.ctypes.data_as(ctypes.c_void_p))
    return dW


def wgrad_points(Aq, As, Bq, Bs, padded, gs, ns, ks):
    Aq, pa = _c(Aq, np.uint8)
    As, pas = _c(As, np.uint8)
    Bq, pb = _c(Bq, np.uint8)
    Bs, pbs = _c(Bs, np.uint8)
    P, pp = _c(padded, np.int32)
    g, pg = _c(gs, np.int64)
    n, pn = _c(ns, np.int64)
    k, pk = _c(ks, np.int64)
    N, Mcap = Aq.shape
    K = Bq.shape[0]
    out = np.empty(g.size, np.float64)
    _load().mxref_wgrad_points(pa, pas, pb, pbs, pp, P.size - 1, N, K, Mcap, pg, pn, pk, g.size,
                               out.ctypes.data_as(ctypes.c_void_p))
    return out


# ---- SwiGLU + MXFP8 of its result (mxref.c states the readings) ----

def silu(x):
    return _load().mxref_silu(float(x))


def block_scale_f64(x):
    a, p = _c(x, np.float64)
    return int(_load().mxref_block_scale_f64(p, a.size))


def quantize_f64_with_scale(x, S):
    a, p = _c(x, np.float64)
    q = np.empty(a.size, np.uint8)
    _load().mxref_quantize_f64_with_scale(p, a.size, int(S), q.ctypes.data_as(ctypes.c_void_p))
    return q.reshape(np.shape(x))


def quantize_rows_f64(x):
    """double [M, K] -> (codes uint8 [M, K], canonical scales uint8 [M, K/32])."""
    a, p = _c(x, np.float64)
    M, K = a.shape
    assert K % 32 == 0
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 32), np.uint8)
    _load().mxref_quantize_rows_f64(p, M, K, q.ctypes.data_as(ctypes.c_void_p), s.ctypes.data_as(ctypes.c_void_p))
    return q, s


def swiglu_quantize(gate, up):
    """gate, up double [M, I] -> (h = silu(gate) up [M, I], codes [M, I], scales [M, I/32])."""
    g, pg = _c(gate, np.float64)
    u, pu = _c(up, np.float64)
    assert g.shape == u.shape and g.ndim == 2 and g.shape[1] % 32 == 0
    M, I = g.shape
    h = np.empty((M, I), np.float64)
    q = np.empty((M, I), np.uint8)
    s = np.empty((M, I // 32), np.uint8)
    _load().mxref_swiglu_quantize(pg, pu, M, I, h.ctypes.data_as(ctypes.c_void_p), q.ctypes.data_as(ctypes.c_void_p),
                                  s.ctypes.data_as(ctypes.c_void_p))
    return h, q, s


def grouped_gemm_swiglu(Xq, Xs, Wgq, Wgs, Wuq, Wus, offsets):
    """MoE first projection and activation: gate = X Wg^T and up = X Wu^T per
    expert (grouped_gemm), then swiglu_quantize.  Wgq, Wuq [G, I, K] codes,
    Wgs, Wus [G, I, K/32] canonical scales.  Returns (h, codes, scales, gate, up);
    rows outside every group have gate = up = 0."""
    gate = grouped_gemm(Xq, Xs, Wgq, Wgs, offsets)
    up = grouped_gemm(Xq, Xs, Wuq, Wus, offsets)
    h, q, s = swiglu_quantize(gate, up)
    return h, q, s, gate, up


def grouped_gemm_swiglu_blocks(Xq, Xs, Wgq, Wgs, Wuq, Wus, offsets, rows, blocks):
    """The same at sampled 32-wide blocks: for each (rows[i], blocks[i]) the
    hidden units [32 b, 32 b + 32) of that row.  Returns (h, codes, scales,
    gate, up): h, codes, gate and up [n, 32], scales [n]."""
    rows = np.asarray(rows, np.int64)
    blocks = np.asarray(blocks, np.int64)
    r = np.repeat(rows, 32)
    c = (blocks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    gate = grouped_gemm_points(Xq, Xs, Wgq, Wgs, offsets, r, c).reshape(-1, 32)
    up = grouped_gemm_points(Xq, Xs, Wuq, Wus, offsets, r, c).reshape(-1, 32)
    h, q, s = swiglu_quantize(gate, up)
    return h, q, s[:, 0], gate, up


def dsilu(x):
    return _load().mxref_dsilu(float(x))


def bf16_round(x):
    """double array -> bf16 bit patterns (uint16), nearest even, one rounding."""
    a, p = _c(x, np.float64)
    out = np.empty(a.shape, np.uint16)
    _load().mxref_bf16_round_n(p, a.size, out.ctypes.data_as(ctypes.c_void_p))
    return out


def swiglu_backward(gate, up, dh):
    """gate, up, dh double arrays of one shape -> (dgate, dup, h) in double."""
    g, pg = _c(gate, np.float64)
    u, pu = _c(up, np.float64)
    d, pd = _c(dh, np.float64)
    assert g.shape == u.shape == d.shape
    out = [np.empty(g.shape, np.float64) for _ in range(3)]
    _load().mxref_swiglu_backward(pg, pu, pd, g.size, *[o.ctypes.data_as(ctypes.c_void_p) for o in out])
    return tuple(out)


# ---- the one-GPU share of dispatch and combine (mxref.c states the readings) ----
def route_plan(experts, G):
    """experts int32 [T, k] -> (offsets int32 [G+1], src int32 [offsets[G]],
    slot_of int32 [T, k]): a stable counting sort of the entries by expert."""
    e, pe = _c(experts, np.int32)
    T, k = e.shape
    offsets = np.empty(G + 1, np.int32)
    src = np.full(max(e.size, 1), -1, np.int32)
    slot_of = np.empty((T, k), np.int32)
    _load().mxref_route_plan(pe, e.size, k, G, offsets.ctypes.data_as(ctypes.c_void_p),
                             src.ctypes.data_as(ctypes.c_void_p), slot_of.ctypes.data_as(ctypes.c_void_p))
    return offsets, src[:offsets[G]], slot_of


def f32_round(x):
    return _load().mxref_f32_round(float(x))


def gather_rows(x_bits, src, scale=None):
    """bf16 bits [T, N], src int32 [M] (, float32 scale [M]) -> bf16 bits [M, N]."""
    x, px = _c(x_bits, np.uint16)
    s, ps = _c(src, np.int32)
    T, N = x.shape
    out = np.empty((s.size, N), np.uint16)
    if scale is None:
        pw = None
    else:
        w, pw = _c(scale, np.float32)
        assert w.size == s.size
    _load().mxref_gather_rows(px, T, N, ps, pw, s.size, out.ctypes.data_as(ctypes.c_void_p))
    return out


def combine(y_bits, slot_of, w=None):
    """bf16 bits [M, N], slot_of int32 [T, k] (, float32 w [T, k]) -> double [T, N]."""
    y, py = _c(y_bits, np.uint16)
    so, pso = _c(slot_of, np.int32)
    M, N = y.shape
    T, k = so.shape
    if w is None:
        pw = None
    else:
        wa, pw = _c(w, np.float32)
        assert wa.shape == so.shape
    out = np.empty((T, N), np.float64)
    _load().mxref_combine(py, M, N, pso, pw, T, k, out.ctypes.data_as(ctypes.c_void_p))
    return out
