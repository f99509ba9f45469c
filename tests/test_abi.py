"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments before launching anything."""
import ctypes
import os
import re

import pytest

import mxfp8_block_scaled_04_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmxmoe.h")

# tests/test_sanitize.py runs this module against a sanitizer build of the
# C-ABI layer (kernel launchers stubbed out) named by MXMOE_ABI_LIB
if os.environ.get("MXMOE_ABI_LIB"):
    mx.LIB_PATH = os.environ["MXMOE_ABI_LIB"]
    mx._lib = None


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_header_symbol():
    lib = mx.load()
    names = header_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(mx.SYMBOLS) == names


def test_debug_build_exports_and_release_has_no_checks():
    dbg = mx.open_library(mx.DEBUG_LIB_PATH)
    for n in header_functions():
        assert hasattr(dbg, n), n
    rel = mx.open_library(mx.RELEASE_LIB_PATH)
    flags = ctypes.c_uint32(7)
    assert rel.mx_debug_flags(ctypes.byref(flags), None) == 5 and flags.value == 0  # MX_ERR_UNSUPPORTED
    assert rel.mx_debug_flags(None, None) == 1


def test_host_helpers():
    assert mx.mx_scale_bytes(40, 512) == 1024
    assert mx.mx_scale_bytes(131072, 7168) == 131072 * 224
    assert mx.mx_scale_bytes(1, 32) == 32 * 8
    assert mx.mx_cols_capacity(300, 3) == 256 * (2 + 2)
    assert mx.mx_cols_capacity(32768, 16) == 256 * (128 + 15)
    assert mx.mx_cols_capacity(0, 1) == 0
    assert mx.load().mx_cols_capacity(5, 0) == -1
    assert mx.status_str(0) == "MX_OK" and mx.status_str(6) == "MX_ERR_HIP"


P = ctypes.c_void_p
FAKE = P(0x100000)  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize(
    "args,want",
    [
        ((FAKE, 4, 33, 40, FAKE, FAKE, None), 2),   # K % 32 != 0
        ((FAKE, -1, 32, 32, FAKE, FAKE, None), 2),  # negative M
        ((FAKE, 4, 64, 32, FAKE, FAKE, None), 2),   # ldx < K
        ((None, 4, 32, 32, FAKE, FAKE, None), 1),   # NULL x
        ((FAKE, 4, 32, 32, None, FAKE, None), 1),   # NULL q
        ((P(0x100004), 4, 32, 32, FAKE, FAKE, None), 3),  # misaligned x
        ((FAKE, 4, 32, 36, FAKE, FAKE, None), 3),   # ldx not a multiple of 8
        ((None, 0, 32, 32, None, None, None), 0),   # M == 0: no work, OK
        # 2^23 units of 32 x 256 at 512 threads each: 2^32 work-items, over the grid limit
        ((FAKE, 32 * (1 << 23), 256, 256, FAKE, FAKE, None), 5),
    ],
)
def test_quantize_rows_validation(args, want):
    assert mx.load().mx_quantize_rows(*args) == want


def test_quantize_cols_validation():
    f = mx.load().mx_quantize_cols
    cap = mx.mx_cols_capacity(300, 3)
    assert f(FAKE, 300, 64, 64, FAKE, 3, FAKE, FAKE, cap - 256, FAKE, None) == 4  # capacity too small
    assert f(FAKE, 300, 64, 64, FAKE, 3, FAKE, FAKE, cap + 8, FAKE, None) == 4    # not multiple of 256
    assert f(FAKE, 300, 60, 64, FAKE, 3, FAKE, FAKE, cap, FAKE, None) == 5        # N % 8 != 0
    assert f(FAKE, 300, 64, 64, FAKE, 0, FAKE, FAKE, cap, FAKE, None) == 2        # G < 1
    assert f(FAKE, 300, 64, 64, FAKE, 5000, FAKE, FAKE, 256 * 6000, FAKE, None) == 2  # G too large
    assert f(FAKE, 300, 64, 64, FAKE, 3, FAKE, FAKE, cap, None, None) == 1        # padded offsets required
    assert f(FAKE, 300, 64, 32, FAKE, 3, FAKE, FAKE, cap, FAKE, None) == 2        # ldx < N


def test_quantize_dual_validation():
    f = mx.load().mx_quantize_dual
    cap = mx.mx_cols_capacity(300, 3)
    ok = (FAKE, 300, 64, 64, FAKE, 3, FAKE, FAKE, FAKE, FAKE, cap, FAKE, None)
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a10=cap - 256) == 4                # capacity too small
    assert call(a2=48, a3=64) == 2                 # N % 32 != 0
    assert call(a3=32) == 2                        # ldx < N
    assert call(a5=0) == 2                         # G < 1
    assert call(a11=None) == 1                     # padded offsets required with groups
    assert call(a6=None) == 1                      # NULL row-wise codes
    assert call(a8=None) == 1                      # NULL column-wise codes
    assert call(a6=P(0x100004)) == 3               # misaligned row-wise codes


def test_grouped_gemm_validation():
    f = mx.load().mx_grouped_gemm
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 512, 128, 288, FAKE, None) == 5  # K % 256 != 0
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 512, 128, 250, FAKE, None) == 2  # K % 32 != 0
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 512, 128, 256, FAKE, None) == 2  # G < 1
    assert f(FAKE, FAKE, None, FAKE, FAKE, 4, 512, 128, 256, FAKE, None) == 1  # NULL W
    assert f(FAKE, FAKE, FAKE, FAKE, None, 4, 512, 128, 256, FAKE, None) == 1  # NULL offsets
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 512, 128, 256, P(0x100002), None) == 3  # misaligned out
    assert f(None, None, None, None, None, 4, 0, 128, 256, None, None) == 0    # M == 0: no work
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 512, 128, 0, FAKE, None) == 5    # K == 0: empty contraction
    assert f(None, None, None, None, None, 4, 0, 128, 0, None, None) == 5      # K == 0 even with no rows


def test_grouped_gemm_swiglu_validation():
    f = mx.load().mx_grouped_gemm_swiglu
    # (Xq, Xs, Wq, Ws, offsets, G, M, I, K, hq, hs, preact, stream)
    F5 = (FAKE,) * 5
    assert f(*F5, 4, 512, 2048, 288, FAKE, FAKE, None, None) == 5        # K % 256 != 0
    assert f(*F5, 4, 512, 2048, 0, FAKE, FAKE, None, None) == 5          # K == 0
    assert f(*F5, 4, 512, 192, 512, FAKE, FAKE, None, None) == 5         # I % 128 != 0
    assert f(*F5, 4, 512, 2048, 250, FAKE, FAKE, None, None) == 2        # K % 32 != 0
    assert f(*F5, 0, 512, 2048, 512, FAKE, FAKE, None, None) == 2        # G < 1
    assert f(*F5, 4, -1, 2048, 512, FAKE, FAKE, None, None) == 2         # M < 0
    assert f(*F5, 4, 512, 2048, 512, None, FAKE, None, None) == 1        # NULL hq
    assert f(*F5, 4, 512, 2048, 512, FAKE, None, None, None) == 1        # NULL hs
    assert f(*F5, 4, 512, 2048, 512, FAKE, P(0x100001), None, None) == 3  # misaligned hs
    assert f(*F5, 4, 512, 2048, 512, FAKE, FAKE, P(0x100002), None) == 3  # misaligned preact
    assert f(*F5, 4, 512, 1 << 22, 512, FAKE, FAKE, None, None) == 5     # 2I past the limit
    assert f(None, None, None, None, None, 4, 0, 2048, 512, None, None, None, None) == 0  # M == 0: no work


def test_swiglu_backward_validation():
    f = mx.load().mx_swiglu_backward
    # (preact, dh, M, I, dpre, h, stream)
    assert f(FAKE, FAKE, 64, 48, FAKE, FAKE, None) == 2            # I % 32 != 0
    assert f(FAKE, FAKE, -1, 64, FAKE, FAKE, None) == 2            # M < 0
    assert f(None, FAKE, 64, 64, FAKE, FAKE, None) == 1            # NULL preact
    assert f(FAKE, FAKE, 64, 64, None, FAKE, None) == 1            # NULL dpre
    assert f(FAKE, FAKE, 64, 64, FAKE, P(0x100008), None) == 3     # misaligned h
    assert f(None, None, 0, 64, None, None, None) == 0             # M == 0: no work


def test_swiglu_backward_quant_validation():
    f = mx.load().mx_swiglu_backward_quant
    cap = mx.mx_cols_capacity(300, 3)
    # (preact, dh, M, I, offsets, G, q, s, qT, sT, hT, hTs, Mcap, padded, stream)
    ok = [FAKE, FAKE, 300, 128, FAKE, 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, cap, FAKE, None]
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a3=96) == 5                        # I % 128 != 0
    assert call(a2=-1) == 2                        # M < 0
    assert call(a5=0) == 2                         # G < 1
    assert call(a12=cap - 256) == 4                # capacity too small
    assert call(a13=None) == 1                     # padded offsets required with groups
    assert call(a0=None) == 1                      # NULL preact
    assert call(a10=None) == 1                     # NULL h codes
    assert call(a8=P(0x100004)) == 3               # misaligned column-wise codes
    assert call(a0=None, a1=None, a2=0, a4=None, a6=None, a7=None, a3=0, a12=0, a13=None) == 0  # no work


def test_route_plan_validation():
    f = mx.load().mx_route_plan
    # (experts, weights, T, k, G, offsets, src, slot_of, slot_weight, stream)
    ok = [FAKE, None, 100, 8, 16, FAKE, FAKE, FAKE, None, None]
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a2=-1) == 2                        # T < 0
    assert call(a3=0) == 2                         # k < 1
    assert call(a4=0) == 2 and call(a4=4097) == 2  # G outside [1, 4096]
    assert call(a2=1 << 28) == 5                   # T k >= 2^31
    assert call(a5=None) == 1                      # NULL offsets
    assert call(a0=None) == 1                      # NULL experts
    assert call(a6=None) == 1                      # NULL src
    assert call(a8=FAKE) == 1                      # slot weights without weights
    assert call(a7=P(0x100002)) == 3               # misaligned slot_of


def test_gather_quantize_validation():
    f = mx.load().mx_gather_quantize
    cap = mx.mx_cols_capacity(300, 3)
    # (x, T, N, ldx, src, row_scale, M, offsets, G, q, s, qT, sT, Mcap, padded, stream)
    ok = [FAKE, 50, 64, 64, FAKE, None, 300, FAKE, 3, FAKE, FAKE, FAKE, FAKE, cap, FAKE, None]
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a13=cap - 256) == 4                # capacity too small for M rows
    assert call(a2=48, a3=64) == 2                 # N % 32 != 0
    assert call(a1=-1) == 2                        # T < 0
    assert call(a6=-1) == 2                        # M < 0
    assert call(a3=32) == 2                        # ldx < N
    assert call(a4=None) == 1                      # NULL src with rows
    assert call(a0=None) == 1                      # NULL x with tokens
    assert call(a14=None) == 1                     # padded offsets required with groups
    assert call(a5=P(0x100002)) == 3               # misaligned row scale
    assert call(a0=P(0x100008)) == 3               # misaligned x
    assert call(a2=0, a7=None, a14=None) == 0      # N == 0, no groups: no work


def test_combine_validation():
    f = mx.load().mx_combine
    # (y, M, N, ldy, slot_of, weights, T, k, out, stream)
    ok = [FAKE, 800, 64, 64, FAKE, None, 100, 8, FAKE, None]
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a2=60, a3=64) == 5                 # N % 8 != 0
    assert call(a3=32) == 2                        # ldy < N
    assert call(a7=0) == 2                         # k < 1
    assert call(a6=-1) == 2                        # T < 0
    assert call(a4=None) == 1                      # NULL slot_of
    assert call(a8=None) == 1                      # NULL out
    assert call(a0=None) == 1                      # NULL y with rows
    assert call(a8=P(0x100008)) == 3               # misaligned out
    assert call(a5=P(0x100002)) == 3               # misaligned weights
    assert call(a6=0, a4=None, a8=None) == 0       # no tokens: no work
    assert call(a6=1 << 24) == 5                   # T workgroups of 256 lanes: 2^32 work-items
    assert call(a2=8 * 256 * 65536, a3=8 * 256 * 65536) == 5  # N / 2048 columns blocks >= 65536


def test_validate_offsets_argument_errors():
    f = mx.load().mx_validate_offsets
    assert f(FAKE, 0, 100, FAKE, None) == 2        # G < 1
    assert f(FAKE, 4097, 100, FAKE, None) == 2     # G too large
    assert f(FAKE, 4, -1, FAKE, None) == 2         # M < 0
    assert f(None, 4, 100, FAKE, None) == 1
    assert f(FAKE, 4, 100, None, None) == 1


def test_stream21_validation():
    f = mx.load().mx_stream21
    assert f(FAKE, FAKE, 24, None) == 2                    # not a multiple of 16 bytes
    assert f(FAKE, FAKE, -16, None) == 2
    assert f(None, FAKE, 64, None) == 1
    assert f(FAKE, P(0x100004), 64, None) == 3
    assert f(None, None, 0, None) == 0
    assert f(FAKE, FAKE, 16 << 32, None) == 5              # 2^32 lanes: over the grid limit


def test_probe_mfma_scale_validation():
    f = mx.load().mx_probe_mfma_scale
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, None) == 2           # T < 0
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 65537, None) == 2        # over 65536 waves
    assert f(FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, None) == 1            # NULL B
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, None) == 1            # NULL D
    assert f(FAKE, FAKE, FAKE, FAKE, P(0x100004), FAKE, 4, None) == 3     # misaligned C
    assert f(None, None, None, None, None, None, 0, None) == 0            # T == 0


def test_dgrad_validation():
    f = mx.load().mx_grouped_gemm_dgrad
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 512, 64, 512, 1024, FAKE, None) == 4   # Wcap < G*K
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 512, 64, 288, 2048, FAKE, None) == 5   # K % 256
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 512, 64, 0, 2048, FAKE, None) == 5     # K == 0
    assert f(FAKE, FAKE, FAKE, FAKE, None, 4, 512, 64, 512, 2048, FAKE, None) == 1   # NULL offsets
    assert f(None, None, None, None, None, 4, 0, 64, 512, 2048, None, None) == 0     # M == 0


def test_wgrad_validation():
    f = mx.load().mx_grouped_gemm_wgrad
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 64, 300, FAKE, None) == 4   # Mcap % 256
    assert f(FAKE, FAKE, FAKE, FAKE, None, 4, 64, 64, 512, FAKE, None) == 1  # NULL offsets
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 64, 512, FAKE, None) == 2  # G < 1
    assert f(None, None, None, None, None, 4, 0, 64, 512, None, None) == 0   # N == 0: no work


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(mx, "_lib", None)
    monkeypatch.setattr(mx, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        mx.load()

