"""Pins for the CPU oracle (``oracle/``), independent of the oracle itself.

Each test checks the oracle against something it does not compute: values
worked by hand from the definition (tests/golden), an independent
table-search encoder, closed forms, invariants of the format, and exact
rational arithmetic.  Definition followed: one E8M0 scale per 32-element
block, the block divided by it, the result cast to FP8 E4M3 (lpnh.cn 2479732
section 1; aigc.bar "秘密武器"), with the scale rule floor(log2 amax) - 8,
saturation to +/-448 and round-to-nearest-even.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# ---------------------------------------------------------------------------
# Independent helpers (not the oracle's code): E4M3FN value table from the
# bit-field definition, nearest-value search with ties to the even code.
# ---------------------------------------------------------------------------


def _e4m3_table():
    vals = np.full(256, np.nan)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 15 and m == 7:
            continue
        vals[c] = s * (m / 8.0) * 2.0 ** -6 if e == 0 else s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3 = _e4m3_table()
POS = E4M3[:0x7F]  # codes 0x00..0x7E, increasing


def table_encode(y):
    """Encode float64 array y by searching the positive E4M3 table."""
    y = np.asarray(y, np.float64)
    sign = np.where(np.signbit(y), 0x80, 0)
    a = np.minimum(np.abs(y), POS[-1])
    hi = np.clip(np.searchsorted(POS, a, side="left"), 0, 126)  # POS[hi] >= a
    lo = np.clip(hi - 1, 0, 126)
    dlo = a - POS[lo]
    dhi = POS[hi] - a
    pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a == POS[hi], hi, pick)
    return (pick | sign).astype(np.uint8)


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


ALL_BF16 = np.arange(65536, dtype=np.uint32)
FINITE_BF16 = ALL_BF16[((ALL_BF16 >> 7) & 0xFF) != 0xFF].astype(np.uint16)


def load_hand_blocks():
    rows = []
    with open(os.path.join(GOLD, "hand_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, xs, s, qs = [p.strip() for p in line.split("|")]
            x = [int(t, 16) for t in xs.split()]
            q = [int(t, 16) for t in qs.split()]
            rows.append((name, x, int(s, 16), q))
    return rows


# ---------------------------------------------------------------------------
# Format decode
# ---------------------------------------------------------------------------


def test_e4m3_decode_matches_format_table():
    for c in range(256):
        v = oracle.e4m3_value(c)
        if np.isnan(E4M3[c]):
            assert math.isnan(v)
        else:
            assert v == E4M3[c], hex(c)
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x38) == 1.0
    assert sum(1 for c in range(256) if not math.isnan(oracle.e4m3_value(c))) == 254


def test_bf16_decode_all_patterns():
    ref = bf16_bits_to_f64(ALL_BF16)
    for b in list(range(0, 65536, 97)) + [0x0001, 0x007F, 0x8001, 0x0080, 0x7F7F, 0xFF7F, 0x8000]:
        v = oracle.bf16_value(b)
        if np.isnan(ref[b]):
            assert math.isnan(v)
        else:
            assert v == ref[b] and math.copysign(1, v) == math.copysign(1, ref[b]), hex(b)


# ---------------------------------------------------------------------------
# Hand-worked blocks
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("blk", load_hand_blocks(), ids=lambda b: b[0])
def test_hand_worked_blocks(blk):
    name, x, S, q = blk
    xb = np.zeros(32, np.uint16)
    xb[: len(x)] = x
    qq, ss = oracle.quantize_rows(xb.reshape(1, 32))
    assert int(ss[0, 0]) == S, name
    want = np.zeros(32, np.uint8)
    want[: len(q)] = q
    assert qq[0].tolist() == want.tolist(), name
    # same block read column-wise (one group of 32 rows)
    qT, sT, P = oracle.quantize_cols(xb.reshape(32, 1))
    assert int(sT[0, 0]) == S
    assert qT[0, :32].tolist() == want.tolist()


# ---------------------------------------------------------------------------
# Scale rule: closed forms over every possible amax
# ---------------------------------------------------------------------------


def test_block_scale_every_amax():
    for a in range(0, 0x7F80):  # every non-negative finite bf16 pattern
        blk = np.zeros(32, np.uint16)
        blk[7] = a
        blk[3] = a | 0x8000 if a else 0  # a negative copy does not change amax
        S = oracle.block_scale(blk)
        # (i) from the exponent field: S = max(E_max - 8, 0), E_max = biased exponent
        emax = a >> 7
        assert S == max(emax - 8, 0), hex(a)
        # (ii) from floor(log2 amax) computed by frexp on the exact value
        v = float(bf16_bits_to_f64([a])[0])
        if v == 0.0:
            assert S == 0
        else:
            _, e = math.frexp(v)
            assert S == min(max(e - 1 - 8, -127), 127) + 127, hex(a)
    assert oracle.block_scale(np.zeros(32, np.uint16)) == 0


def test_block_scale_random_blocks():
    rng = np.random.default_rng(7)
    for _ in range(2000):
        blk = rng.integers(0, 65536, 32).astype(np.uint16)
        blk = np.where(((blk >> 7) & 0xFF) == 0xFF, blk & 0x807F, blk).astype(np.uint16)
        emax = int(((blk >> 7) & 0xFF).max())
        assert oracle.block_scale(blk) == max(emax - 8, 0)


# ---------------------------------------------------------------------------
# Element map: exhaustive against the table-search encoder
# ---------------------------------------------------------------------------


def test_element_map_exhaustive_vs_table_search():
    x64 = bf16_bits_to_f64(FINITE_BF16)
    for S in range(0, 255):
        got = oracle.quantize_with_scale(FINITE_BF16, S)
        want = table_encode(np.ldexp(x64, 127 - S))
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (S, [(hex(FINITE_BF16[i]), hex(got[i]), hex(want[i])) for i in bad[:5]])


def test_encode_special_points():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(464.0) == 0x7E  # tie between 448 and (NaN slot) 480 stays at 448
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00
    assert oracle.e4m3_encode(-(2.0 ** -10)) == 0x80
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02  # 1.5 quanta -> 2 (even)
    assert oracle.e4m3_encode(15 * 2.0 ** -10) == 0x08  # 7.5 quanta -> 8 = smallest normal
    assert oracle.e4m3_encode(1.0625) == 0x38  # tie -> even mantissa
    assert oracle.e4m3_encode(1.1875) == 0x3A


# ---------------------------------------------------------------------------
# Invariants of the quantizer
# ---------------------------------------------------------------------------


def _random_bf16(rng, shape, spread=8):
    x = rng.standard_normal(shape).astype(np.float32) * np.exp2(rng.uniform(-spread, spread, (shape[0], 1))).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation is fine for test data


def test_sign_symmetry():
    rng = np.random.default_rng(1)
    x = _random_bf16(rng, (64, 256))
    q, s = oracle.quantize_rows(x)
    qn, sn = oracle.quantize_rows(x ^ np.uint16(0x8000))
    assert np.array_equal(s, sn)
    assert np.array_equal(qn, q ^ np.uint8(0x80))


def test_power_of_two_covariance():
    rng = np.random.default_rng(2)
    x = _random_bf16(rng, (64, 256), spread=4)
    q, s = oracle.quantize_rows(x)
    for j in (-20, -3, 1, 7, 30):
        e = ((x >> 7) & 0xFF).astype(np.int32)
        nz = e > 0
        xs = x.copy()
        xs[nz] = ((x[nz] & 0x807F) | ((e[nz] + j) << 7)).astype(np.uint16)  # exact x * 2^j
        q2, s2 = oracle.quantize_rows(xs)
        # only blocks that stay clear of the clamp and of bf16 subnormals are covariant
        ok = (s.astype(int) + j > 0) & (s.astype(int) + j <= 246)
        ok_rows = np.repeat(ok, 32, axis=1)
        assert np.array_equal(s2[ok].astype(int), s[ok].astype(int) + j)
        # elements that were bf16 zero stay zero; everything else identical
        assert np.array_equal(q2[ok_rows], q[ok_rows])


def test_top_binade_and_error_bound():
    rng = np.random.default_rng(3)
    x = _random_bf16(rng, (128, 512))
    q, s = oracle.quantize_rows(x)
    qb = q.reshape(128, 16, 32)
    mags = (qb & 0x7F).max(axis=2)
    nz = s > 0
    assert np.all((mags[nz] >= 0x78) & (mags[nz] <= 0x7E))
    xv = bf16_bits_to_f64(x)
    deq = E4M3[q] * np.exp2(np.repeat(s.astype(np.float64) - 127, 32, axis=1))
    y = xv * np.exp2(127 - np.repeat(s.astype(np.float64), 32, axis=1))
    normal = (np.abs(y) >= 2.0 ** -6) & (np.abs(y) <= 448)
    bound = np.exp2(np.floor(np.log2(np.abs(xv[normal]))) - 4)
    assert np.all(np.abs(deq[normal] - xv[normal]) <= bound)


def test_round_trip_of_representable_blocks():
    rng = np.random.default_rng(4)
    pos = [c for c in range(0x7F)]
    for _ in range(300):
        e = int(rng.integers(-100, 100))
        codes = rng.choice(pos, 32)
        codes[rng.integers(0, 32)] = int(rng.integers(0x78, 0x7F))  # max in [256, 448]
        signs = rng.integers(0, 2, 32)
        vals = E4M3[codes] * (1 - 2 * signs) * 2.0 ** e
        bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(bf16_bits_to_f64(bits), vals)  # exactly representable
        q, s = oracle.quantize_rows(bits.reshape(1, 32))
        assert int(s[0, 0]) == e + 127
        want = (codes | (signs << 7)).astype(np.uint8)
        want[codes == 0] = (signs[codes == 0] << 7).astype(np.uint8)
        assert q[0].tolist() == want.tolist()


# ---------------------------------------------------------------------------
# Column-wise quantization against row-wise on transposed, padded slices
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("sizes", [[300], [160, 0, 96, 256], [1, 31, 33, 0, 257, 5]])
def test_cols_equals_rows_of_transposed_group_slices(sizes):
    rng = np.random.default_rng(5)
    M, N = sum(sizes), 48
    x = _random_bf16(rng, (M, N))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    qT, sT, P = oracle.quantize_cols(x, off)
    G = len(sizes)
    assert P[0] == 0
    for g in range(G):
        mg = sizes[g]
        assert P[g + 1] - P[g] == 256 * ((mg + 255) // 256)
        span = P[g + 1] - P[g]
        if span == 0:
            continue
        sl = np.zeros((span, N), np.uint16)
        sl[:mg] = x[off[g] : off[g + 1]]
        qr, sr = oracle.quantize_rows(np.ascontiguousarray(sl.T))
        assert np.array_equal(qT[:, P[g] : P[g + 1]], qr)
        assert np.array_equal(sT[:, P[g] // 32 : P[g + 1] // 32], sr)
    assert np.all(qT[:, P[G]:] == 0) and np.all(sT[:, P[G] // 32 :] == 0)


def test_cols_capacity_bound():
    rng = np.random.default_rng(6)
    for _ in range(500):
        G = int(rng.integers(1, 20))
        sizes = rng.integers(0, 700, G)
        M = int(sizes.sum())
        need = int(sum(256 * ((m + 255) // 256) for m in sizes))
        assert need <= oracle.cols_capacity(M, G)
    with pytest.raises(ValueError):
        oracle.quantize_cols(np.zeros((10, 4), np.uint16), np.array([0, 5, 10], np.int32), Mcap=256)


# ---------------------------------------------------------------------------
# Packed scale layout
# ---------------------------------------------------------------------------


def test_packed_scale_offsets_hand_worked():
    pts = []
    total = None
    with open(os.path.join(GOLD, "packed_scale_offsets.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            if line.startswith("TOTAL"):
                a, b = line[5:].split("|")
                total = (tuple(int(t) for t in a.split()), int(b))
                continue
            rk, rb, o = [p.strip() for p in line.split("|")]
            R, K = (int(t) for t in rk.split())
            r, b = (int(t) for t in rb.split())
            pts.append((R, K, r, b, int(o)))
    for R, K, r, b, o in pts:
        s = np.zeros((R, K // 32), np.uint8)
        s[r, b] = 0xA5
        pk = oracle.pack_scales(s, K)
        assert np.nonzero(pk)[0].tolist() == [o], (r, b)
    (R, K), nbytes = total
    assert oracle.packed_scale_bytes(R, K) == nbytes


def test_pack_unpack_round_trip_and_padding():
    rng = np.random.default_rng(8)
    for R, K in [(1, 32), (33, 288), (64, 7168), (70, 2048)]:
        s = rng.integers(1, 256, (R, K // 32)).astype(np.uint8)
        pk = oracle.pack_scales(s, K)
        assert pk.size == ((R + 31) // 32) * 32 * 8 * ((K + 255) // 256)
        assert np.array_equal(oracle.unpack_scales(pk, R, K), s)
        assert np.count_nonzero(pk) == s.size  # every scale lands once, pads are zero


# ---------------------------------------------------------------------------
# GEMM oracle: exact rational brute force and closed forms
# ---------------------------------------------------------------------------


def _frac_e4m3(c):
    s = -1 if c & 0x80 else 1
    e = (c >> 3) & 0xF
    m = c & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 2 ** 6)
    return s * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


def _frac_deq(q, S):
    return _frac_e4m3(int(q)) * (Fraction(2) ** (int(S) - 127))


def _quantized_operands(rng, M, N, K, G):
    x = _random_bf16(rng, (M, K), spread=6)
    w = _random_bf16(rng, (G * N, K), spread=3)
    Xq, Xs = oracle.quantize_rows(x)
    Wq, Ws = oracle.quantize_rows(w)
    return Xq, Xs, Wq.reshape(G, N, K), Ws.reshape(G, N, K // 32)


def test_grouped_gemm_exact_rational():
    rng = np.random.default_rng(9)
    M, N, K = 7, 3, 96
    sizes = [3, 0, 4]
    off = np.array([0, 3, 3, 7], np.int32)
    Xq, Xs, Wq, Ws = _quantized_operands(rng, M, N, K, 3)
    out = oracle.grouped_gemm(Xq, Xs, Wq, Ws, off)
    for m in range(M):
        g = 0 if m < 3 else 2
        for n in range(N):
            exact = sum(_frac_deq(Xq[m, k], Xs[m, k // 32]) * _frac_deq(Wq[g, n, k], Ws[g, n, k // 32]) for k in range(K))
            assert abs(Fraction(out[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 1000)
    pts_r = np.array([0, 6, 3, 4], np.int64)
    pts_c = np.array([2, 0, 1, 1], np.int64)
    assert np.array_equal(oracle.grouped_gemm_points(Xq, Xs, Wq, Ws, off, pts_r, pts_c), out[pts_r, pts_c])


def test_grouped_gemm_one_hot_closed_form():
    rng = np.random.default_rng(10)
    M, N, K, G = 64, 16, 256, 2
    off = np.array([0, 40, 64], np.int32)
    Xq, Xs, _, _ = _quantized_operands(rng, M, N, K, G)
    Wq = np.zeros((G, N, K), np.uint8)
    Ws = rng.integers(100, 150, (G, N, K // 32)).astype(np.uint8)
    k0 = rng.integers(0, K, (G, N))
    c0 = rng.choice([0x38, 0x40, 0xB0, 0x7E, 0x01], (G, N))
    for g in range(G):
        for n in range(N):
            Wq[g, n, k0[g, n]] = c0[g, n]
    out = oracle.grouped_gemm(Xq, Xs, Wq, Ws, off)
    for m in range(M):
        g = 0 if m < 40 else 1
        for n in range(N):
            k = k0[g, n]
            want = E4M3[Xq[m, k]] * 2.0 ** (int(Xs[m, k // 32]) - 127) * E4M3[c0[g, n]] * 2.0 ** (int(Ws[g, n, k // 32]) - 127)
            assert out[m, n] == want


def test_wgrad_exact_rational():
    rng = np.random.default_rng(11)
    sizes = [5, 0, 40]
    M, N, K = sum(sizes), 3, 2
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    dy = _random_bf16(rng, (M, N), spread=2)
    x = _random_bf16(rng, (M, K), spread=2)
    Aq, As, P = oracle.quantize_cols(dy, off)
    Bq, Bs, P2 = oracle.quantize_cols(x, off)
    assert np.array_equal(P, P2)
    dW = oracle.wgrad(Aq, As, Bq, Bs, P)
    assert np.all(dW[1] == 0)
    for g in (0, 2):
        for n in range(N):
            for k in range(K):
                exact = sum(_frac_deq(Aq[n, t], As[n, t // 32]) * _frac_deq(Bq[k, t], Bs[k, t // 32]) for t in range(P[g], P[g + 1]))
                assert abs(Fraction(dW[g, n, k]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 1000)
    gs = np.array([0, 2, 1], np.int64)
    ns = np.array([1, 2, 0], np.int64)
    ks = np.array([0, 1, 1], np.int64)
    assert np.array_equal(oracle.wgrad_points(Aq, As, Bq, Bs, P, gs, ns, ks), dW[gs, ns, ks])


def test_wgrad_matches_rowwise_gemm_of_padded_slices():
    """wgrad of group g equals the grouped GEMM of the row-quantized, zero-padded,
    transposed group slices (same numbers, a different route through the oracle)."""
    rng = np.random.default_rng(12)
    sizes = [70, 300]
    M, N, K = sum(sizes), 8, 6
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    dy = _random_bf16(rng, (M, N), spread=2)
    x = _random_bf16(rng, (M, K), spread=2)
    Aq, As, P = oracle.quantize_cols(dy, off)
    Bq, Bs, _ = oracle.quantize_cols(x, off)
    dW = oracle.wgrad(Aq, As, Bq, Bs, P)
    for g in range(2):
        span = P[g + 1] - P[g]
        a = np.zeros((span, N), np.uint16)
        a[: sizes[g]] = dy[off[g] : off[g + 1]]
        b = np.zeros((span, K), np.uint16)
        b[: sizes[g]] = x[off[g] : off[g + 1]]
        aq, as_ = oracle.quantize_rows(np.ascontiguousarray(a.T))
        bq, bs = oracle.quantize_rows(np.ascontiguousarray(b.T))
        ref = oracle.grouped_gemm(aq, as_, bq.reshape(1, K, span), bs.reshape(1, K, span // 32), np.array([0, N], np.int32))
        assert np.array_equal(ref, dW[g])


# ---------------------------------------------------------------------------
# SwiGLU of the gate and up projections, quantized to MXFP8 (the activation
# step of the MoE layer that the kucoin.com MoK page (section 02) fuses with the
# quantization): closed forms of silu, a closed-form scale sweep on real
# values, the table-search encoder on off-grid values, and reductions to the
# pinned bf16 quantizer.
# ---------------------------------------------------------------------------


def _ulps(a, b):
    return abs(a - b) / math.ulp(max(abs(a), abs(b)))


def test_silu_closed_forms():
    ln3 = math.log(3.0)
    assert oracle.silu(0.0) == 0.0
    # sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4, sigmoid(-ln 3) = 1/4
    assert _ulps(oracle.silu(ln3), 0.75 * ln3) <= 4
    assert _ulps(oracle.silu(-ln3), -0.25 * ln3) <= 4
    # e^-64 is far below half an ulp of 1: silu(64) is 64 itself
    assert oracle.silu(64.0) == 64.0
    assert -64.0 * 2.0 ** -92 <= oracle.silu(-64.0) < 0.0
    assert oracle.silu(-1000.0) == 0.0


def test_silu_odd_part_identity():
    """silu(x) - silu(-x) = x sigmoid(x) + x sigmoid(-x) = x."""
    rng = np.random.default_rng(20)
    for x in rng.uniform(-30.0, 30.0, 200):
        d = oracle.silu(x) - oracle.silu(-x)
        assert abs(d - x) <= 4 * math.ulp(abs(x)) + 1e-300


def test_block_scale_f64_closed_form_sweep():
    """amax = f 2^e with f in [1, 2): S = clamp(e - 8, -127, 127) + 127, for any
    other elements below amax in magnitude and either sign of amax."""
    rng = np.random.default_rng(21)
    for e in range(-140, 140):
        for f in (1.0, 1.0 + 2.0 ** -40, 1.5, 2.0 - 2.0 ** -45):
            amax = math.ldexp(f, e)
            blk = rng.uniform(-1.0, 1.0, 32) * amax * 0.999
            blk[rng.integers(0, 32)] = amax if rng.integers(0, 2) else -amax
            want = min(max(e - 8, -127), 127) + 127
            assert oracle.block_scale_f64(blk) == want, (e, f)
    assert oracle.block_scale_f64(np.zeros(32)) == 0
    assert oracle.block_scale_f64(-np.zeros(32)) == 0


def test_quantize_f64_matches_table_search_off_grid():
    """Values between the E4M3 grid points, the exact midpoints (ties to even)
    and their neighbours, beyond saturation and in the subnormal range."""
    rng = np.random.default_rng(22)
    pos = POS[np.isfinite(POS)]
    mids = (pos[:-1] + pos[1:]) / 2
    y = np.concatenate([
        rng.uniform(-500.0, 500.0, 4000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 1000),
        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
        [448.0, 463.99, 464.0, 1e30, -1e30, 2.0 ** -10, 2.0 ** -10 + 2.0 ** -60, 3 * 2.0 ** -11, 0.0, -0.0],
    ])
    for S in (127, 100, 140, 0, 254):
        x = np.ldexp(y, S - 127)
        ok = np.isfinite(x) & (np.ldexp(x, 127 - S) == y)  # x exactly y 2^(S-127)
        got = oracle.quantize_f64_with_scale(x[ok], S)
        assert np.array_equal(got, table_encode(y[ok])), S


def test_quantize_rows_f64_equals_bf16_path_on_bf16_values():
    rng = np.random.default_rng(23)
    x = _random_bf16(rng, (96, 256), spread=40)
    x[3, 32:64] = 0
    x[4, 0:32] = rng.integers(1, 0x80, 32).astype(np.uint16)  # bf16 subnormals
    q, s = oracle.quantize_rows(x)
    q2, s2 = oracle.quantize_rows_f64(bf16_bits_to_f64(x))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def _times64_bits(x):
    """bf16 bits of 64 x (exponent field + 6), for normal bf16 x below 2^120."""
    e = (x >> 7) & 0xFF
    assert np.all((e > 0) & (e < 0xF0))
    return ((x & 0x807F) | ((e + 6) << 7)).astype(np.uint16)


def test_swiglu_saturated_gate_reduces_to_quantize_rows():
    """gate = 64: silu(64) = 64 exactly, so h = 64 up and its quantization is the
    bf16 quantizer's on the bits of 64 up (a gate/up mix-up or a wrong silu
    gives other values)."""
    rng = np.random.default_rng(24)
    up = _random_bf16(rng, (40, 256), spread=12)
    up[(up >> 7) & 0xFF == 0] = 0x3F80  # keep every element a normal number
    gate = np.full(up.shape, 64.0)
    h, q, s = oracle.swiglu_quantize(gate, bf16_bits_to_f64(up))
    assert np.array_equal(h, 64.0 * bf16_bits_to_f64(up))
    q_ref, s_ref = oracle.quantize_rows(_times64_bits(up))
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)
    # zero gate: silu(0) = 0, every block is zero with scale byte 0
    h0, q0, s0 = oracle.swiglu_quantize(np.zeros(up.shape), bf16_bits_to_f64(up))
    assert np.all(h0 == 0) and np.all(E4M3[q0] == 0) and np.all(s0 == 0)


def test_swiglu_quantization_invariants():
    """Random gate/up: every nonzero block's largest |y| lies in [2^8, 2^9);
    normal-range elements are within half an E4M3 ulp (2^-4 of their binade),
    subnormal-range ones within half the subnormal quantum, and only |y| beyond
    448 + 16 saturates."""
    rng = np.random.default_rng(25)
    gate = rng.standard_normal((64, 512)) * 3.0
    up = rng.standard_normal((64, 512)) * np.exp2(rng.uniform(-30, 30, (64, 1)))
    h, q, s = oracle.swiglu_quantize(gate, up)
    Sx = np.repeat(s.astype(np.float64), 32, axis=1)
    y = np.ldexp(h, (127 - Sx).astype(np.int64))
    amax_y = np.abs(y).reshape(64, 16, 32).max(axis=2)
    assert np.all((amax_y >= 256.0) & (amax_y < 512.0))
    v = E4M3[q]
    normal = (np.abs(y) >= 2.0 ** -6) & (np.abs(y) <= 448.0)
    assert np.all(np.abs(v - y)[normal] <= np.exp2(np.floor(np.log2(np.abs(y[normal]))) - 4))
    sub = np.abs(y) < 2.0 ** -6
    assert np.all(np.abs(v - y)[sub] <= 2.0 ** -10)
    assert np.all(np.abs(v[np.abs(y) >= 464.0]) == 448.0)
    assert np.all(np.sign(v[v != 0]) == np.sign(y[v != 0]))


def test_grouped_gemm_swiglu_one_hot_routing():
    """Each row of X holds one 1.0 (column km); every gate weight is 64, so
    gate = 64 and up = expert g's up weight at column km: the layer's output is
    the bf16 quantizer's on 64 Wu[g][c][km], with rows past the last group
    zero.  Pins the expert choice and the gate/up roles of the composition."""
    rng = np.random.default_rng(26)
    M, I, K = 48, 64, 256
    off = np.array([0, 12, 12, 40], np.int32)  # rows 40..47 belong to no group
    G = 3
    km = rng.integers(0, K, M)
    Xq = np.zeros((M, K), np.uint8)
    Xq[np.arange(M), km] = 0x38                # 1.0
    Xs = np.full((M, K // 32), 127, np.uint8)
    Wgq = np.full((G, I, K), 0x38, np.uint8)
    Wgs = np.full((G, I, K // 32), 133, np.uint8)  # 1.0 * 2^6
    Wuq = rng.integers(0, 0x7F, (G, I, K)).astype(np.uint8) | (rng.integers(0, 2, (G, I, K)) << 7).astype(np.uint8)
    Wuq[(Wuq & 0x7F) == 0x7F] = 0x40           # no NaN codes
    Wuq[(Wuq & 0x7F) == 0] = 0x30              # and no zeros: up (a sum from +0) is never -0
    Wus = rng.integers(110, 140, (G, I, K // 32)).astype(np.uint8)
    h, q, s, gate, up = oracle.grouped_gemm_swiglu(Xq, Xs, Wgq, Wgs, Wuq, Wus, off)
    upv = np.zeros((M, I))
    for m in range(40):
        g = 0 if m < 12 else 2
        k = km[m]
        upv[m] = E4M3[Wuq[g, :, k]] * np.exp2(Wus[g, :, k // 32].astype(np.float64) - 127)
    assert np.all(gate[:40] == 64.0) and np.all(gate[40:] == 0.0)
    assert np.array_equal(up, upv)
    # 64 up is a bf16 value (3 fraction bits, exponent in range): quantize its bits
    hb = (np.asarray(64.0 * upv, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_bits_to_f64(hb), 64.0 * upv)
    q_ref, s_ref = oracle.quantize_rows(hb)
    assert np.array_equal(q[:40], q_ref[:40]) and np.array_equal(s[:40], s_ref[:40])
    assert np.all(E4M3[q[40:]] == 0) and np.all(s[40:] == 0)


def test_grouped_gemm_swiglu_blocks_match_full():
    rng = np.random.default_rng(27)
    M, I, K, G = 70, 96, 128, 2
    off = np.array([0, 33, 70], np.int32)
    x = _random_bf16(rng, (M, K), spread=3)
    wg = _random_bf16(rng, (G * I, K), spread=2)
    wu = _random_bf16(rng, (G * I, K), spread=2)
    Xq, Xs = oracle.quantize_rows(x)
    Wgq, Wgs = oracle.quantize_rows(wg)
    Wuq, Wus = oracle.quantize_rows(wu)
    args = (Xq, Xs, Wgq.reshape(G, I, K), Wgs.reshape(G, I, K // 32), Wuq.reshape(G, I, K),
            Wus.reshape(G, I, K // 32), off)
    h, q, s, gate, up = oracle.grouped_gemm_swiglu(*args)
    rows = np.array([0, 32, 33, 69, 5], np.int64)
    blocks = np.array([0, 2, 1, 2, 1], np.int64)
    hb, qb, sb, gb, ub = oracle.grouped_gemm_swiglu_blocks(*args, rows, blocks)
    for i, (r, b) in enumerate(zip(rows, blocks)):
        sl = slice(32 * b, 32 * b + 32)
        assert np.array_equal(hb[i], h[r, sl]) and np.array_equal(qb[i], q[r, sl]) and sb[i] == s[r, b]
        assert np.array_equal(gb[i], gate[r, sl]) and np.array_equal(ub[i], up[r, sl])


# ---------------------------------------------------------------------------
# Backward pass of SwiGLU: closed forms, central differences, and the bf16
# rounding of the results against torch's conversion and hand-worked ties.
# ---------------------------------------------------------------------------


def test_dsilu_closed_forms():
    ln3 = math.log(3.0)
    assert oracle.dsilu(0.0) == 0.5
    # sigma(ln 3) = 3/4: silu'(ln 3) = 3/4 (1 + ln 3 / 4); sigma(-ln 3) = 1/4
    assert _ulps(oracle.dsilu(ln3), 0.75 * (1.0 + 0.25 * ln3)) <= 8
    assert _ulps(oracle.dsilu(-ln3), 0.25 * (1.0 - 0.75 * ln3)) <= 64
    assert oracle.dsilu(64.0) == 1.0
    assert -64.0 * 2.0 ** -90 < oracle.dsilu(-64.0) < 0.0
    assert oracle.dsilu(-1000.0) == 0.0


def test_dsilu_central_differences():
    rng = np.random.default_rng(30)
    d = 1e-5
    for x in rng.uniform(-20.0, 20.0, 300):
        fd = (oracle.silu(x + d) - oracle.silu(x - d)) / (2 * d)
        assert abs(fd - oracle.dsilu(x)) <= 1e-8, x


def test_bf16_round_matches_torch_on_float32_values():
    import torch
    rng = np.random.default_rng(31)
    f = (rng.standard_normal(20000) * np.exp2(rng.uniform(-140, 128, 20000))).astype(np.float32)
    # exact midpoints between neighbouring bf16 values (representable in float32)
    b = (rng.integers(0, 0x7F7F, 4000).astype(np.uint32) << 16)
    mids = (b | 0x8000).view(np.float32)
    f = np.concatenate([f, mids, -mids, np.array([0.0, -0.0, 3.3895e38, 1e-45], np.float32)])
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round(f.astype(np.float64)), want)


def test_bf16_round_ties_and_single_rounding():
    # 1 + 2^-8 lies halfway between 1 (even) and 1 + 2^-7; 1 + 3 2^-8 between
    # 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert oracle.bf16_round(1 + 2.0 ** -8) == 0x3F80
    assert oracle.bf16_round(1 + 3 * 2.0 ** -8) == 0x3F82
    # just past the midpoint by less than float32 can hold: rounding through
    # float32 first would land on the tie and go to even instead
    assert oracle.bf16_round((1 + 2.0 ** -8) * (1 + 2.0 ** -30)) == 0x3F81
    assert oracle.bf16_round((1 + 2.0 ** -8) * (1 - 2.0 ** -30)) == 0x3F80
    assert oracle.bf16_round(-(1 + 3 * 2.0 ** -8) * (1 - 2.0 ** -30)) == 0xBF81
    # bf16 subnormals are multiples of 2^-133; the largest rounds up into the normals
    assert oracle.bf16_round(2.0 ** -133) == 0x0001
    assert oracle.bf16_round(3 * 2.0 ** -134) == 0x0002       # 1.5 quanta: tie to even
    assert oracle.bf16_round(2.0 ** -126 - 2.0 ** -140) == 0x0080
    assert oracle.bf16_round(1e300) == 0x7F80


def test_swiglu_backward_closed_forms():
    rng = np.random.default_rng(32)
    up = rng.standard_normal(500)
    dh = rng.standard_normal(500)
    dg, du, h = oracle.swiglu_backward(np.zeros(500), up, dh)
    assert np.array_equal(dg, dh * up * 0.5) and np.all(du == 0) and np.all(h == 0)
    dg, du, h = oracle.swiglu_backward(np.full(500, 64.0), up, dh)
    assert np.array_equal(dg, dh * up) and np.array_equal(du, 64.0 * dh) and np.array_equal(h, 64.0 * up)
    ln3 = math.log(3.0)
    dg, du, h = oracle.swiglu_backward(np.full(500, ln3), up, dh)
    for i in range(0, 500, 37):
        assert _ulps(dg[i], dh[i] * up[i] * 0.75 * (1 + 0.25 * ln3)) <= 16
        assert _ulps(du[i], dh[i] * 0.75 * ln3) <= 8
        assert _ulps(h[i], 0.75 * ln3 * up[i]) <= 8
