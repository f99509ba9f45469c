"""GPU parity of the one-GPU dispatch and combine path against the oracle:
mx_route_plan (bit for bit), mx_gather_quantize (bit for bit: the oracle's
gather, then its row-wise and column-wise quantization) and mx_combine (the
fp32 sum in choice order against the exact sum: within the bf16 rounding
(2^-8 of the value) plus the fp32 rounding of the k steps (k 2^-24 of the
magnitude sum), and at least 99 % of the results equal to the oracle's bf16
rounding of the exact sum)."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_04_amd as mx
import oracle
from mxfp8_block_scaled_04_amd import workloads as W
from tests.mxtest import bits, canonical_scales, combine_ok, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mx.load()


def plan_case(T, k, G, seed, drop=0.0, distinct=True):
    rng = np.random.default_rng(seed)
    if distinct and k <= G:
        e = np.stack([rng.permutation(G)[:k] for _ in range(T)]) if T else np.zeros((0, k), np.int64)
    else:
        e = rng.integers(0, G, (T, k))
    if drop:
        mask = rng.random((T, k)) < drop
        e = np.where(mask, rng.choice([-1, G, -7], (T, k)), e)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    return e.astype(np.int32), w


@pytest.mark.parametrize("T,k,G,drop,distinct", [
    (1, 1, 1, 0.0, True), (0, 4, 8, 0.0, True), (4096, 8, 16, 0.0, True), (1000, 4, 128, 0.1, False),
    (3000, 2, 4096, 0.0, False), (777, 6, 7, 0.3, False), (20000, 1, 3, 0.0, True)])
def test_route_plan_matches_the_oracle(T, k, G, drop, distinct):
    e, w = plan_case(T, k, G, T + G, drop, distinct)
    ed, wd = torch.from_numpy(e).to(DEV), torch.from_numpy(w).to(DEV)
    offsets, src, slot_of, slot_weight = mx.mx_route_plan(ed, G, wd)
    torch.cuda.synchronize()
    o_ref, s_ref, so_ref = oracle.route_plan(e, G)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    n = int(o_ref[-1])
    assert np.array_equal(src.cpu().numpy()[:n], s_ref)
    assert np.array_equal(slot_of.cpu().numpy(), so_ref)
    valid = so_ref >= 0
    sw = np.zeros(max(n, 1), np.float32)
    sw[so_ref[valid]] = w[valid]
    assert np.array_equal(slot_weight.cpu().numpy()[:n], sw[:n])


def special_tokens(T, N, seed):
    """bf16 [T, N]: N(0,1) rows scaled by 2^U(-8, 8), an all-zero block,
    a block of subnormals and an outlier."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, N)).astype(np.float32) * np.exp2(rng.uniform(-8, 8, (T, 1))).astype(np.float32)
    b = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    b[0, 0:32] = 0
    if T > 5:
        b[5, 32:64] = (rng.integers(1, 128, 32) | (rng.integers(0, 2, 32) << 15)).astype(np.uint16)
    b[-1, N - 1] = 0x461C  # 9984
    return torch.from_numpy(b.view(np.int16)).to(DEV).view(torch.bfloat16)


@pytest.mark.parametrize("T,k,G,N,scaled", [(700, 4, 8, 320, False), (700, 4, 8, 320, True),
                                             (300, 2, 3, 64, True), (1, 1, 1, 32, False)])
def test_gather_quantize_matches_the_oracle(T, k, G, N, scaled):
    x = special_tokens(T, N, T + N)
    e, w = plan_case(T, k, G, 7 * T + G, 0.05, False)
    offsets, src, slot_of, slot_weight = mx.mx_route_plan(torch.from_numpy(e).to(DEV), G,
                                                          torch.from_numpy(w).to(DEV))
    M = int(offsets[-1])
    Mcap = mx.mx_cols_capacity(M, G)
    q = torch.full((M, N), 0xEE, dtype=torch.uint8, device=DEV)
    qT = torch.full((N, Mcap), 0xEE, dtype=torch.uint8, device=DEV)
    q, s, qT, sT, P = mx.mx_gather_quantize(x, src, M, offsets, Mcap, slot_weight if scaled else None, q=q, qT=qT)
    torch.cuda.synchronize()
    src_h = src.cpu().numpy()[:M]
    g = oracle.gather_rows(bits(x), src_h, slot_weight.cpu().numpy()[:M] if scaled else None)
    q_ref, s_ref = oracle.quantize_rows(g)
    qT_ref, sT_ref, P_ref = oracle.quantize_cols(g, offsets.cpu().numpy(), Mcap)
    assert np.array_equal(u8(q), q_ref) and np.array_equal(canonical_scales(s, M, N), s_ref)
    assert np.array_equal(P.cpu().numpy(), P_ref)
    assert np.array_equal(u8(qT), qT_ref) and np.array_equal(canonical_scales(sT, N, Mcap), sT_ref)
    if not scaled:
        # the same bytes as the dual quantizer on the gathered rows
        gathered = x.index_select(0, src[:M].long())
        d = mx.mx_quantize_dual(gathered, offsets, Mcap)
        torch.cuda.synchronize()
        assert torch.equal(d[0], q) and torch.equal(d[2], qT)
        assert torch.equal(d[1], s) and torch.equal(d[3], sT)


def test_gather_quantize_out_of_range_sources_are_zero_rows():
    T, N, M = 50, 64, 40
    x = special_tokens(T, N, 1)
    src_h = np.arange(M, dtype=np.int32) % T
    src_h[[3, 17, 39]] = [-1, T, 1 << 30]
    src = torch.from_numpy(src_h).to(DEV)
    q, s, qT, sT, _ = mx.mx_gather_quantize(x, src, M)
    torch.cuda.synchronize()
    g = oracle.gather_rows(bits(x), src_h)
    q_ref, s_ref = oracle.quantize_rows(g)
    assert np.array_equal(u8(q), q_ref) and np.array_equal(canonical_scales(s, M, N), s_ref)
    assert not u8(q)[[3, 17, 39]].any()
    qT_ref, sT_ref, _ = oracle.quantize_cols(g, None, qT.shape[1])
    assert np.array_equal(u8(qT), qT_ref)


def combine_check(out, y, slot_of, w, tokens=None):
    """out bf16 [T, N] (or its rows `tokens`) against the oracle."""
    so = slot_of.cpu().numpy()
    wh = None if w is None else w.cpu().numpy()
    if tokens is not None:
        so = so[tokens]
        wh = None if wh is None else wh[tokens]
    got_b = bits(out) if tokens is None else bits(out[torch.from_numpy(tokens).to(DEV)])
    ok, equal = combine_ok(got_b, bits(y), so, wh)
    assert ok, equal


@pytest.mark.parametrize("T,k,G,N,weighted", [(500, 8, 16, 256, True), (500, 8, 16, 256, False),
                                               (333, 3, 5, 72, True), (1, 1, 1, 8, True)])
def test_combine_matches_the_oracle(T, k, G, N, weighted):
    e, w = plan_case(T, k, G, 3 * T + N, 0.1, False)
    wd = torch.from_numpy(w).to(DEV)
    offsets, src, slot_of, _ = mx.mx_route_plan(torch.from_numpy(e).to(DEV), G)
    M = int(offsets[-1])
    y = W.normal_bf16((max(M, 1), N), 1.0, 11, DEV)[:M]
    out = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    mx.mx_combine(y, slot_of, wd if weighted else None, out=out)
    torch.cuda.synchronize()
    combine_check(out, y, slot_of, wd if weighted else None)


def test_combine_one_hot_weights_are_the_gather():
    T, k, G, N = 400, 4, 8, 128
    e, _ = plan_case(T, k, G, 5, 0.0, True)
    offsets, src, slot_of, _ = mx.mx_route_plan(torch.from_numpy(e).to(DEV), G)
    M = int(offsets[-1])
    y = W.normal_bf16((M, N), 1.0, 12, DEV)
    w = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    w[:, 1] = 1.0
    out = mx.mx_combine(y, slot_of, w)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), y[slot_of[:, 1].long()].view(torch.int16))


def test_dispatch_and_combine_at_the_layer_shape():
    """4096 tokens, top-8 of 16 experts, hidden 7168: the plan in full, the
    gathered quantization on sampled rows and columns, the combine on
    sampled tokens."""
    T, k, G, H = 4096, 8, 16, 7168
    e, w = W.topk_routing(T, k, G, 0.5, 31)
    ed, wd = torch.from_numpy(e).to(DEV), torch.from_numpy(w).to(DEV)
    offsets, src, slot_of, slot_weight = mx.mx_route_plan(ed, G, wd)
    o_ref, s_ref, so_ref = oracle.route_plan(e, G)
    assert np.array_equal(offsets.cpu().numpy(), o_ref) and np.array_equal(slot_of.cpu().numpy(), so_ref)
    assert np.array_equal(src.cpu().numpy(), s_ref)
    M = T * k
    x = W.normal_bf16((T, H), 1.0, 32, DEV)
    Mcap = mx.mx_cols_capacity(M, G)
    q, s, qT, sT, P = mx.mx_gather_quantize(x, src, M, offsets, Mcap, slot_weight)
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    rows = np.unique(np.concatenate([rng.integers(0, M, 200), o_ref[1:-1] - 1, o_ref[1:-1]]))
    g = oracle.gather_rows(bits(x), s_ref[rows], w.reshape(-1)[np.argsort(so_ref.reshape(-1))][rows])
    q_ref, s_ref_rows = oracle.quantize_rows(g)
    assert np.array_equal(u8(q)[rows], q_ref)
    cols = np.array([0, 1, 100, 4095, 7167])
    full = oracle.gather_rows(bits(x[:, torch.from_numpy(cols).to(DEV)]), s_ref,
                              w.reshape(-1)[np.argsort(so_ref.reshape(-1))])
    qT_ref, _, _ = oracle.quantize_cols(full, o_ref, Mcap)
    assert np.array_equal(u8(qT)[cols], qT_ref)
    y = W.normal_bf16((M, H), 1.0, 34, DEV)
    out = mx.mx_combine(y, slot_of, wd)
    torch.cuda.synchronize()
    combine_check(out, y, slot_of, wd, tokens=np.unique(rng.integers(0, T, 64)))
