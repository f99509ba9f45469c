"""Pins of the oracle's dispatch and combine functions (route_plan, f32_round,
gather_rows, combine) against definitions computed another way: a plain sort
of (expert, entry) pairs, numpy's and torch's own float conversions, hand-
worked rounding cases and closed forms of the combine."""
import numpy as np
import pytest
import torch

import oracle


def brute_plan(experts, G):
    """Slots by sorting the routed entries on (expert, entry index)."""
    T, k = experts.shape
    entries = sorted((int(e), j) for j, e in enumerate(experts.reshape(-1)) if 0 <= e < G)
    src = np.array([j // k for _, j in entries], np.int32)
    slot_of = np.full(T * k, -1, np.int32)
    for slot, (_, j) in enumerate(entries):
        slot_of[j] = slot
    counts = np.bincount([e for e, _ in entries], minlength=G) if entries else np.zeros(G, np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return offsets, src, slot_of.reshape(T, k)


@pytest.mark.parametrize("seed", range(6))
def test_route_plan_is_the_stable_sort_by_expert(seed):
    rng = np.random.default_rng(seed)
    T, k, G = int(rng.integers(1, 40)), int(rng.integers(1, 5)), int(rng.integers(1, 7))
    experts = rng.integers(-1, G + 1, (T, k)).astype(np.int32)  # -1 and G: dropped
    got = oracle.route_plan(experts, G)
    want = brute_plan(experts, G)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


def test_route_plan_hand_worked():
    experts = np.array([[1, 0], [1, 2], [0, 1]], np.int32)
    offsets, src, slot_of = oracle.route_plan(experts, 3)
    assert offsets.tolist() == [0, 2, 5, 6]
    assert src.tolist() == [0, 2, 0, 1, 2, 1]
    assert slot_of.tolist() == [[2, 0], [3, 5], [1, 4]]


def test_route_plan_inverse_maps():
    rng = np.random.default_rng(9)
    T, k, G = 500, 8, 16
    experts = np.stack([rng.permutation(G)[:k] for _ in range(T)]).astype(np.int32)
    offsets, src, slot_of = oracle.route_plan(experts, G)
    assert offsets[-1] == T * k and sorted(slot_of.reshape(-1).tolist()) == list(range(T * k))
    for t in range(T):
        for j in range(k):
            slot = slot_of[t, j]
            assert src[slot] == t
            assert offsets[experts[t, j]] <= slot < offsets[experts[t, j] + 1]


def test_f32_round_against_numpy():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-140, 120, 20000))
    x = np.concatenate([x, x * (1 + 2.0 ** -30)])
    got = np.array([oracle.f32_round(v) for v in x])
    assert np.array_equal(got, x.astype(np.float32).astype(np.float64))


def test_f32_round_hand_worked():
    u = 2.0 ** -23
    assert oracle.f32_round(1 + u / 2) == 1.0                     # tie to even
    assert oracle.f32_round(1 + 3 * u / 2) == 1 + 2 * u           # tie to even (up)
    assert oracle.f32_round(2.0 ** -150) == 0.0                   # half the smallest subnormal: tie to 0
    assert oracle.f32_round(3 * 2.0 ** -150) == 2.0 ** -148
    assert oracle.f32_round((2 - u / 2) * 2.0 ** 127) == np.inf   # rounds past the largest float
    assert oracle.f32_round(-(2 - u) * 2.0 ** 127) == -(2 - u) * 2.0 ** 127


def bf16_bits(v):
    return torch.tensor(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_gather_rows_without_scale_is_indexing():
    rng = np.random.default_rng(4)
    x = rng.integers(0, 1 << 16, (30, 64)).astype(np.uint16)
    src = np.array([3, 0, 29, 3, -1, 30, 7], np.int32)
    got = oracle.gather_rows(x, src)
    for r, s in enumerate(src):
        assert np.array_equal(got[r], x[s] if 0 <= s < 30 else np.zeros(64, np.uint16))


def test_gather_rows_scaled_against_torch():
    """fp32 product, then bf16: numpy's float32 product and torch's
    float32 -> bf16 conversion compute the same two roundings."""
    rng = np.random.default_rng(5)
    xv = (rng.standard_normal((40, 96)) * np.exp2(rng.integers(-20, 20, (40, 1)))).astype(np.float32)
    x = bf16_bits(xv)
    xb = (x.astype(np.uint32) << 16).view(np.float32)
    src = rng.integers(0, 40, 50).astype(np.int32)
    scale = rng.uniform(0, 1, 50).astype(np.float32)
    got = oracle.gather_rows(x, src, scale)
    want = bf16_bits(xb[src] * scale[:, None])  # float32 * float32: one RNE rounding
    assert np.array_equal(got, want)


def test_gather_rows_double_rounding_reading():
    """The scaled row is the fp32 product rounded to bf16, not the exact
    product rounded once.  x = 1 + 2^-7 (bf16), w = 0x1.02fa0cp+0 (fp32): the
    exact product lies just above the bf16 midpoint m = 1 + 2^-6 + 2^-8, so
    one rounding gives 1 + 3 2^-7 (0x3f83); its fp32 rounding is m itself,
    which ties to the even neighbour 1 + 2^-6 (0x3f82)."""
    a = 1 + 2.0 ** -7
    m = 1 + 2.0 ** -6 + 2.0 ** -8
    w = np.array([float.fromhex("0x1.02fa0cp+0")], np.float32)
    p = a * float(w[0])                                    # exact in double
    assert p > m and oracle.f32_round(p) == m
    assert oracle.bf16_round(np.array([p]))[0] == 0x3F83   # the single-rounding reading
    got = oracle.gather_rows(bf16_bits([a]).reshape(1, 1), np.array([0], np.int32), w)[0, 0]
    assert got == 0x3F82


def test_combine_one_hot_and_plain_sum():
    rng = np.random.default_rng(6)
    M, N, T, k = 40, 32, 10, 4
    y = bf16_bits(rng.standard_normal((M, N)))
    yv = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    slot_of = np.stack([rng.permutation(M)[:k] for _ in range(T)]).astype(np.int32)
    slot_of[0, 1] = -1                                      # a dropped entry
    w = np.zeros((T, k), np.float32)
    w[:, 2] = 1.0
    assert np.array_equal(oracle.combine(y, slot_of, w), yv[slot_of[:, 2]])
    plain = oracle.combine(y, slot_of)
    want = np.zeros((T, N))
    for t in range(T):
        for j in range(k):
            if slot_of[t, j] >= 0:
                want[t] += yv[slot_of[t, j]]
    assert np.array_equal(plain, want)


def test_combine_hand_worked_and_linear():
    y = bf16_bits([[1.0, -2.0], [0.5, 4.0], [3.0, 0.25]])
    slot_of = np.array([[2, 0], [1, -1]], np.int32)
    w = np.array([[0.5, 0.25], [2.0, 8.0]], np.float32)
    assert oracle.combine(y, slot_of, w).tolist() == [[1.5 + 0.25, 0.125 - 0.5], [1.0, 8.0]]
    w2 = np.array([[0.125, 1.0], [0.5, 0.0]], np.float32)
    assert np.array_equal(oracle.combine(y, slot_of, w + w2),
                          oracle.combine(y, slot_of, w) + oracle.combine(y, slot_of, w2))
