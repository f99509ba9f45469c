"""GPU parity of the grouped GEMM kernels against the fp64 oracle:
|gpu - ref| <= 8e-3 |ref| + 1e-3 rms(ref) for every checked element (the
bf16 output rounding alone contributes up to 2^-9 |ref|), and bit-exact
results where the exact product is representable in bf16 (one-hot weights).
Operands are quantized by the GPU kernels, and every test first asserts
that their codes and packed scales are exactly the oracle's quantization of
the same bf16 tensors; the oracle GEMM then runs on the oracle's operands, so
each check covers the chain from the bf16 inputs.  The large workloads are
checked on the sample the measurement recipe fixes (tests/parity.py); tests
named *multi_tile* check every output element of grids where each persistent
workgroup runs at least two tiles (the cross-tile pipeline, the store-count
waits after an epilogue, alternating round directions of wgrad)."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_04_amd as mx
import oracle
from mxfp8_block_scaled_04_amd import workloads as W
from tests.mxtest import bits, bf16_to_f64, canonical_scales, gemm_tolerance_ok, u8
from tests.parity import (assert_cols_are_oracle, assert_rows_are_oracle, gathered, gemm_sample, oracle_full,
                          oracle_points, oracle_wgrad_full, oracle_wgrad_points)

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mx.load()


def quantize_pair(x, w):
    """Quantize X [M, K] and W [G, N, K] on the GPU and assert that codes and
    packed scales are exactly the oracle's.  Returns the device tensors and
    the oracle's operands (codes, canonical scales) for the oracle GEMM."""
    G, N, K = w.shape
    Xq, Xs = mx.mx_quantize_rows(x)
    Wq, Ws = mx.mx_quantize_rows(w.reshape(G * N, K))
    torch.cuda.synchronize()
    xq, xs = assert_rows_are_oracle(x, Xq, Xs)
    wq, ws = assert_rows_are_oracle(w.reshape(G * N, K), Wq, Ws)
    host = (xq, xs, wq.reshape(G, N, K), ws.reshape(G, N, K // 32))
    return Xq, Xs, Wq.reshape(G, N, K), Ws, host


def nan_filled(shape):
    return torch.full(shape, NAN_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)


def test_gemm_tiny_moe_full():
    d = W.tiny_moe(seed=0, device=DEV)
    Xq, Xs, Wq, Ws, host = quantize_pair(d["x"], d["w"])
    off = torch.from_numpy(d["offsets"]).to(DEV)
    out = mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, off, out=nan_filled((d["M"], d["N"])))
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm(*host, d["offsets"])
    got = bf16_to_f64(out)
    ok, ratio = gemm_tolerance_ok(got, ref)
    assert ok, ratio


def test_gemm_one_hot_bit_exact():
    """One nonzero weight per output column: each output is a single product
    of two E4M3 values times two powers of two, exact in bf16."""
    rng = np.random.default_rng(3)
    M, N, K, G = 300, 200, 512, 3
    sizes = [120, 0, 180]
    off = W.offsets_from_sizes(sizes)
    x = torch.from_numpy((rng.standard_normal((M, K)) * 4).astype(np.float32)).to(torch.bfloat16).to(DEV)
    w = np.zeros((G, N, K), np.float32)
    k0 = rng.integers(0, K, (G, N))
    vals = rng.choice([1.0, -2.0, 0.5, 1.5, -3.0, 0.25], (G, N))
    for g in range(G):
        for n in range(N):
            w[g, n, k0[g, n]] = vals[g, n]
    wt = torch.from_numpy(w).to(torch.bfloat16).to(DEV)
    Xq, Xs, Wq, Ws, host = quantize_pair(x, wt)
    out = mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, torch.from_numpy(off).to(DEV), out=nan_filled((M, N)))
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm(*host, off)
    ref_bf16 = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(ref_bf16.float(), torch.from_numpy(ref.astype(np.float32)))  # exact in bf16
    assert np.array_equal(bits(out), bits(ref_bf16))


@pytest.mark.parametrize("sizes,N,K", [([1, 31, 33, 0, 257, 5], 72, 512), ([0, 0, 700], 300, 256), ([513], 256, 768), ([40] * 10, 40, 256)])
def test_gemm_ragged_full(sizes, N, K):
    M, G = sum(sizes), len(sizes)
    off = W.offsets_from_sizes(sizes)
    x = W.normal_bf16((M, K), 1.0, M + N, DEV)
    w = W.normal_bf16((G, N, K), 0.02, M + K, DEV)
    Xq, Xs, Wq, Ws, host = quantize_pair(x, w)
    out = mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, torch.from_numpy(off).to(DEV), out=nan_filled((M, N)))
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm(*host, off)
    ok, ratio = gemm_tolerance_ok(bf16_to_f64(out), ref)
    assert ok, ratio


def multi_tile_sizes(M, G, seed, N, nwg=256, rounds=2):
    """Dirichlet(0.5) group sizes over M rows whose 256 x 256 tile count is
    at least rounds x nwg (so every persistent workgroup runs >= rounds tiles)."""
    sizes = W.dirichlet_sizes(M, G, 0.5, seed)
    tiles = sum(-(-int(m) // 256) for m in sizes) * -(-N // 256)
    assert tiles >= rounds * nwg, tiles
    return list(sizes)


def test_gemm_multi_tile_full():
    """16384 x 2048 x 256, 16 Dirichlet(0.5) groups: every output element,
    with each workgroup running 2-3 tiles (>= 512 tiles on 256 workgroups)."""
    M, N, K, G = 16384, 2048, 256, 16
    sizes = multi_tile_sizes(M, G, 7, N)
    off = W.offsets_from_sizes(sizes)
    x = W.normal_bf16((M, K), 1.0, 41, DEV)
    w = W.normal_bf16((G, N, K), 0.02, 42, DEV)
    Xq, Xs, Wq, Ws, host = quantize_pair(x, w)
    out = mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, torch.from_numpy(off).to(DEV), out=nan_filled((M, N)))
    torch.cuda.synchronize()
    ref = oracle_full(*host, off)
    ok, ratio = gemm_tolerance_ok(bf16_to_f64(out), ref)
    assert ok, ratio


def test_gemm_group_permutation_bitwise():
    """Experts permuted together with their row blocks permute the output row
    blocks bit for bit: a row's result depends on its expert and its data,
    not on where its group sits (row tiles, bands, workgroups, XCDs).  Group
    sizes put rows at every offset mod 256 and mix full, partial and empty
    row tiles."""
    sizes = [300, 0, 45, 513, 7, 128, 129, 256, 1]
    G, N, K = len(sizes), 384, 512
    M = sum(sizes)
    off = W.offsets_from_sizes(sizes)
    x = W.normal_bf16((M, K), 1.0, 11, DEV)
    w = W.normal_bf16((G, N, K), 0.02, 12, DEV)
    perm = np.random.default_rng(3).permutation(G)
    sizes_p = [sizes[g] for g in perm]
    off_p = W.offsets_from_sizes(sizes_p)
    rows_p = np.concatenate([np.arange(off[g], off[g + 1]) for g in perm]).astype(np.int64)
    x_p = x[torch.from_numpy(rows_p).to(DEV)].contiguous()
    w_p = w[torch.from_numpy(perm).to(DEV)].contiguous()
    outs = []
    for xx, ww, oo in ((x, w, off), (x_p, w_p, off_p)):
        Xq, Xs, Wq, Ws, _ = quantize_pair(xx, ww)
        outs.append(mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, torch.from_numpy(oo).to(DEV), out=nan_filled((M, N))))
    torch.cuda.synchronize()
    a = bits(outs[0])[rows_p]
    b = bits(outs[1])
    assert np.array_equal(a, b), int(np.count_nonzero(a != b))


def test_gemm_ragged_expert_permutation_bitwise_full():
    """The ragged workload (65536 x 2048 x 7168, 128 Zipf experts with empty
    and 1-31-row groups) in the benchmark's launch configuration, its experts
    permuted together with their row blocks: every output element of the
    permuted run equals the original's permuted row, bit for bit (a check of
    the expert-aware tile order over the whole output, next to the oracle
    sample of the ragged parity test)."""
    d = W.moe_ragged(seed=0, device=DEV)
    sizes, off = d["sizes"], d["offsets"]
    G, N, K, M = d["G"], d["N"], d["K"], d["M"]
    perm = np.random.default_rng(9).permutation(G)
    off_p = W.offsets_from_sizes([int(sizes[g]) for g in perm])
    rows_p = torch.from_numpy(np.concatenate([np.arange(off[g], off[g + 1]) for g in perm]).astype(np.int64)).to(DEV)
    outs = []
    for xx, ww, oo in ((d["x"], d["w"], off), (d["x"][rows_p], d["w"][torch.from_numpy(perm).to(DEV)], off_p)):
        Xq, Xs = mx.mx_quantize_rows(xx.contiguous())
        Wq, Ws = mx.mx_quantize_rows(ww.contiguous().reshape(G * N, K))
        outs.append(mx.mx_grouped_gemm(Xq, Xs, Wq.reshape(G, N, K), Ws, torch.from_numpy(oo).to(DEV),
                                       out=nan_filled((M, N))))
        del Xq, Xs, Wq, Ws
    torch.cuda.synchronize()
    a = outs[0][rows_p].view(torch.int16)
    b = outs[1].view(torch.int16)
    assert torch.equal(a, b), int((a != b).sum())


def test_down_backward_expert_permutation_bitwise_full():
    """dgrad and wgrad of the down projection (32768 rows, 16 Dirichlet
    experts, 7168 x 2048) in the benchmark's launch configuration, experts
    permuted together with their row blocks: dX rows and dW experts permute
    bit for bit over the whole outputs (the wgrad longest-first order changes
    with the permutation, the results may not)."""
    d = W.moe_down_backward(seed=0, device=DEV)
    sizes, off = d["sizes"], d["offsets"]
    G, N, K, M = d["G"], d["N"], d["K"], d["M"]
    perm = np.random.default_rng(10).permutation(G)
    off_p = W.offsets_from_sizes([int(sizes[g]) for g in perm])
    rows_p = torch.from_numpy(np.concatenate([np.arange(off[g], off[g + 1]) for g in perm]).astype(np.int64)).to(DEV)
    perm_t = torch.from_numpy(perm).to(DEV)
    woff = torch.arange(0, G + 1, dtype=torch.int32, device=DEV) * N
    res = []
    for dy, x, w, oo in ((d["dy"], d["x"], d["w"], off), (d["dy"][rows_p], d["x"][rows_p], d["w"][perm_t], off_p)):
        o = torch.from_numpy(oo).to(DEV)
        dyq, dys = mx.mx_quantize_rows(dy.contiguous())
        wT, wTs, _ = mx.mx_quantize_cols(w.contiguous().reshape(G * N, K), woff)
        dx = mx.mx_grouped_gemm_dgrad(dyq, dys, wT, wTs, o, G, out=nan_filled((M, K)))
        A, As, P = mx.mx_quantize_cols(dy.contiguous(), o)
        B, Bs, _ = mx.mx_quantize_cols(x.contiguous(), o)
        dW = mx.mx_grouped_gemm_wgrad(A, As, B, Bs, P, dW=nan_filled((G * N, K)).view(G, N, K))
        res.append((dx, dW))
        del dyq, dys, wT, wTs, A, As, B, Bs
    torch.cuda.synchronize()
    (dx0, dW0), (dx1, dW1) = res
    assert torch.equal(dx0[rows_p].view(torch.int16), dx1.view(torch.int16))
    assert torch.equal(dW0[perm_t].view(torch.int16), dW1.view(torch.int16))


def test_gemm_zero_rows_is_noop():
    Xq = torch.empty((0, 256), dtype=torch.uint8, device=DEV)
    Xs = torch.empty(0, dtype=torch.uint8, device=DEV)
    Wq = torch.zeros((2, 64, 256), dtype=torch.uint8, device=DEV)
    Ws = torch.zeros(mx.mx_scale_bytes(128, 256), dtype=torch.uint8, device=DEV)
    off = torch.zeros(3, dtype=torch.int32, device=DEV)
    out = mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, off)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


def sampled_check(x, w, sizes, seed):
    """The workload in the benchmark's launch configuration, checked on the
    recipe's sample (a 128 x 128 tile per non-empty group, 4096 uniform
    points, every element of groups below 32 rows); every output row of a
    group must have been written (NaN prefill)."""
    M, K = x.shape
    G, N, _ = w.shape
    off = W.offsets_from_sizes(sizes)
    Xq, Xs, Wq, Ws, host = quantize_pair(x, w)
    out = mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, torch.from_numpy(off).to(DEV), out=nan_filled((M, N)))
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item(), "an output row was not written"
    rows, cols = gemm_sample(M, N, off, seed)
    ref = oracle_points(*host, off, rows, cols)
    ok, ratio = gemm_tolerance_ok(gathered(out, rows, cols), ref)
    assert ok, ratio
    return out


def test_gemm_gate_up_sampled():
    d = W.moe_gate_up(seed=0, device=DEV)
    sampled_check(d["x"], d["w"], d["sizes"], 0)


def test_gemm_ragged_and_dense_sampled():
    d = W.moe_ragged(seed=0, device=DEV)
    sampled_check(d["x"], d["w"], d["sizes"], 1)
    sampled_check(d["x"], d["w_dense"], [d["M"]], 2)


def test_gemm_down_forward_sampled():
    d = W.moe_down_backward(seed=0, device=DEV)
    sampled_check(d["x"], d["w"], d["sizes"], 3)


def dgrad_check(dy, w, sizes, seed, sample=True):
    """dX = dY W per expert: dY row-quantized along N_out; W^T from the
    column-wise quantization of W viewed as [G*N_out, K_in] with one group per
    expert, consumed in place by mx_grouped_gemm_dgrad."""
    G, Nout, Kin = w.shape
    M = dy.shape[0]
    dyq, dys = mx.mx_quantize_rows(dy)
    woff_h = (np.arange(G + 1) * Nout).astype(np.int32)
    wT, wTs, P = mx.mx_quantize_cols(w.reshape(G * Nout, Kin), torch.from_numpy(woff_h).to(DEV))
    off = W.offsets_from_sizes(sizes)
    out = mx.mx_grouped_gemm_dgrad(dyq, dys, wT, wTs, torch.from_numpy(off).to(DEV), G, out=nan_filled((M, Kin)))
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item()
    # both operands are exactly the oracle's quantizations of the bf16 inputs
    dq, ds = assert_rows_are_oracle(dy, dyq, dys)
    wT_h, wTs_h, _ = assert_cols_are_oracle(w.reshape(G * Nout, Kin), woff_h, wT, wTs, P)
    # oracle operands: W^T of expert g = columns [g Nout, (g+1) Nout) of the
    # column-quantized weights, as a [G, Kin, Nout] stack
    Bq = np.stack([wT_h[:, g * Nout:(g + 1) * Nout] for g in range(G)])
    Bs = np.stack([wTs_h[:, g * Nout // 32:(g + 1) * Nout // 32] for g in range(G)])
    if sample:
        rows, cols = gemm_sample(M, Kin, off, seed)
        ref = oracle_points(dq, ds, Bq, Bs, off, rows, cols)
        ok, ratio = gemm_tolerance_ok(gathered(out, rows, cols), ref)
    else:
        ref = oracle_full(dq, ds, Bq, Bs, off)
        ok, ratio = gemm_tolerance_ok(bf16_to_f64(out), ref)
    assert ok, ratio


def test_gemm_dgrad_small_full():
    sizes = [5, 0, 300, 40]
    G, Nout, Kin = 4, 512, 72
    dy = W.normal_bf16((sum(sizes), Nout), 1.0, 21, DEV)
    w = W.normal_bf16((G, Nout, Kin), 0.02, 22, DEV)
    dgrad_check(dy, w, sizes, 0, sample=False)


def test_gemm_dgrad_sampled():
    d = W.moe_down_backward(seed=0, device=DEV)
    dgrad_check(d["dy"], d["w"], d["sizes"], 4)


def test_gemm_dgrad_multi_tile_full():
    """dX [16384, 2048] = dY [16384, 256] W (16 experts, Dirichlet(0.5)):
    every element, each workgroup running >= 2 tiles."""
    M, Nout, Kin, G = 16384, 256, 2048, 16
    sizes = multi_tile_sizes(M, G, 8, Kin)
    dy = W.normal_bf16((M, Nout), 1.0, 43, DEV)
    w = W.normal_bf16((G, Nout, Kin), 0.02, 44, DEV)
    dgrad_check(dy, w, sizes, 0, sample=False)


@pytest.mark.parametrize("sizes,N,K", [([5, 0, 300, 40], 64, 48), ([256], 296, 264), ([0, 0], 32, 32), ([700, 1], 256, 256)])
def test_wgrad_full(sizes, N, K):
    M = sum(sizes)
    off = W.offsets_from_sizes(sizes)
    dy = W.normal_bf16((M, N), 1.0, 11 + M, DEV)
    x = W.normal_bf16((M, K), 1.0, 12 + M, DEV)
    off_dev = torch.from_numpy(off).to(DEV)
    A, As, P = mx.mx_quantize_cols(dy, off_dev)
    B, Bs, P2 = mx.mx_quantize_cols(x, off_dev)
    G = len(sizes)
    dW = mx.mx_grouped_gemm_wgrad(A, As, B, Bs, P, dW=nan_filled((G, N, K)))
    torch.cuda.synchronize()
    Aq, Asc, Pr = assert_cols_are_oracle(dy, off, A, As, P)
    Bq, Bsc, _ = assert_cols_are_oracle(x, off, B, Bs, P2)
    ref = oracle.wgrad(Aq, Asc, Bq, Bsc, Pr)
    ok, ratio = gemm_tolerance_ok(bf16_to_f64(dW), ref)
    assert ok, ratio
    for g in range(G):
        if sizes[g] == 0:
            assert torch.count_nonzero(dW[g].float()).item() == 0


def test_wgrad_multi_tile_full():
    """40 groups (taken longest first, rounds in alternating directions),
    dW [40, 1024, 1024] over 4096 Dirichlet(0.5)-routed rows: every element,
    640 tiles on 256 workgroups (two tile rounds for all, a third for some)."""
    M, N, K, G = 4096, 1024, 1024, 40
    sizes = list(W.dirichlet_sizes(M, G, 0.5, 9))
    sizes = [max(1, s) for s in sizes]  # every group non-empty: 40 x 16 tiles
    sizes[int(np.argmax(sizes))] -= sum(sizes) - M
    off = W.offsets_from_sizes(sizes)
    dy = W.normal_bf16((M, N), 1.0, 45, DEV)
    x = W.normal_bf16((M, K), 1.0, 46, DEV)
    off_dev = torch.from_numpy(off).to(DEV)
    A, As, P = mx.mx_quantize_cols(dy, off_dev)
    B, Bs, P2 = mx.mx_quantize_cols(x, off_dev)
    dW = mx.mx_grouped_gemm_wgrad(A, As, B, Bs, P, dW=nan_filled((G, N, K)))
    torch.cuda.synchronize()
    Aq, Asc, Pr = assert_cols_are_oracle(dy, off, A, As, P)
    Bq, Bsc, _ = assert_cols_are_oracle(x, off, B, Bs, P2)
    ref = oracle_wgrad_full(Aq, Asc, Bq, Bsc, Pr)
    ok, ratio = gemm_tolerance_ok(bf16_to_f64(dW), ref)
    assert ok, ratio


def test_wgrad_down_backward_sampled():
    d = W.moe_down_backward(seed=0, device=DEV)
    off = d["offsets"]
    off_dev = torch.from_numpy(off).to(DEV)
    A, As, P = mx.mx_quantize_cols(d["dy"], off_dev)
    B, Bs, P2 = mx.mx_quantize_cols(d["x"], off_dev)
    G, N, K = d["G"], d["N"], d["K"]
    dW = mx.mx_grouped_gemm_wgrad(A, As, B, Bs, P, dW=nan_filled((G, N, K)))
    torch.cuda.synchronize()
    assert not torch.isnan(dW).any().item()
    Aq, Asc, Pr = assert_cols_are_oracle(d["dy"], off, A, As, P)
    Bq, Bsc, _ = assert_cols_are_oracle(d["x"], off, B, Bs, P2)
    # the recipe's sample mapped to dW [G][N][K]: a 128 x 128 tile of every
    # expert's dW (the contraction is the group), 4096 uniform points, and
    # the last element of every expert
    rng = np.random.default_rng(5)
    gs, ns, ks = [rng.integers(0, G, 4096)], [rng.integers(0, N, 4096)], [rng.integers(0, K, 4096)]
    for g in range(G):
        n0 = 128 * int(rng.integers(0, N // 128))
        k0 = 128 * int(rng.integers(0, K // 128))
        nn, kk = np.meshgrid(np.arange(n0, n0 + 128), np.arange(k0, k0 + 128), indexing="ij")
        gs.append(np.full(nn.size, g))
        ns.append(nn.ravel())
        ks.append(kk.ravel())
        gs.append(np.array([g]))
        ns.append(np.array([N - 1]))
        ks.append(np.array([K - 1]))
    gs, ns, ks = (np.concatenate(a).astype(np.int64) for a in (gs, ns, ks))
    ref = oracle_wgrad_points(Aq, Asc, Bq, Bsc, Pr, gs, ns, ks)
    got = bf16_to_f64(dW[torch.from_numpy(gs).to(DEV), torch.from_numpy(ns).to(DEV), torch.from_numpy(ks).to(DEV)])
    ok, ratio = gemm_tolerance_ok(got, ref)
    assert ok, ratio


@pytest.mark.parametrize("offs,M,want", [
    ([0, 160, 160, 256, 512], 512, 0),      # the tiny MoE routing
    ([16, 76, 76, 150], 170, 0),            # rows outside every group are allowed
    ([0, 10, 5, 20], 20, 3),                # decreasing at index 2
    ([-1, 5, 9], 9, 1),                     # negative first entry
    ([0, 5, 11], 10, 3),                    # past M
    ([0] * 4097, 0, 0),                     # 4096 empty groups
])
def test_validate_offsets(offs, M, want):
    r = mx.mx_validate_offsets(torch.tensor(offs, dtype=torch.int32, device=DEV), M)
    torch.cuda.synchronize()
    assert int(r.item()) == want


def test_wgrad_many_groups_natural_order():
    """300 groups (above the 256 that are ranked longest first): the natural
    tile order; mixed lengths, empty groups; sampled against the oracle."""
    rng = np.random.default_rng(21)
    sizes = list(rng.choice([0, 1, 40, 300, 600], 300))
    M, N, K = int(sum(sizes)), 64, 96
    off = W.offsets_from_sizes(sizes)
    dy = W.normal_bf16((M, N), 1.0, 31, DEV)
    x = W.normal_bf16((M, K), 1.0, 32, DEV)
    off_dev = torch.from_numpy(off).to(DEV)
    A, As, P = mx.mx_quantize_cols(dy, off_dev)
    B, Bs, _ = mx.mx_quantize_cols(x, off_dev)
    G = len(sizes)
    dW = mx.mx_grouped_gemm_wgrad(A, As, B, Bs, P, dW=nan_filled((G, N, K)))
    torch.cuda.synchronize()
    Aq, Asc, Pr = assert_cols_are_oracle(dy, off, A, As, P)
    Bq, Bsc, _ = assert_cols_are_oracle(x, off, B, Bs)
    gs = rng.integers(0, G, 3000)
    ns = rng.integers(0, N, 3000)
    ks = rng.integers(0, K, 3000)
    ref = oracle.wgrad_points(Aq, Asc, Bq, Bsc, Pr, gs, ns, ks)
    got = bf16_to_f64(dW)[gs, ns, ks]
    ok, ratio = gemm_tolerance_ok(got, ref)
    assert ok, ratio
    empty = [g for g in range(G) if sizes[g] == 0]
    assert torch.count_nonzero(dW[empty].float()).item() == 0


def test_gemm_4096_groups():
    """The largest group count: 4096 experts, most of them empty, a few with
    1-300 rows; every output row of a group checked at sampled columns."""
    rng = np.random.default_rng(22)
    G, N, K = 4096, 128, 256
    sizes = np.zeros(G, np.int64)
    busy = rng.choice(G, 40, replace=False)
    sizes[busy] = rng.integers(1, 300, 40)
    M = int(sizes.sum())
    off = W.offsets_from_sizes(list(sizes))
    x = W.normal_bf16((M, K), 1.0, 33, DEV)
    w = W.normal_bf16((G, N, K), 0.02, 34, DEV)
    Xq, Xs, Wq, Ws, host = quantize_pair(x, w)
    out = mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, torch.from_numpy(off).to(DEV), out=nan_filled((M, N)))
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item()
    rows = np.arange(M)
    cols = rng.integers(0, N, M)
    ref = oracle.grouped_gemm_points(*host, off, rows, cols)
    ok, ratio = gemm_tolerance_ok(bf16_to_f64(out)[rows, cols], ref)
    assert ok, ratio
