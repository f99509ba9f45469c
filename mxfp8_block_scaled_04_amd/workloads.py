"""Seeded synthetic inputs for the five workloads (no quantization or GEMM
arithmetic here: only shapes, value distributions and routing).

The public write-ups give no tensor shapes or data; these workloads stand in
for the "typical MoE GEMM" and the quantize-bandwidth benchmark they describe
(aigc.bar "被忽视的量化税"; lpnh.cn 2479732 sections 1 and 4).  The MoE shapes
use hidden size 7168 and expert width 2048 (the Kimi-2.5 shape named on the
kucoin.com MoK page), 4096 tokens x top-8 routed rows.

All randomness comes from numpy PCG64 (routing) and torch.Generator (tensor
values) seeded by the caller; bf16 values are the round-to-nearest-even
conversion of float32 samples.
"""
import numpy as np
import torch

HIDDEN = 7168
EXPERT_DIM = 2048


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, std, seed, device):
    g = _gen(seed, device)
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(0.0, std, generator=g)
    return x.to(torch.bfloat16)


def offsets_from_sizes(sizes):
    return np.concatenate([[0], np.cumsum(np.asarray(sizes, dtype=np.int64))]).astype(np.int32)


# ---------------------------------------------------------------- routing


def dirichlet_sizes(total, experts, alpha, seed):
    """Group sizes ~ multinomial(total, Dirichlet(alpha * 1))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    p = rng.dirichlet(np.full(experts, alpha))
    return rng.multinomial(total, p).astype(np.int64)


def zipf_sizes(total, experts, s, seed, n_empty=8, n_tiny=8):
    """Group sizes ~ multinomial(total, p), p proportional to rank^-s over a
    seeded permutation of the experts; then n_empty seeded experts are forced
    to 0 rows and n_tiny others to U{1..31} rows, the difference going to the
    largest group (so that empty and 1-31-row groups are always present)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ranks = rng.permutation(experts) + 1
    p = ranks.astype(np.float64) ** (-s)
    p /= p.sum()
    sizes = rng.multinomial(total, p).astype(np.int64)
    order = rng.permutation(experts)
    biggest = int(np.argmax(sizes))
    order = order[order != biggest]
    for e in order[:n_empty]:
        sizes[e] = 0
    for e in order[n_empty:n_empty + n_tiny]:
        sizes[e] = int(rng.integers(1, 32))
    sizes[biggest] += total - int(sizes.sum())
    assert sizes.sum() == total and sizes.min() >= 0
    return sizes


def topk_routing(tokens, k, experts, alpha, seed):
    """Top-k routing of `tokens` tokens to k distinct experts each: expert
    popularity p ~ Dirichlet(alpha * 1), each token's experts drawn from p
    without replacement; routing weights U(0, 1) normalized to sum to 1 per
    token.  Returns (experts int32 [tokens, k], weights float32 [tokens, k])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    p = rng.dirichlet(np.full(experts, alpha))
    e = np.stack([rng.choice(experts, k, replace=False, p=p) for _ in range(tokens)]) if tokens else \
        np.zeros((0, k), np.int64)
    w = rng.uniform(0.0, 1.0, (tokens, k))
    w /= np.maximum(w.sum(axis=1, keepdims=True), 1e-30)
    return e.astype(np.int32), w.astype(np.float32)


# ---------------------------------------------------------------- workloads


def tiny_moe(seed=0, device="cpu"):
    """Tiny MoE GEMM: X bf16 [512, 256] with rows N(0,1) * 2^U(-8,8), one
    all-zero block (row 0, k 0..31), one block of bf16 subnormals (row 200,
    k 32..63, random nonzero mantissa and sign), one 1e4 outlier (row 300,
    k 100); 4 experts with group sizes [160, 0, 96, 256]; W bf16
    [4, 128, 256] ~ N(0, 0.02)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    M, K, N, G = 512, 256, 128, 4
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= np.exp2(rng.uniform(-8, 8, (M, 1))).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16).copy()
    bits[0, 0:32] = 0
    mant = rng.integers(1, 128, 32).astype(np.uint16)
    sign = (rng.integers(0, 2, 32).astype(np.uint16) << 15).astype(np.uint16)
    bits[200, 32:64] = mant | sign
    bits[300, 100] = 0x461C  # bf16(1e4) = 9984
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    w = normal_bf16((G, N, K), 0.02, seed + 1, "cpu")
    sizes = np.array([160, 0, 96, 256], np.int64)
    return dict(x=x.to(device), w=w.to(device), sizes=sizes, offsets=offsets_from_sizes(sizes), M=M, N=N, K=K, G=G)


def quant_bandwidth(seed=0, device="cuda", M=131072, K=HIDDEN):
    """bf16 [131072, 7168] ~ N(0,1) with floor(0.001 * numel) positions,
    chosen without replacement, multiplied by 100 (heavy-tailed outliers)."""
    g = _gen(seed, device)
    x = torch.empty((M, K), dtype=torch.float32, device=device)
    x.normal_(0.0, 1.0, generator=g)
    n_out = (M * K) // 1000
    idx = torch.randperm(M * K, generator=g, device=device)[:n_out]
    x.view(-1)[idx] *= 100.0
    del idx
    return x.to(torch.bfloat16)


def moe_gate_up(seed=0, device="cuda", M=32768, K=HIDDEN, N=2 * EXPERT_DIM, G=16):
    """Forward gate+up projection: 32768 routed rows (4096 tokens x top-8),
    K = 7168, N = 4096 (fused 2 x 2048), 16 local experts, group sizes
    multinomial over Dirichlet(0.5) expert probabilities; X ~ N(0,1),
    W ~ N(0, 0.02)."""
    sizes = dirichlet_sizes(M, G, 0.5, seed)
    x = normal_bf16((M, K), 1.0, seed + 1, device)
    w = normal_bf16((G, N, K), 0.02, seed + 2, device)
    return dict(x=x, w=w, sizes=sizes, offsets=offsets_from_sizes(sizes), M=M, N=N, K=K, G=G)


def moe_down_backward(seed=0, device="cuda", M=32768, K=EXPERT_DIM, N=HIDDEN, G=16):
    """Down projection + backward with the same routing as the gate+up case:
    X [32768, 2048], W [16, 7168, 2048], dY [32768, 7168] ~ N(0, 1)."""
    sizes = dirichlet_sizes(M, G, 0.5, seed)
    x = normal_bf16((M, K), 1.0, seed + 1, device)
    w = normal_bf16((G, N, K), 0.02, seed + 2, device)
    dy = normal_bf16((M, N), 1.0, seed + 3, device)
    return dict(x=x, w=w, dy=dy, sizes=sizes, offsets=offsets_from_sizes(sizes), M=M, N=N, K=K, G=G)


def moe_ragged(seed=0, device="cuda", M=65536, K=HIDDEN, N=EXPERT_DIM, G=128):
    """Ragged stress case: 128 experts over 65536 rows, Zipf(1.2) sizes with
    forced empty and 1-31-row groups; X ~ N(0,1), W [128, 2048, 7168] ~
    N(0, 0.02); the dense twin is one W [2048, 7168] with the same M, K, N."""
    sizes = zipf_sizes(M, G, 1.2, seed)
    x = normal_bf16((M, K), 1.0, seed + 1, device)
    w = normal_bf16((G, N, K), 0.02, seed + 2, device)
    w_dense = normal_bf16((1, N, K), 0.02, seed + 3, device)
    return dict(x=x, w=w, w_dense=w_dense, sizes=sizes, offsets=offsets_from_sizes(sizes), M=M, N=N, K=K, G=G)


# ---------------------------------------------------------------- samples


def gemm_sample(M, N, offsets, seed, tile=128, n_random=4096):
    """Output points of a grouped GEMM [M, N] at which the fp64 oracle is
    evaluated on the large workloads (parity checks and the CPU-baseline
    timing share it):
      * one tile x tile output tile per non-empty group, at a seeded position
        inside the group (row start a multiple of `tile` from the group's
        first row, column start a multiple of `tile`), clipped to the group
        and to N;
      * n_random seeded uniform (m, n) pairs;
      * every output element of the groups with fewer than 32 rows;
      * the last row of every non-empty group at its first and last column.
    Returns (rows, cols) int64 arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = [rng.integers(0, M, n_random)]
    cols = [rng.integers(0, N, n_random)]
    G = len(offsets) - 1
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi <= lo:
            continue
        r0 = lo + tile * int(rng.integers(0, -(-(hi - lo) // tile)))
        c0 = tile * int(rng.integers(0, -(-N // tile)))
        r = np.arange(r0, min(r0 + tile, hi))
        c = np.arange(c0, min(c0 + tile, N))
        rows.append(np.repeat(r, c.size))
        cols.append(np.tile(c, r.size))
        if hi - lo < 32:
            r = np.arange(lo, hi)
            rows.append(np.repeat(r, N))
            cols.append(np.tile(np.arange(N), r.size))
        rows.append(np.array([hi - 1, hi - 1]))
        cols.append(np.array([0, N - 1]))
    return np.concatenate(rows).astype(np.int64), np.concatenate(cols).astype(np.int64)
