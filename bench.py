#!/usr/bin/env python3
"""Benchmark of the MXFP8 hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--seed S] [--no-gemm] [--no-layer] [--no-layer-unfused]
                    [--no-routed] [--no-plain-layer] [--no-cpu]
                    [--gemm-cases gate_up,swiglu,ragged,down] [--copy-calibration]

Prints ONE JSON line.  The headline (``value``) is the quantize bandwidth on
the quantize-only workload, bf16 [131072, 7168] ~ N(0,1) with 0.1 % of the
elements scaled by 100: one step = one row-wise pass + one column-wise
(transposed) pass, each writing fp8 codes and packed E8M0 scales.
Throughput = algorithmic bytes (2 B read + 1 B + 1/32 B written per element,
per pass; the byte count of the lpnh.cn 2479732 section 4 benchmark with bf16
input) / GPU time, inputs resident in HBM.

``quantize_dual`` times the dual-layout quantize on the same input (one read,
row-wise and column-wise results: 2 B read + 2 x (1 + 1/32) B written per
element) next to the two separate passes.

The ``gemm`` object times the grouped GEMMs on the MoE workloads (TFLOP/s =
2 M N K over real rows / GPU time): gate+up (32768 x 7168 -> 4096, 16 experts),
the same with the quantizing SwiGLU epilogue (MXFP8 [32768, 2048] out), the
ragged 128-expert case next to the dense GEMM of the same size, and the down
projection forward / dgrad / wgrad.

``moe_layer`` runs one MoE layer's expert computation forward + backward on
that routing (quantize, gate+up GEMM with the quantizing SwiGLU epilogue, down
GEMM; then dgrad, the SwiGLU backward fused with the quantization of its
results, wgrad; weights re-quantized each step) and reports each stage's time
and the quantize / GEMM time ratio, next to the same step with the SwiGLU
backward and its quantizations as separate calls.  ``moe_layer_routed`` is one
GPU's share of the expert-parallel layer: 4096 tokens routed top-8 to 16
local experts, with the route plan, the dispatch (gather + MXFP8), the combine
and their backward around the same expert computation.

``roofline`` describes the dominant kernel of the step (its own launch time
from HIP events on the launch stream, next to the average of the committed
rocprofv3 kernel trace and the HBM bytes of the committed counter profile,
both keyed by a hash of the kernel's sources); ``roofline_gemm`` does the
same for the gate+up GEMM, with the MFMA busy fraction and the shader clock
the chip held during it.  Each GEMM case also reports its work decomposition
(256 x 256 tiles, rounds of one tile per CU, row padding).  ``cpu_baseline``
times the CPU oracle on the whole quantize input (and on one thread over a
part of it): a reported baseline, not a target.
"""
import argparse
import concurrent.futures
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_TBS = 8.0          # MI355X HBM3E, TB/s
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense MXFP8 MFMA, TFLOP/s
METRIC = "MXFP8 quantize TB/s; grouped-GEMM TFLOP/s; each as % of HBM/MFMA peak"


def quant_bytes(M, K):
    return 2 * M * K + M * K + M * K // 32


# sources each kernel is built from (its .hip file and the headers it includes)
KERNEL_SOURCES = {
    "quantize": ("quantize.hip", "mx_device.h", "mx_internal.h", "mx_debug.h"),
    "quantize_dual": ("quantize_dual.hip", "mx_bf16.h", "mx_device.h", "mx_internal.h", "mx_debug.h"),
    "grouped_gemm": ("grouped_gemm.hip", "mx_device.h", "mx_internal.h", "mx_debug.h"),
}


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mxfp8_block_scaled_04_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_profile(name, digest):
    """key: value lines of the committed rocprofv3 summary profiles/<name>.txt,
    or None when it is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", name + ".txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != digest:
        return None
    return vals


def profile_float(vals, key):
    try:
        return float(vals[key]) if vals is not None else None
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events on the stream the kernels are launched on."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def run(self, fn, steps):
        self.a.record()
        for _ in range(steps):
            fn()
        self.b.record()
        self.b.synchronize()
        return self.a.elapsed_time(self.b) / steps  # ms per launch


def host_threads():
    """Host threads the oracle may use: the CPUs this process may run on,
    at most 16 (the host CPU share that goes with one GPU of an 8-GPU node)."""
    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:
        visible = os.cpu_count() or 1
    return max(1, min(visible, 16)), visible


def oracle_quantize_pass(oracle, bits, threads):
    """The oracle (as it stands) on bf16 bits [M, K]: the row-wise pass, then
    the column-wise pass (one group; 256-row slabs are independent), each
    split over `threads` host threads (ctypes releases the GIL).  Returns the
    wall time of each pass."""
    import numpy as np

    M = bits.shape[0]
    chunks = [c for c in np.array_split(np.arange(M), threads) if c.size]
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda r: oracle.quantize_rows(bits[r[0]:r[-1] + 1]), chunks))
    t_rows = time.perf_counter() - t0
    slabs = [(i, min(i + 256, M)) for i in range(0, M, 256)]
    groups = [g for g in np.array_split(np.arange(len(slabs)), threads) if g.size]

    def run_cols(gi):
        for i in gi:
            a, b = slabs[i]
            oracle.quantize_cols(bits[a:b])

    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        list(ex.map(run_cols, groups))
    return t_rows, time.perf_counter() - t0


def cpu_baseline(x_bits, seed, one_thread_rows):
    """The CPU oracle on the whole quantize workload (row-wise then
    column-wise pass) over the host threads, plus the same on one thread
    over its first `one_thread_rows` rows; both as algorithmic TB/s."""
    import oracle

    threads, visible = host_threads()
    M, K = x_bits.shape
    t_rows, t_cols = oracle_quantize_pass(oracle, x_bits, threads)
    tbs = 2 * quant_bytes(M, K) / (t_rows + t_cols) / 1e12
    m1 = min(one_thread_rows, M)
    t1r, t1c = oracle_quantize_pass(oracle, x_bits[:m1], 1)
    return {"value": tbs, "unit": "TB/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole quantize workload, {M} x {K} bf16 (seed {seed}): row-wise then column-wise "
                      f"pass on {threads} host threads ({visible} CPUs visible, at most 16 used); "
                      f"{t_rows:.2f} s + {t_cols:.2f} s wall",
            "one_thread": {"value": 2 * quant_bytes(m1, K) / (t1r + t1c) / 1e12, "unit": "TB/s", "cores": 1,
                           "sample": f"first {m1} rows x {K}, row-wise then column-wise pass; "
                                     f"{t1r:.2f} s + {t1c:.2f} s wall"},
            "gemm_oracle": gemm_oracle_rate(seed, threads),
            "gemm_oracle_gate_up": gemm_oracle_gate_up_sample(seed, threads)}


def gemm_oracle_rate(seed, cores):
    """The fp64 grouped-GEMM oracle on the tiny MoE workload in full (33.6
    MFLOP, rows split over host threads), as GFLOP/s."""
    import numpy as np
    import oracle
    from mxfp8_block_scaled_04_amd import workloads as W

    d = W.tiny_moe(seed=seed, device="cpu")
    G, N, K, M = d["G"], d["N"], d["K"], d["M"]
    xb = d["x"].contiguous().view(__import__("torch").int16).numpy().view(np.uint16)
    wb = d["w"].reshape(G * N, K).contiguous().view(__import__("torch").int16).numpy().view(np.uint16)
    Xq, Xs = oracle.quantize_rows(xb)
    Wq, Ws = oracle.quantize_rows(wb)
    Wq, Ws = Wq.reshape(G, N, K), Ws.reshape(G, N, K // 32)
    off = d["offsets"]
    rows = np.arange(M)
    parts = np.array_split(rows, cores)
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(cores) as ex:
        list(ex.map(lambda r: oracle.grouped_gemm_points(Xq, Xs, Wq, Ws, off, np.repeat(r, N),
                                                          np.tile(np.arange(N), len(r))), parts))
    t = time.perf_counter() - t0
    return {"gflops": 2.0 * M * N * K / t / 1e9, "s": t, "cores": cores,
            "sample": f"tiny MoE workload in full: {M} x {N} x {K}, {G} experts (seed {seed})"}


def gemm_oracle_gate_up_sample(seed, cores, device="cuda"):
    """The fp64 grouped-GEMM oracle on a deterministic sample of the gate+up
    workload (32768 x 4096 x 7168, 16 experts): a 128 x 128 output patch at
    the start of every non-empty group (clipped to the group) plus 4096
    uniform points.  The oracle quantizes the bf16 operands first (not
    timed); the points are split over host threads.  Reported as GFLOP/s of
    the sample and the full GEMM's time extrapolated at that rate."""
    import numpy as np
    import torch
    import oracle
    from mxfp8_block_scaled_04_amd import workloads as W

    d = W.moe_gate_up(seed=seed, device=device)
    G, N, K, M = d["G"], d["N"], d["K"], d["M"]
    off = d["offsets"]

    def host_bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    xb = host_bits(d["x"])
    wb = host_bits(d["w"].reshape(G * N, K))
    del d

    def quant_all(bits):
        parts = np.array_split(np.arange(bits.shape[0]), cores)
        with concurrent.futures.ThreadPoolExecutor(cores) as ex:
            res = list(ex.map(lambda r: oracle.quantize_rows(bits[r[0]:r[-1] + 1]), parts))
        return np.concatenate([q for q, _ in res]), np.concatenate([s for _, s in res])

    Xq, Xs = quant_all(xb)
    del xb
    Wq, Ws = quant_all(wb)
    del wb
    Wq, Ws = Wq.reshape(G, N, K), Ws.reshape(G, N, K // 32)
    rows, cols = W.gemm_sample(M, N, off, seed)
    parts = np.array_split(np.arange(rows.size), cores)
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(cores) as ex:
        list(ex.map(lambda p: oracle.grouped_gemm_points(Xq, Xs, Wq, Ws, off, rows[p], cols[p]), parts))
    t = time.perf_counter() - t0
    rate = 2.0 * rows.size * K / t
    return {"gflops": rate / 1e9, "s": t, "cores": cores, "points": int(rows.size),
            "extrapolated_full_s": 2.0 * M * N * K / rate,
            "sample": f"gate+up workload {M} x {N} x {K}, {G} experts (seed {seed}): a 128 x 128 tile per "
                      f"non-empty group + 4096 uniform points + every element of the groups below 32 rows "
                      f"(the parity tests' sample); full-size time extrapolated, not measured"}


def launch_stats(torch, fn, n):
    """Median / min / max of n launches, one event pair each."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    evs[-1][1].synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    return {"median": ts[len(ts) // 2], "min": ts[0], "max": ts[-1], "n": n}


def bench_quant(torch, mx, W, args):
    x = W.quant_bandwidth(seed=args.seed, device="cuda")
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty(mx.mx_scale_bytes(M, K), dtype=torch.uint8, device="cuda")
    Mcap = mx.mx_cols_capacity(M, 1)
    qT = torch.empty((K, Mcap), dtype=torch.uint8, device="cuda")
    sT = torch.empty(mx.mx_scale_bytes(K, Mcap), dtype=torch.uint8, device="cuda")

    def rows():
        mx.mx_quantize_rows(x, q, s)

    def cols():
        mx.mx_quantize_cols(x, None, Mcap, qT, sT)

    def dual():
        mx.mx_quantize_dual(x, None, Mcap, q, s, qT, sT)

    for _ in range(args.warmup):
        rows()
        cols()
        dual()
    torch.cuda.synchronize()
    tm = Timer(torch)
    t0 = time.perf_counter()
    ms_rows = tm.run(rows, args.steps)
    ms_cols = tm.run(cols, args.steps)
    ms_dual = tm.run(dual, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-launch spread (an event pair around each launch)
    spread = {name: launch_stats(torch, fn, args.steps) for name, fn in (("rows", rows), ("cols", cols))}
    # measured streaming ceiling: mx_stream21 reads the whole input and
    # writes half its bytes (the quantizers' 2:1 ratio, no arithmetic)
    flat = x.view(-1).view(torch.uint8)
    dst = torch.empty(flat.numel() // 2, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        mx.mx_stream21(flat, dst)
    ms_copy = tm.run(lambda: mx.mx_stream21(flat, dst), args.steps)
    copy_tbs = (flat.numel() + dst.numel()) / ms_copy / 1e9
    del dst, flat
    nbytes = quant_bytes(M, K)
    dual_bytes = 2 * M * K + 2 * (M * K + M * K // 32)  # one read, both results written
    res = {
        "M": M, "K": K, "ms_rows": ms_rows, "ms_cols": ms_cols, "wall_s": wall,
        "bytes_per_pass": nbytes,
        "tbs_rows": nbytes / ms_rows / 1e9, "tbs_cols": nbytes / ms_cols / 1e9,
        "launch_ms": spread, "copy_tbs": copy_tbs,
        "dual": {"ms": ms_dual, "bytes": dual_bytes, "tbs": dual_bytes / ms_dual / 1e9,
                 "frac_hbm_peak": dual_bytes / ms_dual / 1e9 / HBM_PEAK_TBS,
                 "ms_rows_plus_cols": ms_rows + ms_cols, "speedup_vs_two_passes": (ms_rows + ms_cols) / ms_dual},
    }
    sample = None
    if not args.no_cpu:
        sample = x.cpu().contiguous().view(torch.int16).numpy().view("uint16")
    del x, q, s, qT, sT
    torch.cuda.empty_cache()
    return res, sample


GEMM_CASES = ("gate_up", "swiglu", "ragged", "down")


def tile_stats(torch, sizes, N):
    """Work decomposition of a row-grouped GEMM launch: every group padded to
    whole 256-row tiles, 256-column tiles, one persistent workgroup per CU
    taking one tile per round."""
    import numpy as np

    sizes = np.asarray(sizes, np.int64)
    row_tiles = int(((sizes + 255) // 256).sum())
    tiles = row_tiles * ((N + 255) // 256)
    wgs = min(torch.cuda.get_device_properties(0).multi_processor_count, tiles) if tiles else 0
    return {"row_tiles": row_tiles, "padded_rows_frac": row_tiles * 256 / max(int(sizes.sum()), 1) - 1,
            "tiles": tiles, "workgroups": wgs, "rounds": tiles / wgs if wgs else 0.0,
            "rounds_run": -(-tiles // wgs) if wgs else 0}


def tflops(M, N, K, ms):
    return 2.0 * M * N * K / (ms * 1e-3) / 1e12


def bench_gemm(torch, mx, W, args):
    out = {}
    tm = Timer(torch)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        return tm.run(fn, args.steps)

    cases = set(args.gemm_cases.split(","))
    unknown = cases - set(GEMM_CASES)
    if unknown:
        raise SystemExit(f"bench.py: unknown GEMM case(s) {sorted(unknown)}; choose from {GEMM_CASES}")
    if cases & {"gate_up", "swiglu"}:
        gate_up_cases(torch, mx, W, args, timed, cases, out)
    if "ragged" in cases:
        ragged_case(torch, mx, W, args, timed, out)
    if "down" in cases:
        down_case(torch, mx, W, args, timed, out)
    return out


def gate_up_cases(torch, mx, W, args, timed, cases, out):
    # gate+up projection, 16 experts
    d = W.moe_gate_up(seed=args.seed, device="cuda")
    G, N, K = d["G"], d["N"], d["K"]
    Xq, Xs = mx.mx_quantize_rows(d["x"])
    Wq, Ws = mx.mx_quantize_rows(d["w"].reshape(G * N, K))
    Wq = Wq.reshape(G, N, K)
    off = torch.from_numpy(d["offsets"]).to("cuda")
    ms = None
    if "gate_up" in cases:
        y = torch.empty((d["M"], N), dtype=torch.bfloat16, device="cuda")
        ms = timed(lambda: mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, off, out=y))
        qx = timed(lambda: mx.mx_quantize_rows(d["x"], Xq, Xs))
        out["gate_up"] = {"M": d["M"], "N": N, "K": K, "G": G, "ms": ms, "tflops": tflops(d["M"], N, K, ms),
                          "frac_mfma_peak": tflops(d["M"], N, K, ms) / MFMA_FP8_PEAK_TFLOPS,
                          "quantize_x_ms": qx, "quantize_over_gemm": qx / ms,
                          "work": tile_stats(torch, d["sizes"], N)}
        del y
    del Wq, Ws
    torch.cuda.empty_cache()
    if "swiglu" not in cases:
        return

    # the same projection with the quantizing SwiGLU epilogue: h = silu(gate) up
    # as MXFP8 [M, N/2] + scales instead of bf16 [M, N]
    I = N // 2
    Wi, Wis = mx.mx_quantize_rows(mx.swiglu_interleave(d["w"]).reshape(G * N, K))
    Wi = Wi.reshape(G, N, K)
    hq = torch.empty((d["M"], I), dtype=torch.uint8, device="cuda")
    hs = torch.empty(mx.mx_scale_bytes(d["M"], I), dtype=torch.uint8, device="cuda")
    ms_sw = timed(lambda: mx.mx_grouped_gemm_swiglu(Xq, Xs, Wi, Wis, off, hq=hq, hs=hs))
    out["gate_up_swiglu"] = {
        "M": d["M"], "N": N, "K": K, "G": G, "ms": ms_sw, "tflops": tflops(d["M"], N, K, ms_sw),
        "frac_mfma_peak": tflops(d["M"], N, K, ms_sw) / MFMA_FP8_PEAK_TFLOPS,
        "over_bf16_gemm": None if ms is None else ms_sw / ms,
        # bytes of the activation written by the fused kernel, and those of
        # the unfused route (bf16 [M, N] written, read back, codes + scales written)
        "bytes_out_fused": d["M"] * I * (1 + 1 / 32),
        "bytes_unfused": d["M"] * N * 2 * 2 + d["M"] * I * (1 + 1 / 32),
    }
    del d, Xq, Xs, Wi, Wis, hq, hs
    torch.cuda.empty_cache()


def ragged_case(torch, mx, W, args, timed, out):
    # ragged 128 experts vs dense
    d = W.moe_ragged(seed=args.seed, device="cuda")
    G, N, K, M = d["G"], d["N"], d["K"], d["M"]
    Xq, Xs = mx.mx_quantize_rows(d["x"])
    Wq, Ws = mx.mx_quantize_rows(d["w"].reshape(G * N, K))
    Wq = Wq.reshape(G, N, K)
    Dq, Ds = mx.mx_quantize_rows(d["w_dense"].reshape(N, K))
    Dq = Dq.reshape(1, N, K)
    off = torch.from_numpy(d["offsets"]).to("cuda")
    off1 = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ms_g = timed(lambda: mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, off, out=y))
    ms_d = timed(lambda: mx.mx_grouped_gemm(Xq, Xs, Dq, Ds, off1, out=y))
    # roofline of this shape: the larger of the MFMA time and the time to
    # stream the fp8 weights once (the case sits near the ridge point)
    roof_ms = max(2.0 * M * N * K / (MFMA_FP8_PEAK_TFLOPS * 1e12), G * N * K * (1 + 1 / 32) / (HBM_PEAK_TBS * 1e12)) * 1e3
    out["ragged"] = {"M": M, "N": N, "K": K, "G": G, "ms_grouped": ms_g, "ms_dense": ms_d,
                     "roofline_ms": roof_ms, "frac_roofline_grouped": roof_ms / ms_g,
                     "tflops_grouped": tflops(M, N, K, ms_g), "tflops_dense": tflops(M, N, K, ms_d),
                     "grouped_over_dense": ms_g / ms_d,
                     "frac_mfma_peak_grouped": tflops(M, N, K, ms_g) / MFMA_FP8_PEAK_TFLOPS,
                     "work_grouped": tile_stats(torch, d["sizes"], N), "work_dense": tile_stats(torch, [M], N)}
    del d, Xq, Xs, Wq, Ws, Dq, Ds, y
    torch.cuda.empty_cache()


def down_case(torch, mx, W, args, timed, out):
    # down projection forward / dgrad / wgrad
    d = W.moe_down_backward(seed=args.seed, device="cuda")
    G, N, K, M = d["G"], d["N"], d["K"], d["M"]
    off = torch.from_numpy(d["offsets"]).to("cuda")
    Xq, Xs = mx.mx_quantize_rows(d["x"])
    Wq, Ws = mx.mx_quantize_rows(d["w"].reshape(G * N, K))
    Wq = Wq.reshape(G, N, K)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ms_f = timed(lambda: mx.mx_grouped_gemm(Xq, Xs, Wq, Ws, off, out=y))
    dyq, dys = mx.mx_quantize_rows(d["dy"])
    woff = torch.arange(0, G + 1, dtype=torch.int32, device="cuda") * N
    wT, wTs, _ = mx.mx_quantize_cols(d["w"].reshape(G * N, K), woff)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    ms_dg = timed(lambda: mx.mx_grouped_gemm_dgrad(dyq, dys, wT, wTs, off, G, out=dx))
    A, As, P = mx.mx_quantize_cols(d["dy"], off)
    B, Bs, _ = mx.mx_quantize_cols(d["x"], off)
    dW = torch.empty((G, N, K), dtype=torch.bfloat16, device="cuda")
    ms_wg = timed(lambda: mx.mx_grouped_gemm_wgrad(A, As, B, Bs, P, dW=dW))
    ms_qc = timed(lambda: mx.mx_quantize_cols(d["dy"], off, A.shape[1], A, As, P))
    out["down_backward"] = {
        "M": M, "N": N, "K": K, "G": G,
        "ms_fwd": ms_f, "tflops_fwd": tflops(M, N, K, ms_f), "work_fwd": tile_stats(torch, d["sizes"], N),
        "ms_dgrad": ms_dg, "tflops_dgrad": tflops(M, K, N, ms_dg),
        "ms_wgrad": ms_wg, "tflops_wgrad": tflops(N, K, M, ms_wg),
        "quantize_cols_dy_ms": ms_qc,
    }
    del d
    torch.cuda.empty_cache()


def bench_layer(torch, mx, W, args):
    """One MoE layer's expert computation, forward + backward, on the gate+up /
    down workloads' routing (32768 rows, H 7168, I 2048, 16 experts): per-stage
    GPU time from events recorded between the calls, averaged over the timed
    steps, plus the step total timed without them, eagerly and replayed from a
    HIP graph.  The layer runs with its fused SwiGLU backward + quantization;
    the step with its independent calls on two streams (``two_streams``) and
    the step with the SwiGLU backward unfused are timed after it for
    comparison."""
    from mxfp8_block_scaled_04_amd.moe_layer import KIND, MoELayer

    d1 = W.moe_gate_up(seed=args.seed, device="cuda")
    d2 = W.moe_down_backward(seed=args.seed, device="cuda")
    assert (d1["offsets"] == d2["offsets"]).all()
    M, H, I = d1["M"], d1["K"], d1["N"] // 2
    X, dY = d1["x"], d2["dy"]
    W1 = mx.swiglu_interleave(d1["w"])
    W2 = d2["w"]
    off = torch.from_numpy(d1["offsets"]).to("cuda")
    del d1, d2
    torch.cuda.empty_cache()
    tm = Timer(torch)

    def run(fuse):
        layer = MoELayer(off, M, H, I, fuse_swiglu_backward=fuse)
        step = lambda mark=None: layer.step(X, dY, W1, W2, mark)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        names, events = [], []

        def mark(name):
            ev = torch.cuda.Event(enable_timing=True)
            ev.record()
            names.append(name)
            events.append(ev)

        stage = {}
        for _ in range(args.steps):
            names.clear()
            events.clear()
            mark("start")
            step(mark)
            events[-1].synchronize()
            for i in range(1, len(events)):
                stage[names[i]] = stage.get(names[i], 0.0) + events[i - 1].elapsed_time(events[i]) / args.steps
        ms_step = tm.run(step, args.steps)
        # the same step recorded once as a HIP graph and replayed (every call
        # it makes only launches kernels on the current stream)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        ms_graph = tm.run(graph.replay, args.steps)
        del graph
        overlapped = None
        if fuse:
            # the same step with its independent calls on two streams
            ovl = lambda: layer.step_overlapped(X, dY, W1, W2)
            for _ in range(args.warmup):
                ovl()
            torch.cuda.synchronize()
            ms_ovl = tm.run(ovl, args.steps)
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                ovl()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                ovl()
            torch.cuda.synchronize()
            overlapped = {"ms_step": ms_ovl, "ms_step_graph": tm.run(graph.replay, args.steps)}
            del graph
        flops, G = layer.flops(), layer.G
        del layer
        torch.cuda.empty_cache()
        return stage, ms_step, ms_graph, flops, G, overlapped

    stage, ms_step, ms_graph, flops, G, overlapped = run(True)
    unfused = None
    if not args.no_layer_unfused:
        stage_u, ms_step_u, ms_graph_u, _, _, _ = run(False)
        unfused = {"ms_step": ms_step_u, "ms_step_graph": ms_graph_u, "ms_by_stage": stage_u}
    kinds = {}
    for n, ms in stage.items():
        kinds[KIND[n]] = kinds.get(KIND[n], 0.0) + ms
    # quantization of activations and gradients, the fused SwiGLU backward
    # stage included (its elementwise work is counted with it)
    quant_act = sum(ms for n, ms in stage.items() if KIND[n] == "quant" and not n.startswith("W"))
    out = {
        "workload": f"MoE layer fwd+bwd, M {M}, H {H}, I {I}, {G} experts (Dirichlet(0.5) routing)",
        "ms_step": ms_step, "tflops": flops / (ms_step * 1e-3) / 1e12, "ms_step_graph": ms_graph,
        "ms_by_kind": kinds, "ms_by_stage": stage,
        "quant_activations_ms": quant_act,
        "quant_activations_over_gemm": quant_act / kinds["gemm"],
        "quant_all_over_gemm": kinds["quant"] / kinds["gemm"],
        "two_streams": overlapped,
        "unfused_swiglu_backward": unfused,
    }
    del X, dY, W1, W2
    torch.cuda.empty_cache()
    return out


def bench_routed(torch, mx, W, args):
    """One GPU's share of an expert-parallel MoE layer: 4096 tokens routed
    top-8 to 16 local experts (Dirichlet(0.5) expert popularity), H 7168,
    I 2048; route plan, dispatch (gather + MXFP8), the expert computation,
    combine, and their backward.  Per-stage GPU time from events between the
    calls, the step timed without them, eagerly and as a HIP graph, and the
    HBM rates of the dispatch and combine kernels (algorithmic bytes)."""
    from mxfp8_block_scaled_04_amd.moe_layer import KIND, RoutedMoELayer

    T, k, G, H, I = 4096, 8, 16, 7168, 2048
    e, w = W.topk_routing(T, k, G, 0.5, args.seed)
    ed, wd = torch.from_numpy(e).to("cuda"), torch.from_numpy(w).to("cuda")
    X = W.normal_bf16((T, H), 1.0, args.seed + 101, "cuda")
    dOut = W.normal_bf16((T, H), 1.0, args.seed + 102, "cuda")
    W1 = mx.swiglu_interleave(W.normal_bf16((G, 2 * I, H), 0.02, args.seed + 103, "cuda"))
    W2 = W.normal_bf16((G, H, I), 0.02, args.seed + 104, "cuda")
    R = RoutedMoELayer(T, k, G, H, I)
    step = lambda mark=None: R.step(X, dOut, ed, wd, W1, W2, mark)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    names, events = [], []

    def mark(name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        names.append(name)
        events.append(ev)

    stage = {}
    for _ in range(args.steps):
        names.clear()
        events.clear()
        mark("start")
        step(mark)
        events[-1].synchronize()
        for i in range(1, len(events)):
            stage[names[i]] = stage.get(names[i], 0.0) + events[i - 1].elapsed_time(events[i]) / args.steps
    tm = Timer(torch)
    ms_step = tm.run(step, args.steps)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    ms_graph = tm.run(graph.replay, args.steps)
    del graph
    M = T * k
    # algorithmic HBM bytes: the gathered quantization reads M bf16 rows and
    # writes both layouts (2 x (1 + 1/32) B per element); the combine reads
    # the k expert rows of every token and writes its bf16 row
    quant_bytes_ = 2 * M * H + 2 * M * H * (1 + 1 / 32)
    comb_y_bytes = 2 * M * H + 2 * T * H
    comb_dx_bytes = 2 * M * H + 2 * T * H
    rate = lambda b, ms: b / (ms * 1e-3) / 1e12
    kinds = {}
    for n, ms in stage.items():
        kinds[KIND[n]] = kinds.get(KIND[n], 0.0) + ms
    out = {
        "workload": f"routed MoE layer fwd+bwd, {T} tokens top-{k} of {G} local experts (Dirichlet(0.5) "
                    f"popularity), H {H}, I {I}: {M} routed rows",
        "ms_step": ms_step, "ms_step_graph": ms_graph, "tflops": R.flops() / (ms_step * 1e-3) / 1e12,
        "ms_by_kind": kinds, "ms_by_stage": stage,
        "tbs": {
            "dispatch + quantize X": rate(quant_bytes_, stage["D dispatch + quantize X"]),
            "reverse combine + quantize dOut": rate(quant_bytes_, stage["C' reverse combine + quantize dOut"]),
            "combine": rate(comb_y_bytes, stage["C combine"]),
            "reverse dispatch": rate(comb_dx_bytes, stage["D' reverse dispatch"]),
        },
        "tbs_note": "algorithmic bytes / stage time (the stage includes the launch gaps around its kernels); "
                    "frac_hbm_peak divides by 8 TB/s",
    }
    out["frac_hbm_peak"] = {n: v / HBM_PEAK_TBS for n, v in out["tbs"].items()}
    del R, X, dOut, W1, W2
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-gemm", action="store_true", help="skip the grouped-GEMM section")
    ap.add_argument("--no-layer", action="store_true", help="skip the MoE-layer chain")
    ap.add_argument("--no-routed", action="store_true", help="skip the routed MoE layer (dispatch and combine)")
    ap.add_argument("--no-plain-layer", action="store_true",
                    help="skip the MoE layer on pre-grouped rows (the routed layer still runs)")
    ap.add_argument("--no-layer-unfused", action="store_true",
                    help="skip the comparison step of the MoE layer with the SwiGLU backward unfused")
    ap.add_argument("--gemm-cases", default=",".join(GEMM_CASES),
                    help="comma-separated subset of the GEMM section's workloads to run (%(default)s); "
                         "a profiler run of one case sees only its dispatches")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows-1t", type=int, default=8192,
                    help="rows of the one-thread oracle figure (the threaded figure runs the whole input)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (read 1 GiB, write 1 GiB) a few times, "
                         "so that HBM counters can be scaled against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding over several GPUs is a design note, not code", file=sys.stderr)
        sys.exit(2)

    import torch
    import mxfp8_block_scaled_04_amd as mx
    from mxfp8_block_scaled_04_amd import workloads as W

    mx.load()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    quant, sample = bench_quant(torch, mx, W, args)
    gemm = None if args.no_gemm else bench_gemm(torch, mx, W, args)
    layer = None if args.no_layer or args.no_plain_layer else bench_layer(torch, mx, W, args)
    routed = None if args.no_layer or args.no_routed else bench_routed(torch, mx, W, args)
    cpu = None if sample is None else cpu_baseline(sample, args.seed, args.cpu_rows_1t)

    ms_step = quant["ms_rows"] + quant["ms_cols"]
    value = 2 * quant["bytes_per_pass"] / (ms_step * 1e-3) / 1e12
    kname = "quantize_cols_kernel" if quant["ms_cols"] >= quant["ms_rows"] else "quantize_rows_kernel"
    dom_ms = max(quant["ms_rows"], quant["ms_cols"])
    achieved = quant["bytes_per_pass"] / (dom_ms * 1e-3) / 1e9  # GB/s
    qdigest = source_digest(*KERNEL_SOURCES["quantize"])
    pmc = read_profile(kname + "_pmc", qdigest)
    trace = read_profile(kname + "_trace", qdigest)
    trace_us = profile_float(trace, "avg_us")
    roofline = {
        "bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_TBS * 1000, "unit": "GB/s",
        "frac": achieved / (HBM_PEAK_TBS * 1000), "traffic": profile_float(pmc, "hbm_bytes_per_launch"),
        "algorithmic_bytes_per_launch": quant["bytes_per_pass"],
        "timing": "mean launch time from HIP events on the launch stream over the timed launches of this run",
        "source_sha256": qdigest,
        # the same quantity from the committed rocprofv3 kernel trace (another
        # run of this command on these kernel sources; null if they changed)
        "kernel_trace": None if trace_us is None else {
            "avg_us": trace_us, "achieved": quant["bytes_per_pass"] / (trace_us * 1e-6) / 1e9,
            "frac": quant["bytes_per_pass"] / (trace_us * 1e-6) / 1e9 / (HBM_PEAK_TBS * 1000),
            "file": f"profiles/{kname}_trace.txt"},
    }
    roofline_gemm = None
    if gemm is not None and "gate_up" in gemm:
        gu = gemm["gate_up"]
        flops = 2.0 * gu["M"] * gu["N"] * gu["K"]
        gdigest = source_digest(*KERNEL_SOURCES["grouped_gemm"])
        gpmc = read_profile("grouped_gemm_gate_up_pmc", gdigest)
        gtrace = read_profile("grouped_gemm_gate_up_trace", gdigest)
        gtrace_us = profile_float(gtrace, "avg_us")
        roofline_gemm = {
            "bound": "mfma", "kernel": "grouped_gemm_kernel",
            "workload": f"gate+up {gu['M']} x {gu['N']} x {gu['K']}, {gu['G']} experts",
            "achieved": flops / (gu["ms"] * 1e-3) / 1e12, "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": flops / (gu["ms"] * 1e-3) / 1e12 / MFMA_FP8_PEAK_TFLOPS,
            "traffic": profile_float(gpmc, "hbm_bytes_per_launch"),
            "algorithmic_flops_per_launch": flops,
            "mfma_busy": profile_float(gpmc, "mfma_busy"),
            # the shader clock the chip held during this kernel (GRBM_GUI_ACTIVE
            # cycles per XCD over the dispatch time, from the counter profile):
            # the 5.0 PFLOP/s peak assumes 2.4 GHz
            "clock_ghz": profile_float(gpmc, "clock_ghz"),
            "frac_of_peak_at_clock": None if profile_float(gpmc, "clock_ghz") is None else
            flops / (gu["ms"] * 1e-3) / 1e12 / (MFMA_FP8_PEAK_TFLOPS * profile_float(gpmc, "clock_ghz") / 2.4),
            "timing": "mean launch time from HIP events on the launch stream over the timed launches of this run",
            "source_sha256": gdigest,
            "kernel_trace": None if gtrace_us is None else {
                "avg_us": gtrace_us, "achieved": flops / (gtrace_us * 1e-6) / 1e12,
                "frac": flops / (gtrace_us * 1e-6) / 1e12 / MFMA_FP8_PEAK_TFLOPS,
                "file": "profiles/grouped_gemm_gate_up_trace.txt"},
        }
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->fp8_e4m3+e8m0",
        "data": "synthetic (seeded N(0,1) bf16, 0.1% outliers x100)",
        "config": {"workload": "quantize_bandwidth bf16 [131072, 7168], row-wise + column-wise pass",
                   "seed": args.seed, "frac_hbm_peak": value / HBM_PEAK_TBS,
                   "tbs_rows": quant["tbs_rows"], "tbs_cols": quant["tbs_cols"],
                   "ms_rows": quant["ms_rows"], "ms_cols": quant["ms_cols"],
                   "launch_ms": quant["launch_ms"], "copy_tbs_measured": quant["copy_tbs"],
                   "frac_copy_ceiling": value / quant["copy_tbs"]},
        "roofline": roofline,
        "roofline_gemm": roofline_gemm,
        "cpu_baseline": cpu,
        "quantize_dual": dict(quant["dual"], workload="bf16 [131072, 7168] -> row-wise + column-wise MXFP8, one read"),
        "gemm": gemm,
        "moe_layer": layer,
        "moe_layer_routed": routed,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
