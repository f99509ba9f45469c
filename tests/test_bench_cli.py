"""bench.py's command line on the CPU: more than one GPU is refused with a
message before anything touches a GPU, and the host-side helpers that the
benchmark line is built from behave as documented."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_flags():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--no-gemm", "--no-layer", "--no-routed", "--no-plain-layer", "--no-cpu",
                 "--gemm-cases", "--copy-calibration"):
        assert flag in r.stdout, flag


def test_algorithmic_bytes_and_profile_digests():
    M, K = 131072, 7168
    assert bench.quant_bytes(M, K) == 2 * M * K + M * K + M * K // 32 == 2847932416
    for name, srcs in bench.KERNEL_SOURCES.items():
        d = bench.source_digest(*srcs)
        assert len(d) == 16 and int(d, 16) >= 0, name
    # a profile taken on other sources is not used
    assert bench.read_profile("quantize_cols_kernel_trace", "0" * 16) is None
    # the committed summaries that the benchmark line quotes were taken on the current sources
    for name, key in (("quantize_cols_kernel_trace", "quantize"), ("quantize_rows_kernel_pmc", "quantize"),
                      ("quantize_dual_kernel_trace", "quantize_dual"), ("grouped_gemm_gate_up_trace", "grouped_gemm"),
                      ("grouped_gemm_gate_up_pmc", "grouped_gemm")):
        prof = bench.read_profile(name, bench.source_digest(*bench.KERNEL_SOURCES[key]))
        assert prof is not None, f"profiles/{name}.txt was taken on other sources"
