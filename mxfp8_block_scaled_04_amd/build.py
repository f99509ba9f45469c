"""Build libmxmoe.so (the HIP kernels and the C ABI) for gfx950, in-tree,
and its debug twin libmxmoe_debug.so (the same sources with MXMOE_DEBUG:
device-side contract checks, read by mx_debug_flags).

    python -m mxfp8_block_scaled_04_amd.build

Each source is compiled to an object under _build/ (debug objects under
_build/debug/), in parallel, then linked.  Always rebuilds.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmxmoe.so")
DEBUG_LIB = os.path.join(HERE, "libmxmoe_debug.so")
SOURCES = ["api.cpp", "quantize.hip", "quantize_dual.hip", "grouped_gemm.hip", "swiglu_backward.hip", "stream.hip", "offsets.hip", "probe.hip",
           "swiglu_backward_quant.hip", "routing.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU ops are disabled for every HIP source (plain float code
# only; no v_pk_*_f32).
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall",
]


def _compile(src, debug=False):
    out = os.path.join(BUILD, "debug") if debug else BUILD
    obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + (["-DMXMOE_DEBUG=1"] if debug else []) + ["-x", "hip", "-c", os.path.join(CSRC, src),
                                                                     "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build():
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + [(src, True) for src in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], DEBUG_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
