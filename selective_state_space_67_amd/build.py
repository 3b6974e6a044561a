"""Build libssmscan.so for gfx950 with hipcc, in place (next to this file).

Usage: python -m selective_state_space_67_amd.build [--verbose]
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.cpp", "scan_fwd.hip", "scan_fwd_f32_plain.hip", "scan_fwd_f32_reset.hip", "scan_fwd_bf16_plain.hip",
           "scan_fwd_bf16_reset.hip", "scan_fwd_n16.hip", "scan_fwd_wavefront.hip", "scan_bwd.hip", "state_update.hip",
           "scan_cplx.hip", "scan_cplx_bwd.hip", "fill.hip", "scan_noalloc.hip", "log.cpp"]
OUT = os.path.join(HERE, "libssmscan.so")
OBJ = os.path.join(ROOT, "_build")
ARCH = "gfx950"

# Packed FP32 instructions are disabled: only plain float32 VALU arithmetic.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
NOISE = "is not a recognized feature for this target"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel) and link libssmscan.so."""
    os.makedirs(OBJ, exist_ok=True)
    common = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
              "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *DEVICE_FLAGS]
    objs = [os.path.join(OBJ, os.path.splitext(src)[0] + ".o") for src in SOURCES]
    jobs = [common + ["-c", "-o", obj, os.path.join(CSRC, src)] for src, obj in zip(SOURCES, objs)]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
        for fut in [pool.submit(_run, cmd, verbose) for cmd in jobs]:
            fut.result()
    _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", OUT + ".tmp"] + objs, verbose)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
