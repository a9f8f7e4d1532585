"""Compile libgqa_decode.so (HIP, gfx950 only) in-tree.

The shared library holds the split-KV pieces kernel, the log-sum-exp
combine kernel and the C-ABI declared in include/gqa_decode.h. It is built
ahead of time for gfx950 (MI355X); there is no JIT path and no other target.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgqa_decode.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["gqa_decode_kernels.hip", "gqa_decode_api.cpp"]
# Measurement kernels of bench.py (streaming-read ceiling, VALU load for the
# counter check): a library of their own, outside the decode ABI.
BENCH_LIB_PATH = os.path.join(PKG_DIR, "libgqa_bench.so")
BENCH_SOURCES = ["bench_kernels.hip"]

# Device-code flags. Packed fp32 instructions are switched off: hipcc would
# otherwise fuse pairs of fp32 FMAs into v_pk_fma_f32.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-mcode-object-version=5",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernels' first 4 argument dwords arrive in scalar registers
    "-mllvm", "-amdgpu-kernarg-preload-count=4",
]


def hipcc() -> str:
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError(f"hipcc not found (looked for {path})")
    return path


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile the decode library and the bench kernels' library; always
    rebuilds. Returns the decode library's path."""
    _compile(LIB_PATH, SOURCES, verbose, extra_flags)
    _compile(BENCH_LIB_PATH, BENCH_SOURCES, verbose, None)
    return LIB_PATH


def _compile(out_path, sources, verbose, extra_flags):
    tmp = out_path + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []), "-shared",
           "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host compiler pass warns that it does not know the packed-fp32
    # feature; keep only other diagnostics.
    noise = "is not a recognized feature for this target"
    diag = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{diag}")
    if verbose and diag.strip():
        print(diag, file=sys.stderr)
    os.replace(tmp, out_path)


if __name__ == "__main__":
    print(build(verbose=True))
