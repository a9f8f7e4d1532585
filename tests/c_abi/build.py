"""Build the C program that drives libgqa_decode.so through the C ABI alone.

gcc compiles it as C11 against include/gqa_decode.h and the HIP runtime
headers, and links it to the in-tree library (found at run time through an
rpath relative to the program) and to libamdhip64.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SOURCE = os.path.join(HERE, "decode_from_c.c")
PROGRAM = os.path.join(HERE, "decode_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_program() -> str:
    """Compile the program (always rebuilds); returns its path."""
    cmd = ["gcc", "-std=c11", "-Wall", "-O2", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SOURCE,
           "-L", os.path.join(ROOT, "gqa_token_decode_amd"), "-lgqa_decode",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../gqa_token_decode_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", PROGRAM]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    return PROGRAM


def ensure_c_program() -> str:
    """The program, rebuilt if missing or older than its source, the header or the library."""
    deps = [SOURCE, os.path.join(ROOT, "include", "gqa_decode.h"),
            os.path.join(ROOT, "gqa_token_decode_amd", "libgqa_decode.so")]
    if (not os.path.exists(PROGRAM)
            or os.path.getmtime(PROGRAM) < max(os.path.getmtime(d) for d in deps if os.path.exists(d))):
        build_c_program()
    return PROGRAM
