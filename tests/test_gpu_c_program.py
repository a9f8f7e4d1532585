"""GPU parity through the C ABI from a plain C program (no Python, no torch
in the decoding process): tests/c_abi/decode_from_c.c reads q, kv and the
lengths from files, calls gqa_decode with HIP runtime memory and writes the
output, which is checked against the CPU oracle with the page's bar. The
program first runs the same decode through gqa_decode_ex_noalloc and exits
with status 4 unless both outputs are byte for byte the same.
"""
import importlib.util
import os
import subprocess

import numpy as np
import pytest

from oracle.reference import decode_ragged, round_fp16
import workloads

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _program():
    spec = importlib.util.spec_from_file_location("gqa_c_abi_build",
                                                  os.path.join(HERE, "c_abi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.ensure_c_program()


@pytest.mark.parametrize("spec", ["page_b4_c256", "b1_c256_len200", (257, [257, 0, 1, 200, 65])])
def test_c_program_matches_oracle(spec, tmp_path):
    w = (workloads.get(spec) if isinstance(spec, str)
         else workloads.build("c program", 97, spec[0], spec[1], fill="nan"))
    print(f"case c program {w.name}", flush=True)
    files = {k: str(tmp_path / f"{k}.bin") for k in ("q", "kv", "lens", "out")}
    np.ascontiguousarray(w.q).tofile(files["q"])
    w.dense_kv().tofile(files["kv"])
    w.seq_lens.astype(np.int32).tofile(files["lens"])
    res = subprocess.run([_program(), files["q"], files["kv"], files["lens"], files["out"],
                          str(w.batch), str(w.capacity), repr(float(w.q_scale))],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "output identical to gqa_decode" in res.stdout
    got = np.fromfile(files["out"], dtype=np.float16).reshape(w.q.shape).astype(np.float64)
    ref = round_fp16(decode_ragged(w.q, w.k_valid, w.v_valid, w.q_scale)).astype(np.float64)
    d = np.abs(got - ref)
    print(f"c program {w.name}: max|d|={d.max():.3e} mean|d|={d.mean():.3e}", flush=True)
    assert d.max() <= 2e-3 and d.mean() <= 2e-4
