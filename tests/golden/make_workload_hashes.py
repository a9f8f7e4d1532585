"""Write tests/golden/workload_sha256.json: SHA-256 fingerprints of the
seeded synthetic inputs of every named workload (the input recipe, not any
expected result). Lengths and q for every workload; the K and V arrays too
for the small ones; also the bf16, E4M3 and block-scaled FP4 encodings of
the smallest. Run from the repository root: python tests/golden/make_workload_hashes.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

FULL = ["b1_c256_len200", "b8_c4096_nanfill", "page_b1_c64", "page_b4_c256", "page_b1_c1024",
        "page_b1_c4096"]
TYPED = [("b1_c256_len200", e) for e in ("bf16", "e4m3", "nvfp4")]


def digest(arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(a.tobytes())
    return h.hexdigest()


def fingerprint(name: str, elem: str = "f16") -> dict:
    w = workloads.get(name, elem, with_kv=name in FULL)
    d = {"lengths": digest([w.seq_lens]), "q": digest([w.q])}
    if name in FULL:
        d["k"] = digest(w.k_valid)
        d["v"] = digest(w.v_valid)
        if elem == "nvfp4":
            d["k_scales"] = digest(w.k_scales)
            d["v_scales"] = digest(w.v_scales)
    return d


def main() -> None:
    out = {"note": "SHA-256 of the seeded inputs (workloads.py); fingerprints of the input "
                   "recipe, not expected results. Written by tests/golden/make_workload_hashes.py.",
           "f16": {n: fingerprint(n) for n in workloads.WORKLOADS},
           "typed": {f"{n}/{e}": fingerprint(n, e) for n, e in TYPED}}
    path = os.path.join(ROOT, "tests", "golden", "workload_sha256.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"wrote {path}")


if __name__ == "__main__":
    main()
