"""Benchmark of the FP16 GQA single-token decode on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                [--no-cpu-baseline] [--graph]

One step = one gqa_decode call (split-KV pieces kernel + combine kernel)
over one batch of the named synthetic workload, inputs resident in HBM.
To keep every step reading from HBM rather than from the 256 MB
Infinity Cache, the step cycles through R copies of the KV cache whose
valid bytes add up to at least 1 GiB.

Prints ONE JSON line:
  value       KV-read throughput: sum(L_b) * 4096 B / step time (GB/s)
  roofline    the pieces kernel's algorithmic KV bytes per launch divided
              by its average duration (HIP events recorded by the library
              on the launch stream, inside the timed region), against the
              8 TB/s HBM peak; `traffic` is the measured HBM bytes per launch
              from rocprofv3 counters when a committed summary matches the
              current kernel source, else null
  cpu_baseline  the float64 CPU oracle on the host cores, same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode µs/step + achieved KV-read HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "b8_c4096_nanfill"
KERNEL_SOURCE = os.path.join(ROOT, "gqa_token_decode_amd", "csrc", "gqa_decode_kernels.hip")
ROTATE_TARGET_BYTES = 1 << 30


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_from_profiles(workload: str):
    """HBM bytes per partial-kernel launch from a committed counter summary.

    Looks for profiles/*traffic*<workload>*.md with lines
    `kernel_source_sha256: <hex>` and `traffic_bytes_per_launch: <int>`;
    returns None unless the hash matches the current kernel source.
    """
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    want = kernel_source_hash()
    for f in sorted(os.listdir(pdir)):
        if "traffic" not in f or workload not in f or not f.endswith((".md", ".txt")):
            continue
        text = open(os.path.join(pdir, f)).read()
        h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
        t = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
        if h and t and h.group(1) == want:
            return int(t.group(1))
    return None


def cpu_baseline(w, min_seconds: float):
    import numpy as np

    from oracle.reference import decode_ragged

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    reps, t0 = 0, time.perf_counter()
    while True:
        decode_ragged(w.q, w.k_valid, w.v_valid, w.q_scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    gbs = w.kv_bytes_read * reps / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole workload {w.name}, {reps} pass(es) in {el:.1f} s "
                      f"(float64 numpy, {threads} BLAS threads, "
                      f"{len(os.sched_getaffinity(0))} host cores visible)",
            "seconds_per_step": round(el / reps, 4)}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--graph", action="store_true",
                    help="also time the steps replayed from one captured HIP graph")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the decode shards by batch or KV head with no communication, "
              "but multi-GPU runs are not part of it).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gqa_token_decode_amd as g
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.get(args.workload)
    kv_bytes = w.kv_bytes_read
    sum_len = int(w.valid_lengths.sum())

    q = torch.from_numpy(w.q).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    kv0 = w.kv_to_device(dev)
    rot = max(1, math.ceil(ROTATE_TARGET_BYTES / max(kv_bytes, 1)))
    rot = min(rot, max(1, int(40e9 // kv0.numel() // 2)))     # keep the copies under ~40 GB
    kvs = [kv0] + [kv0.clone() for _ in range(rot - 1)]
    out = torch.empty_like(q)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        g.gqa_decode(q, kvs[i % rot], lens, out=out, q_scale=w.q_scale)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    with g.KernelTimer() as kt:
        for i in range(args.steps):
            g.gqa_decode(q, kvs[i % rot], lens, out=out, q_scale=w.q_scale)
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = e0.elapsed_time(e1) / args.steps
    pieces_us = kt.pieces_ms / kt.calls * 1e3
    combine_us = kt.combine_ms / kt.calls * 1e3

    graph_us = None
    if args.graph:
        gr = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            # The workspace is cached per stream: create it before capture.
            g.gqa_decode(q, kvs[0], lens, out=out, q_scale=w.q_scale)
            s.synchronize()
            with torch.cuda.graph(gr, stream=s):
                for i in range(rot):
                    g.gqa_decode(q, kvs[i], lens, out=out, q_scale=w.q_scale)
        torch.cuda.synchronize()
        reps = max(1, args.steps // rot)
        gr.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / (reps * rot)

    # Quick numerical sanity (full parity lives in the GPU tests).
    res = out.float().cpu().numpy()
    assert np.all(np.isfinite(res)), "non-finite decode output"

    achieved = kv_bytes / (pieces_us * 1e-6) / 1e9
    traffic = traffic_from_profiles(args.workload)
    line = {
        "metric": METRIC,
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "description": workloads.describe(args.workload),
            "batch": w.batch, "capacity": w.capacity, "q_heads": 32, "kv_heads": 8,
            "head_dim": 128, "sum_valid_len": sum_len, "kv_bytes_per_step": kv_bytes,
            "kv_copies_rotated": rot, "accumulate": "f32",
        },
        "kernel_us": {"pieces": round(pieces_us, 3), "combine": round(combine_us, 3),
                      "sum": round(pieces_us + combine_us, 3)},
        "hbm_frac_of_step": round(kv_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "wall_ms_timed_region": round(wall_ms, 3),
        "roofline": {
            "bound": "hbm",
            "kernel": "gqa_decode_pieces",
            "achieved": round(achieved, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }
    if graph_us is not None:
        line["graph_us_per_step"] = round(graph_us, 3)
        line["graph_GBps"] = round(kv_bytes / (graph_us * 1e-6) / 1e9, 3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
