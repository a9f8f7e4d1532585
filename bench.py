"""Benchmark of the FP16 GQA single-token decode on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                [--elem f16|bf16|e4m3|nvfp4] [--page-size P] [--q-heads H --kv-heads H]
                [--no-cpu-baseline] [--copy-calibration-mib N]
python bench.py --summarize-pmc FETCH_DIR WRITE_DIR [--workload NAME]
python bench.py --summarize-sq DIR [--workload NAME] [--elem E]

One step = one gqa_decode call (split-KV pieces kernel + combine kernel)
over one batch of the named synthetic workload, inputs resident in HBM.
To keep every step reading from HBM rather than from the 256 MB
Infinity Cache, the steps cycle through R copies of the KV cache whose
valid bytes add up to at least 1 GiB (R <= 32; smaller workloads stay
partly cache-resident, reported as kv_copies_rotated).

Timed region: K steps captured once in a HIP graph and replayed, bracketed
by device synchronisation (a decode loop replays captured steps; this
removes host launch cost, not GPU work). The same K steps issued as eager
API calls are timed separately (api_us_per_step: what a caller issuing one
call after another sees per step), then once more with the library's
start/stop HIP events attached to each kernel dispatch on the launch stream
(kernel_us: the kernels' execution time, without launch gaps).

Single calls, cold and warm (latency_us): before each cold sample a 1 GiB
scratch buffer is overwritten, which evicts the L2 caches and the Infinity
Cache, then one eager call is timed between two events on its stream
(median, p10, p90); warm samples repeat one call on the same KV copy behind
a short spin kernel, so the KV bytes may be cache-resident when they fit.
Both kinds of sample wait behind GPU work, so host launch time stays out.

Prints ONE JSON line:
  value       KV-read throughput: sum(L_b) * 4096 B / step time (GB/s)
  roofline    the pieces kernel's algorithmic KV bytes per launch divided
              by its average event-measured execution time, against the 8 TB/s
              HBM peak; `traffic` is the measured HBM bytes per launch
              from rocprofv3 counters when a committed summary matches the
              current kernel source, else null
  cpu_baseline  the float64 CPU oracle on the host cores, same workload
  parity_vs_oracle  max/mean |d| of the benchmarked output against the
              oracle's result from the CPU leg, rounded to the output type
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
ROTATE_MAX_COPIES = 32
CALIBRATION_COPIES = 5


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


def cpu_baseline(w, min_seconds: float, gpu_out=None):
    import numpy as np

    from oracle.formats import bf16_to_f64, e4m3_to_f64, nvfp4_to_f64
    from oracle.reference import decode_ragged

    # the oracle takes the element values widened exactly
    if w.elem == "bf16":
        q = bf16_to_f64(w.q)
        kval = [bf16_to_f64(k) for k in w.k_valid]
        vval = [bf16_to_f64(v) for v in w.v_valid]
    elif w.elem == "e4m3":
        q = w.q
        kval = [e4m3_to_f64(k) for k in w.k_valid]
        vval = [e4m3_to_f64(v) for v in w.v_valid]
    elif w.elem == "nvfp4":
        q = w.q
        kval = [nvfp4_to_f64(k, s) for k, s in zip(w.k_valid, w.k_scales)]
        vval = [nvfp4_to_f64(v, s) for v, s in zip(w.v_valid, w.v_scales)]
    else:
        q, kval, vval = w.q, w.k_valid, w.v_valid
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    reps, t0 = 0, time.perf_counter()
    ref = None
    while True:
        ref = decode_ragged(q, kval, vval, w.q_scale, k_scale=w.k_scale, v_scale=w.v_scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    gbs = w.kv_bytes_read * reps / el / 1e9
    parity = None
    if gpu_out is not None:
        # the benchmarked output against the oracle's, rounded once to the
        # output type (fp16; bf16 for bf16 runs)
        if w.elem == "bf16":
            from oracle.formats import round_bf16
            ref_t = bf16_to_f64(round_bf16(ref))
        else:
            from oracle.reference import round_fp16
            ref_t = round_fp16(ref).astype(np.float64)
        d = np.abs(gpu_out - ref_t)
        parity = {"max_abs_diff": float(d.max()), "mean_abs_diff": float(d.mean()),
                  "bar": ("within about 1 bf16 ulp of the rounded oracle" if w.elem == "bf16"
                          else "max <= 2e-3, mean <= 2e-4")}
    res = {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole workload {w.name}, {reps} pass(es) in {el:.1f} s "
                      f"(float64 numpy, {threads} BLAS threads, "
                      f"{len(os.sched_getaffinity(0))} host cores visible)",
            "seconds_per_step": round(el / reps, 4)}
    return res, parity


def single_call_latency(step, dev, samples: int):
    """Median/p10/p90 (us) of one eager call timed between two events on the
    current stream: cold (a 1 GiB write before each call evicts the L2s and
    the Infinity Cache) and warm (the same KV copy again). Each sample is
    queued behind GPU work (the write, or a short spin kernel for warm
    samples), so the host's launch time is not inside the events."""
    import numpy as np
    import torch

    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    spin = getattr(torch.cuda, "_sleep", None)    # torch's spin kernel (a private helper)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(i, cold):
        if cold:
            flush.fill_(i & 0xFF)
        elif spin is not None:
            spin(200000)                  # tens of microseconds of GPU work
        a.record(stream)
        step(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3

    res = {}
    for name, cold in (("cold", True), ("warm", False)):
        timed(0, cold)                                   # untimed first call
        t = np.array([timed(i if cold else 0, cold) for i in range(samples)])
        res[name] = {"p10": round(float(np.percentile(t, 10)), 3),
                     "p50": round(float(np.percentile(t, 50)), 3),
                     "p90": round(float(np.percentile(t, 90)), 3)}
    res["samples"] = samples
    res["warm_queued_behind_spin"] = spin is not None   # else host launch time is included
    del flush
    torch.cuda.empty_cache()
    return res


def _counter_rows(d: str):
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, counter, match):
    """(dispatch id, counter value summed over instances) for matching kernels."""
    vals = {}
    for r in rows:
        if r.get("Counter_Name") != counter or not match(r.get("Kernel_Name", "")):
            continue
        key = int(r["Dispatch_Id"])
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return sorted(vals.items())


SQ_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
               "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
               "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "GRBM_GUI_ACTIVE")


def summarize_sq(d: str, workload: str, elem: str) -> str:
    """Mean per pieces-kernel dispatch of one rocprofv3 --pmc run of the
    SQ_COUNTERS, with utilisations normalised to the chip's cycles:
    GRBM_GUI_ACTIVE is read as summed over the 8 XCDs, so one XCD's active
    cycles are GRBM/8, and the chip has 1024 SIMDs and 256 CUs in them.
    VALU busy = 4 * SQ_ACTIVE_INST_VALU (counted in 4-cycle units) / SIMD
    cycles; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMD cycles; LDS bank
    conflicts = SQ_LDS_BANK_CONFLICT / CU cycles."""
    rows = _counter_rows(d)
    is_ours = lambda n: "gqa_decode_pieces" in n
    mean = {}
    n = 0
    for c in SQ_COUNTERS:
        vals = [v for _, v in _per_dispatch(rows, c, is_ours)]
        if not vals:
            raise SystemExit(f"{c}: no decode dispatches in {d}")
        mean[c] = sum(vals) / len(vals)
        n = len(vals)
    xcd_cycles = mean["GRBM_GUI_ACTIVE"] / 8
    simd_cycles, cu_cycles = xcd_cycles * 1024, xcd_cycles * 256
    lines = [f"# SQ counters of gqa_decode_pieces ({elem}) on {workload}", "",
             f"kernel_source_sha256: {kernel_source_hash()}",
             f"dispatches: {n}", "", "Mean per dispatch:", "", "```"]
    lines += [f"{c:26s} {mean[c]:16.1f}" for c in SQ_COUNTERS]
    lines += ["```", "",
              f"VALU busy: {100 * 4 * mean['SQ_ACTIVE_INST_VALU'] / simd_cycles:.1f}% of SIMD cycles",
              f"MFMA busy: {100 * mean['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.1f}% of SIMD cycles",
              f"LDS bank conflicts: {100 * mean['SQ_LDS_BANK_CONFLICT'] / cu_cycles:.1f}% of CU cycles",
              f"VALU instructions per MFMA: {mean['SQ_INSTS_VALU'] / max(mean['SQ_INSTS_MFMA'], 1):.1f}",
              ""]
    return "\n".join(lines)


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str, copy_mib: int) -> str:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, both of
    `bench.py --copy-calibration-mib N`) into HBM bytes per pieces-kernel
    launch. Each counter (KiB per dispatch) is scaled by what it reads for
    the calibration copies, which move exactly N MiB each way."""
    is_ours = lambda n: "gqa_decode_pieces" in n
    is_copy = lambda n: ("copyBuffer" in n or "direct_copy" in n or "copy_kernel" in n)
    out = {}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d)
        ours = _per_dispatch(rows, counter, is_ours)
        if not ours:
            raise SystemExit(f"{counter}: no decode dispatches in {d}")
        # The calibration copies are the first copies after the last decode.
        copies = [v for k, v in _per_dispatch(rows, counter, is_copy) if k > ours[-1][0]]
        copies = copies[:CALIBRATION_COPIES]
        if len(copies) < CALIBRATION_COPIES:
            raise SystemExit(f"{counter}: found {len(copies)} calibration copies in {d}")
        factor = copy_mib * 1048576 / (sum(copies) / len(copies) * 1024)
        vals = [v for _, v in ours]
        out[counter] = (sum(vals) / len(vals) * 1024 * factor, factor, len(vals))
    traffic = int(out["FETCH_SIZE"][0] + out["WRITE_SIZE"][0])
    return "\n".join([
        f"# HBM traffic of gqa_decode_pieces on {workload}",
        "",
        f"kernel_source_sha256: {kernel_source_hash()}",
        f"traffic_bytes_per_launch: {traffic}",
        f"fetch_bytes_per_launch: {int(out['FETCH_SIZE'][0])} (copy scale factor {out['FETCH_SIZE'][1]:.4f}, {out['FETCH_SIZE'][2]} dispatches)",
        f"write_bytes_per_launch: {int(out['WRITE_SIZE'][0])} (copy scale factor {out['WRITE_SIZE'][1]:.4f}, {out['WRITE_SIZE'][2]} dispatches)",
        "",
    ])


def _paginate(kv, page_size, seed):
    """The cache [B, 2, 8, C, 128] as shuffled HND pages [B * C/P, 2, 8, P,
    128] and its block table [B, C/P] (C padded to a multiple of P)."""
    import numpy as np
    import torch

    B, _, H, C, D = kv.shape
    P = page_size
    maxp = -(-C // P)
    raw = kv.view(torch.int16 if kv.element_size() == 2 else torch.uint8)
    if maxp * P != C:
        pad = torch.zeros((B, 2, H, maxp * P - C, D), dtype=raw.dtype, device=kv.device)
        raw = torch.cat([raw, pad], dim=3)
    ordered = raw.reshape(B, 2, H, maxp, P, D).permute(0, 3, 1, 2, 4, 5).reshape(B * maxp, 2, H, P, D)
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(B * maxp)).to(kv.device)
    pages = torch.empty_like(ordered)
    pages[perm] = ordered
    table = perm.to(torch.int32).reshape(B, maxp).contiguous()
    return pages.view(kv.dtype), table


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--elem", default="f16", choices=["f16", "bf16", "e4m3", "nvfp4"],
                    help="element type: f16 (default), bf16 (q, kv, out), e4m3 (fp16 q and "
                         "out, FP8 E4M3 kv with per-tensor scales), or nvfp4 (fp16 q and out, "
                         "block-scaled FP4 kv: gqa_decode_fp4); non-f16 types use the typed "
                         "entry points")
    ap.add_argument("--page-size", type=int, default=0,
                    help="> 0: read the cache as shuffled HND pages of this many positions "
                         "(gqa_decode_paged); 0: the contiguous cache")
    ap.add_argument("--q-heads", type=int, default=32,
                    help="query heads (with --kv-heads: other head counts, same lengths)")
    ap.add_argument("--kv-heads", type=int, default=8, help="KV heads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--latency-samples", type=int, default=100,
                    help="single-call samples, cold and warm each (0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run plain device copies of this size (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-sq", metavar="DIR")
    args = ap.parse_args(argv)

    if args.summarize_sq:
        print(summarize_sq(args.summarize_sq, args.workload, args.elem))
        return 0
    if args.summarize_pmc:
        print(summarize_pmc(*args.summarize_pmc, args.workload, args.copy_calibration_mib or 256))
        return 0

    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the decode shards by batch or KV head with no communication, "
              "but no multi-GPU path is implemented).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gqa_token_decode_amd as g
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.get(args.workload, args.elem, q_heads=args.q_heads, kv_heads=args.kv_heads)
    kv_bytes = w.kv_bytes_read
    sum_len = int(w.valid_lengths.sum())

    q = w.q_to_device(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    kv0 = w.kv_to_device(dev)
    fp4 = args.elem == "nvfp4"
    sc0 = w.scales_to_device(dev) if fp4 else None
    alloc = kv0.numel() * kv0.element_size() + (sc0.numel() if fp4 else 0)
    rot = max(1, math.ceil(ROTATE_TARGET_BYTES / max(kv_bytes, 1)))
    rot = min(rot, ROTATE_MAX_COPIES, max(1, int(40e9 // alloc)))
    kvs = [kv0] + [kv0.clone() for _ in range(rot - 1)]
    scs = ([sc0] + [sc0.clone() for _ in range(rot - 1)]) if fp4 else None
    out = torch.empty_like(q)
    tables = None
    if args.page_size > 0:
        kvs, tables = zip(*[_paginate(kv, args.page_size, seed=i) for i, kv in enumerate(kvs)])
        if fp4:   # the same pages (same seed): the scale pages share the block table
            scs = [_paginate(sc, args.page_size, seed=i)[0] for i, sc in enumerate(scs)]
    torch.cuda.synchronize()

    def step(i):
        if fp4:
            g.gqa_decode_fp4(q, kvs[i % rot], scs[i % rot], lens, out=out,
                             block_table=None if tables is None else tables[i % rot],
                             q_scale=w.q_scale, k_scale=w.k_scale, v_scale=w.v_scale)
        elif tables is not None:
            g.gqa_decode_paged(q, kvs[i % rot], tables[i % rot], lens, out=out,
                               q_scale=w.q_scale, k_scale=w.k_scale, v_scale=w.v_scale)
        else:
            g.gqa_decode(q, kvs[i % rot], lens, out=out, q_scale=w.q_scale, k_scale=w.k_scale,
                         v_scale=w.v_scale)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps replayed from one captured graph.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        step(0)                      # the workspace is cached per stream: create it first
        gs.synchronize()
        with torch.cuda.graph(graph, stream=gs):
            for i in range(args.steps):
                step(i)
    torch.cuda.synchronize()
    graph.replay()                   # untimed: the first replay uploads the graph
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(gs)
    with torch.cuda.stream(gs):
        graph.replay()
    e1.record(gs)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # The same steps as eager API calls: plain, then with per-kernel events
    # (the events add work between dispatches, so they are not in the API time).
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    api_ms_per_step = e0.elapsed_time(e1) / args.steps
    with g.KernelTimer() as kt:
        for i in range(args.steps):
            step(i)
    torch.cuda.synchronize()
    pieces_us = kt.pieces_ms / kt.calls * 1e3
    combine_us = kt.combine_ms / kt.calls * 1e3

    latency = None
    if args.latency_samples > 0:
        latency = single_call_latency(step, dev, args.latency_samples)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 1048576
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(CALIBRATION_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Quick numerical sanity (full parity lives in the GPU tests).
    res = out.float().cpu().numpy()
    assert np.all(np.isfinite(res)), "non-finite decode output"

    achieved = kv_bytes / (pieces_us * 1e-6) / 1e9
    default_heads = (args.q_heads, args.kv_heads) == (32, 8)
    traffic = (traffic_from_profiles(args.workload)
               if args.elem == "f16" and default_heads and args.page_size == 0 else None)
    line = {
        "metric": METRIC,
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "api_us_per_step": round(api_ms_per_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.elem,
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "description": workloads.describe(args.workload),
            "batch": w.batch, "capacity": w.capacity, "q_heads": w.q_heads,
            "kv_heads": w.kv_heads,
            "head_dim": 128, "sum_valid_len": sum_len, "kv_bytes_per_step": kv_bytes,
            "kv_copies_rotated": rot, "accumulate": "f32",
            "kv_layout": (f"paged, {args.page_size} positions per page, shuffled"
                          if args.page_size > 0 else "contiguous"),
        },
        "bytes_per_step": {
            "kv": kv_bytes,
            "q": q.numel() * q.element_size(),
            "out": out.numel() * out.element_size(),
            "seq_lens": lens.numel() * lens.element_size(),
            "algorithmic_total": kv_bytes + q.numel() * q.element_size()
                                 + out.numel() * out.element_size()
                                 + lens.numel() * lens.element_size(),
            # device memory the library holds for this shape (partials,
            # segment table), allocated once and reused
            "workspace_allocated": (g.workspace_bytes(w.batch, w.capacity)
                                    if default_heads else None),
        },
        "latency_us": latency,
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
    if not args.no_cpu_baseline:
        # the last eager step's output (every KV copy holds the same values)
        if out.dtype == torch.bfloat16:
            from oracle.formats import bf16_to_f64
            got = bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
        else:
            got = out.cpu().numpy().astype(np.float64)
        line["cpu_baseline"], parity = cpu_baseline(w, args.cpu_seconds, got)
        line["parity_vs_oracle"] = parity
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
