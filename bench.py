"""Benchmark of the FP16 GQA single-token decode on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--also NAMES|none]
                [--elem f16|bf16|e4m3|nvfp4] [--page-size P] [--q-heads H --kv-heads H]
                [--no-cpu-baseline] [--copy-calibration-mib N] [--valu-calibration]
python bench.py --summarize-pmc FETCH_DIR WRITE_DIR [--workload NAME] [--elem E]
python bench.py --summarize-sq DIR [--workload NAME] [--elem E] [--kernel NAME]
python bench.py --summarize-trace DIR [--workload NAME] [--elem E] [--steps K] [--warmup W]

One step = one gqa_decode call (split-KV pieces kernel + combine kernel)
over one batch of the named synthetic workload, inputs resident in HBM.
The headline workload is the largest single-GPU configuration, batch 2 with
131072- and 65537-row sequences (805 MB of K/V per step); the other
configurations are measured in the same run (graph-replayed step and the
pieces kernel's execution time) and reported under "workloads".
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

Read ceiling (read_ceiling): a plain streaming-read kernel (libgqa_bench.so)
reads the same number of bytes, rotating over copies like the decode steps;
its median time is the fastest these bytes stream on this GPU, and
frac_of_read_ceiling = that time / the pieces kernel's time (for the
headline and, as read_ceiling_us / frac_of_read_ceiling, for each entry of
`workloads`).

Prints ONE JSON line:
  value       KV-read throughput: sum(L_b) * 4096 B / step time (GB/s)
  roofline    the pieces kernel's algorithmic KV bytes per launch divided
              by its average event-measured execution time, against the 8 TB/s
              HBM peak; `traffic` is the measured HBM bytes per launch
              from rocprofv3 counters when a committed summary matches the
              current kernel source, else null; step_frac is the same bytes
              over the whole graph-replayed step (pieces + combine)
  cpu_baseline  the float64 CPU oracle on the host cores, same workload
              (BLAS threads of the host), plus a 1-thread figure and the CPU model
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
DEFAULT_WORKLOAD = "b2_c131072_long"
# the other configurations, measured in the same run
ALSO_DEFAULT = ["b1_c256_len200", "b8_c4096_nanfill", "b32_c8192_qs05", "b64_c16384_skewed"]
KERNEL_SOURCE = os.path.join(ROOT, "gqa_token_decode_amd", "csrc", "gqa_decode_kernels.hip")
ROTATE_TARGET_BYTES = 1 << 30
ROTATE_MAX_COPIES = 32
CALIBRATION_COPIES = 5


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_from_profiles(workload: str, elem: str = "f16"):
    """HBM bytes per pieces-kernel launch from a committed counter summary.

    Looks for profiles/*traffic*<workload>*.md with lines
    `kernel_source_sha256: <hex>`, `elem: <type>` (f16 if absent) and
    `traffic_bytes_per_launch: <int>`; returns None unless the hash matches
    the current kernel source and the element type matches.
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
        e = re.search(r"^elem:\s*(\S+)", text, re.M)
        if h and t and h.group(1) == want and (e.group(1) if e else "f16") == elem:
            return int(t.group(1))
    return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, min_seconds: float, gpu_out=None, one_thread_seconds: float = 3.0):
    """The oracle as it stands on the host: repeated passes over the whole
    workload for at least min_seconds with the BLAS library's own thread
    count, then passes with one BLAS thread for at least one_thread_seconds
    (threadpoolctl; skipped if it is missing)."""
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
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = len(os.sched_getaffinity(0))

    def passes(seconds):
        reps, t0 = 0, time.perf_counter()
        while True:
            out = decode_ragged(q, kval, vval, w.q_scale, k_scale=w.k_scale, v_scale=w.v_scale)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return out, reps, el

    ref, reps, el = passes(min_seconds)
    gbs = w.kv_bytes_read * reps / el / 1e9
    one = None
    if threadpool_limits is not None and one_thread_seconds > 0:
        with threadpool_limits(limits=1):
            _, r1, e1 = passes(one_thread_seconds)
        one = {"value": round(w.kv_bytes_read * r1 / e1 / 1e9, 4), "unit": "GB/s",
               "seconds_per_step": round(e1 / r1, 4), "passes": r1}
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
           "seconds_per_step": round(el / reps, 4),
           "cpu_model": cpu_model(),
           "one_thread": one}
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


def _dispatch_ns(rows, match):
    """Mean kernel duration (ns) over the matching dispatches of a counter run."""
    spans = {}
    for r in rows:
        if match(r.get("Kernel_Name", "")) and r.get("Start_Timestamp") and r.get("End_Timestamp"):
            spans[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return sum(spans.values()) / len(spans) if spans else None


def summarize_sq(d: str, workload: str, elem: str, kernel: str = "gqa_decode_pieces",
                 valu_reference=None) -> str:
    """Mean per dispatch of `kernel` of one rocprofv3 --pmc run of the
    SQ_COUNTERS, normalised to the chip's SIMD cycles. GRBM_GUI_ACTIVE is
    the sum over the 8 XCDs (checked: divided by the dispatch's duration it
    gives 8 x the clock, e.g. 16.0 GHz for 8 XCDs at 2.0 GHz), so the chip
    had GRBM/8 x 1024 SIMD cycles (128 SIMDs per XCD) and GRBM/8 x 256 CU
    cycles. Reported: VALU instructions issued per SIMD cycle (SQ_INSTS_VALU,
    wave instructions; SQ_ACTIVE_INST_VALU reads the same count on gfx950),
    and that rate as a share of the rate of valu_load, a kernel that keeps
    every SIMD's VALU busy with independent FMAs (`bench.py
    --valu-calibration`; valu_reference is its rate, or the path of its
    summary); MFMA busy cycles and LDS bank-conflict cycles as counted, over
    SIMD and CU cycles."""
    rows = _counter_rows(d)
    is_ours = lambda n: kernel in n
    mean = {}
    n = 0
    for c in SQ_COUNTERS:
        vals = [v for _, v in _per_dispatch(rows, c, is_ours)]
        if not vals:
            raise SystemExit(f"{c}: no {kernel} dispatches in {d}")
        mean[c] = sum(vals) / len(vals)
        n = len(vals)
    if isinstance(valu_reference, str):
        m = re.search(r"valu_issue_per_simd_cycle:\s*([0-9.]+)", open(valu_reference).read())
        valu_reference = float(m.group(1)) if m else None
    xcd_cycles = mean["GRBM_GUI_ACTIVE"] / 8
    simd_cycles, cu_cycles = xcd_cycles * 1024, xcd_cycles * 256
    dur = _dispatch_ns(rows, is_ours)
    issue = mean["SQ_INSTS_VALU"] / simd_cycles
    lines = [f"# SQ counters of {kernel} ({elem}) on {workload}", "",
             f"kernel_source_sha256: {kernel_source_hash()}",
             f"dispatches: {n}", "", "Mean per dispatch:", "", "```"]
    lines += [f"{c:26s} {mean[c]:16.1f}" for c in SQ_COUNTERS]
    lines += ["```", ""]
    if dur:
        lines.append(f"Duration {dur / 1e3:.2f} us; GRBM_GUI_ACTIVE / duration = "
                     f"{mean['GRBM_GUI_ACTIVE'] / dur:.2f} GHz (8 XCDs at "
                     f"{mean['GRBM_GUI_ACTIVE'] / dur / 8:.2f} GHz)")
    lines += [f"valu_issue_per_simd_cycle: {issue:.4f}"]
    if valu_reference:
        lines.append(f"VALU issue as a share of the VALU-saturating kernel's: "
                     f"{100 * issue / valu_reference:.1f}% (its rate {valu_reference:.4f})")
    lines += [f"MFMA busy: {100 * mean['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.1f}% of SIMD cycles",
              f"LDS bank conflicts: {100 * mean['SQ_LDS_BANK_CONFLICT'] / cu_cycles:.1f}% of CU cycles",
              f"VALU instructions per MFMA: {mean['SQ_INSTS_VALU'] / max(mean['SQ_INSTS_MFMA'], 1):.1f}",
              ""]
    return "\n".join(lines)


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str, copy_mib: int,
                  elem: str = "f16") -> str:
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
        f"# HBM traffic of gqa_decode_pieces on {workload} ({elem})",
        "",
        f"kernel_source_sha256: {kernel_source_hash()}",
        f"elem: {elem}",
        f"traffic_bytes_per_launch: {traffic}",
        f"fetch_bytes_per_launch: {int(out['FETCH_SIZE'][0])} (copy scale factor {out['FETCH_SIZE'][1]:.4f}, {out['FETCH_SIZE'][2]} dispatches)",
        f"write_bytes_per_launch: {int(out['WRITE_SIZE'][0])} (copy scale factor {out['WRITE_SIZE'][1]:.4f}, {out['WRITE_SIZE'][2]} dispatches)",
        "",
    ])


def _trace_rows(d: str):
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_trace.csv under {d}")
    with open(files[0]) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return rows


def _stats_rows(d: str):
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        return []
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def trace_phases(warmup: int, steps: int):
    """Decode calls of one bench.py run (--also none, --latency-samples 0) in
    issue order: (phase, number of calls)."""
    return [("warm-up (eager)", warmup), ("first call on the capture stream (eager)", 1),
            ("graph replay, untimed upload", steps), ("graph replay, timed", steps),
            ("eager API pass", steps), ("eager pass with dispatch events (kernel_us)", steps)]


def summarize_trace(d: str, workload: str, elem: str, warmup: int, steps: int,
                    command: str = "") -> str:
    """Per-phase mean durations of the decode kernels in one rocprofv3
    --kernel-trace run of bench.py (--also none, --latency-samples 0; the
    same --steps and --warmup as given here). Dispatches of each kernel are
    taken in start order and cut into the bench's phases; in graph replays a
    kernel's recorded start can precede the end of the previous step's
    combine, which lengthens the recorded durations there, so the phase that
    bench.py's kernel_us and roofline use (eager with dispatch events) is
    the one to compare with them."""
    rows = _trace_rows(d)
    names = {"pieces": "gqa_decode_pieces", "combine": "gqa_decode_combine"}
    per = {k: [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
               for r in rows if v in r["Kernel_Name"]] for k, v in names.items()}
    phases = trace_phases(warmup, steps)
    total = sum(n for _, n in phases)
    lines = [f"# Kernel trace of gqa_decode on {workload} ({elem})", "",
             f"kernel_source_sha256: {kernel_source_hash()}", f"elem: {elem}", ""]
    if command:
        lines += ["Command (from the repository root on the GPU host):", "", f"    {command}", ""]
    lines += [f"Decode calls: {total} (warm-up {warmup}, steps {steps}); dispatches found: "
              + ", ".join(f"{k} {len(v)}" for k, v in per.items()), "",
              "Mean duration per phase (us):", "", "| phase | calls | pieces | combine |",
              "|---|---|---|---|"]
    means = {}
    for k, durs in per.items():
        if durs and len(durs) != total:
            raise SystemExit(f"{names[k]}: {len(durs)} dispatches, expected {total} "
                             "(run with --also none --latency-samples 0)")
    i = 0
    for name, n in phases:
        row = [name, str(n)]
        for k in names:
            durs = per[k][i:i + n]
            m = sum(durs) / len(durs) / 1e3 if durs else None
            means[(name, k)] = m
            row.append(f"{m:.3f}" if m is not None else "-")
        lines.append("| " + " | ".join(row) + " |")
        i += n
    stats = _stats_rows(d)
    if stats:
        lines += ["", "rocprofv3 --stats over all dispatches (run_kernel_stats.csv, ns):", "", "```",
                  '"Name","Calls","AverageNs","MinNs","MaxNs"']
        for r in stats:
            if any(v in r.get("Name", "") for v in names.values()):
                lines.append(f'"{r["Name"]}",{r["Calls"]},{r["AverageNs"]},{r["MinNs"]},{r["MaxNs"]}')
        lines.append("```")
    ev = trace_phases(warmup, steps)[-1][0]
    lines += ["", f"pieces_us_eager_events: {means[(ev, 'pieces')]:.3f}"]
    if means[(ev, "combine")] is not None:
        lines.append(f"combine_us_eager_events: {means[(ev, 'combine')]:.3f}")
    lines.append("")
    return "\n".join(lines)


def bench_lib():
    import ctypes

    path = os.path.join(ROOT, "gqa_token_decode_amd", "libgqa_bench.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build first (__graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    fp = ctypes.POINTER(ctypes.c_float)
    lib.gqa_bench_stream_read.argtypes = [vp, sz, sz, i32, i32, i32, i32, vp, vp, fp]
    lib.gqa_bench_stream_read.restype = i32
    lib.gqa_bench_valu_load.argtypes = [i32, i32, i32, vp, vp, fp]
    lib.gqa_bench_valu_load.restype = i32
    return lib


def read_ceiling(nbytes: int, dev, reps: int = 15):
    """Median time of a plain streaming read of nbytes (rounded down to 16),
    rotating over copies that add up to >= 1 GiB like the decode steps; the
    best of 1 or 2 workgroups per CU and 4 or 8 KiB per wave in flight."""
    import ctypes

    import numpy as np
    import torch

    nbytes = nbytes // 16 * 16
    if nbytes < 16:
        return None
    lib = bench_lib()
    stride = (nbytes + 4095) // 4096 * 4096
    copies = min(ROTATE_MAX_COPIES, max(1, math.ceil(ROTATE_TARGET_BYTES / nbytes)))
    buf = torch.zeros(copies * stride, dtype=torch.uint8, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(cus * 8, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    best = None
    for wpc in (1, 2):
        for kib in (4, 8):
            us = (ctypes.c_float * reps)()
            rc = lib.gqa_bench_stream_read(buf.data_ptr(), nbytes, stride, copies, reps, wpc, kib,
                                           sink.data_ptr(), stream, us)
            if rc != 0:
                raise RuntimeError("streaming-read kernel failed")
            med = float(np.median(np.array(us[1:] if reps > 1 else us)))
            if best is None or med < best[0]:
                best = (med, wpc, kib)
    del buf
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "us": round(best[0], 3), "gbs": round(nbytes / best[0] / 1e3, 1),
            "copies": copies, "wgs_per_cu": best[1], "kib_in_flight_per_wave": best[2]}


def valu_calibration(dev, iters: int = 20000, reps: int = 5):
    """Run the VALU-saturating kernel (for the SQ counter check)."""
    import ctypes

    import torch

    lib = bench_lib()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(cus * 8, dtype=torch.int32, device=dev)
    us = (ctypes.c_float * reps)()
    rc = lib.gqa_bench_valu_load(iters, reps, 8, sink.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream, us)
    if rc != 0:
        raise RuntimeError("VALU load kernel failed")
    waves = cus * 8 * 4
    return {"kernel": "valu_load", "workgroups": cus * 8, "fma_per_wave": 8 * iters,
            "us": [round(x, 2) for x in us],
            "expected_valu_fma": waves * 8 * iters}


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


def _device_state(w, args, dev):
    """Device tensors of workload w, rotated over KV copies, and its step."""
    import torch

    import gqa_token_decode_amd as g

    q = w.q_to_device(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    kv0 = w.kv_to_device(dev)
    fp4 = args.elem == "nvfp4"
    sc0 = w.scales_to_device(dev) if fp4 else None
    alloc = kv0.numel() * kv0.element_size() + (sc0.numel() if fp4 else 0)
    rot = max(1, math.ceil(ROTATE_TARGET_BYTES / max(w.kv_bytes_read, 1)))
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

    return {"q": q, "lens": lens, "out": out, "rot": rot, "step": step}


def _time_steps(st, steps: int, warmup: int, eager_api: bool = True):
    """Graph-replayed step time (the timed region), the eager API pass and
    the per-kernel event times, in ms per step / us."""
    import torch

    import gqa_token_decode_amd as g

    step = st["step"]
    for i in range(warmup):
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
            for i in range(steps):
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
    res = {"wall_ms": (time.perf_counter() - t0) * 1e3,
           "ms_per_step": e0.elapsed_time(e1) / steps}
    # The same steps as eager API calls: plain, then with per-kernel events
    # (the events add work between dispatches, so they are not in the API time).
    stream = torch.cuda.current_stream()
    if eager_api:
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        res["api_ms_per_step"] = e0.elapsed_time(e1) / steps
    with g.KernelTimer() as kt:
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    res["pieces_us"] = kt.pieces_ms / kt.calls * 1e3
    res["combine_us"] = kt.combine_ms / kt.calls * 1e3
    del graph
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads measured in the same run (graph step and "
                         "kernel times), or 'none'; default: the other configurations when the "
                         "headline is the default workload, else none")
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
    ap.add_argument("--no-read-ceiling", action="store_true")
    ap.add_argument("--latency-samples", type=int, default=100,
                    help="single-call samples, cold and warm each (0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-one-thread-seconds", type=float, default=3.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run plain device copies of this size (counter calibration)")
    ap.add_argument("--valu-calibration", action="store_true",
                    help="also run the VALU-saturating kernel (SQ counter normalisation check)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-sq", metavar="DIR")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--kernel", default="gqa_decode_pieces",
                    help="--summarize-sq: the kernel whose dispatches are summarised")
    ap.add_argument("--command", default="", help="--summarize-trace: the profiled command")
    ap.add_argument("--valu-reference", default=None,
                    help="--summarize-sq: the valu_load summary (its issue rate is the reference)")
    args = ap.parse_args(argv)

    if args.summarize_sq:
        print(summarize_sq(args.summarize_sq, args.workload, args.elem, args.kernel,
                           args.valu_reference))
        return 0
    if args.summarize_pmc:
        print(summarize_pmc(*args.summarize_pmc, args.workload, args.copy_calibration_mib or 256,
                            args.elem))
        return 0
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.workload, args.elem, args.warmup,
                              args.steps, args.command))
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
    default_heads = (args.q_heads, args.kv_heads) == (32, 8)
    if args.also is None:
        also = ALSO_DEFAULT if args.workload == DEFAULT_WORKLOAD else []
    else:
        also = [] if args.also == "none" else [a for a in args.also.split(",") if a]
    w = workloads.get(args.workload, args.elem, q_heads=args.q_heads, kv_heads=args.kv_heads)
    kv_bytes = w.kv_bytes_read
    sum_len = int(w.valid_lengths.sum())

    st = _device_state(w, args, dev)
    q, out, lens, rot, step = st["q"], st["out"], st["lens"], st["rot"], st["step"]
    tm = _time_steps(st, args.steps, args.warmup)
    ms_per_step, pieces_us, combine_us = tm["ms_per_step"], tm["pieces_us"], tm["combine_us"]

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
    valu = valu_calibration(dev) if args.valu_calibration else None

    # Quick numerical sanity (full parity lives in the GPU tests).
    res = out.float().cpu().numpy()
    assert np.all(np.isfinite(res)), "non-finite decode output"
    if out.dtype == torch.bfloat16:
        from oracle.formats import bf16_to_f64
        got = bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    else:
        got = out.cpu().numpy().astype(np.float64)
    ceiling = None if args.no_read_ceiling else read_ceiling(kv_bytes, dev)
    del st, q, out, lens, step
    torch.cuda.empty_cache()

    # The other configurations, same run: graph step and kernel times.
    others = {}
    for name in also:
        wo = workloads.get(name, args.elem, q_heads=args.q_heads, kv_heads=args.kv_heads)
        so = _device_state(wo, args, dev)
        to = _time_steps(so, args.steps, args.warmup, eager_api=False)
        kb = wo.kv_bytes_read
        others[name] = {
            "sum_valid_len": int(wo.valid_lengths.sum()), "kv_bytes_per_step": kb,
            "us_per_step": round(to["ms_per_step"] * 1e3, 3),
            "gbs": round(kb / (to["ms_per_step"] * 1e-3) / 1e9, 1),
            "step_frac": round(kb / (to["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "pieces_us": round(to["pieces_us"], 3), "combine_us": round(to["combine_us"], 3),
            "pieces_frac": round(kb / (to["pieces_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "kv_copies_rotated": so["rot"],
        }
        if not args.no_read_ceiling:
            c = read_ceiling(kb, dev)
            if c:
                others[name]["read_ceiling_us"] = c["us"]
                others[name]["frac_of_read_ceiling"] = round(c["us"] / to["pieces_us"], 4)
        del so, wo
        torch.cuda.empty_cache()

    achieved = kv_bytes / (pieces_us * 1e-6) / 1e9
    traffic = (traffic_from_profiles(args.workload, args.elem)
               if default_heads and args.page_size == 0 else None)
    line = {
        "metric": METRIC,
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "api_us_per_step": round(tm["api_ms_per_step"] * 1e3, 3),
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
            "q": w.q.size * 2,
            "out": w.q.size * 2,
            "seq_lens": w.seq_lens.size * 4,
            "algorithmic_total": kv_bytes + 2 * w.q.size * 2 + w.seq_lens.size * 4,
            # device memory the library holds for this shape (partials,
            # segment table), allocated once and reused
            "workspace_allocated": (g.workspace_bytes(w.batch, w.capacity)
                                    if default_heads else None),
        },
        "latency_us": latency,
        "kernel_us": {"pieces": round(pieces_us, 3), "combine": round(combine_us, 3),
                      "sum": round(pieces_us + combine_us, 3)},
        "hbm_frac_of_step": round(kv_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "wall_ms_timed_region": round(tm["wall_ms"], 3),
        "roofline": {
            "bound": "hbm",
            "kernel": "gqa_decode_pieces",
            "achieved": round(achieved, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
            "step_frac": round(kv_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "read_ceiling": ceiling,
        "frac_of_read_ceiling": (round(ceiling["us"] / pieces_us, 4) if ceiling else None),
        "workloads": others or None,
    }
    if valu is not None:
        line["valu_calibration"] = valu
    if not args.no_cpu_baseline:
        # the last eager step's output (every KV copy holds the same values)
        line["cpu_baseline"], parity = cpu_baseline(w, args.cpu_seconds, got,
                                                    args.cpu_one_thread_seconds)
        line["parity_vs_oracle"] = parity
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
