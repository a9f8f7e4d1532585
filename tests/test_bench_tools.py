"""CPU tests of bench.py's host-side tooling: the one-GPU guard and the
rocprofv3 counter summaries (synthetic counter files with known values)."""
import csv
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(w.fieldnames, r)))


PIECES = "void gqa::(anonymous namespace)::gqa_decode_pieces<0, false, true>(int const*, int, int)"
OTHER = "void gqa::(anonymous namespace)::gqa_decode_combine<0, true>(int2 const*, int, int)"


def test_more_than_one_gpu_is_refused(capsys):
    assert _bench().main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_sq_summary_normalisation(tmp_path):
    b = _bench()
    # 8 XCDs x 1000 active cycles: 1,024,000 SIMD cycles and 256,000 CU cycles
    per = {"GRBM_GUI_ACTIVE": 8000, "SQ_ACTIVE_INST_VALU": 204800,
           "SQ_VALU_MFMA_BUSY_CYCLES": 102400, "SQ_LDS_BANK_CONFLICT": 2560,
           "SQ_INSTS_VALU": 204800, "SQ_INSTS_MFMA": 100, "SQ_WAVE_CYCLES": 1,
           "SQ_BUSY_CYCLES": 1, "SQ_ACTIVE_INST_LDS": 1}
    rows = []
    for disp in (1, 3):
        for c, v in per.items():
            # two instances per dispatch (values are summed), e.g. two XCD halves
            rows += [(disp, PIECES, c, v / 2), (disp, PIECES, c, v / 2)]
    for c in per:
        rows.append((2, OTHER, c, 1e9))          # another kernel: ignored
    _write_counters(str(tmp_path / "sq"), rows)
    text = b.summarize_sq(str(tmp_path / "sq"), "wl", "f16", valu_reference=0.4)
    assert "dispatches: 2" in text
    assert "valu_issue_per_simd_cycle: 0.2000" in text
    assert "share of the VALU-saturating kernel's: 50.0%" in text
    assert "MFMA busy: 10.0% of SIMD cycles" in text
    assert "LDS bank conflicts: 1.0% of CU cycles" in text
    assert "VALU instructions per MFMA: 2048.0" in text
    assert b.kernel_source_hash() in text
    ref = tmp_path / "ref.md"
    ref.write_text("valu_issue_per_simd_cycle: 0.8000\n")
    assert "25.0%" in b.summarize_sq(str(tmp_path / "sq"), "wl", "f16", valu_reference=str(ref))


def test_traffic_summary_scales_by_the_calibration_copies(tmp_path):
    b = _bench()
    mib = 256
    # FETCH_SIZE reads half of each copy's bytes (KiB), WRITE_SIZE all of them
    fetch = [(1, PIECES, "FETCH_SIZE", 1000.0), (2, PIECES, "FETCH_SIZE", 1200.0)]
    fetch += [(10 + i, "copyBuffer", "FETCH_SIZE", mib * 1024 / 2) for i in range(5)]
    write = [(1, PIECES, "WRITE_SIZE", 30.0), (2, PIECES, "WRITE_SIZE", 10.0)]
    write += [(10 + i, "copyBuffer", "WRITE_SIZE", mib * 1024.0) for i in range(5)]
    _write_counters(str(tmp_path / "f"), fetch)
    _write_counters(str(tmp_path / "w"), write)
    text = b.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "wl", mib)
    # fetch: mean 1100 KiB x 2 = 2200 KiB; write: mean 20 KiB x 1
    assert f"traffic_bytes_per_launch: {2200 * 1024 + 20 * 1024}" in text
    assert "copy scale factor 2.0000" in text and "copy scale factor 1.0000" in text


def test_traffic_summary_needs_the_calibration_copies(tmp_path):
    b = _bench()
    _write_counters(str(tmp_path / "f"), [(1, PIECES, "FETCH_SIZE", 1.0)])
    _write_counters(str(tmp_path / "w"), [(1, PIECES, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit, match="calibration copies"):
        b.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "wl", 256)


def test_trace_summary_cuts_dispatches_into_the_bench_phases(tmp_path):
    b = _bench()
    d = tmp_path / "tr"
    os.makedirs(d)
    warmup, steps = 2, 3
    phases = b.trace_phases(warmup, steps)
    # pieces take 10 + phase index us, combines 1 us; another kernel in between
    rows, t = [], 0
    for k, (_, n) in enumerate(phases):
        for _ in range(n):
            rows.append((PIECES, t, t + (10 + k) * 1000))
            rows.append(("stream_read", t + 50000, t + 60000))
            rows.append((OTHER, t + 100000, t + 101000))
            t += 1000000
    rows.reverse()                        # the file's order does not matter: start time does
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerows(rows)
    text = b.summarize_trace(str(d), "wl", "f16", warmup, steps, "python3 bench.py ...")
    assert "pieces_us_eager_events: 15.000" in text
    assert "combine_us_eager_events: 1.000" in text
    assert "| graph replay, timed | 3 | 13.000 | 1.000 |" in text
    assert "python3 bench.py ..." in text
    with pytest.raises(SystemExit, match="expected"):
        b.summarize_trace(str(d), "wl", "f16", warmup + 1, steps)


def test_traffic_lookup_matches_source_hash_and_element_type(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    h = b.kernel_source_hash()
    (tmp_path / "profiles" / "gqa_decode_pieces_traffic_wl.md").write_text(
        f"kernel_source_sha256: {h}\ntraffic_bytes_per_launch: 123\n")
    (tmp_path / "profiles" / "gqa_decode_pieces_traffic_e4m3_wl.md").write_text(
        f"kernel_source_sha256: {h}\nelem: e4m3\ntraffic_bytes_per_launch: 45\n")
    (tmp_path / "profiles" / "gqa_decode_pieces_traffic_old_wl.md").write_text(
        f"kernel_source_sha256: {'0' * 64}\nelem: nvfp4\ntraffic_bytes_per_launch: 7\n")
    assert b.traffic_from_profiles("wl") == 123
    assert b.traffic_from_profiles("wl", "e4m3") == 45
    assert b.traffic_from_profiles("wl", "nvfp4") is None      # stale source hash
    assert b.traffic_from_profiles("other") is None
