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
    per = {"GRBM_GUI_ACTIVE": 8000, "SQ_ACTIVE_INST_VALU": 128000,
           "SQ_VALU_MFMA_BUSY_CYCLES": 102400, "SQ_LDS_BANK_CONFLICT": 2560,
           "SQ_INSTS_VALU": 900, "SQ_INSTS_MFMA": 100, "SQ_WAVE_CYCLES": 1,
           "SQ_BUSY_CYCLES": 1, "SQ_ACTIVE_INST_LDS": 1}
    rows = []
    for disp in (1, 3):
        for c, v in per.items():
            # two instances per dispatch (values are summed), e.g. two XCD halves
            rows += [(disp, PIECES, c, v / 2), (disp, PIECES, c, v / 2)]
    for c in per:
        rows.append((2, OTHER, c, 1e9))          # another kernel: ignored
    _write_counters(str(tmp_path / "sq"), rows)
    text = b.summarize_sq(str(tmp_path / "sq"), "wl", "f16")
    assert "dispatches: 2" in text
    assert "VALU busy: 50.0% of SIMD cycles" in text
    assert "MFMA busy: 10.0% of SIMD cycles" in text
    assert "LDS bank conflicts: 1.0% of CU cycles" in text
    assert "VALU instructions per MFMA: 9.0" in text
    assert b.kernel_source_hash() in text


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
