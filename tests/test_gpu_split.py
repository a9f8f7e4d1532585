"""GPU parity of the two-length split against the oracle.

With more than one workgroup per CU the cost line is cut into longer pieces
for the first workgroup of each CU and shorter ones (second_share / 64 of
their length) for the rest, when the pieces are long (at least 1024 cost
units on average). These tests force the split (GQA_DECODE_WG_PER_CU=2,
GQA_DECODE_SECOND_SHARE) on workloads long enough to take it, at shares from
1/64 to equal, and check the page bar against the oracle; both launch forms
then cut the work the same way and must agree bitwise.
"""
import numpy as np
import pytest

from oracle.formats import nvfp4_to_f64
from oracle.reference import decode_ragged, round_fp16
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_TOL, MEAN_TOL = 2e-3, 2e-4


def _torch():
    import torch
    return torch


def _g():
    import gqa_token_decode_amd as g
    return g


@pytest.fixture(autouse=True)
def _restore_auto_form():
    yield
    _g().set_launch_form("auto")


def _workload(elem):
    # 4 x 8 segments of up to 24000 rows: ~640K cost units, above 512 x 1024
    return workloads.build(f"split {elem}", 150, 24000, [24000, 19001, 17, 23999], fill="nan",
                           elem=elem)


def _run(w):
    torch = _torch()
    g = _g()
    q, kv = w.q_to_device(DEV), w.kv_to_device(DEV)
    lens = torch.from_numpy(w.seq_lens).to(DEV)
    if w.elem == "nvfp4":
        out = g.gqa_decode_fp4(q, kv, w.scales_to_device(DEV), lens, q_scale=w.q_scale)
    else:
        out = g.gqa_decode(q, kv, lens, q_scale=w.q_scale)
    torch.cuda.synchronize()
    return out


def _oracle(w):
    if w.elem == "nvfp4":
        k = [nvfp4_to_f64(c, s) for c, s in zip(w.k_valid, w.k_scales)]
        v = [nvfp4_to_f64(c, s) for c, s in zip(w.v_valid, w.v_scales)]
        return decode_ragged(w.q, k, v, w.q_scale)
    return decode_ragged(w.q, w.k_valid, w.v_valid, w.q_scale)


@pytest.mark.parametrize("elem", ["f16", "nvfp4"])
def test_two_length_pieces_match_oracle_and_launch_forms_agree(monkeypatch, elem):
    torch = _torch()
    w = _workload(elem)
    ref16 = round_fp16(_oracle(w)).astype(np.float64)
    monkeypatch.setenv("GQA_DECODE_WG_PER_CU", "2")
    for share in ("1", "23", "40", "64"):
        monkeypatch.setenv("GQA_DECODE_SECOND_SHARE", share)
        outs = []
        for form in ("two", "single"):
            _g().set_launch_form(form)
            out = _run(w)
            outs.append(out.view(torch.int16).cpu().numpy())
            d = np.abs(out.cpu().numpy().astype(np.float64) - ref16)
            print(f"{elem} share {share} {form}: max|d|={d.max():.3e} mean|d|={d.mean():.3e}",
                  flush=True)
            assert d.max() <= MAX_TOL and d.mean() <= MEAN_TOL, (share, form)
        assert np.array_equal(outs[0], outs[1]), f"share {share}: launch forms differ"
