"""Seeded random sweep on the GPU against the CPU oracle.

Each case draws, from its own seed: the batch size, the capacity, the
lengths (zero, one and the full capacity planted among ragged values), the
head counts, the element format (fp16, bf16, E4M3 or block-scaled FP4), the
layout (contiguous, or paged with a shuffled page pool), q_scale, a forced
split length and the launch form. The output is checked against the oracle
with the format's bar, and sequences of length zero must return zeros.
"""
import numpy as np
import pytest

import workloads
from test_gpu_fp4 import _paginate_fp4, oracle_fp4
from test_gpu_fp4 import check as check_fp4
from test_gpu_layouts import _paginate
from test_gpu_typed import check_bf16, check_f16, oracle_of

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HEADS = [(32, 8), (64, 8), (28, 4), (16, 16), (8, 1), (12, 4), (6, 2), (40, 8)]
CAPACITIES = [1, 2, 31, 32, 33, 64, 127, 500, 1024, 2049, 3000]
N_CASES = 120


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


def draw_case(i):
    rng = np.random.default_rng(5000 + i)
    batch = int(rng.integers(1, 25))
    cap = int(rng.choice(CAPACITIES))
    lens = rng.integers(0, cap + 1, batch)
    for v in (0, 1, cap):
        if rng.random() < 0.5:
            lens[rng.integers(batch)] = v
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    elem = str(rng.choice(["f16", "bf16", "e4m3", "nvfp4"]))
    page = 0
    if rng.random() < 0.4:
        page = int(rng.choice([p for p in (16, 32, 64, 128) if elem != "nvfp4" or p >= 32]))
    return {
        "seed": 6000 + i, "batch": batch, "cap": cap, "lens": [int(x) for x in lens],
        "hq": hq, "hkv": hkv, "elem": elem, "page": page,
        "q_scale": float(rng.choice([1.0, 0.5, 0.125])),
        "chunk": int(rng.choice([0, 0, 1, 7, 64, 300])),
        "form": str(rng.choice(["auto", "two", "single"])),
    }


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_matches_oracle(i):
    torch = _torch()
    g = _g()
    c = draw_case(i)
    print(f"case random {i}: {c}", flush=True)
    w = workloads.build(f"random {i}", c["seed"], c["cap"], c["lens"], fill="nan",
                        elem=c["elem"], q_heads=c["hq"], kv_heads=c["hkv"],
                        q_scale=c["q_scale"])
    g.set_launch_form(c["form"])
    q = w.q_to_device(DEV)
    lens = torch.from_numpy(w.seq_lens).to(DEV)
    kv = w.kv_to_device(DEV)
    common = {"q_scale": w.q_scale, "chunk_len": c["chunk"], "k_scale": w.k_scale,
              "v_scale": w.v_scale}
    if c["elem"] == "nvfp4":
        scales = w.scales_to_device(DEV)
        table = None
        if c["page"]:
            kv, scales, table = _paginate_fp4(kv, scales, w.valid_lengths, c["page"], seed=i)
        out = g.gqa_decode_fp4(q, kv, scales, lens, block_table=table, **common)
    elif c["page"]:
        pages, table = _paginate(kv, w.valid_lengths, c["page"], seed=i)
        out = g.gqa_decode_paged(q, pages, table, lens, **common)
    else:
        out = g.gqa_decode(q, kv, lens, **common)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (c["batch"], c["hq"], 128)
    label = f"random {i} ({c['elem']}, page {c['page']}, {c['form']})"
    if c["elem"] == "nvfp4":
        check_fp4(out, oracle_fp4(w), label)
    elif c["elem"] == "bf16":
        check_bf16(out, oracle_of(w), label)
    else:
        check_f16(out, oracle_of(w), label)
    raw = out.view(torch.int16).cpu().numpy()
    for b in range(c["batch"]):
        if c["lens"][b] == 0:
            assert np.all(raw[b] == 0), b
