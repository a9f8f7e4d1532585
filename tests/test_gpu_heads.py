"""GPU parity for head counts other than the page's 32 query / 8 KV heads.

Query head h reads KV head h // (Hq / Hkv); up to 8 query heads share a KV
head (they fill columns of the same 16-wide MFMA operand, so every K/V row
still crosses HBM once per KV head). Each case is checked against the CPU
oracle with the element type's bar, and the two launch forms against each
other bitwise.
"""
import numpy as np
import pytest

import workloads
from test_gpu_layouts import _paginate
from test_gpu_typed import check_bf16, check_f16, oracle_of

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

HEADS = [(64, 8), (28, 4), (16, 16), (32, 16), (8, 1), (40, 8), (12, 4), (1, 1), (6, 2),
         (48, 6)]


def _torch():
    import torch
    return torch


def _g():
    import gqa_token_decode_amd as g
    return g


def _bits(t):
    torch = _torch()
    return t.view(torch.int16).cpu().numpy()


@pytest.fixture(autouse=True)
def _restore_auto_form():
    yield
    _g().set_launch_form("auto")


def _check(w, out, label):
    if w.elem == "bf16":
        check_bf16(out, oracle_of(w), label)
    else:
        check_f16(out, oracle_of(w), label)


def _run(w, kv=None, **kw):
    torch = _torch()
    lens = torch.from_numpy(w.seq_lens).to(DEV)
    out = _g().gqa_decode(w.q_to_device(DEV), w.kv_to_device(DEV) if kv is None else kv, lens,
                          q_scale=w.q_scale, k_scale=w.k_scale, v_scale=w.v_scale, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("hq,hkv", HEADS)
def test_head_counts_match_oracle(hq, hkv):
    print(f"case heads {hq}/{hkv}", flush=True)
    lens = [600, 1, 0, 257, 33, 600]
    w = workloads.build(f"heads {hq}/{hkv}", 40 + hq + hkv, 600, lens, fill="nan",
                        q_heads=hq, kv_heads=hkv)
    out = _run(w)
    assert tuple(out.shape) == (len(lens), hq, 128)
    assert np.all(_bits(out)[2] == 0)                    # empty sequence
    _check(w, out, f"heads {hq}/{hkv}")
    # length one returns its V row exactly
    for h in range(hq):
        v = w.v_valid[1][h // (hq // hkv), 0]
        assert np.array_equal(out[1, h].cpu().numpy(), v), h
    # forced splits
    for chunk in (7, 100):
        _check(w, _run(w, chunk_len=chunk), f"heads {hq}/{hkv} chunk {chunk}")


@pytest.mark.parametrize("hq,hkv", [(64, 8), (28, 4), (8, 1), (16, 16)])
@pytest.mark.parametrize("elem", ["bf16", "e4m3"])
def test_head_counts_other_formats(hq, hkv, elem):
    print(f"case heads {hq}/{hkv} {elem}", flush=True)
    w = workloads.build(f"heads {elem}", 50 + hq, 500, [500, 3, 0, 77, 260], fill="nan",
                        elem=elem, q_heads=hq, kv_heads=hkv)
    _check(w, _run(w), f"heads {hq}/{hkv} {elem}")
    _check(w, _run(w, chunk_len=50), f"heads {hq}/{hkv} {elem} chunk 50")


@pytest.mark.parametrize("hq,hkv", [(64, 8), (28, 4), (16, 16)])
def test_head_counts_launch_forms_agree_bitwise(hq, hkv):
    torch = _torch()
    g = _g()
    w = workloads.build("heads forms", 60 + hq, 3000, [3000, 1500, 2, 2999], fill="nan",
                        q_heads=hq, kv_heads=hkv)
    kv = w.kv_to_device(DEV)
    res = []
    for form in ("two", "single"):
        g.set_launch_form(form)
        res.append(_bits(_run(w, kv=kv)))
    assert np.array_equal(res[0], res[1])
    _check(w, torch.from_numpy(res[1].view(np.float16)), f"heads {hq}/{hkv} forms")


@pytest.mark.parametrize("hq,hkv", [(64, 8), (12, 4)])
def test_head_counts_large_batch_block_planner(hq, hkv):
    # more than 64 sequences: the workgroup-wide planner
    rng = np.random.default_rng(70)
    lens = rng.integers(0, 300, 100, endpoint=True)
    w = workloads.build("heads big batch", 70, 300, lens, q_heads=hq, kv_heads=hkv)
    _check(w, _run(w), f"heads {hq}/{hkv} batch 100")


@pytest.mark.parametrize("hq,hkv", [(64, 8), (28, 4), (16, 16)])
@pytest.mark.parametrize("elem", ["f16", "bf16", "e4m3"])
def test_head_counts_paged(hq, hkv, elem):
    print(f"case heads {hq}/{hkv} paged {elem}", flush=True)
    w = workloads.build("heads paged", 80 + hq, 512, [512, 1, 0, 300, 17], fill="nan",
                        q_heads=hq, kv_heads=hkv, elem=elem)
    kv = w.kv_to_device(DEV)
    pages, table = _paginate(kv, w.valid_lengths, 32, seed=hq)
    torch = _torch()
    lens = torch.from_numpy(w.seq_lens).to(DEV)
    out = _g().gqa_decode_paged(w.q_to_device(DEV), pages, table, lens, q_scale=w.q_scale,
                                k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    _check(w, out, f"heads {hq}/{hkv} paged {elem}")


def test_head_counts_strided_q_equals_contiguous_bitwise():
    # q as heads 8..71 of a packed [B, 80, 128] projection output, 64/8 heads
    torch = _torch()
    w = workloads.build("heads strided", 90, 400, [400, 9, 200], q_heads=64, kv_heads=8)
    q = w.q_to_device(DEV)
    packed = torch.zeros((q.shape[0], 80, 128), dtype=q.dtype, device=DEV)
    packed[:, 8:72] = q
    kv = w.kv_to_device(DEV)
    lens = torch.from_numpy(w.seq_lens).to(DEV)
    base = _g().gqa_decode(q, kv, lens)
    got = _g().gqa_decode(packed[:, 8:72], kv, lens)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(got), _bits(base))


def test_bad_head_ratios_are_rejected():
    torch = _torch()
    g = _g()
    lens = torch.ones(2, dtype=torch.int32, device=DEV)
    kv = torch.zeros((2, 2, 8, 16, 128), dtype=torch.float16, device=DEV)
    for hq in (72, 30, 4):
        q = torch.zeros((2, hq, 128), dtype=torch.float16, device=DEV)
        with pytest.raises(ValueError, match="heads"):
            g.gqa_decode(q, kv, lens)
