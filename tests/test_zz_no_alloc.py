"""The allocation-free entry point (gqa_decode_ex_noalloc) against the
cached-workspace one (gqa_decode_ex), through the C ABI.

Both run the same kernels with the same split; only where the partial
results, segment descriptors and tickets live differs (a fixed device array
in the library instead of a per-stream workspace), so the outputs must agree
bitwise. Two calls in a row, the second with a smaller input, check that
nothing of the first call's scratch contents leaks into the second; both
launch forms run (the single launch uses the scratch's tickets, which every
call must leave zero). A shape whose partials do not fit the scratch is
refused with nothing enqueued.
"""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BAD_SHAPE = -2


def _torch():
    import torch
    return torch


def _g():
    import gqa_token_decode_amd as g
    return g


def _bits(t):
    torch = _torch()
    return t.view(torch.int16).cpu().numpy()


def _inputs(w):
    torch = _torch()
    return w.q_to_device(DEV), w.kv_to_device(DEV), torch.from_numpy(w.seq_lens).to(DEV)


def _decode_ex(q, kv, lens, out, w, chunk_len):
    """gqa_decode_ex through ctypes, with the tensors' strides and heads."""
    import ctypes

    g = _g()
    lib = g.load_library()
    lay = g._Layout(q.stride(0), q.stride(1), kv.stride(0), kv.stride(1), kv.stride(2),
                    kv.stride(3), None, 0, 0, 0, q.shape[1], kv.shape[2])
    dtype = 2 if w.elem == "e4m3" else 0
    st = lib.gqa_decode_ex(q.data_ptr(), kv.data_ptr(), lens.data_ptr(), out.data_ptr(), dtype,
                           ctypes.byref(lay), w.q_scale, w.k_scale, w.v_scale, q.shape[0],
                           kv.shape[3], chunk_len, _torch().cuda.current_stream().cuda_stream)
    assert st == 0, lib.gqa_decode_last_error().decode()


def _both(w, chunk_len=0):
    """(bits from gqa_decode_ex, bits from gqa_decode_ex_noalloc)."""
    torch = _torch()
    g = _g()
    q, kv, lens = _inputs(w)
    ref = torch.full_like(q, float("nan"))
    _decode_ex(q, kv, lens, ref, w, chunk_len)
    out = torch.full_like(q, float("nan"))
    g.gqa_decode_noalloc(q, kv, lens, out=out, q_scale=w.q_scale, k_scale=w.k_scale,
                         v_scale=w.v_scale, chunk_len=chunk_len)
    torch.cuda.synchronize()
    return _bits(ref), _bits(out)


@pytest.fixture(autouse=True)
def _restore_auto_form():
    yield
    _g().set_launch_form("auto")


@pytest.mark.parametrize("form", ["auto", "two", "single"])
@pytest.mark.parametrize("elem", ["f16", "e4m3"])
def test_noalloc_matches_the_workspace_entry_point_on_two_calls(form, elem):
    _g().set_launch_form(form)
    cases = [
        workloads.build("noalloc big", 140, 512,
                        lambda r: r.integers(1, 512, 96, endpoint=True), fill="nan", elem=elem,
                        q_heads=64, kv_heads=8),
        workloads.build("noalloc small", 141, 300, [300, 1, 0, 257, 31], fill="nan", elem=elem,
                        q_heads=64, kv_heads=8),
    ]
    for w in cases:
        print(f"case noalloc {form} {elem} {w.name}", flush=True)
        ref, got = _both(w)
        assert not np.any(np.isnan(got.view(np.float16))), w.name
        assert np.array_equal(ref, got), f"{w.name} ({form}, {elem})"


def test_noalloc_long_sequences_with_forced_split():
    w1 = workloads.build("noalloc long", 142, 65536, [65536, 40000, 9])
    w2 = workloads.build("noalloc shorter", 143, 4096, [4096, 1])
    for w, chunk in ((w1, 0), (w1, 2000), (w2, 0), (w2, 64)):
        print(f"case noalloc {w.name} chunk {chunk}", flush=True)
        ref, got = _both(w, chunk)
        assert np.array_equal(ref, got), f"{w.name} chunk {chunk}"


def test_noalloc_refuses_shapes_beyond_its_scratch_with_nothing_enqueued():
    torch = _torch()
    g = _g()
    # one-row pieces over 3 x 8 x 4096 rows: ~100 MB of partials
    w = workloads.build("noalloc too big", 144, 4096, [4096, 4096, 4096])
    q, kv, lens = _inputs(w)
    out = torch.full_like(q, float("nan"))
    torch.cuda.synchronize()
    with pytest.raises(g.GqaDecodeError) as err:
        g.gqa_decode_noalloc(q, kv, lens, out=out, chunk_len=1)
    assert err.value.status == BAD_SHAPE and "scratch" in str(err.value)
    torch.cuda.synchronize()
    assert np.all(np.isnan(out.float().cpu().numpy()))      # nothing was enqueued
    with pytest.raises(ValueError):
        g.gqa_decode_noalloc(q, kv, lens, out=None)
