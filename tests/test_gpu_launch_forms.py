"""The single-launch form (the last workgroup of each cut segment merges its
partials, found through a per-segment atomic ticket) against the two-kernel
form (pieces kernel, then combine kernel).

Both forms cut the work identically and merge partials in the same fixed
order, so every output must match bitwise, for every element type, layout
and split. The ticket counts must return to zero after every call: repeated
calls with changing lengths (hence changing numbers of pieces per segment),
with the output poisoned before each call, must keep matching.
"""
import numpy as np
import pytest

import workloads
from test_gpu_typed import check_bf16, check_f16, oracle_of

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


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


def _assert_same(two, single, label):
    if np.array_equal(two, single):
        return
    diff = np.flatnonzero(two.ravel() != single.ravel())
    a = two.ravel()[diff].view(np.float16).astype(np.float64)
    b = single.ravel()[diff].view(np.float16).astype(np.float64)
    raise AssertionError(
        f"{label}: {diff.size} of {two.size} elements differ (first at flat index {diff[0]}); "
        f"max |two - single| = {np.nanmax(np.abs(a - b)):.3e}; two {a[:4]} single {b[:4]}")


def _both_forms(call):
    """Run call() in the two-kernel form, then the single-launch form, with a
    NaN-poisoned output each time; return both results' bits."""
    torch = _torch()
    g = _g()
    res = []
    for form in ("two", "single"):
        g.set_launch_form(form)
        out = call()
        torch.cuda.synchronize()
        res.append(_bits(out))
    return res


CASES = [
    # (workload name or (capacity, lengths), elem, chunk_len)
    ("b8_c4096_nanfill", "f16", 0),
    ("b64_c16384_skewed", "f16", 0),
    ((40000, [40000, 20001]), "f16", 0),        # ~40 pieces per segment
    ("page_b1_c4096", "f16", 0),
    ("page_b4_c256", "f16", 0),
    ("b1_c256_len200", "f16", 0),
    ("b8_c4096_nanfill", "bf16", 0),
    ("b8_c4096_nanfill", "e4m3", 0),
    ((700, [700, 1, 0, 333, 129, 64, 2, 700]), "f16", 0),
    ((700, [700, 1, 0, 333, 129, 64, 2, 700]), "f16", 7),
    ((700, [700, 1, 0, 333, 129, 64, 2, 700]), "e4m3", 50),
    ((5000, [5000, 4999, 17]), "bf16", 100),
]


def _workload(spec, elem, seed=60):
    if isinstance(spec, str):
        return workloads.get(spec, elem)
    cap, lens = spec
    return workloads.build(f"forms {cap}", seed, cap, lens, fill="nan", elem=elem)


@pytest.mark.parametrize("spec,elem,chunk", CASES)
def test_single_launch_equals_two_launches_bitwise(spec, elem, chunk):
    torch = _torch()
    g = _g()
    w = _workload(spec, elem)
    print(f"case forms {spec if isinstance(spec, str) else spec[0]} {elem} chunk {chunk}",
          flush=True)
    q, kv = w.q_to_device(DEV), w.kv_to_device(DEV)
    lens = torch.from_numpy(w.seq_lens).to(DEV)
    out = torch.empty_like(q)

    def call():
        out.view(torch.int16).fill_(0x7E00)
        return g.gqa_decode(q, kv, lens, out=out, q_scale=w.q_scale, k_scale=w.k_scale,
                            v_scale=w.v_scale, chunk_len=chunk)

    two, single = _both_forms(call)
    _assert_same(two, single, f"{spec if isinstance(spec, str) else spec[0]} {elem} {chunk}")
    if w.batch * w.capacity <= 8 * 4096:
        if elem == "bf16":
            check_bf16(out, oracle_of(w), f"single launch {elem}")
        else:
            check_f16(out, oracle_of(w), f"single launch {elem}")


def test_tickets_return_to_zero_across_calls():
    # Lengths change from call to call, so a segment is cut into a different
    # number of pieces each time; a ticket left nonzero by one call would make
    # a later call skip (or repeat) a merge, leaving NaN or stale rows.
    torch = _torch()
    g = _g()
    rng = np.random.default_rng(61)
    cap = 3000
    base = workloads.build("tickets", 61, cap, [cap] * 6, elem="f16")
    q, kv = base.q_to_device(DEV), base.kv_to_device(DEV)
    out = torch.empty_like(q)
    for rep in range(8):
        lens_np = rng.integers(0, cap, 6, endpoint=True).astype(np.int32)
        lens = torch.from_numpy(lens_np).to(DEV)

        def call():
            out.view(torch.int16).fill_(0x7E00)
            return g.gqa_decode(q, kv, lens, out=out, chunk_len=[0, 64, 300][rep % 3])

        two, single = _both_forms(call)
        _assert_same(two, single, f"call {rep}, lengths {lens_np.tolist()}")


def test_single_launch_in_a_graph_with_lengths_changed_on_the_device():
    torch = _torch()
    g = _g()
    g.set_launch_form("single")
    w = workloads.build("forms graph", 62, 2048, [2048, 5, 700, 1500], elem="f16")
    q, kv = w.q_to_device(DEV), w.kv_to_device(DEV)
    lens = torch.from_numpy(w.seq_lens).to(DEV)
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.gqa_decode(q, kv, lens, out=out)        # eager first: creates workspace and tickets
    s.synchronize()
    eager = _bits(out)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            g.gqa_decode(q, kv, lens, out=out)
    torch.cuda.synchronize()
    for rep in range(4):
        out.view(torch.int16).fill_(0x7E00)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), eager), f"replay {rep}"
    new_lens = [100, 2048, 0, 777]
    lens.copy_(torch.tensor(new_lens, dtype=torch.int32))
    out.view(torch.int16).fill_(0x7E00)
    graph.replay()
    torch.cuda.synchronize()
    g.set_launch_form("two")
    ref = g.gqa_decode(q, kv, torch.tensor(new_lens, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), _bits(ref))


@pytest.mark.parametrize("cap", ["1", "3", "7"])
@pytest.mark.parametrize("spec", [
    # many segments, each cut into a few pieces: one combine unit per segment
    ("batch 40", 125, 8192, lambda r: r.integers(1, 8192, 40, endpoint=True)),
    # few long segments: one combine unit per (segment, query head)
    ("two long", 126, 65536, [65536, 40000]),
])
def test_combine_workgroups_taking_units_in_turns_match_bitwise(monkeypatch, cap, spec):
    # The combine kernel's grid is capped (1024 workgroups by default, 65536
    # at most; any batch then stays within one dispatch); each workgroup
    # takes units w, w + grid, ... A tiny cap makes every workgroup take
    # many units in turn, with the barrier between turns.
    torch = _torch()
    g = _g()
    name, seed, cap_rows, lens = spec
    w = workloads.build(f"turns {name}", seed, cap_rows, lens, fill="nan")
    q, kv, ln = w.q_to_device(DEV), w.kv_to_device(DEV), torch.from_numpy(w.seq_lens).to(DEV)
    g.set_launch_form("two")
    ref = _bits(g.gqa_decode(q, kv, ln, q_scale=w.q_scale))
    torch.cuda.synchronize()
    monkeypatch.setenv("GQA_DECODE_COMBINE_MAX_GRID", cap)
    out = torch.full_like(q, float("nan"))
    g.gqa_decode(q, kv, ln, out=out, q_scale=w.q_scale)
    torch.cuda.synchronize()
    _assert_same(ref, _bits(out), f"{name}, combine grid {cap}")


# (batch, capacity, q heads, KV heads): on both sides of each bound of the
# automatic choice (capacity <= 512 with at most 131072 cache rows, or
# capacity <= 1024 with at most 32768 rows; rows = batch x KV heads x capacity)
AUTO_SHAPES = [
    (1, 512, 32, 8), (32, 512, 32, 8), (33, 512, 32, 8),
    (4, 1024, 32, 8), (5, 1024, 32, 8), (1, 1025, 32, 8), (1, 2048, 32, 8),
    (32, 1024, 8, 1), (33, 1024, 8, 1), (3, 999, 24, 3),
]


def _auto_single(batch, capacity, kv_heads):
    rows = batch * kv_heads * capacity
    return (capacity <= 512 and rows <= 131072) or (capacity <= 1024 and rows <= 32768)


@pytest.mark.parametrize("batch,capacity,hq,hkv", AUTO_SHAPES)
def test_auto_form_follows_its_documented_bounds(batch, capacity, hq, hkv):
    # A single launch runs no combine kernel, so the library's kernel timer
    # records no combine time for it; a two-kernel call always records some.
    torch = _torch()
    g = _g()
    gen = torch.Generator(device=DEV).manual_seed(batch * 10007 + capacity)
    q = torch.randn(batch, hq, 128, device=DEV, generator=gen).half()
    kv = torch.randn(batch, 2, hkv, capacity, 128, device=DEV, generator=gen).half()
    lens = torch.full((batch,), capacity, dtype=torch.int32, device=DEV)
    g.set_launch_form("auto")
    g.gqa_decode(q, kv, lens)                    # workspace and tickets exist
    torch.cuda.synchronize()
    with g.KernelTimer() as t:
        out = g.gqa_decode(q, kv, lens)
        torch.cuda.synchronize()
    want_single = _auto_single(batch, capacity, hkv)
    assert t.calls == 1
    assert (t.combine_ms == 0.0) == want_single, (
        f"B={batch} C={capacity} Hkv={hkv}: combine {t.combine_ms * 1e3:.2f} us, "
        f"expected {'single launch' if want_single else 'two kernels'}")
    g.set_launch_form("single" if want_single else "two")
    _assert_same(_bits(g.gqa_decode(q, kv, lens)), _bits(out), f"B={batch} C={capacity}")
