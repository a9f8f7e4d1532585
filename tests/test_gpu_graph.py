"""The decode inside HIP graphs and on concurrent streams.

A captured graph holds only kernel nodes (the host never reads the lengths
and the workspace exists before capture), so every replay must reproduce the
eager result bitwise, also with other eager work and synchronisations
between replays and with lengths changed on the device between replays.
Two streams decoding at once use separate workspaces and must not disturb
each other.
"""
import numpy as np
import pytest

import workloads

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


@pytest.mark.parametrize("elem", ["f16", "e4m3"])
def test_graph_replays_match_eager_bitwise(elem):
    torch = _torch()
    g = _g()
    ws = [workloads.build(f"graph {elem} {i}", 90 + i, 2048, lens, elem=elem)
          for i, lens in enumerate([[2048, 5, 700], [1, 1500, 33], [0, 64, 2048]])]
    qs = [w.q_to_device(DEV) for w in ws]
    kvs = [w.kv_to_device(DEV) for w in ws]
    lens = [torch.from_numpy(w.seq_lens).to(DEV) for w in ws]
    outs = [torch.empty_like(q) for q in qs]

    def calls():
        for w, q, kv, ln, o in zip(ws, qs, kvs, lens, outs):
            g.gqa_decode(q, kv, ln, out=o, q_scale=w.q_scale, k_scale=w.k_scale,
                         v_scale=w.v_scale)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()                        # eager on the capture stream: creates its workspace
    s.synchronize()
    eager = [_bits(o) for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            calls()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()      # unrelated eager work
        graph.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for i, o in enumerate(outs):
            assert np.array_equal(_bits(o), eager[i]), f"replay {rep}, call {i}"
    # lengths live on the device: change them in place and replay
    lens[0].copy_(torch.tensor([3, 2048, 0], dtype=torch.int32))
    graph.replay()
    torch.cuda.synchronize()
    w2 = workloads.build("graph relen", 90, 2048, [2048, 5, 700], elem=elem)
    q2, kv2 = w2.q_to_device(DEV), w2.kv_to_device(DEV)
    ref = g.gqa_decode(q2, kv2, torch.tensor([3, 2048, 0], dtype=torch.int32, device=DEV),
                       q_scale=w2.q_scale, k_scale=w2.k_scale, v_scale=w2.v_scale)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(outs[0]), _bits(ref))


@pytest.mark.parametrize("form", ["two", "single"])
def test_two_streams_decode_concurrently(form):
    # Each stream has its own workspace (and, in the single launch, its own
    # segment tickets): interleaved calls on two streams must not see each
    # other's partials or tickets.
    torch = _torch()
    g = _g()
    g.set_launch_form(form)
    a = workloads.get("b8_c4096_nanfill")
    b = workloads.build("stream b", 95, 8192, [8192, 100, 4000, 1, 7000, 3, 8000, 2], elem="f16")
    qa, kva, la = a.q_to_device(DEV), a.kv_to_device(DEV), torch.from_numpy(a.seq_lens).to(DEV)
    qb, kvb, lb = b.q_to_device(DEV), b.kv_to_device(DEV), torch.from_numpy(b.seq_lens).to(DEV)
    ref_a = _bits(g.gqa_decode(qa, kva, la))
    ref_b = _bits(g.gqa_decode(qb, kvb, lb))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs_a, outs_b = [], []
    for _ in range(10):
        with torch.cuda.stream(s1):
            outs_a.append(g.gqa_decode(qa, kva, la))
        with torch.cuda.stream(s2):
            outs_b.append(g.gqa_decode(qb, kvb, lb))
    torch.cuda.synchronize()
    for oa, ob in zip(outs_a, outs_b):
        assert np.array_equal(_bits(oa), ref_a)
        assert np.array_equal(_bits(ob), ref_b)


@pytest.mark.parametrize("form", ["two", "single"])
def test_graph_survives_workspace_growth_on_its_stream(form):
    # A graph captured on stream s holds s's workspace (and, in the single
    # launch, its ticket array). A later, larger eager call on s needs
    # bigger buffers: the library must leave the captured ones allocated, so
    # replays still write where the graph expects, and must not hand them to
    # anyone else (torch allocations made meanwhile are filled with NaN to
    # catch such reuse).
    torch = _torch()
    g = _g()
    g.set_launch_form(form)
    try:
        small = workloads.build(f"grow small {form}", 120, 256, [256, 37, 200])
        big = workloads.build(f"grow big {form}", 121, 256,
                              lambda r: r.integers(1, 256, 200, endpoint=True))
        qs, kvs = small.q_to_device(DEV), small.kv_to_device(DEV)
        ls = torch.from_numpy(small.seq_lens).to(DEV)
        qb, kvb = big.q_to_device(DEV), big.kv_to_device(DEV)
        lb = torch.from_numpy(big.seq_lens).to(DEV)
        out_s = torch.empty_like(qs)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            # a fresh stream: its first call sizes the buffers for the small batch
            g.gqa_decode(qs, kvs, ls, out=out_s, q_scale=small.q_scale)
        s.synchronize()
        eager_small = _bits(out_s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                g.gqa_decode(qs, kvs, ls, out=out_s, q_scale=small.q_scale)
        torch.cuda.synchronize()
        # a larger batch on the same stream: new, larger buffers
        with torch.cuda.stream(s):
            out_b = g.gqa_decode(qb, kvb, lb, q_scale=big.q_scale)
        s.synchronize()
        eager_big = _bits(out_b)
        junk = [torch.full((n,), float("nan"), device=DEV) for n in (1 << 12, 1 << 16, 1 << 20)]
        for rep in range(3):
            out_s.fill_(float("nan"))
            with torch.cuda.stream(s):
                graph.replay()
                out_b2 = g.gqa_decode(qb, kvb, lb, q_scale=big.q_scale)
            s.synchronize()
            assert np.array_equal(_bits(out_s), eager_small), f"{form}: replay {rep}"
            assert np.array_equal(_bits(out_b2), eager_big), f"{form}: eager after replay {rep}"
        del junk
    finally:
        g.set_launch_form("auto")


def test_growth_under_capture_is_refused_with_nothing_enqueued():
    # A call under capture that needs a larger workspace than its stream has
    # fails with GQA_ERR_ALLOC before enqueuing anything; the stream's
    # buffers stay usable for calls of the size they serve.
    torch = _torch()
    g = _g()
    small = workloads.build("capture small", 122, 1024, [1024, 3])
    big = workloads.build("capture big", 123, 1024,
                          lambda r: r.integers(1, 1024, 300, endpoint=True))
    qs, kvs, ls = small.q_to_device(DEV), small.kv_to_device(DEV), torch.from_numpy(small.seq_lens).to(DEV)
    qb, kvb, lb = big.q_to_device(DEV), big.kv_to_device(DEV), torch.from_numpy(big.seq_lens).to(DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ref = g.gqa_decode(qs, kvs, ls, q_scale=small.q_scale)
    s.synchronize()
    ref_bits = _bits(ref)
    out_b = torch.empty_like(qb)
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(g.GqaDecodeError) as err:
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                g.gqa_decode(qb, kvb, lb, out=out_b, q_scale=big.q_scale)
    assert err.value.status == -7, str(err.value)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        again = g.gqa_decode(qs, kvs, ls, q_scale=small.q_scale)
    s.synchronize()
    assert np.array_equal(_bits(again), ref_bits)
