"""GPU parity of the block-scaled FP4 cache (gqa_decode_fp4) against the CPU
oracle, through the C ABI.

Every FP4 element value (an E2M1 value times an E4M3 block scale) is an
fp16 value, and the kernel forms it exactly before the fp16 arithmetic of
the other paths; the oracle takes the same exact values (decoded from the
codes by oracle.formats.nvfp4_to_f64). So the page's fp16 bar applies:
max |gpu - fp16(oracle)| <= 2e-3 and mean <= 2e-4.
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


class _Deq:
    """Per-(b, g) dequantised K or V rows of an nvfp4 workload, on access."""

    def __init__(self, codes, scales):
        self.codes, self.scales = codes, scales

    def __getitem__(self, b):
        codes, scales = self.codes[b], self.scales[b]

        class _Seq:
            def __getitem__(self, g):
                return nvfp4_to_f64(codes[g], scales[g])

            def __len__(self):
                return len(codes)

        return _Seq()


def oracle_fp4(w, k_scale=1.0, v_scale=1.0):
    return decode_ragged(w.q, _Deq(w.k_valid, w.k_scales), _Deq(w.v_valid, w.v_scales),
                         w.q_scale, k_scale=k_scale * w.k_scale, v_scale=v_scale * w.v_scale)


def check(out, ref64, label):
    got = out.cpu().numpy().astype(np.float64)
    ref16 = round_fp16(ref64).astype(np.float64)
    d = np.abs(got - ref16)
    print(f"{label}: max|d|={d.max():.3e} mean|d|={d.mean():.3e}", flush=True)
    assert np.all(np.isfinite(got)), label
    assert d.max() <= MAX_TOL and d.mean() <= MEAN_TOL, label


def bits(t):
    torch = _torch()
    return t.view(torch.int16).cpu().numpy()


def run(w, codes=None, scales=None, **kw):
    torch = _torch()
    lens = torch.from_numpy(w.seq_lens).to(DEV)
    codes = w.kv_to_device(DEV) if codes is None else codes
    scales = w.scales_to_device(DEV) if scales is None else scales
    kw.setdefault("q_scale", w.q_scale)
    out = _g().gqa_decode_fp4(w.q_to_device(DEV), codes, scales, lens, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["b1_c256_len200", "b8_c4096_nanfill", "b64_c16384_skewed"]
                         + workloads.PAGE_SHAPES)
def test_fp4_workloads_match_oracle(name):
    print(f"case fp4 {name}", flush=True)
    w = workloads.get(name, "nvfp4")
    check(run(w), oracle_fp4(w), f"fp4 {name}")


@pytest.mark.parametrize("chunk_len", [0, 7, 32, 143])
def test_fp4_ragged_lengths_odd_capacity(chunk_len):
    lens = [0, 1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, -5, 1000]
    print(f"case fp4 ragged chunk {chunk_len}", flush=True)
    w = workloads.build("fp4 ragged", 81, 257, lens, fill="nan", elem="nvfp4")
    out = run(w, chunk_len=chunk_len)
    check(out, oracle_fp4(w), f"fp4 ragged chunk {chunk_len}")
    b = bits(out)
    assert np.all(b[0] == 0) and np.all(b[16] == 0)           # empty and negative lengths


def test_fp4_length_one_returns_the_dequantised_v_row():
    print("case fp4 length one", flush=True)
    w = workloads.build("fp4 len1", 82, 64, [1, 1, 1], elem="nvfp4", sigma_v=3.0)
    out = run(w).cpu().numpy()
    for b in range(3):
        for h in range(32):
            v = nvfp4_to_f64(w.v_valid[b][h // 4, 0], w.v_scales[b][h // 4, 0])
            assert np.array_equal(out[b, h].astype(np.float64), v), (b, h)


def test_fp4_contents_beyond_length_have_no_effect():
    print("case fp4 fill", flush=True)
    lens = [300, 1, 77, 128]
    a = workloads.build("fp4 fill", 83, 300, lens, fill="nan", elem="nvfp4")
    z = workloads.build("fp4 fill", 83, 300, lens, fill="zero", elem="nvfp4")
    assert np.array_equal(bits(run(a)), bits(run(z)))


def test_fp4_tensor_scales():
    print("case fp4 scales", flush=True)
    w = workloads.build("fp4 scales", 84, 500, [500, 250, 3], elem="nvfp4")
    out = run(w, k_scale=0.375, v_scale=1.75, q_scale=0.5)
    w.q_scale = 0.5
    check(out, oracle_fp4(w, k_scale=0.375, v_scale=1.75), "fp4 k/v scales")


def test_fp4_nhd_view_equals_contiguous_bitwise():
    torch = _torch()
    print("case fp4 nhd", flush=True)
    w = workloads.build("fp4 nhd", 85, 600, [600, 311, 1, 40], elem="nvfp4")
    codes, scales = w.kv_to_device(DEV), w.scales_to_device(DEV)
    base = run(w, codes, scales)
    nhd_c = codes.permute(0, 3, 1, 2, 4).contiguous()          # [B, C, 2, 8, 64]
    nhd_s = scales.permute(0, 3, 1, 2, 4).contiguous()         # [B, C, 2, 8, 8]
    got = run(w, nhd_c.permute(0, 2, 3, 1, 4), nhd_s.permute(0, 2, 3, 1, 4))
    assert np.array_equal(bits(got), bits(base))
    # scale rows padded to 16 bytes
    padded = torch.zeros(scales.shape[:4] + (16,), dtype=torch.uint8, device=DEV)
    padded[..., :8] = scales
    got2 = run(w, codes, padded[..., :8])
    assert np.array_equal(bits(got2), bits(base))


def _paginate_fp4(codes, scales, lens, page_size, seed, spare=3):
    """Scatter each sequence's code and scale rows into pages of a shuffled
    pool (garbage in unused pages and rows); block table entries past a
    sequence's pages are -1."""
    torch = _torch()
    B, _, H, C, _ = codes.shape
    P = page_size
    max_pages = -(-C // P)
    num_pages = B * max_pages + spare
    rng = np.random.default_rng(seed)
    perm = rng.permutation(num_pages)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    cp = torch.randint(0, 256, (num_pages, 2, H, P, 64), dtype=torch.uint8, device=DEV,
                       generator=gen)
    sp = torch.full((num_pages, 2, H, P, 8), workloads.E4M3_NAN_CODE, dtype=torch.uint8,
                    device=DEV)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    for b in range(B):
        for j in range(-(-int(lens[b]) // P)):
            pid = int(perm[b * max_pages + j])
            table[b, j] = pid
            hi = min((j + 1) * P, C)
            cp[pid, :, :, :hi - j * P] = codes[b, :, :, j * P:hi]
            sp[pid, :, :, :hi - j * P] = scales[b, :, :, j * P:hi]
    return cp, sp, torch.from_numpy(table).to(DEV)


@pytest.mark.parametrize("page_size,chunk", [(32, 0), (64, 0), (256, 0), (32, 50)])
def test_fp4_paged_cache(page_size, chunk):
    print(f"case fp4 paged {page_size} chunk {chunk}", flush=True)
    lens = [700, 1, 0, 333, 64, 65, 31]
    w = workloads.build("fp4 paged", 86 + page_size, 700, lens, elem="nvfp4")
    cp, sp, table = _paginate_fp4(w.kv_to_device(DEV), w.scales_to_device(DEV),
                                  w.valid_lengths, page_size, seed=page_size)
    out = run(w, cp, sp, block_table=table, chunk_len=chunk)
    check(out, oracle_fp4(w), f"fp4 paged {page_size} chunk {chunk}")


@pytest.mark.parametrize("hq,hkv", [(64, 8), (28, 4), (8, 1)])
def test_fp4_head_counts_paged(hq, hkv):
    print(f"case fp4 heads {hq}/{hkv} paged", flush=True)
    w = workloads.build("fp4 heads paged", 91 + hq, 300, [300, 1, 0, 97, 64], fill="nan",
                        elem="nvfp4", q_heads=hq, kv_heads=hkv)
    cp, sp, table = _paginate_fp4(w.kv_to_device(DEV), w.scales_to_device(DEV),
                                  w.valid_lengths, 32, seed=hq)
    check(run(w, cp, sp, block_table=table), oracle_fp4(w), f"fp4 heads {hq}/{hkv} paged")


@pytest.mark.parametrize("hq,hkv", [(64, 8), (28, 4), (16, 16), (8, 1), (6, 2)])
def test_fp4_head_counts(hq, hkv):
    print(f"case fp4 heads {hq}/{hkv}", flush=True)
    w = workloads.build("fp4 heads", 87 + hq, 400, [400, 3, 0, 129, 260], fill="nan",
                        elem="nvfp4", q_heads=hq, kv_heads=hkv)
    check(run(w), oracle_fp4(w), f"fp4 heads {hq}/{hkv}")
    check(run(w, chunk_len=45), oracle_fp4(w), f"fp4 heads {hq}/{hkv} chunk 45")


@pytest.mark.parametrize("spec,chunk", [((3000, [3000, 1500, 2, 2999]), 0),
                                        ((700, [700, 1, 0, 333, 129, 64, 2, 700]), 0),
                                        ((700, [700, 1, 0, 333, 129, 64, 2, 700]), 7),
                                        ((40000, [40000, 20001]), 0)])
def test_fp4_launch_forms_agree_bitwise(spec, chunk):
    torch = _torch()
    g = _g()
    cap, lens = spec
    print(f"case fp4 forms {cap} chunk {chunk}", flush=True)
    w = workloads.build("fp4 forms", 88, cap, lens, fill="nan", elem="nvfp4")
    codes, scales = w.kv_to_device(DEV), w.scales_to_device(DEV)
    res = []
    for form in ("two", "single"):
        g.set_launch_form(form)
        out = torch.full(w.q.shape, float("nan"), dtype=torch.float16, device=DEV)
        res.append(bits(run(w, codes, scales, out=out, chunk_len=chunk)))
    assert np.array_equal(res[0], res[1])
    if cap <= 3000:
        check(torch.from_numpy(res[1].view(np.float16)), oracle_fp4(w), f"fp4 forms {cap}")


def test_fp4_paged_table_entries_beyond_lengths_and_invalid_ids():
    # Entries past a sequence's pages are never read (any value gives the
    # same bits); an out-of-range id inside a length reads zero codes and
    # scales (zero K and V rows) without a fault, other sequences unchanged.
    torch = _torch()
    print("case fp4 paged table", flush=True)
    w = workloads.build("fp4 paged table", 89, 256, [256, 200, 64], elem="nvfp4")
    codes, scales = w.kv_to_device(DEV), w.scales_to_device(DEV)
    cp, sp, table = _paginate_fp4(codes, scales, w.valid_lengths, 32, seed=9)
    base = bits(run(w, cp, sp, block_table=table))
    tail = table.clone()
    tail[tail < 0] = 1 << 30
    assert np.array_equal(bits(run(w, cp, sp, block_table=tail)), base)
    bad = table.clone()
    bad[1, 2] = cp.shape[0] + 7
    bad[1, 3] = -5
    got = run(w, cp, sp, block_table=bad)
    assert np.all(np.isfinite(got.float().cpu().numpy()))
    assert np.array_equal(bits(got)[[0, 2]], base[[0, 2]])
    # equal to the cache with sequence 1's rows 64..127 zeroed (codes and scales)
    codes0, scales0 = codes.clone(), scales.clone()
    codes0[1, :, :, 64:128] = 0
    scales0[1, :, :, 64:128] = 0
    cp0, sp0, table0 = _paginate_fp4(codes0, scales0, w.valid_lengths, 32, seed=9)
    assert np.array_equal(bits(got)[1], bits(run(w, cp0, sp0, block_table=table0))[1])


def test_fp4_graph_replays_match_eager_bitwise():
    # Captured calls hold only kernel nodes: every replay reproduces the eager
    # bits, with unrelated eager work between replays and with lengths
    # changed on the device.
    torch = _torch()
    g = _g()
    print("case fp4 graph", flush=True)
    ws = [workloads.build(f"fp4 graph {i}", 95 + i, 2048, lens, elem="nvfp4")
          for i, lens in enumerate([[2048, 5, 700], [1, 1500, 33], [0, 64, 2048]])]
    qs = [w.q_to_device(DEV) for w in ws]
    codes = [w.kv_to_device(DEV) for w in ws]
    scales = [w.scales_to_device(DEV) for w in ws]
    lens = [torch.from_numpy(w.seq_lens).to(DEV) for w in ws]
    outs = [torch.empty_like(q) for q in qs]

    def calls():
        for q, c, sc, ln, o in zip(qs, codes, scales, lens, outs):
            g.gqa_decode_fp4(q, c, sc, ln, out=o)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    s.synchronize()
    eager = [bits(o) for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            calls()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()
        graph.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for i, o in enumerate(outs):
            assert np.array_equal(bits(o), eager[i]), f"replay {rep}, call {i}"
    lens[0].copy_(torch.tensor([3, 2048, 0], dtype=torch.int32))
    graph.replay()
    torch.cuda.synchronize()
    ref = g.gqa_decode_fp4(qs[0], codes[0], scales[0],
                           torch.tensor([3, 2048, 0], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(bits(outs[0]), bits(ref))
