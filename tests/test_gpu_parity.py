"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar (element-wise over every output, rows of empty sequences included):
max |gpu - fp16(oracle)| <= 2e-3 and mean |gpu - fp16(oracle)| <= 2e-4,
where fp16(oracle) is one nearest-even rounding of the float64 result.
Exact properties of the method (length-1 rows, contents beyond a length,
power-of-two scaling of V, fixed-split reproducibility, independence of
batch entries and heads) are checked bitwise.
"""
import numpy as np
import pytest

import oracle
from oracle.reference import decode_ragged, round_fp16
import workloads

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL = 2e-3, 2e-4
DEV = "cuda:0"


def _torch():
    import torch
    return torch


def _g():
    import gqa_token_decode_amd as g
    return g


def _device_inputs(w, kv=None):
    torch = _torch()
    q = torch.from_numpy(w.q).to(DEV)
    lens = torch.from_numpy(w.seq_lens).to(DEV)
    if kv is None:
        kv = w.kv_to_device(DEV)
    return q, kv, lens


def run(w, chunk_len=0, kv=None, q_scale=None):
    torch = _torch()
    q, kv, lens = _device_inputs(w, kv)
    out = _g().gqa_decode(q, kv, lens, q_scale=w.q_scale if q_scale is None else q_scale,
                          chunk_len=chunk_len)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(got, ref64, label):
    ref16 = round_fp16(ref64).astype(np.float64)
    g64 = got.astype(np.float64)
    assert np.all(np.isfinite(g64)), f"{label}: non-finite output"
    d = np.abs(g64 - ref16)
    print(f"{label}: max|d|={d.max():.3e} mean|d|={d.mean():.3e} "
          f"max|gpu-oracle64|={np.abs(g64 - ref64).max():.3e}", flush=True)
    assert d.max() <= MAX_TOL, f"{label}: max |d| {d.max():.3e} at {np.unravel_index(d.argmax(), d.shape)}"
    assert d.mean() <= MEAN_TOL, f"{label}: mean |d| {d.mean():.3e}"


def oracle_of(w, q_scale=None):
    return decode_ragged(w.q, w.k_valid, w.v_valid, w.q_scale if q_scale is None else q_scale)


# ---------------------------------------------------------------- workloads
@pytest.mark.parametrize("name", workloads.SYNTHETIC)
def test_parity_synthetic_workloads_full_size(name):
    print(f"case {name}", flush=True)
    w = workloads.get(name)
    check(run(w), oracle_of(w), name)


@pytest.mark.parametrize("name", workloads.PAGE_SHAPES)
def test_parity_page_shapes(name):
    w = workloads.get(name)
    check(run(w), oracle_of(w), name)


@pytest.mark.parametrize("chunk_len,expected_chunks", [(1000, 1), (500, 2), (143, 7), (1, 1000)])
def test_forced_chunk_counts(chunk_len, expected_chunks):
    w = workloads.build("forced", 31, 1024, [1000], sigma_k=2.0)
    assert -(-1000 // chunk_len) == expected_chunks
    check(run(w, chunk_len=chunk_len), oracle_of(w), f"chunk_len={chunk_len}")


@pytest.mark.parametrize("chunk_len", [0, 7, 64])
def test_ragged_lengths_odd_capacity_and_clamping(chunk_len):
    lens = [0, 1, 2, 3, 4, 5, 15, 16, 17, 63, 64, 65, 255, 256, 257, -5, 1000]
    w = workloads.build("ragged", 32, 257, lens, fill="nan")
    got = run(w, chunk_len=chunk_len)
    for b in (0, 15):                    # L = 0 and L < 0: zero rows
        assert np.all(got[b] == 0)
    check(got, oracle_of(w), f"ragged chunk_len={chunk_len}")


@pytest.mark.parametrize("batch,cap,lo,hi", [(100, 512, 0, 300), (300, 128, 1, 64), (1000, 64, 0, 40)])
def test_large_batches_use_the_block_level_plan(batch, cap, lo, hi):
    # Batches above 64 locate their rows with workgroup-wide scans (and
    # above 256 with several passes over the lengths). The two short caches
    # (128 and 64 rows, 2400 and 8000 segments) also run two workgroups per
    # CU, and their combine kernels take more segments than workgroups
    # (each workgroup merges several in turn).
    w = workloads.build(f"batch{batch}", 42 + batch, cap,
                        lambda r: r.integers(lo, hi, batch, endpoint=True), fill="nan")
    got = run(w)
    for b in np.flatnonzero(w.valid_lengths == 0):
        assert np.all(got[b] == 0)
    check(got, oracle_of(w), f"batch {batch}")
    check(run(w, chunk_len=37), oracle_of(w), f"batch {batch}, chunk_len 37")


def test_long_sequence_with_one_row_tail():
    w = workloads.build("tail", 33, 65600, [65537, 65600, 1])
    check(run(w), oracle_of(w), "65537-row tail")


@pytest.mark.parametrize("q_scale", [0.0, -1.0, 4.0, 30.0])
def test_scale_variants(q_scale):
    w = workloads.build("scales", 34, 700, [700, 333, 129])
    check(run(w, q_scale=q_scale), oracle_of(w, q_scale), f"q_scale={q_scale}")


def test_extreme_magnitudes_stay_finite_within_the_fp32_error_bound():
    # V near the fp16 maximum and K scaled by 40: no overflow in the fp32
    # accumulators or the output conversion. Neither the absolute bar nor a
    # one-ulp bar applies here. Two near-equal weights on V values of opposite
    # sign leave an output far below the terms it sums (109 against 52000),
    # and the fp32 scores carry an absolute error that scales with their
    # terms' magnitude A = scale * max_i sum_d |q_d k_id| (about 360 here).
    # A weight is then off by that error relative to itself, and an output by
    # that much of mag = sum_i p_i |v_i| / sum_i p_i. The bound, with
    # sixteen fp32 roundings' worth of slack on the scores (measured: under
    # half of it): one fp16 ulp of the output plus 2^-20 (1 + A) mag, here
    # 3.4e-4 mag; a 1% error in a weight would exceed it about 30-fold.
    rng = np.random.default_rng(77)
    w = workloads.build("extreme", 77, 900, [900, 17, 1])
    k = [(kk.astype(np.float32) * 40).astype(np.float16) for kk in w.k_valid]
    v = [(np.sign(vv.astype(np.float32)) * 65504 * rng.uniform(0.5, 1.0, vv.shape))
         .astype(np.float16) for vv in w.v_valid]
    big = workloads.Workload("extreme big", w.q, w.seq_lens, w.capacity, w.q_scale, k, v)
    ref16 = round_fp16(oracle_of(big)).astype(np.float16)
    mag = decode_ragged(w.q, k, [np.abs(x) for x in v], w.q_scale)
    scale = w.q_scale / np.sqrt(128.0)
    A = np.zeros(mag.shape[:2])
    for b in range(w.batch):
        for h in range(32):
            A[b, h] = scale * np.max(np.abs(k[b][h // 4].astype(np.float64))
                                     @ np.abs(w.q[b, h].astype(np.float64)))
    # fp16 ulp of each reference value from its binade (np.spacing would
    # step past 65504 to infinity)
    r = np.abs(ref16.astype(np.float64))
    _, ex = np.frexp(r)
    ulp = np.where(r > 0, np.ldexp(1.0, np.maximum(ex - 1, -14) - 10), 2.0 ** -24)
    bound = ulp + 2.0 ** -20 * (1.0 + A[:, :, None]) * mag
    for chunk in (0, 64):
        got = run(big, chunk_len=chunk).astype(np.float64)
        assert np.all(np.isfinite(got))
        d = np.abs(got - ref16.astype(np.float64))
        print(f"extreme chunk {chunk}: max|d|={d.max():.3f}, max|d|/bound={np.max(d / bound):.3f}, "
              f"max|out|={np.abs(got).max():.0f}", flush=True)
        assert np.all(d <= bound), np.unravel_index(np.argmax(d / bound), d.shape)
        assert np.abs(got).max() > 30000                 # the case reaches the top binade


# ---------------------------------------------------------------- exact properties
def test_length_one_returns_v_row_bitwise():
    w = workloads.build("len1", 35, 96, [1, 1, 1], fill="nan")
    got = run(w)
    for b in range(3):
        for h in range(32):
            assert np.array_equal(got[b, h].view(np.uint16), w.v_valid[b][h // 4, 0].view(np.uint16))


@pytest.mark.parametrize("chunk_len", [0, 100])
def test_contents_beyond_length_have_no_effect_bitwise(chunk_len):
    base = workloads.build("fill", 36, 3000, [2999, 1500, 17, 3000])
    nanw = workloads.build("fill", 36, 3000, [2999, 1500, 17, 3000], fill="nan")
    torch = _torch()
    garbage = base.kv_to_device(DEV)
    # Random finite garbage (incl. huge values) beyond each length.
    for b, L in enumerate(base.seq_lens):
        tail = garbage[b, :, :, L:]
        tail.copy_((torch.randn_like(tail, dtype=torch.float32) * 3e4).to(torch.float16))
    a = run(base, chunk_len=chunk_len)
    b_ = run(nanw, chunk_len=chunk_len)
    c = run(base, chunk_len=chunk_len, kv=garbage)
    assert np.array_equal(a.view(np.uint16), b_.view(np.uint16))
    assert np.array_equal(a.view(np.uint16), c.view(np.uint16))


def test_repeated_runs_are_bitwise_identical():
    w = workloads.get("b8_c4096_nanfill")
    torch = _torch()
    q, kv, lens = _device_inputs(w)
    g = _g()
    outs = []
    for _ in range(5):
        outs.append(g.gqa_decode(q, kv, lens, q_scale=w.q_scale).cpu().numpy().view(np.uint16))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("chunk_len", [0, 256])
def test_batch_entries_are_independent(chunk_len):
    # With the lengths unchanged the split is unchanged, so replacing another
    # sequence's q/K/V must leave this sequence's output bit-identical. A
    # batch of one splits differently (pieces follow the flattened row
    # order), so it is held to the parity bar instead.
    w = workloads.build("indep", 37, 2048, [2048, 5, 1031, 777])
    full = run(w, chunk_len=chunk_len)
    other = workloads.build("indep2", 99, 2048, [2048, 5, 1031, 777], sigma_k=3.0)
    for b in range(w.batch):
        mix_q = other.q.copy()
        mix_q[b] = w.q[b]
        mix_k = [w.k_valid[i] if i == b else other.k_valid[i] for i in range(w.batch)]
        mix_v = [w.v_valid[i] if i == b else other.v_valid[i] for i in range(w.batch)]
        mixed = workloads.Workload("mixed", mix_q, w.seq_lens, w.capacity, w.q_scale, mix_k, mix_v)
        assert np.array_equal(run(mixed, chunk_len=chunk_len)[b].view(np.uint16),
                              full[b].view(np.uint16))
        one = workloads.Workload("one", w.q[b:b + 1], w.seq_lens[b:b + 1], w.capacity, w.q_scale,
                                 w.k_valid[b:b + 1], w.v_valid[b:b + 1])
        check(run(one, chunk_len=chunk_len), oracle_of(one), f"batch entry {b} alone")


@pytest.mark.parametrize("chunk_len", [0, 300])
def test_heads_are_independent_bitwise(chunk_len):
    # The split depends on the lengths only, and each query head is its own
    # MFMA column with its own softmax state: replacing the other KV heads'
    # K/V and the other groups' q must leave a group's outputs bit-identical,
    # and so must replacing one q head inside the group for its neighbours.
    lens = [1500, 700, 3, 1]
    w = workloads.build("heads indep", 41, 1500, lens)
    full = run(w, chunk_len=chunk_len)
    other = workloads.build("heads indep 2", 42, 1500, lens, sigma_k=3.0)
    for g in (0, 5):
        hs = slice(4 * g, 4 * g + 4)
        mix_q = other.q.copy()
        mix_q[:, hs] = w.q[:, hs]
        mix_k, mix_v = [], []
        for b in range(w.batch):
            k, v = other.k_valid[b].copy(), other.v_valid[b].copy()
            k[g], v[g] = w.k_valid[b][g], w.v_valid[b][g]
            mix_k.append(k)
            mix_v.append(v)
        mixed = workloads.Workload("heads mixed", mix_q, w.seq_lens, w.capacity, w.q_scale,
                                   mix_k, mix_v)
        got = run(mixed, chunk_len=chunk_len)
        assert np.array_equal(got[:, hs].view(np.uint16), full[:, hs].view(np.uint16)), g
        # one q head of the group replaced: its three neighbours are unchanged
        q1 = w.q.copy()
        q1[:, 4 * g + 1] = other.q[:, 4 * g + 1]
        one = workloads.Workload("one head", q1, w.seq_lens, w.capacity, w.q_scale,
                                 w.k_valid, w.v_valid)
        got1 = run(one, chunk_len=chunk_len)
        for h in (4 * g, 4 * g + 2, 4 * g + 3):
            assert np.array_equal(got1[:, h].view(np.uint16), full[:, h].view(np.uint16)), h
        check(got1, oracle_of(one), f"one q head replaced, group {g}")


def test_doubling_v_doubles_output_bitwise():
    # Doubling V doubles every fp32 accumulator exactly, so the fp16 result
    # doubles exactly wherever it is a normal fp16 number. (In the fp16
    # subnormal range, rounding 2x and doubling round(x) can differ.)
    w = workloads.build("v2", 38, 1500, [1500, 999])
    w2 = workloads.Workload("v2x", w.q, w.seq_lens, w.capacity, w.q_scale, w.k_valid,
                            [(v.astype(np.float32) * 2).astype(np.float16) for v in w.v_valid])
    a, b = run(w), run(w2)
    normal = np.abs(b.astype(np.float32)) >= 2.0 ** -13
    assert normal.mean() > 0.99
    doubled = (a.astype(np.float32) * 2).astype(np.float16)
    bad = int(np.sum(doubled.view(np.uint16)[normal] != b.view(np.uint16)[normal]))
    assert bad == 0, f"{bad} normal outputs differ from exactly doubled ones"


def test_permuting_positions_stays_within_bar():
    w = workloads.build("perm", 39, 2000, [2000, 1234])
    rng = np.random.default_rng(5)
    k2, v2 = [], []
    for b in range(w.batch):
        p = rng.permutation(w.k_valid[b].shape[1])
        k2.append(w.k_valid[b][:, p].copy())
        v2.append(w.v_valid[b][:, p].copy())
    wp = workloads.Workload("permuted", w.q, w.seq_lens, w.capacity, w.q_scale, k2, v2)
    ref = oracle_of(w)
    check(run(w), ref, "original order")
    check(run(wp), ref, "permuted order")


def test_constant_v_returns_constant_within_one_ulp():
    w = workloads.build("constv", 40, 900, [900, 450], sigma_k=2.0)
    rng = np.random.default_rng(6)
    const = rng.standard_normal((w.batch, 8, 1, 128)).astype(np.float16)
    vv = [np.broadcast_to(const[b], w.v_valid[b].shape).copy() for b in range(w.batch)]
    wc = workloads.Workload("constv", w.q, w.seq_lens, w.capacity, w.q_scale, w.k_valid, vv)
    got = run(wc).astype(np.float64)
    for b in range(w.batch):
        for h in range(32):
            c = const[b, h // 4, 0]
            ulp = np.spacing(np.abs(c)).astype(np.float64)
            assert np.all(np.abs(got[b, h] - c.astype(np.float64)) <= ulp)


# ---------------------------------------------------------------- API behaviour
def test_out_argument_and_side_stream():
    torch = _torch()
    g = _g()
    w = workloads.get("page_b4_c256")
    q, kv, lens = _device_inputs(w)
    out = torch.full_like(q, float("nan"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        r = g.gqa_decode(q, kv, lens, out=out, q_scale=w.q_scale)
    s.synchronize()
    assert r.data_ptr() == out.data_ptr()
    check(out.cpu().numpy(), oracle_of(w), "side stream")


def test_workspace_reuse_after_a_larger_call():
    # A large multi-chunk call leaves partials in the cached workspace; a
    # following small call must not see them.
    big = workloads.get("b2_c131072_long")
    small = workloads.build("small", 41, 4096, [4096, 3000, 1])
    run(big)
    check(run(small), oracle_of(small), "after large call")


@pytest.mark.parametrize("form", ["two", "single"])
def test_poisoned_partials_do_not_leak_into_the_next_call(form):
    # The library's cached workspace cannot be written from outside, so it
    # is poisoned through the API: a call whose valid rows hold NaN fills
    # every partial slot it uses with NaN. The next call on the same stream
    # (same workspace, same split) must return exactly the bits of the same
    # call on a fresh stream (another workspace).
    torch = _torch()
    g = _g()
    print(f"case poisoned partials {form}", flush=True)
    g.set_launch_form(form)
    try:
        w = workloads.build("poison", 43, 600, [600, 421, 2, 599], fill="nan")
        q, kv, lens = _device_inputs(w)
        bad = kv.clone()
        bad.view(torch.int16).fill_(0x7E00)                  # NaN everywhere
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        outs = []
        for chunk in (0, 37):
            with torch.cuda.stream(s1):
                poisoned = g.gqa_decode(q, bad, lens, chunk_len=chunk)
                after = g.gqa_decode(q, kv, lens, chunk_len=chunk)
            with torch.cuda.stream(s2):
                fresh = g.gqa_decode(q, kv, lens, chunk_len=chunk)
            torch.cuda.synchronize()
            assert np.isnan(poisoned.float().cpu().numpy()).all()
            a = after.view(torch.int16).cpu().numpy()
            f = fresh.view(torch.int16).cpu().numpy()
            assert np.array_equal(a, f), f"chunk {chunk}"
            outs.append(after.cpu().numpy())
        check(outs[0], oracle_of(w), f"after poisoned partials ({form})")
    finally:
        g.set_launch_form("auto")


def test_workspace_limit_reports_allocation_failure(monkeypatch):
    # A call that needs a new workspace larger than GQA_DECODE_WORKSPACE_LIMIT
    # fails with GQA_ERR_ALLOC and enqueues nothing; without the limit the
    # same call on the same stream then succeeds.
    torch = _torch()
    g = _g()
    print("case workspace limit", flush=True)
    w = workloads.build("ws limit", 44, 2048, [2048, 1500])
    q, kv, lens = _device_inputs(w)
    out = torch.full(q.shape, float("nan"), dtype=torch.float16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    monkeypatch.setenv("GQA_DECODE_WORKSPACE_LIMIT", "4096")
    with torch.cuda.stream(s):
        with pytest.raises(g.GqaDecodeError) as err:
            g.gqa_decode(q, kv, lens, out=out)
    assert err.value.status == -7 and "GQA_DECODE_WORKSPACE_LIMIT" in str(err.value)
    torch.cuda.synchronize()
    assert np.isnan(out.float().cpu().numpy()).all()          # nothing was enqueued
    monkeypatch.delenv("GQA_DECODE_WORKSPACE_LIMIT")
    with torch.cuda.stream(s):
        g.gqa_decode(q, kv, lens, out=out)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle_of(w), "after the workspace limit is lifted")


def test_errors_are_raised_on_gpu():
    torch = _torch()
    g = _g()
    w = workloads.get("page_b1_c64")
    q, kv, lens = _device_inputs(w)
    with pytest.raises(g.GqaDecodeError) as e:
        g.gqa_decode(q, kv, lens, out=q)             # out aliases q
    assert e.value.status == -4
    buf = torch.empty(q.numel() + 4, dtype=torch.float16, device=DEV)
    qmis = buf[4:].view(q.shape)                     # 8-byte offset: not 16-byte aligned
    qmis.copy_(q)
    with pytest.raises(g.GqaDecodeError) as e:
        g.gqa_decode(qmis, kv, lens)
    assert e.value.status == -3
    assert g.workspace_bytes(64, 16384) > 0


def test_kernel_timer_reports_kernel_time():
    torch = _torch()
    g = _g()
    w = workloads.get("b32_c8192_qs05")
    q, kv, lens = _device_inputs(w)
    g.gqa_decode(q, kv, lens, q_scale=w.q_scale)
    with g.KernelTimer() as t:
        for _ in range(3):
            g.gqa_decode(q, kv, lens, q_scale=w.q_scale)
    torch.cuda.synchronize()
    # capacity 8192: the automatic choice runs two kernels
    assert t.calls == 3 and t.pieces_ms > 0 and t.combine_ms > 0
    g.set_launch_form("single")
    try:
        with g.KernelTimer() as t:
            g.gqa_decode(q, kv, lens, q_scale=w.q_scale)
        torch.cuda.synchronize()
    finally:
        g.set_launch_form("auto")
    assert t.calls == 1 and t.pieces_ms > 0 and t.combine_ms == 0
