"""Pins for the CPU oracle against things other than itself.

Each check is chosen so that a plausible slip in the oracle fails at least
one of them: a dropped 1/sqrt(128) or q_scale (brute force, SDPA, closed
forms), a wrong query-to-KV head map (SDPA with enable_gqa, per-group
constants), K and V swapped (length-1 closed form), an off-by-one length
or rows read past the length (NaN beyond L, length-1/2 forms), a sign
error in the scale (large +/- q_scale picks argmax / argmin), a missing
max subtraction (large q_scale overflows), and double rounding in the final
fp16 conversion.

Definition followed: FlashInfer PR #5052 analysis page ("SM110 FP16 GQA
decode"), section 1 docstring and section 3 SDPA comparator.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from oracle.reference import decode, decode_head, decode_ragged, effective_scale, round_fp16
import workloads

H, G, D = 32, 8, 128
HERE = os.path.dirname(os.path.abspath(__file__))


def _rand_inputs(rng, B, C, sigma_k=1.0):
    q = rng.standard_normal((B, H, D)).astype(np.float16)
    kv = rng.standard_normal((B, 2, G, C, D)).astype(np.float16)
    kv[:, 0] = (kv[:, 0].astype(np.float32) * sigma_k).astype(np.float16)
    return q, kv


# ---------------------------------------------------------------- P1 brute
@pytest.mark.parametrize("C", [1, 2, 3, 5, 8])
def test_matches_fsum_brute_force_every_length(C):
    rng = np.random.default_rng(100 + C)
    lens = list(range(C + 1)) + [-3, C + 5]      # every L in [0, C] plus clamping
    B = len(lens)
    q, kv = _rand_inputs(rng, B, C)
    qf = q.astype(np.float64).tolist()
    kvf = kv.astype(np.float64).tolist()
    for q_scale in (0.0, 0.5, 1.0, 3.7, -1.0):
        got = decode(q, kv, np.array(lens, np.int32), q_scale)
        ref = np.array(brute.decode_brute(qf, kvf, lens, q_scale))
        scale = max(1.0, float(np.abs(ref).max()))
        assert np.abs(got - ref).max() <= 1e-12 * scale, (C, q_scale)


def test_matches_mpmath_at_40_digits():
    rng = np.random.default_rng(7)
    q, kv = _rand_inputs(rng, 1, 9, sigma_k=2.0)
    lens = np.array([9], np.int32)
    for q_scale in (1.0, 2.5):
        got = decode(q, kv, lens, q_scale)
        for h in (0, 5, 31):
            g = h // 4
            ref = brute.decode_head_mp(q[0, h].astype(float).tolist(),
                                       kv[0, 0, g].astype(float).tolist(),
                                       kv[0, 1, g].astype(float).tolist(), q_scale)
            assert np.abs(got[0, h] - np.array(ref)).max() <= 1e-14


# ---------------------------------------------------------------- P2 library routine
def _sdpa_f64(q, kv, lens, q_scale):
    import torch
    import torch.nn.functional as F

    B, C = q.shape[0], kv.shape[3]
    tq = torch.from_numpy(q.astype(np.float64)).unsqueeze(2)          # [B,32,1,128]
    tk = torch.from_numpy(kv[:, 0].astype(np.float64))                # [B,8,C,128]
    tv = torch.from_numpy(kv[:, 1].astype(np.float64))
    L = torch.from_numpy(np.clip(np.asarray(lens, np.int64), 0, C))
    mask = (torch.arange(C)[None, :] < L[:, None])[:, None, None, :]  # [B,1,1,C]
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                       scale=effective_scale(q_scale), enable_gqa=True)
    return o.squeeze(2).numpy()


@pytest.mark.parametrize("name", workloads.PAGE_SHAPES)
def test_matches_torch_sdpa_float64_page_shapes(name):
    w = workloads.get(name)
    kv = w.dense_kv()
    got = decode(w.q, kv, w.seq_lens, w.q_scale)
    ref = _sdpa_f64(w.q, kv, w.seq_lens, w.q_scale)
    assert np.abs(got - ref).max() <= 1e-12


def test_matches_torch_sdpa_float64_odd_capacity():
    rng = np.random.default_rng(11)
    q, kv = _rand_inputs(rng, 3, 257, sigma_k=2.0)
    lens = np.array([257, 1, 130], np.int32)
    for q_scale in (1.0, 0.5, -2.0):
        got = decode(q, kv, lens, q_scale)
        ref = _sdpa_f64(q, kv, lens, q_scale)
        assert np.abs(got - ref).max() <= 1e-12


def test_sdpa_and_oracle_agree_that_empty_prefix_gives_zeros():
    import torch

    rng = np.random.default_rng(12)
    q, kv = _rand_inputs(rng, 2, 16)
    lens = np.array([0, 16], np.int32)
    got = decode(q, kv, lens, 1.0)
    assert np.all(got[0] == 0.0)
    ref = _sdpa_f64(q, kv, lens, 1.0)
    if not np.all(np.isfinite(ref[0])):
        pytest.skip(f"torch {torch.__version__} SDPA returns non-finite rows for an empty mask")
    assert np.all(ref[0] == 0.0)
    assert np.abs(got[1] - ref[1]).max() <= 1e-12


# ---------------------------------------------------------------- P3 closed forms
def test_length_one_returns_v_row_exactly():
    rng = np.random.default_rng(13)
    q, kv = _rand_inputs(rng, 2, 5)
    got = decode(q, kv, np.array([1, 1], np.int32), 3.0)
    for b in range(2):
        for h in range(H):
            assert np.array_equal(got[b, h], kv[b, 1, h // 4, 0].astype(np.float64))


def test_length_two_is_a_sigmoid_mix():
    rng = np.random.default_rng(14)
    q, kv = _rand_inputs(rng, 1, 4)
    q_scale = 1.7
    got = decode(q, kv, np.array([2], np.int32), q_scale)
    c = float(np.float32(q_scale)) / math.sqrt(128)
    for h in range(H):
        g = h // 4
        qv = q[0, h].astype(float)
        k0, k1 = kv[0, 0, g, 0].astype(float), kv[0, 0, g, 1].astype(float)
        d = c * (math.fsum(qv * k0) - math.fsum(qv * k1))   # s0 - s1
        w0 = 1.0 / (1.0 + math.exp(-d))
        w1 = 1.0 / (1.0 + math.exp(d))
        ref = w0 * kv[0, 1, g, 0].astype(float) + w1 * kv[0, 1, g, 1].astype(float)
        assert np.abs(got[0, h] - ref).max() <= 1e-13


def test_zero_scale_gives_mean_of_valid_rows():
    rng = np.random.default_rng(15)
    q, kv = _rand_inputs(rng, 2, 40)
    lens = np.array([37, 40], np.int32)
    got = decode(q, kv, lens, 0.0)
    for b in range(2):
        for g in range(G):
            V = kv[b, 1, g, :lens[b]].astype(float)
            mean = np.array([math.fsum(V[:, d]) / lens[b] for d in range(D)])
            for h in range(4 * g, 4 * g + 4):
                assert np.abs(got[b, h] - mean).max() <= 1e-14


def test_equal_keys_give_mean_of_valid_rows():
    rng = np.random.default_rng(16)
    q, kv = _rand_inputs(rng, 1, 33)
    kv[0, 0, :, :, :] = kv[0, 0, :, :1, :]           # every key row equal
    got = decode(q, kv, np.array([33], np.int32), 2.0)
    for g in range(G):
        V = kv[0, 1, g].astype(float)
        mean = np.array([math.fsum(V[:, d]) / 33 for d in range(D)])
        assert np.abs(got[0, 4 * g:4 * g + 4] - mean).max() <= 1e-14


def test_constant_v_rows_return_the_constant():
    rng = np.random.default_rng(17)
    q, kv = _rand_inputs(rng, 2, 64, sigma_k=2.0)
    const = rng.standard_normal((2, G, 1, D)).astype(np.float16)
    kv[:, 1] = np.broadcast_to(const, (2, G, 64, D))
    got = decode(q, kv, np.array([64, 50], np.int32), 1.0)
    for b in range(2):
        for h in range(H):
            ref = const[b, h // 4, 0].astype(float)
            assert np.abs(got[b, h] - ref).max() <= 1e-15 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_large_scale_selects_extreme_score_row(sign):
    # With a huge |q_scale| the softmax becomes a hard max over q.k (or a
    # hard min for a negative scale). Integer-valued q and K make the dot
    # products exact and distinct.
    rng = np.random.default_rng(18)
    C = 24
    q = rng.integers(-3, 4, (1, H, D)).astype(np.float16)
    kv = np.zeros((1, 2, G, C, D), np.float16)
    kv[0, 0] = rng.integers(-3, 4, (G, C, D)).astype(np.float16)
    kv[0, 1] = rng.standard_normal((G, C, D)).astype(np.float16)
    got = decode(q, kv, np.array([C], np.int32), sign * 1e5)
    for h in range(H):
        g = h // 4
        dots = [int(np.dot(q[0, h].astype(np.int64), kv[0, 0, g, i].astype(np.int64)))
                for i in range(C)]
        order = sorted(range(C), key=lambda i: sign * dots[i], reverse=True)
        if sign * dots[order[0]] == sign * dots[order[1]]:
            continue  # tie: the max is shared by two rows
        assert np.abs(got[0, h] - kv[0, 1, g, order[0]].astype(float)).max() <= 1e-12


def test_each_query_head_reads_kv_head_h_div_4():
    # V of KV head g is the constant g+1; output head h must read h//4 + 1.
    rng = np.random.default_rng(19)
    q, kv = _rand_inputs(rng, 1, 8)
    for g in range(G):
        kv[0, 1, g] = np.float16(g + 1)
    got = decode(q, kv, np.array([8], np.int32), 1.0)
    for h in range(H):
        assert np.abs(got[0, h] - float(h // 4 + 1)).max() <= 1e-14


# ---------------------------------------------------------------- P4 invariants
def test_permuting_valid_positions_is_invariant():
    rng = np.random.default_rng(20)
    q, kv = _rand_inputs(rng, 2, 100)
    lens = np.array([100, 77], np.int32)
    ref = decode(q, kv, lens, 1.0)
    kv2 = kv.copy()
    for b in range(2):
        perm = rng.permutation(lens[b])
        kv2[b][:, :, :lens[b]] = kv[b][:, :, perm]
    got = decode(q, kv2, lens, 1.0)
    assert np.abs(got - ref).max() <= 1e-12


def test_contents_beyond_length_have_no_effect():
    rng = np.random.default_rng(21)
    q, kv = _rand_inputs(rng, 3, 50)
    lens = np.array([1, 25, 49], np.int32)
    ref = decode(q, kv, lens, 1.0)
    kv2 = kv.copy()
    for b in range(3):
        kv2[b, :, :, lens[b]:] = np.float16(np.nan)
        kv2[b, 0, :, lens[b]:][..., ::7] = np.float16(np.inf)
    got = decode(q, kv2, lens, 1.0)
    assert np.array_equal(got, ref)


def test_scaling_v_by_two_scales_output_exactly():
    rng = np.random.default_rng(22)
    q, kv = _rand_inputs(rng, 1, 64)
    lens = np.array([61], np.int32)
    ref = decode(q, kv, lens, 1.0)
    kv2 = kv.copy()
    kv2[:, 1] *= np.float16(2)
    assert np.array_equal(decode(q, kv2, lens, 1.0), 2.0 * ref)


def test_doubling_k_and_halving_scale_is_exact():
    rng = np.random.default_rng(23)
    q, kv = _rand_inputs(rng, 1, 64)
    lens = np.array([64], np.int32)
    ref = decode(q, kv, lens, 1.5)
    kv2 = kv.copy()
    kv2[:, 0] *= np.float16(2)
    assert np.array_equal(decode(q, kv2, lens, 0.75), ref)


def test_batch_entries_are_independent_and_ragged_form_agrees():
    w = workloads.get("page_b4_c256")
    full = decode(w.q, w.dense_kv(), w.seq_lens, w.q_scale)
    rag = decode_ragged(w.q, w.k_valid, w.v_valid, w.q_scale)
    assert np.array_equal(full, rag)
    for b in range(w.batch):
        one = decode(w.q[b:b + 1], w.dense_kv()[b:b + 1], w.seq_lens[b:b + 1], w.q_scale)
        assert np.array_equal(one[0], full[b])


def test_sampled_rows_match_full_decode():
    w = workloads.get("page_b4_c256")
    kv = w.dense_kv()
    full = decode(w.q, kv, w.seq_lens, w.q_scale)
    rows = [(0, 3), (2, 17), (3, 31)]
    part = decode(w.q, kv, w.seq_lens, w.q_scale, rows=rows)
    for b, h in rows:
        assert np.array_equal(part[b, h], full[b, h])


# ---------------------------------------------------------------- final rounding
def test_fp16_rounding_is_single_and_nearest_even():
    # 1 + 2^-11 + 2^-40 lies just above the midpoint of 1 and 1 + 2^-10:
    # a direct conversion rounds up; going through float32 would first drop
    # the 2^-40 and then tie-break down to 1.0.
    x = 1.0 + 2.0 ** -11 + 2.0 ** -40
    assert round_fp16(np.array([x])).view(np.uint16)[0] == 0x3C01
    assert np.float16(np.float32(x)).view(np.uint16) == 0x3C00
    assert round_fp16(np.array([1.0 + 2.0 ** -11])).view(np.uint16)[0] == 0x3C00  # tie -> even
    assert round_fp16(np.array([65520.0]))[0] == np.inf                            # overflow


# ---------------------------------------------------------------- inputs
def test_generator_is_reproducible_and_follows_recipe():
    a, b = workloads.get("b8_c4096_nanfill"), workloads.get("b8_c4096_nanfill")
    assert np.array_equal(a.q.view(np.uint16), b.q.view(np.uint16))
    assert np.array_equal(a.seq_lens, b.seq_lens)
    for x, y in zip(a.k_valid, b.k_valid):
        assert np.array_equal(x.view(np.uint16), y.view(np.uint16))
    assert a.batch == 8 and a.capacity == 4096 and a.fill == "nan"
    assert np.all((a.seq_lens >= 1) & (a.seq_lens <= 4096))
    kv = a.dense_kv()
    for i in range(8):
        L = int(a.seq_lens[i])
        assert np.all(np.isnan(kv[i, :, :, L:].astype(np.float32)))
        assert not np.any(np.isnan(kv[i, :, :, :L].astype(np.float32)))


def test_skewed_lengths_recipe():
    rng = np.random.default_rng(4)
    lens = workloads._cfg4_lengths(rng)
    assert lens.shape == (64,)
    assert np.sum((lens >= 16) & (lens <= 512)) == 58
    assert np.sum((lens >= 8192) & (lens <= 16384)) == 6


def test_page_shapes_match_golden_fixture():
    with open(os.path.join(HERE, "golden", "page4_shapes.json")) as f:
        gold = json.load(f)
    for s in gold["shapes"]:
        w = workloads.get(s["name"])
        assert w.batch == s["batch"] and w.capacity == s["capacity"]
        assert w.seq_lens.tolist() == s["lengths"]


# ---------------------------------------------------------------- extension: bf16, K/V scales
def test_bf16_widening_matches_torch_for_every_pattern():
    import torch

    from oracle.formats import bf16_to_f64

    bits = np.arange(1 << 16, dtype=np.uint16)
    got = bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_rounding_matches_torch_on_float32_values():
    import torch

    from oracle.formats import round_bf16

    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # subnormal range
        (rng.standard_normal(2000) * 1e38).astype(np.float32),      # near overflow
        np.float32([0.0, -0.0, 1e-45, -1e-45, 3.3895e38]),
    ])
    # exact ties: midpoints between neighbouring bfloat16 numbers
    lo = rng.integers(0x0080, 0x7F00, 5000).astype(np.uint32)
    ties = ((lo << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    got = round_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (got == ref).all()


def test_bf16_rounding_is_direct_from_float64():
    from oracle.formats import bf16_to_f64, round_bf16

    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7; 2^-40 above it must round
    # up, while a float32 step would first drop the 2^-40 and then tie to 1.
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8 + 2.0 ** -40)])
    assert bf16_to_f64(round_bf16(x)).tolist() == [1 + 2.0 ** -7, 1.0, 1 + 2 * 2.0 ** -7,
                                                    -(1 + 2.0 ** -7)]
    assert np.isinf(bf16_to_f64(round_bf16(np.array([3.5e38, -3.5e38])))).all()
    assert bf16_to_f64(round_bf16(np.array([2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134]))).tolist() \
        == [2.0 ** -133, 0.0, 2.0 ** -132]


@pytest.mark.parametrize("C", [1, 3, 6])
def test_scales_match_brute_force_with_scaled_rows(C):
    # brute force multiplies every stored K and V element by its scale first;
    # the oracle folds k_scale into the score scale and v_scale into the output
    rng = np.random.default_rng(200 + C)
    lens = list(range(C + 1))
    q, kv = _rand_inputs(rng, len(lens), C)
    qf, kvf = q.astype(np.float64).tolist(), kv.astype(np.float64).tolist()
    for q_scale, k_scale, v_scale in ((1.0, 0.37, 1.0), (0.5, 1.0, -2.5), (1.3, 3.1, 0.011)):
        got = decode(q, kv, np.array(lens, np.int32), q_scale, k_scale=k_scale, v_scale=v_scale)
        ref = np.array(brute.decode_brute(qf, kvf, lens, q_scale, k_scale=k_scale,
                                          v_scale=v_scale))
        assert np.abs(got - ref).max() <= 1e-12 * max(1.0, float(np.abs(ref).max()))


def test_scales_match_torch_sdpa_on_scaled_tensors():
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(12)
    B, C = 3, 70
    q, kv = _rand_inputs(rng, B, C)
    lens = np.array([70, 5, 33], np.int32)
    ks, vs = 0.8125, 1.75
    tq = torch.from_numpy(q.astype(np.float64)).unsqueeze(2)
    tk = torch.from_numpy(kv[:, 0].astype(np.float64)) * float(np.float32(ks))
    tv = torch.from_numpy(kv[:, 1].astype(np.float64)) * float(np.float32(vs))
    mask = (torch.arange(C)[None, :] < torch.from_numpy(lens.astype(np.int64))[:, None])[:, None, None, :]
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=effective_scale(0.9),
                                         enable_gqa=True).squeeze(2).numpy()
    got = decode(q, kv, lens, 0.9, k_scale=ks, v_scale=vs)
    assert np.abs(got - ref).max() <= 1e-12


def test_bf16_inputs_match_sdpa_on_widened_values():
    import torch
    import torch.nn.functional as F

    from oracle.formats import bf16_to_f64

    rng = np.random.default_rng(13)
    B, C = 2, 40
    qb = torch.from_numpy(rng.standard_normal((B, H, D)).astype(np.float32)).to(torch.bfloat16)
    kvb = torch.from_numpy(rng.standard_normal((B, 2, G, C, D)).astype(np.float32)).to(torch.bfloat16)
    q64 = bf16_to_f64(qb.view(torch.int16).numpy().view(np.uint16))
    kv64 = bf16_to_f64(kvb.view(torch.int16).numpy().view(np.uint16))
    lens = np.array([40, 17], np.int32)
    got = decode(q64, kv64, lens, 1.0)
    mask = (torch.arange(C)[None, :] < torch.from_numpy(lens.astype(np.int64))[:, None])[:, None, None, :]
    ref = F.scaled_dot_product_attention(qb.double().unsqueeze(2), kvb[:, 0].double(),
                                         kvb[:, 1].double(), attn_mask=mask,
                                         scale=effective_scale(1.0), enable_gqa=True)
    assert np.abs(got - ref.squeeze(2).numpy()).max() <= 1e-12


def test_e4m3_decoding_matches_torch_for_every_code():
    import torch

    from oracle.formats import e4m3_to_f64

    codes = np.arange(256, dtype=np.uint8)
    got = e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert ((got == ref) | (np.isnan(got) & np.isnan(ref))).all()
    # fixed points of the format: largest finite, smallest subnormal and
    # normal, one, signed zero, NaN codes
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert got[0x38] == 1.0 and got[0xB8] == -1.0
    assert got[0x80] == 0.0 and np.signbit(got[0x80])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.isfinite(np.delete(got, [0x7F, 0xFF])).all()


def test_e4m3_cache_matches_sdpa_on_dequantised_tensors():
    import torch
    import torch.nn.functional as F

    from oracle.formats import e4m3_to_f64

    w = workloads.build("e4m3 pin", 57, 90, [90, 33, 1], elem="e4m3")
    kv = w.dense_kv()
    kv64 = e4m3_to_f64(kv)
    got = decode(w.q, kv64, w.seq_lens, 1.0, k_scale=w.k_scale, v_scale=w.v_scale)
    tkv = torch.from_numpy(kv).view(torch.float8_e4m3fn).to(torch.float64)
    tk, tv = tkv[:, 0] * w.k_scale, tkv[:, 1] * w.v_scale
    C = kv.shape[3]
    mask = (torch.arange(C)[None, :] < torch.from_numpy(w.seq_lens.astype(np.int64))[:, None])[:, None, None, :]
    ref = F.scaled_dot_product_attention(torch.from_numpy(w.q.astype(np.float64)).unsqueeze(2),
                                         tk, tv, attn_mask=mask, scale=effective_scale(1.0),
                                         enable_gqa=True).squeeze(2).numpy()
    assert np.abs(got - ref).max() <= 1e-12


# ---------------------------------------------------------------- block-scaled FP4
# The FP4 E2M1 element format as tabulated in the OCP Microscaling Formats
# (MX) v1.0 specification (FP4 E2M1 section): the eight non-negative codes
# and their values; codes 8..15 are their negatives.
E2M1_TABLE = {0b0000: 0.0, 0b0001: 0.5, 0b0010: 1.0, 0b0011: 1.5,
              0b0100: 2.0, 0b0101: 3.0, 0b0110: 4.0, 0b0111: 6.0}


def _e2m1_from_table(code):
    v = E2M1_TABLE[code & 7]
    return -v if code & 8 else v


def test_e2m1_decoding_matches_the_format_table():
    from oracle.formats import e2m1_to_f64

    got = e2m1_to_f64(np.arange(16))
    for c in range(16):
        assert got[c] == _e2m1_from_table(c), c
    assert np.signbit(got[8]) and not np.signbit(got[0])


def test_block_scaled_fp4_rows_match_element_by_element_brute_force():
    # Each element decoded on its own from the table, its byte and nibble,
    # and its block's scale (torch's E4M3 decoding): catches a swapped nibble
    # order, a wrong block size or a scale applied to the wrong block.
    import torch

    from oracle.formats import nvfp4_to_f64

    rng = np.random.default_rng(901)
    packed = rng.integers(0, 256, (3, 5, 64), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (3, 5, 8), dtype=np.uint8)   # finite, positive codes
    scales[0, 0] = [0x38, 0x40, 0x30, 0x48, 0x01, 0x7E, 0x39, 0x08]
    got = nvfp4_to_f64(packed, scales)
    sc = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for a in range(3):
        for r in range(5):
            for i in range(128):
                byte = int(packed[a, r, i // 2])
                code = byte & 15 if i % 2 == 0 else byte >> 4
                want = _e2m1_from_table(code) * sc[a, r, i // 16]
                assert got[a, r, i] == want, (a, r, i)
    # one row written out: byte 0x21 holds elements (0.5, 1.0), byte 0xF7
    # holds (6, -6); scales 2 and 0.5 for the first two blocks
    row = np.zeros(64, np.uint8)
    row[0], row[1], row[8] = 0x21, 0xF7, 0x93
    scl = np.zeros(8, np.uint8)
    scl[0], scl[1] = 0x40, 0x30
    v = nvfp4_to_f64(row, scl)
    assert list(v[:4]) == [1.0, 2.0, 12.0, -12.0]
    assert list(v[16:18]) == [0.75, -0.25] and not v[4:16].any() and not v[18:].any()


def test_block_scaled_fp4_encoding_keeps_representable_values():
    # Input preparation check: a row whose blocks hold exact E2M1 multiples
    # of an E4M3 scale, with the block maximum at 6 x scale, is encoded and
    # decoded back unchanged.
    from oracle.formats import nvfp4_to_f64

    rng = np.random.default_rng(902)
    mags = np.array(sorted(E2M1_TABLE.values()))
    x = rng.choice(mags, (4, 128)) * rng.choice([-1.0, 1.0], (4, 128))
    x[:, ::16] = 6.0
    blk_scale = np.repeat(rng.choice([0.25, 0.5, 1.0, 1.5, 3.0], (4, 8)), 16, axis=1)
    x = (x * blk_scale).astype(np.float32)
    packed, scales = workloads.encode_nvfp4(x)
    assert np.array_equal(nvfp4_to_f64(packed, scales), x.astype(np.float64))


def test_block_scaled_fp4_cache_matches_sdpa_on_dequantised_tensors():
    import torch
    import torch.nn.functional as F

    from oracle.formats import nvfp4_to_f64

    w = workloads.build("nvfp4 pin", 58, 70, [70, 17, 1, 0], elem="nvfp4", fill="nan")
    kv64 = nvfp4_to_f64(w.dense_kv(), w.dense_scales())
    assert kv64.shape == (4, 2, 8, 70, 128)
    got = decode(w.q, kv64, w.seq_lens, 1.0)
    # SDPA on tensors dequantised with the table and torch's E4M3 decoding;
    # NaN rows beyond the lengths are masked (and zeroed, as SDPA would still
    # multiply them by a zero weight)
    table = np.array([_e2m1_from_table(c) for c in range(16)])
    raw = w.dense_kv().astype(np.int64)
    codes = np.stack([raw & 15, raw >> 4], axis=-1).reshape(raw.shape[:-1] + (128,))
    sc = torch.from_numpy(w.dense_scales()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    deq = table[codes] * np.repeat(sc, 16, axis=-1)
    C = deq.shape[3]
    valid = np.arange(C)[None, :] < w.seq_lens.astype(np.int64)[:, None]
    deq = np.where(valid[:, None, None, :, None], deq, 0.0)
    mask = torch.from_numpy(valid)[:, None, None, :]
    ref = F.scaled_dot_product_attention(torch.from_numpy(w.q.astype(np.float64)).unsqueeze(2),
                                         torch.from_numpy(deq[:, 0]), torch.from_numpy(deq[:, 1]),
                                         attn_mask=mask, scale=effective_scale(1.0),
                                         enable_gqa=True).squeeze(2).numpy()
    ref[3] = 0.0                       # empty prefix: zeros (SDPA gives NaN for a fully masked row)
    assert np.abs(got - ref).max() <= 1e-12


# ---------------------------------------------------------------- other head counts
# The page fixes 32 query and 8 KV heads; the library also takes other
# counts (Hq a multiple of Hkv, Hq / Hkv <= 8), with query head h reading KV
# head h // (Hq / Hkv) as SDPA's enable_gqa does for any ratio.
HEAD_COUNTS = [(64, 8), (28, 4), (16, 16), (32, 16), (8, 1), (40, 8), (12, 4), (1, 1)]


def _rand_heads(rng, B, C, Hq, Hkv):
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    kv = rng.standard_normal((B, 2, Hkv, C, D)).astype(np.float16)
    return q, kv


@pytest.mark.parametrize("Hq,Hkv", HEAD_COUNTS)
def test_other_head_counts_match_brute_force(Hq, Hkv):
    rng = np.random.default_rng(700 + Hq + Hkv)
    C = 3
    lens = [0, 1, 2, 3, 7]
    q, kv = _rand_heads(rng, len(lens), C, Hq, Hkv)
    got = decode(q, kv, np.array(lens, np.int32), 1.3)
    ref = np.array(brute.decode_brute(q.astype(np.float64).tolist(),
                                      kv.astype(np.float64).tolist(), lens, 1.3,
                                      n_kv_heads=Hkv))
    assert got.shape == (len(lens), Hq, D)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, float(np.abs(ref).max()))


@pytest.mark.parametrize("Hq,Hkv", HEAD_COUNTS)
def test_other_head_counts_match_torch_sdpa(Hq, Hkv):
    rng = np.random.default_rng(800 + Hq + Hkv)
    q, kv = _rand_heads(rng, 3, 67, Hq, Hkv)
    lens = np.array([67, 1, 40], np.int32)
    got = decode(q, kv, lens, 0.75)
    ref = _sdpa_f64(q, kv, lens, 0.75)
    assert np.abs(got - ref).max() <= 1e-12
    # the ragged form reads the same heads
    k_valid = [kv[b, 0, :, :lens[b]] for b in range(3)]
    v_valid = [kv[b, 1, :, :lens[b]] for b in range(3)]
    assert np.abs(decode_ragged(q, k_valid, v_valid, 0.75) - got).max() <= 1e-15


@pytest.mark.parametrize("Hq,Hkv", [(64, 8), (28, 4), (8, 1), (12, 4)])
def test_other_head_counts_use_contiguous_groups(Hq, Hkv):
    # V of KV head g is the constant g + 1: query head h must return
    # h // (Hq / Hkv) + 1 (a strided map h % Hkv would differ).
    rng = np.random.default_rng(900 + Hq)
    q, kv = _rand_heads(rng, 1, 5, Hq, Hkv)
    for g in range(Hkv):
        kv[0, 1, g] = np.float16(g + 1)
    got = decode(q, kv, np.array([5], np.int32), 1.0)
    grp = Hq // Hkv
    for h in range(Hq):
        assert np.abs(got[0, h] - float(h // grp + 1)).max() <= 1e-14


def test_one_query_head_per_kv_head_is_per_head_attention():
    # Hq == Hkv: every head attends over its own K/V, the textbook
    # multi-head case, written out here with a softmax per head.
    rng = np.random.default_rng(901)
    Hh, C = 6, 9
    q, kv = _rand_heads(rng, 1, C, Hh, Hh)
    got = decode(q, kv, np.array([C], np.int32), 1.0)
    for h in range(Hh):
        K = kv[0, 0, h].astype(np.float64)
        V = kv[0, 1, h].astype(np.float64)
        s = (K @ q[0, h].astype(np.float64)) / math.sqrt(D)
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.abs(got[0, h] - p @ V).max() <= 1e-13


def test_workload_inputs_match_recorded_fingerprints():
    # The seeded inputs are byte-for-byte those recorded when the fixture
    # was written (tests/golden/make_workload_hashes.py): a change of the
    # input recipe, or of the random streams under it, shows up here.
    import importlib.util

    path = os.path.join(HERE, "golden", "make_workload_hashes.py")
    spec = importlib.util.spec_from_file_location("make_workload_hashes", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(os.path.join(HERE, "golden", "workload_sha256.json")) as f:
        gold = json.load(f)
    for name in workloads.WORKLOADS:
        assert mod.fingerprint(name) == gold["f16"][name], name
    for name, elem in mod.TYPED:
        assert mod.fingerprint(name, elem) == gold["typed"][f"{name}/{elem}"], (name, elem)
