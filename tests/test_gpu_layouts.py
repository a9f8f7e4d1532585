"""GPU parity of strided views and paged caches (gqa_decode_ex through the
binding) against the CPU oracle and against the contiguous entry point.

Strided views change only addresses, so their results must equal the
contiguous call's bitwise (same split, same arithmetic). A paged cache keeps
pieces and segments 16-row aligned, so its split differs from the contiguous
one: it is checked against the oracle with the element type's bar, and
bitwise against itself under a different placement of the same pages.
"""
import numpy as np
import pytest

import workloads
from test_gpu_typed import check_bf16, check_f16, oracle_of

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ELEMS = ["f16", "bf16", "e4m3"]


def _torch():
    import torch
    return torch


def _g():
    import gqa_token_decode_amd as g
    return g


def _check(w, out, label):
    if w.elem == "bf16":
        check_bf16(out, oracle_of(w), label)
    else:
        check_f16(out, oracle_of(w), label)


def _bits(t):
    torch = _torch()
    if t.element_size() == 2:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.uint8).cpu().numpy()


def _raw(t):
    """Integer view of a 1- or 2-byte tensor (float8 tensors are filled and
    copied through it)."""
    torch = _torch()
    return t.view(torch.int16 if t.element_size() == 2 else torch.uint8)


def _zeros_like_shape(shape, like):
    torch = _torch()
    raw_dtype = torch.int16 if like.element_size() == 2 else torch.uint8
    return torch.zeros(shape, dtype=raw_dtype, device=DEV).view(like.dtype)


def _decode(w, q, kv, **kw):
    torch = _torch()
    lens = torch.from_numpy(w.seq_lens).to(DEV)
    out = _g().gqa_decode(q, kv, lens, q_scale=w.q_scale, k_scale=w.k_scale, v_scale=w.v_scale,
                          **kw)
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------- strided views
@pytest.mark.parametrize("elem", ELEMS)
def test_nhd_cache_view_equals_contiguous_bitwise(elem):
    # an NHD cache [B, C, 2, 8, 128] seen as [B, 2, 8, C, 128]: rows of one
    # head are 2 * 8 * 128 elements apart
    torch = _torch()
    w = workloads.build(f"nhd {elem}", 80, 700, [700, 333, 1, 0, 129], fill="nan", elem=elem)
    kv = w.kv_to_device(DEV)
    q = w.q_to_device(DEV)
    nhd = _raw(kv).permute(0, 3, 1, 2, 4).contiguous().view(kv.dtype)   # [B, C, 2, 8, 128]
    view = nhd.permute(0, 2, 3, 1, 4)                    # [B, 2, 8, C, 128], strided
    assert not view.is_contiguous()
    base = _decode(w, q, kv)
    got = _decode(w, q, view)
    assert np.array_equal(_bits(got), _bits(base))
    _check(w, got, f"nhd view {elem}")
    for chunk in (7, 100):
        assert np.array_equal(_bits(_decode(w, q, view, chunk_len=chunk)),
                              _bits(_decode(w, q, kv, chunk_len=chunk)))


@pytest.mark.parametrize("elem", ELEMS)
def test_packed_q_and_padded_rows_equal_contiguous_bitwise(elem):
    # q as heads 8..39 of a packed [B, 48, 128] projection output; kv rows
    # padded to 2x their width ([..., 256] sliced to 128)
    torch = _torch()
    w = workloads.build(f"packed {elem}", 81, 300, [300, 7, 64], elem=elem)
    q = w.q_to_device(DEV)
    kv = w.kv_to_device(DEV)
    packed = torch.zeros((q.shape[0], 48, 128), dtype=q.dtype, device=DEV)
    packed[:, 8:40] = q
    qv = packed[:, 8:40]
    wide = _zeros_like_shape(kv.shape[:4] + (256,), kv)
    _raw(wide)[..., :128] = _raw(kv)
    kvv = wide[..., :128]
    assert not qv.is_contiguous() and not kvv.is_contiguous()
    base = _decode(w, q, kv)
    assert np.array_equal(_bits(_decode(w, qv, kv)), _bits(base))
    assert np.array_equal(_bits(_decode(w, q, kvv)), _bits(base))
    assert np.array_equal(_bits(_decode(w, qv, kvv)), _bits(base))


# ---------------------------------------------------------------- paged caches
def _paginate(kv, lens, page_size, seed, spare=5, bad_tail=None):
    """Scatter each sequence's rows into pages of a shuffled pool. Returns
    (kv_pages [num_pages, 2, Hkv, P, 128], block_table [B, max_pages])."""
    torch = _torch()
    B, _, H, C, D = kv.shape
    P = page_size
    max_pages = -(-C // P)
    num_pages = B * max_pages + spare
    rng = np.random.default_rng(seed)
    perm = rng.permutation(num_pages)
    pages = _zeros_like_shape((num_pages, 2, H, P, D), kv)
    rp, rk = _raw(pages), _raw(kv)
    table = np.full((B, max_pages), -1 if bad_tail is None else bad_tail, dtype=np.int32)
    for b in range(B):
        used = -(-int(lens[b]) // P)
        for j in range(used):
            pid = int(perm[b * max_pages + j])
            table[b, j] = pid
            rows = rk[b, :, :, j * P:min((j + 1) * P, C)]
            rp[pid, :, :, :rows.shape[2]] = rows
    return pages, torch.from_numpy(table).to(DEV)


def _decode_paged(w, pages, table, **kw):
    torch = _torch()
    lens = torch.from_numpy(w.seq_lens).to(DEV)
    out = _g().gqa_decode_paged(w.q_to_device(DEV), pages, table, lens, q_scale=w.q_scale,
                                k_scale=w.k_scale, v_scale=w.v_scale, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("page_size", [16, 32, 256])
def test_paged_cache_matches_oracle(elem, page_size):
    print(f"case paged {elem} P={page_size}", flush=True)
    lens = [1024, 1, 0, 17, 300, 1000, 33, 512]
    w = workloads.build(f"paged {elem}", 82, 1024, lens, fill="nan", elem=elem)
    kv = w.kv_to_device(DEV)
    pages, table = _paginate(kv, w.valid_lengths, page_size, seed=page_size)
    got = _decode_paged(w, pages, table)
    for b in np.flatnonzero(w.valid_lengths == 0):
        assert np.all(_bits(got)[b] == 0)
    _check(w, got, f"paged {elem} P={page_size}")
    # the same pages placed elsewhere: bitwise the same result
    pages2, table2 = _paginate(kv, w.valid_lengths, page_size, seed=1000 + page_size)
    assert np.array_equal(_bits(_decode_paged(w, pages2, table2)), _bits(got))
    # forced pieces (rounded up to 16 rows)
    _check(w, _decode_paged(w, pages, table, chunk_len=50), f"paged {elem} P={page_size} chunk 50")


@pytest.mark.parametrize("elem", ["f16", "e4m3"])
def test_paged_table_entries_beyond_lengths_are_never_read(elem):
    w = workloads.build(f"paged tail {elem}", 83, 512, [100, 512, 3, 40], elem=elem)
    kv = w.kv_to_device(DEV)
    pages, table = _paginate(kv, w.valid_lengths, 32, seed=3, bad_tail=-1)
    base = _decode_paged(w, pages, table)
    _, table_bad = _paginate(kv, w.valid_lengths, 32, seed=3, bad_tail=2 ** 30)
    assert np.array_equal(_bits(_decode_paged(w, pages, table_bad)), _bits(base))


def test_paged_invalid_page_id_inside_a_length_reads_zeros_without_fault():
    # The kernel checks page ids against num_pages; an out-of-range id inside
    # a sequence's length reads as zeros. Other sequences are unaffected.
    torch = _torch()
    w = workloads.build("paged bad id", 84, 256, [256, 200, 64], elem="f16")
    kv = w.kv_to_device(DEV)
    pages, table = _paginate(kv, w.valid_lengths, 32, seed=4)
    base = _bits(_decode_paged(w, pages, table))
    bad = table.clone()
    bad[1, 2] = pages.shape[0] + 7
    bad[1, 3] = -5
    got = _decode_paged(w, pages, bad)
    assert np.all(np.isfinite(got.float().cpu().numpy()))
    assert np.array_equal(_bits(got)[[0, 2]], base[[0, 2]])
    # zeros in place of sequence 1's rows 64..127 equal a cache with those rows zeroed
    kv0 = kv.clone()
    _raw(kv0)[1, :, :, 64:128] = 0
    pages0, table0 = _paginate(kv0, w.valid_lengths, 32, seed=4)
    assert np.array_equal(_bits(got)[1], _bits(_decode_paged(w, pages0, table0))[1])
