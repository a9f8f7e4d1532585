"""GPU decode at the size limits: the largest capacity (2^22 positions per
sequence, 16 GiB of K/V per sequence) and a very large batch, for the fp16
cache and the block-scaled FP4 cache.

At the largest capacity the inputs are built on the device: K is zero except
a few rows whose scores dominate by more than 40 (every other row's weight
is below e^-40, far under fp16 resolution even summed over 2^22 rows), so
the exact result is the plain average of those rows' V, computed here in
float64 from the few rows. A row just past the length gets an even larger
score: reading it would change the result. For the large batch, sampled
sequences are checked against the CPU oracle on their own rows.
"""
import numpy as np
import pytest

from oracle.reference import decode_ragged, round_fp16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CAP = 1 << 22


def _torch():
    import torch
    return torch


def _g():
    import gqa_token_decode_amd as g
    return g


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    _torch().cuda.empty_cache()


def test_maximum_capacity_reads_far_rows_and_nothing_beyond():
    torch = _torch()
    g = _g()
    print("case max capacity 2^22", flush=True)
    B, H, G, D = 2, 32, 8, 128
    lens = [CAP, CAP - 3]
    # (b, rows with a dominant score inside the length, row beyond the length or None)
    picks = [(0, [0, CAP - 1], None), (1, [5, CAP // 2 + 7, CAP - 4], CAP - 3)]
    kv = torch.zeros((B, 2, G, CAP, D), dtype=torch.float16, device=DEV)
    rng = np.random.default_rng(31)
    q = torch.ones((B, H, D), dtype=torch.float16, device=DEV)
    expect = np.zeros((B, H, D))
    for b, rows, beyond in picks:
        vals = rng.standard_normal((len(rows), G, D)).astype(np.float16)
        for i, r in enumerate(rows):
            kv[b, 0, :, r, :] = 4.0                  # score 128 * 4 / sqrt(128) = 45.3
            kv[b, 1, :, r, :] = torch.from_numpy(vals[i]).to(DEV)
        if beyond is not None:
            kv[b, 0, :, beyond, :] = 8.0             # would dominate if it were read
            kv[b, 1, :, beyond, :] = 100.0
        mean = vals.astype(np.float64).mean(axis=0)  # [G, D]
        for h in range(H):
            expect[b, h] = mean[h // 4]
    out = g.gqa_decode(q, kv, torch.tensor(lens, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    d = np.abs(got - round_fp16(expect).astype(np.float64))
    print(f"max capacity: max|d|={d.max():.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert d.max() <= 2e-3
    # the same with a forced split
    for kw in ({"chunk_len": 100000},):
        again = g.gqa_decode(q, kv, torch.tensor(lens, dtype=torch.int32, device=DEV), **kw)
        torch.cuda.synchronize()
        d2 = np.abs(again.float().cpu().numpy() - got)
        assert d2.max() <= 2e-3, kw
    del kv


def test_batch_of_65536_sampled_against_the_oracle():
    torch = _torch()
    g = _g()
    print("case batch 65536", flush=True)
    B, C, H, G, D = 1 << 16, 24, 32, 8, 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(32)
    lens = torch.randint(0, C + 1, (B,), dtype=torch.int32, device=DEV, generator=gen)
    q = torch.randn((B, H, D), dtype=torch.float16, device=DEV, generator=gen)
    kv = torch.randn((B, 2, G, C, D), dtype=torch.float16, device=DEV, generator=gen)
    out = g.gqa_decode(q, kv, lens)
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    sample = np.concatenate([[0, B - 1], rng.choice(B, 30, replace=False)])
    lens_h = lens.cpu().numpy()
    idx = torch.from_numpy(sample).to(DEV)
    q_h = q[idx].cpu().numpy()
    kv_s = kv[idx].cpu().numpy()
    k_valid = [kv_s[i, 0, :, :lens_h[b]] for i, b in enumerate(sample)]
    v_valid = [kv_s[i, 1, :, :lens_h[b]] for i, b in enumerate(sample)]
    ref = round_fp16(decode_ragged(q_h, k_valid, v_valid, 1.0)).astype(np.float64)
    got = out[idx].float().cpu().numpy().astype(np.float64)
    d = np.abs(got - ref)
    print(f"batch 65536 sampled: max|d|={d.max():.3e} mean|d|={d.mean():.3e}", flush=True)
    assert d.max() <= 2e-3 and d.mean() <= 2e-4
    for i, b in enumerate(sample):
        if lens_h[b] == 0:
            assert np.all(got[i] == 0)


def test_fp4_maximum_capacity_reads_far_rows_and_nothing_beyond():
    # The FP4 cache at capacity 2^22 (8 GiB of codes, 1 GiB of scales): K
    # codes are zero except a few rows of E2M1 code 6 (value 4) under scale
    # 1, whose scores (128 * 4 / sqrt(128) = 45.3) dominate by more than 40;
    # V at those rows holds random codes under scales up to 0.5. A row just
    # past the length has K value 12 (code 7, scale 2): reading it would
    # change the result.
    torch = _torch()
    g = _g()
    from oracle.formats import nvfp4_to_f64
    print("case fp4 max capacity 2^22", flush=True)
    B, H, G, D = 2, 32, 8, 128
    lens = [CAP, CAP - 3]
    picks = [(0, [0, CAP - 1], None), (1, [5, CAP // 2 + 7, CAP - 4], CAP - 3)]
    codes = torch.zeros((B, 2, G, CAP, D // 2), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((B, 2, G, CAP, 8), dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(34)
    q = torch.ones((B, H, D), dtype=torch.float16, device=DEV)
    expect = np.zeros((B, H, D))
    for b, rows, beyond in picks:
        vcodes = rng.integers(0, 256, (len(rows), G, D // 2), dtype=np.uint8)
        vscales = rng.choice(np.array([0x20, 0x28, 0x2C, 0x30], np.uint8), (len(rows), G, 8))
        for i, r in enumerate(rows):
            codes[b, 0, :, r, :] = 0x66                 # two E2M1 codes 6 (value 4) per byte
            scales[b, 0, :, r, :] = 0x38                # E4M3 1.0
            codes[b, 1, :, r, :] = torch.from_numpy(vcodes[i]).to(DEV)
            scales[b, 1, :, r, :] = torch.from_numpy(vscales[i]).to(DEV)
        if beyond is not None:
            codes[b, 0, :, beyond, :] = 0x77            # value 6 ...
            scales[b, 0, :, beyond, :] = 0x40           # ... times 2
            codes[b, 1, :, beyond, :] = 0x77
            scales[b, 1, :, beyond, :] = 0x40
        mean = nvfp4_to_f64(vcodes, vscales).mean(axis=0)   # [G, D]
        for h in range(H):
            expect[b, h] = mean[h // 4]
    out = g.gqa_decode_fp4(q, codes, scales, torch.tensor(lens, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    d = np.abs(got - round_fp16(expect).astype(np.float64))
    print(f"fp4 max capacity: max|d|={d.max():.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert d.max() <= 2e-3
    again = g.gqa_decode_fp4(q, codes, scales, torch.tensor(lens, dtype=torch.int32, device=DEV),
                             chunk_len=100000)
    torch.cuda.synchronize()
    assert np.abs(again.float().cpu().numpy() - got).max() <= 2e-3
    del codes, scales


def test_fp4_batch_of_65536_sampled_against_the_oracle():
    # Random codes and finite scales drawn on the device; sampled sequences
    # are decoded on the CPU from their own codes and scales.
    torch = _torch()
    g = _g()
    from oracle.formats import nvfp4_to_f64
    print("case fp4 batch 65536", flush=True)
    B, C, H, G, D = 1 << 16, 24, 32, 8, 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(35)
    lens = torch.randint(0, C + 1, (B,), dtype=torch.int32, device=DEV, generator=gen)
    q = torch.randn((B, H, D), dtype=torch.float16, device=DEV, generator=gen)
    codes = torch.randint(0, 256, (B, 2, G, C, D // 2), dtype=torch.uint8, device=DEV,
                          generator=gen)
    # E4M3 scales 0.125 .. 0.5 (codes 0x20 .. 0x30): |K|, |V| <= 3
    scales = torch.randint(0x20, 0x31, (B, 2, G, C, 8), dtype=torch.uint8, device=DEV,
                           generator=gen)
    out = g.gqa_decode_fp4(q, codes, scales, lens)
    torch.cuda.synchronize()
    rng = np.random.default_rng(36)
    sample = np.concatenate([[0, B - 1], rng.choice(B, 30, replace=False)])
    lens_h = lens.cpu().numpy()
    idx = torch.from_numpy(sample).to(DEV)
    q_h = q[idx].cpu().numpy()
    kv64 = nvfp4_to_f64(codes[idx].cpu().numpy(), scales[idx].cpu().numpy())
    k_valid = [kv64[i, 0, :, :lens_h[b]] for i, b in enumerate(sample)]
    v_valid = [kv64[i, 1, :, :lens_h[b]] for i, b in enumerate(sample)]
    ref = round_fp16(decode_ragged(q_h, k_valid, v_valid, 1.0)).astype(np.float64)
    got = out[idx].float().cpu().numpy().astype(np.float64)
    d = np.abs(got - ref)
    print(f"fp4 batch 65536 sampled: max|d|={d.max():.3e} mean|d|={d.mean():.3e}", flush=True)
    assert d.max() <= 2e-3 and d.mean() <= 2e-4
    for i, b in enumerate(sample):
        if lens_h[b] == 0:
            assert np.all(got[i] == 0)
