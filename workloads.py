"""Seeded synthetic inputs for single-token FP16 GQA decode.

This module only draws and lays out inputs; it holds none of the decode
arithmetic. Both the CPU oracle (through the tests and the benchmark's CPU
leg) and the HIP path consume what it produces.

Shapes follow the decode API documented on the FlashInfer PR #5052 analysis
page ("SM110 FP16 GQA decode", section 1, the ``sm110_gqa_decode``
docstring): ``q [batch, 32, 128]`` fp16, stacked ``kv [batch, 2, 8,
capacity, 128]`` fp16 (index 0 of axis 1 is K, 1 is V), int32
``sequence_lengths [batch]``. The named workloads are the five synthetic
configurations of this library plus the four benchmark shapes printed in the
same page's performance tables.

Draw order (fixed, so a seed reproduces the same bytes):
  1. sequence lengths (if random),
  2. q = standard_normal((B, 32, 128), float32) * sigma_q -> fp16 (RNE),
  3. for b in 0..B-1: K_b = standard_normal((8, L_b, 128)) * sigma_k -> fp16,
     then V_b the same way with sigma_v.
Only the valid prefix [0, L_b) of each sequence is drawn. Slots beyond L_b
are filled with zeros, or with a quiet NaN when the workload says so; a
correct decode never reads them.

Element types: "f16" (default), or "bf16" for the library's bfloat16 entry
point: the same float32 draws rounded to bfloat16 (nearest even) instead of
fp16, kept as uint16 bit patterns on the host (numpy has no bfloat16). Or
"e4m3": q as fp16, and each K (V) draw divided by the per-tensor scale
k_scale (v_scale), a power of two, and rounded to OCP FP8 E4M3 (nearest
even, by torch's float8_e4m3fn conversion), kept as uint8 codes. With
k_scale = v_scale = 2^-4 a unit-variance draw is coded at variance 256:
well inside the format's range (largest finite 448) and above its subnormals.
Or "nvfp4": q as fp16, and K/V as block-scaled FP4: each block of 16
consecutive elements of a row gets the scale amax / 6 rounded to E4M3
(nearest even, torch's float8_e4m3fn), and each element the E2M1 code
nearest to x / scale (ties to the even code, magnitudes above 6 saturate);
two codes per byte, element 2m in the low nibble. The packed codes are kept
as uint8 [Hkv, L, 64] and the scales as uint8 [Hkv, L, 8]; k_scale = v_scale
= 1. Beyond the lengths the "nan" fill writes code bytes 0xFF and NaN scale
codes 0x7F.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional

import numpy as np

NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
HEAD_DIM = 128

FP16_QNAN_BITS = 0x7E00
BF16_QNAN_BITS = 0x7FC0
E4M3_NAN_CODE = 0x7F
E4M3_SCALE = 2.0 ** -4
FP4_BLOCK = 16
FP4_FILL_BYTE = 0xFF
# E2M1 magnitudes in code order (code = 2 * exponent field + mantissa bit)
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
# midpoints between neighbouring magnitudes
_E2M1_MID = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2


@dataclasses.dataclass
class Workload:
    """One decode step's inputs, with the valid K/V prefixes kept ragged.

    ``k_valid[b]`` and ``v_valid[b]`` are fp16 arrays of shape
    ``[Hkv, L_b, 128]`` (Hkv = 8 unless built with other head counts); the
    dense stacked cache is materialised on demand by
    :meth:`dense_kv` (host) or :meth:`kv_to_device` (GPU), so that a 4 GiB
    cache is never built on the host unless asked for.
    """

    name: str
    q: np.ndarray                 # fp16 [B, Hq, 128] (uint16 bit patterns for bf16)
    seq_lens: np.ndarray          # int32 [B]
    capacity: int
    q_scale: float
    k_valid: List[np.ndarray]     # fp16 [Hkv, L_b, 128] per b
    v_valid: List[np.ndarray]     # fp16 [Hkv, L_b, 128] per b
    fill: str = "zero"            # "zero" or "nan": contents beyond L_b
    elem: str = "f16"             # "f16", "bf16", "e4m3" or "nvfp4" (kv only)
    k_scale: float = 1.0          # e4m3: the stored codes stand for K / k_scale
    v_scale: float = 1.0
    k_scales: Optional[List[np.ndarray]] = None   # nvfp4: uint8 [Hkv, L_b, 8] E4M3 block scales
    v_scales: Optional[List[np.ndarray]] = None

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def kv_heads(self) -> int:
        return int(self.k_valid[0].shape[0]) if self.k_valid else NUM_KV_HEADS

    @property
    def valid_lengths(self) -> np.ndarray:
        """Lengths clamped to [0, capacity], as the decode interprets them."""
        return np.clip(self.seq_lens.astype(np.int64), 0, self.capacity)

    @property
    def kv_bytes_read(self) -> int:
        """K+V bytes of the valid prefixes: sum(L_b) * 2 * Hkv * (bytes per
        head row: 256 for 16-bit types, 128 for e4m3, 64 + 8 for nvfp4)."""
        return int(self.valid_lengths.sum()) * 2 * self.kv_heads * self.kv_row_bytes

    @property
    def kv_row_bytes(self) -> int:
        if self.elem == "nvfp4":
            return HEAD_DIM // 2 + HEAD_DIM // FP4_BLOCK
        return HEAD_DIM * self.kv_elem_bytes

    @property
    def kv_elem_bytes(self) -> int:
        """Bytes per stored element of kv (nvfp4: the packed code bytes)."""
        return 1 if self.elem in ("e4m3", "nvfp4") else 2

    @property
    def kv_row_elems(self) -> int:
        """Stored elements per kv head row (nvfp4: 64 code bytes)."""
        return HEAD_DIM // 2 if self.elem == "nvfp4" else HEAD_DIM

    def fill_value_bits(self) -> int:
        if self.fill != "nan":
            return 0
        return {"bf16": BF16_QNAN_BITS, "e4m3": E4M3_NAN_CODE,
                "nvfp4": FP4_FILL_BYTE}.get(self.elem, FP16_QNAN_BITS)

    def _host_dtype(self):
        return {"bf16": np.uint16, "e4m3": np.uint8, "nvfp4": np.uint8}.get(self.elem, np.float16)

    def _torch_dtype(self):
        import torch

        return {"bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn,
                "nvfp4": torch.uint8}.get(self.elem, torch.float16)

    def q_to_device(self, device):
        """q as a device tensor of the workload's element type."""
        import torch

        t = torch.from_numpy(self.q)
        if self.elem == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(device)

    def dense_kv(self) -> np.ndarray:
        """Host ``[B, 2, Hkv, C, 128]`` cache (fp16, or bf16 bit patterns,
        or codes; nvfp4: ``[B, 2, Hkv, C, 64]`` packed bytes) with the fill
        beyond L_b."""
        B, C = self.batch, self.capacity
        kv = np.empty((B, 2, self.kv_heads, C, self.kv_row_elems), dtype=self._host_dtype())
        if kv.dtype == np.uint8:
            kv[...] = self.fill_value_bits()
        else:
            kv.view(np.uint16)[...] = self.fill_value_bits()
        for b in range(B):
            L = self.k_valid[b].shape[1]
            kv[b, 0, :, :L, :] = self.k_valid[b]
            kv[b, 1, :, :L, :] = self.v_valid[b]
        return kv

    def kv_to_device(self, device):
        """Build the dense cache directly in device memory (torch tensor)."""
        import torch

        B, C = self.batch, self.capacity
        kv = torch.empty((B, 2, self.kv_heads, C, self.kv_row_elems), dtype=self._torch_dtype(),
                         device=device)
        if self.elem in ("e4m3", "nvfp4"):
            raw, host_raw = kv.view(torch.uint8), np.uint8
            raw.fill_(self.fill_value_bits())
        else:
            raw, host_raw = kv.view(torch.int16), np.int16
            raw.fill_(np.int16(np.uint16(self.fill_value_bits())).item())
        for b in range(B):
            L = self.k_valid[b].shape[1]
            if L:
                raw[b, 0, :, :L, :].copy_(torch.from_numpy(self.k_valid[b].view(host_raw)))
                raw[b, 1, :, :L, :].copy_(torch.from_numpy(self.v_valid[b].view(host_raw)))
        return kv

    def dense_scales(self) -> np.ndarray:
        """nvfp4: host ``[B, 2, Hkv, C, 8]`` E4M3 block scales (NaN codes
        beyond L_b for the "nan" fill, zeros otherwise)."""
        assert self.elem == "nvfp4"
        B, C = self.batch, self.capacity
        sc = np.full((B, 2, self.kv_heads, C, HEAD_DIM // FP4_BLOCK),
                     E4M3_NAN_CODE if self.fill == "nan" else 0, dtype=np.uint8)
        for b in range(B):
            L = self.k_scales[b].shape[1]
            sc[b, 0, :, :L] = self.k_scales[b]
            sc[b, 1, :, :L] = self.v_scales[b]
        return sc

    def scales_to_device(self, device):
        """nvfp4: the block scales as a device uint8 tensor [B, 2, Hkv, C, 8]."""
        import torch

        assert self.elem == "nvfp4"
        B, C = self.batch, self.capacity
        sc = torch.empty((B, 2, self.kv_heads, C, HEAD_DIM // FP4_BLOCK), dtype=torch.uint8,
                         device=device)
        sc.fill_(E4M3_NAN_CODE if self.fill == "nan" else 0)
        for b in range(B):
            L = self.k_scales[b].shape[1]
            if L:
                sc[b, 0, :, :L].copy_(torch.from_numpy(self.k_scales[b]))
                sc[b, 1, :, :L].copy_(torch.from_numpy(self.v_scales[b]))
        return sc


def encode_nvfp4(x: np.ndarray):
    """float32 [..., 128] -> (packed uint8 [..., 64], scales uint8 [..., 8]).

    Input preparation only (the decode never encodes): per block of 16, the
    scale amax / 6 rounded to E4M3, then each element's nearest E2M1 code
    for x / scale. Works one leading slice at a time to bound host memory.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim > 2:
        parts = [encode_nvfp4(x[i]) for i in range(x.shape[0])]
        shp = x.shape[:-1]
        if not parts:
            return (np.zeros(shp + (x.shape[-1] // 2,), np.uint8),
                    np.zeros(shp + (x.shape[-1] // FP4_BLOCK,), np.uint8))
        return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])
    import torch

    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // FP4_BLOCK, FP4_BLOCK))
    amax = np.abs(blocks).max(axis=-1, initial=0.0)
    sc_codes = torch.from_numpy((amax / np.float32(6.0)).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    sc_vals = torch.from_numpy(sc_codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    den = np.where(sc_vals > 0, sc_vals, 1.0)[..., None]
    y = np.where(sc_vals[..., None] > 0, blocks.astype(np.float64) / den, 0.0)
    mag = np.abs(y)
    # index into the sorted magnitudes (= the code without its sign): the
    # number of midpoints below |y|, plus one at the midpoints whose upper
    # neighbour is the even code (ties go to the even code)
    code = np.zeros(mag.shape, dtype=np.uint8)
    for k, mid in enumerate(_E2M1_MID):
        code += mag > mid
        if k % 2 == 1:
            code += mag == mid
    code |= (y < 0).astype(np.uint8) << 3
    code = code.reshape(x.shape)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.astype(np.uint8), sc_codes.astype(np.uint8)


def _normal(rng: np.random.Generator, shape, sigma: float, elem: str,
            code_scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    if elem == "e4m3":
        import torch

        y = x / np.float32(code_scale)           # exact: a power-of-two scale
        return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    if elem == "bf16":
        import torch

        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x.astype(np.float16)


def build(
    name: str,
    seed: int,
    capacity: int,
    lengths: Callable[[np.random.Generator], np.ndarray] | List[int] | np.ndarray,
    *,
    q_scale: float = 1.0,
    sigma_q: float = 1.0,
    sigma_k: float = 1.0,
    sigma_v: float = 1.0,
    fill: str = "zero",
    elem: str = "f16",
    q_heads: int = NUM_Q_HEADS,
    kv_heads: int = NUM_KV_HEADS,
    with_kv: bool = True,
) -> Workload:
    """Draw a workload. ``lengths`` is a list or a callable taking the rng.

    Lengths may lie outside [0, capacity] (tests of clamping); only
    ``clip(L_b, 0, capacity)`` rows are drawn. Draw order: lengths, q, then
    per sequence K and V (the same order for any head counts).
    ``with_kv=False`` stops after q (lengths and q are the same; the K/V
    lists hold empty arrays): for checks of the first draws only.
    """
    rng = np.random.default_rng(seed)
    if callable(lengths):
        lens = np.asarray(lengths(rng), dtype=np.int64)
    else:
        lens = np.asarray(lengths, dtype=np.int64)
    B = int(lens.shape[0])
    assert elem in ("f16", "bf16", "e4m3", "nvfp4"), elem
    kv_scale = E4M3_SCALE if elem == "e4m3" else 1.0
    q = _normal(rng, (B, q_heads, HEAD_DIM), sigma_q,
                "f16" if elem in ("e4m3", "nvfp4") else elem)
    k_valid, v_valid = [], []
    k_scales, v_scales = ([], []) if elem == "nvfp4" else (None, None)
    for b in range(B):
        L = int(min(max(lens[b], 0), capacity)) if with_kv else 0
        if elem == "nvfp4":
            for sigma, vals, scs in ((sigma_k, k_valid, k_scales), (sigma_v, v_valid, v_scales)):
                x = rng.standard_normal((kv_heads, L, HEAD_DIM), dtype=np.float32)
                if sigma != 1.0:
                    x = x * np.float32(sigma)
                packed, sc = encode_nvfp4(x)
                vals.append(packed)
                scs.append(sc)
            continue
        k_valid.append(_normal(rng, (kv_heads, L, HEAD_DIM), sigma_k, elem, kv_scale))
        v_valid.append(_normal(rng, (kv_heads, L, HEAD_DIM), sigma_v, elem, kv_scale))
    return Workload(name, q, lens.astype(np.int32), int(capacity), float(q_scale),
                    k_valid, v_valid, fill, elem, kv_scale, kv_scale, k_scales, v_scales)


def build_sink(
    name: str,
    seed: int,
    capacity: int,
    lengths: List[int],
    *,
    sink_period: int,
    sink_rows: tuple = (0, 16, 32, 48),
    c: float = 1.0,
    elem: str = "f16",
    sigma_k: float = 0.25,
    sink_gain: float = 1.5,
    q_scale: float = 1.0,
) -> Workload:
    """Attention-sink inputs: long runs of keys with small scores under a
    few dominant ("sink") keys, the shape of a decode whose first tokens
    take most of the attention.

    Every query head of a KV group uses one query vector u ~ N(0, 1) (fp16).
    Key row i of a sequence is a sink when i % sink_period is in sink_rows
    (sink_period = 0: only the rows in sink_rows themselves); a sink key is
    sink_gain * u, so with sink_gain 1.5 its score, about
    sink_gain * |u|^2 / sqrt(128), lies some 17 nats above the other keys,
    which are N(0, sigma_k^2). V is 0 on sink rows and c * U(0.5, 1.5)
    elsewhere, so the output is c times the small share of the non-sink
    rows. Encodings: "f16" stores the values as fp16 (v_scale 1); "e4m3"
    stores K / 2^-4 and V / (c 2^-4) as E4M3 codes with k_scale 2^-4 and
    v_scale c 2^-4; "nvfp4" stores K and V / c as block-scaled FP4 with
    v_scale c.
    """
    import torch

    assert elem in ("f16", "e4m3", "nvfp4"), elem
    rng = np.random.default_rng(seed)
    lens = np.asarray(lengths, dtype=np.int64)
    B, Hq, Hkv = int(lens.shape[0]), NUM_Q_HEADS, NUM_KV_HEADS
    G = Hq // Hkv
    u = rng.standard_normal((B, Hkv, HEAD_DIM), dtype=np.float32).astype(np.float16)
    q = np.repeat(u, G, axis=1)                      # heads 4g .. 4g + 3 share u[b, g]
    k_valid, v_valid = [], []
    k_scales, v_scales = ([], []) if elem == "nvfp4" else (None, None)
    v_div = 1.0 if elem == "f16" else float(c)
    for b in range(B):
        L = int(min(max(lens[b], 0), capacity))
        rows = np.arange(L)
        sink = np.isin(rows % sink_period if sink_period > 0 else rows, sink_rows)
        k = rng.standard_normal((Hkv, L, HEAD_DIM), dtype=np.float32) * np.float32(sigma_k)
        k[:, sink, :] = np.float32(sink_gain) * u[b].astype(np.float32)[:, None, :]
        v = rng.uniform(0.5, 1.5, (Hkv, L, HEAD_DIM)).astype(np.float32)
        v *= np.float32(c / v_div)
        v[:, sink, :] = 0.0
        if elem == "f16":
            k_valid.append(k.astype(np.float16))
            v_valid.append(v.astype(np.float16))
        elif elem == "e4m3":
            to8 = lambda x: torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            k_valid.append(to8(k / np.float32(E4M3_SCALE)))
            v_valid.append(to8(v / np.float32(E4M3_SCALE)))
        else:
            for x, vals, scs in ((k, k_valid, k_scales), (v, v_valid, v_scales)):
                packed, sc = encode_nvfp4(x)
                vals.append(packed)
                scs.append(sc)
    ks = E4M3_SCALE if elem == "e4m3" else 1.0
    vs = (E4M3_SCALE * c) if elem == "e4m3" else (float(c) if elem == "nvfp4" else 1.0)
    return Workload(name, q, lens.astype(np.int32), int(capacity), float(q_scale),
                    k_valid, v_valid, "zero", elem, ks, vs, k_scales, v_scales)


def _cfg4_lengths(rng: np.random.Generator) -> np.ndarray:
    # 90% short-prefix sequences, 10% long ones: 58 + 6 of 64, then shuffled.
    short = rng.integers(16, 512, 58, endpoint=True)
    long_ = rng.integers(8192, 16384, 6, endpoint=True)
    return rng.permutation(np.concatenate([short, long_]))


# Name -> (description, factory of the element type). The five synthetic
# decode workloads, then the four benchmark shapes printed in the PR #5052
# page's timing tables (batch/capacity/valid lengths exactly as printed there).
WORKLOADS: Dict[str, tuple] = {
    "b1_c256_len200": (
        "batch 1, capacity 256, length 200, N(0,1), q_scale 1.0",
        lambda e, **kw: build("b1_c256_len200", 1, 256, [200], elem=e, **kw),
    ),
    "b8_c4096_nanfill": (
        "batch 8, capacity 4096, lengths U[1,4096], N(0,1), NaN beyond each length, q_scale 1.0",
        lambda e, **kw: build("b8_c4096_nanfill", 2, 4096,
                        lambda r: r.integers(1, 4096, 8, endpoint=True), fill="nan",
                        elem=e, **kw),
    ),
    "b32_c8192_qs05": (
        "batch 32, capacity 8192, lengths U[1024,8192], N(0,1), q_scale 0.5",
        lambda e, **kw: build("b32_c8192_qs05", 3, 8192,
                        lambda r: r.integers(1024, 8192, 32, endpoint=True), q_scale=0.5,
                        elem=e, **kw),
    ),
    "b64_c16384_skewed": (
        "batch 64, capacity 16384, 58 lengths U[16,512] + 6 lengths U[8192,16384] shuffled, "
        "q,V ~ N(0,1), K ~ N(0, std 2), q_scale 1.0",
        lambda e, **kw: build("b64_c16384_skewed", 4, 16384, _cfg4_lengths, sigma_k=2.0, elem=e, **kw),
    ),
    "b2_c131072_long": (
        "batch 2, capacity 131072, lengths [131072, 65537], N(0,1), q_scale 1.0",
        lambda e, **kw: build("b2_c131072_long", 5, 131072, [131072, 65537], elem=e, **kw),
    ),
    "page_b1_c64": (
        "page shape: batch 1, capacity 64, lengths [1]",
        lambda e, **kw: build("page_b1_c64", 11, 64, [1], elem=e, **kw),
    ),
    "page_b4_c256": (
        "page shape: batch 4, capacity 256, lengths [64, 127, 191, 256]",
        lambda e, **kw: build("page_b4_c256", 12, 256, [64, 127, 191, 256], elem=e, **kw),
    ),
    "page_b1_c1024": (
        "page shape: batch 1, capacity 1024, lengths [1024]",
        lambda e, **kw: build("page_b1_c1024", 13, 1024, [1024], elem=e, **kw),
    ),
    "page_b1_c4096": (
        "page shape: batch 1, capacity 4096, lengths [3968]",
        lambda e, **kw: build("page_b1_c4096", 14, 4096, [3968], elem=e, **kw),
    ),
}

# The five synthetic workloads in order (small first).
SYNTHETIC = ["b1_c256_len200", "b8_c4096_nanfill", "b32_c8192_qs05",
             "b64_c16384_skewed", "b2_c131072_long"]
PAGE_SHAPES = ["page_b1_c64", "page_b4_c256", "page_b1_c1024", "page_b1_c4096"]


def get(name: str, elem: str = "f16", q_heads: int = NUM_Q_HEADS,
        kv_heads: int = NUM_KV_HEADS, with_kv: bool = True) -> Workload:
    """Named workload; elem="bf16", "e4m3" or "nvfp4" draws it (same seed and
    recipe) in that element type, and other head counts draw it with Hq
    query and Hkv KV heads (same lengths). with_kv=False: lengths and q only
    (see build)."""
    kw = {} if with_kv else {"with_kv": False}
    if (q_heads, kv_heads) != (NUM_Q_HEADS, NUM_KV_HEADS):
        kw.update(q_heads=q_heads, kv_heads=kv_heads)
    return WORKLOADS[name][1](elem, **kw)


def describe(name: str) -> str:
    return WORKLOADS[name][0]
