"""Element formats used by the decode's extended entry points (test
infrastructure; see the package docstring).

bfloat16: the upper 16 bits of an IEEE binary32 value (1 sign bit, 8
exponent bits with bias 127, 7 fraction bits). Widening is exact; narrowing
rounds to nearest, ties to even, directly from float64 (no float32 step, so
there is no double rounding). Subnormals are kept (spacing 2^-133); values
beyond the largest finite bfloat16 become infinities.

Block-scaled FP4 ("NVFP4-like", the K/V page format named on the FlashInfer
NVFP4 paged-context attention page: E2M1 values with E4M3 block scales).
Readings (the page names the format only): every 16 consecutive elements of
a 128-element head row share one E4M3 scale, so a row has 8 scales; two
elements share a byte, element 2m in the low nibble of byte m and element
2m + 1 in the high nibble; the element's value is its E2M1 value times its
block's scale; a per-tensor scale, when there is one, is the decode's
k_scale / v_scale.
"""
from __future__ import annotations

import numpy as np

_BF16_MIN_NORMAL_EXP = -126      # smallest normal exponent (as for binary32)
_BF16_FRACTION_BITS = 7
_BF16_MAX = float.fromhex("0x1.fep127")


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16 array) as float64."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    # spacing of bfloat16 numbers around |x|: 2^(e - 7) for |x| in [2^e, 2^(e+1)),
    # and the subnormal spacing 2^(-126 - 7) below 2^-126
    _, e = np.frexp(np.abs(xf))              # |x| = f * 2^e, f in [0.5, 1)
    e = np.maximum(e - 1, _BF16_MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, e - _BF16_FRACTION_BITS)
    r = np.rint(xf / quantum) * quantum      # exact: division by a power of two, rint is RNE
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[finite] = r[finite]
    out[~finite] = x[~finite]
    bits = out.astype(np.float32).view(np.uint32) >> np.uint32(16)   # exact: out is a bfloat16 value
    return bits.astype(np.uint16)


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact value of OCP FP8 E4M3 codes (uint8 array) as float64.

    Bit fields s eeee mmm: exponent bias 7; e = 0 encodes subnormals
    m * 2^-9; e = 15 with m = 7 is NaN (the format has no infinities), so
    the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def e2m1_to_f64(codes) -> np.ndarray:
    """Exact value of FP4 E2M1 codes (integers 0..15) as float64.

    Bit fields s ee m: exponent bias 1; e = 0 encodes the subnormals m * 0.5
    (0 and 0.5), otherwise (1 + m / 2) * 2^(e - 1). No infinities or NaN;
    the largest magnitude is 6.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64)))
    return sign * mag


FP4_BLOCK = 16      # elements per E4M3 block scale


def nvfp4_to_f64(packed, scales) -> np.ndarray:
    """Exact values of block-scaled FP4 rows as float64.

    packed: uint8 [..., n / 2] (element 2m in the low nibble of byte m,
    element 2m + 1 in the high nibble); scales: uint8 [..., n / 16] E4M3
    codes, scale k covering elements 16k .. 16k + 15. Returns [..., n].
    """
    p = np.asarray(packed).astype(np.int64)
    lo, hi = p & 15, p >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))
    vals = e2m1_to_f64(codes)
    sc = e4m3_to_f64(scales)
    assert sc.shape[-1] * FP4_BLOCK == vals.shape[-1], (sc.shape, vals.shape)
    return vals * np.repeat(sc, FP4_BLOCK, axis=-1)
