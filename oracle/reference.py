"""float64 reference for single-token FP16 GQA decode (test infrastructure).

Source: FlashInfer PR #5052 analysis page ("SM110 FP16 GQA decode").
  * Section 1, the ``sm110_gqa_decode`` docstring: q is ``[batch, 32, 128]``,
    the stacked cache ``kv`` is ``[batch, 2, 8, capacity, 128]``, lengths are
    int32 ``[batch]``, and the scores are multiplied by ``q_scale`` on top of
    the usual ``1/sqrt(128)``.
  * Section 2: fixed 32 query heads, 8 KV heads, head dim 128 (4:1 grouping).
  * Section 3: the PyTorch SDPA comparator -- a boolean mask over the
    capacity axis, ``scale = 1/sqrt(128)`` and ``enable_gqa=True``.

Readings where the page is silent (each listed with its reason in the
design notes):
  * axis 1 of ``kv``: index 0 is K, index 1 is V;
  * query head h uses KV head h // 4 (contiguous groups, as SDPA's
    ``enable_gqa`` repeats each KV head 4 times);
  * a length masks the prefix [0, L) of the capacity axis; lengths are
    clamped to [0, capacity]; an empty prefix gives a zero output row;
  * q_scale is a float32 ABI value; the effective scale is
    float32(q_scale) / sqrt(128) applied to the exact dot product.

Rows at or beyond L are sliced away, never read, so their contents (NaN or
garbage) cannot influence the result.

Extension beyond the page (other head counts): with Hq query heads and Hkv
KV heads (Hq a multiple of Hkv), query head h uses KV head h // (Hq / Hkv),
the contiguous grouping that SDPA's ``enable_gqa`` applies for any ratio;
the head counts are read from the shapes of q and kv. The page's 32/8 case
is the default everywhere.

Extension beyond the page (the library's typed entry point): stored K and V
values may stand for k_scale * K and v_scale * V (per-tensor scales, float32
at the ABI). The definition is unchanged with K and V replaced by those
products; here k_scale joins the score scale and v_scale multiplies the
normalised output, which is the same real number.
"""
from __future__ import annotations

import math

import numpy as np

NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
HEAD_DIM = 128
GROUP = NUM_Q_HEADS // NUM_KV_HEADS  # 4 query heads share one KV head


def effective_scale(q_scale: float, k_scale: float = 1.0) -> float:
    """Score scale: float32(q_scale) * float32(k_scale) / sqrt(128)."""
    return float(np.float32(q_scale)) * float(np.float32(k_scale)) / math.sqrt(HEAD_DIM)


def decode_head(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query row over L key/value rows, in float64.

    q_row: [128]; K, V: [L, 128]. Returns [128]. L == 0 gives zeros.
    """
    q_row = np.asarray(q_row, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(HEAD_DIM, dtype=np.float64)
    s = scale * (K @ q_row)          # scores, one per valid position
    w = np.exp(s - s.max())          # unnormalised softmax weights
    return (w @ V) / w.sum()


def _group_of(n_q_heads: int, n_kv_heads: int) -> int:
    assert n_q_heads >= 1 and n_kv_heads >= 1 and n_q_heads % n_kv_heads == 0, \
        (n_q_heads, n_kv_heads)
    return n_q_heads // n_kv_heads


def decode(q: np.ndarray, kv: np.ndarray, seq_lens, q_scale: float = 1.0,
           rows=None, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Decode one token for every (batch, query head); float64 result.

    q: [B, Hq, 128] (Hq = 32 on the page); kv: [B, 2, Hkv, C, 128] (Hkv = 8),
    any float dtype holding the element values exactly (fp16, or bf16
    widened with formats.bf16_to_f64); seq_lens: int [B]. ``rows``
    optionally restricts the work to a list of (b, h) pairs; the other
    output rows are left as NaN (used for sampled checks on large inputs).
    """
    q = np.asarray(q)
    B, Hq = q.shape[0], q.shape[1]
    Hkv, C = kv.shape[2], kv.shape[3]
    assert q.shape == (B, Hq, HEAD_DIM)
    assert kv.shape == (B, 2, Hkv, C, HEAD_DIM)
    group = _group_of(Hq, Hkv)
    lens = np.asarray(seq_lens).astype(np.int64)
    scale = effective_scale(q_scale, k_scale)
    vs = float(np.float32(v_scale))
    out = np.full((B, Hq, HEAD_DIM), np.nan if rows is not None else 0.0)
    wanted = None
    if rows is not None:
        wanted = {}
        for b, h in rows:
            wanted.setdefault(int(b), set()).add(int(h))
    for b in range(B):
        if wanted is not None and b not in wanted:
            continue
        L = int(min(max(lens[b], 0), C))
        for g in range(Hkv):
            heads = [h for h in range(g * group, (g + 1) * group)
                     if wanted is None or h in wanted[b]]
            if not heads:
                continue
            K = kv[b, 0, g, :L, :].astype(np.float64)
            V = kv[b, 1, g, :L, :].astype(np.float64)
            for h in heads:
                out[b, h] = vs * decode_head(q[b, h].astype(np.float64), K, V, scale)
    return out


def decode_ragged(q: np.ndarray, k_valid, v_valid, q_scale: float = 1.0,
                  k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Same definition, taking each sequence's valid K/V rows directly.

    k_valid[b], v_valid[b]: [Hkv, L_b, 128]. Avoids building a dense cache.
    """
    B, Hq = q.shape[0], q.shape[1]
    Hkv = len(k_valid[0]) if B else NUM_KV_HEADS
    group = _group_of(Hq, Hkv)
    scale = effective_scale(q_scale, k_scale)
    vs = float(np.float32(v_scale))
    out = np.zeros((B, Hq, HEAD_DIM))
    for b in range(B):
        assert len(k_valid[b]) == Hkv and len(v_valid[b]) == Hkv
        for g in range(Hkv):
            K = np.asarray(k_valid[b][g], dtype=np.float64)
            V = np.asarray(v_valid[b][g], dtype=np.float64)
            for h in range(g * group, (g + 1) * group):
                out[b, h] = vs * decode_head(q[b, h].astype(np.float64), K, V, scale)
    return out


def round_fp16(x: np.ndarray) -> np.ndarray:
    """One correctly rounded (nearest-even) float64 -> fp16 conversion.

    numpy converts double to half directly, so there is no intermediate
    float32 rounding (no double rounding).
    """
    return np.asarray(x, dtype=np.float64).astype(np.float16)
