"""Brute-force decode on tiny inputs (test infrastructure, pins the oracle).

Independent of ``oracle.reference``: scalar Python loops over the same
definition (FlashInfer PR #5052 analysis page, section 1 docstring and the
section 3 SDPA comparator), with exactly rounded sums (``math.fsum``) in
float64, and an arbitrary-precision variant using mpmath. No numpy
arithmetic is used on the values.
"""
from __future__ import annotations

import math


def _head_float(qv, Krows, Vrows, scale):
    L = len(Krows)
    if L == 0:
        return [0.0] * len(qv)
    scores = [scale * math.fsum(a * b for a, b in zip(qv, k)) for k in Krows]
    top = max(scores)
    w = [math.exp(s - top) for s in scores]
    den = math.fsum(w)
    D = len(qv)
    return [math.fsum(w[i] * Vrows[i][d] for i in range(L)) / den for d in range(D)]


def decode_brute(q, kv, seq_lens, q_scale, n_kv_heads=8, k_scale=1.0, v_scale=1.0):
    """q: nested lists [B][H][D]; kv: nested [B][2][G][C][D]; floats.

    Returns nested lists [B][H][D]. Query head h reads KV head h // (H/G).
    k_scale and v_scale (float32 values) multiply every stored K and V
    element before anything else, as their definition says.
    """
    import numpy as np  # only to turn the scales into their float32 values

    B = len(q)
    H = len(q[0])
    group = H // n_kv_heads
    scale = float(np.float32(q_scale)) / math.sqrt(len(q[0][0]))
    ks, vs = float(np.float32(k_scale)), float(np.float32(v_scale))
    if ks != 1.0 or vs != 1.0:
        kv = [[[[[x * (ks if kind == 0 else vs) for x in row] for row in head]
                for head in part] for kind, part in enumerate(seq)] for seq in kv]
    out = []
    for b in range(B):
        C = len(kv[b][0][0])
        L = min(max(int(seq_lens[b]), 0), C)
        rows = []
        for h in range(H):
            g = h // group
            rows.append(_head_float(q[b][h], kv[b][0][g][:L], kv[b][1][g][:L], scale))
        out.append(rows)
    return out


def decode_head_mp(qv, Krows, Vrows, q_scale, digits=40):
    """One head in mpmath at ``digits`` significant digits; returns floats."""
    import mpmath
    import numpy as np

    with mpmath.workdps(digits):
        scale = mpmath.mpf(float(np.float32(q_scale))) / mpmath.sqrt(len(qv))
        L = len(Krows)
        if L == 0:
            return [0.0] * len(qv)
        scores = [scale * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b) for a, b in zip(qv, k))
                  for k in Krows]
        top = max(scores)
        w = [mpmath.exp(s - top) for s in scores]
        den = mpmath.fsum(w)
        return [float(mpmath.fsum(w[i] * mpmath.mpf(Vrows[i][d]) for i in range(L)) / den)
                for d in range(len(qv))]
