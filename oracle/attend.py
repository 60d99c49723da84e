"""Renormalised softmax attention over a selected set (HashAttention study
notes, sec. 2.1: z_i = <q, k_i> / sqrt(d); the sparse output is
sum_{i in I} e^{z_i} v_i / sum_{j in I} e^{z_j}, with the denominator's index
corrected as the notes point out; the selected rows are read by index from
the full cache, page size one, sec. 2.5).

All arithmetic in float64; q is float32 and K/V are bf16, both widened
exactly.  The maximum logit is subtracted before exponentiating, which leaves
the ratio unchanged.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attend_rows(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float) -> np.ndarray:
    """q float [d]; k_rows, v_rows bf16 bits [m][d] -> float64 [d]."""
    K = bf16_bits_to_f64(k_rows)
    V = bf16_bits_to_f64(v_rows)
    z = (K @ np.asarray(q, np.float64)) * scale
    e = np.exp(z - z.max())
    return (e @ V) / e.sum()


def attend(q, K, V, idx, block_tokens: int = 1, per_query_head: bool = False,
           scale: float | None = None) -> np.ndarray:
    """Batched sparse attention.

    q   float32 [R][Hq][d]
    K,V bf16 bits [R][Hkv][n][d]
    idx int [R][Hsel][m]: token rows (block_tokens == 1) or block ids of
        block_tokens rows each; Hsel = Hq if per_query_head else Hkv
    Query head h reads KV head h // (Hq / Hkv).
    Returns float64 [R][Hq][d].
    """
    q = np.asarray(q)
    R, Hq, d = q.shape
    Hkv = K.shape[1]
    grp = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.zeros((R, Hq, d), np.float64)
    for r in range(R):
        for h in range(Hq):
            g = h // grp
            sel = np.asarray(idx[r, h if per_query_head else g], np.int64)
            if block_tokens > 1:
                sel = (sel[:, None] * block_tokens + np.arange(block_tokens)[None, :]).reshape(-1)
            out[r, h] = attend_rows(q[r, h], K[r, g, sel], V[r, g, sel], scale)
    return out
