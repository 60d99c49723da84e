"""Per-block min/max key summaries (OasisKV review, background section on
Quest-style block summaries, and the core-method section: each logical block
keeps per-dimension minimum and maximum key vectors, the query is scored
against them, and each KV head ranks the whole context on its own).

Block score for query q against block b: sum_j max(q_j * mn_bj, q_j * mx_bj),
an upper bound of q . k for every key k in the block.  A GQA group scores a
block by the sum of its heads' bounds.

Reading taken: summaries are the bf16 keys' block min and max rounded to fp16
outwards (min rounded down, max rounded up), so the bound survives the
rounding.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f32(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32)


def summaries(k_bf16: np.ndarray, block: int = 16):
    """k_bf16 uint16 [n][d] -> (mn, mx) float16 [nb][d], nb = ceil(n / block).
    A last, partly filled block is summarised over the tokens it holds."""
    x = bf16_bits_to_f32(k_bf16)
    n, d = x.shape
    nb = -(-n // block)
    lo = np.stack([x[b * block:min(n, (b + 1) * block)].min(axis=0) for b in range(nb)])
    hi = np.stack([x[b * block:min(n, (b + 1) * block)].max(axis=0) for b in range(nb)])
    mn = lo.astype(np.float16)
    mx = hi.astype(np.float16)
    mn = np.where(mn.astype(np.float32) > lo, np.nextafter(mn, np.float16(-np.inf)), mn)
    mx = np.where(mx.astype(np.float32) < hi, np.nextafter(mx, np.float16(np.inf)), mx)
    return mn.astype(np.float16), mx.astype(np.float16)


def block_scores(mn: np.ndarray, mx: np.ndarray, q_grp: np.ndarray) -> np.ndarray:
    """mn, mx float16 [nb][d]; q_grp float32 [H][d] -> float64 [nb]."""
    a = mn.astype(np.float64)
    b = mx.astype(np.float64)
    s = np.zeros(a.shape[0], np.float64)
    for qh in np.asarray(q_grp, np.float64):
        s += np.maximum(a * qh[None, :], b * qh[None, :]).sum(axis=1)
    return s


def expand_blocks(block_ids: np.ndarray, block: int) -> np.ndarray:
    """Block ids -> the token rows they cover, in order."""
    b = np.asarray(block_ids, np.int64)
    return (b[:, None] * block + np.arange(block)[None, :]).reshape(-1)
