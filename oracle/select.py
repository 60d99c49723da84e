"""Top-k selection (HashAttention study notes, sec. 2.1 three-stage inference
and sec. 3.1 protocol; Fathom summary, top-k=512 setting; OasisKV review,
per-KV-head global top-K over block summaries).

Ordering: by key (largest first for scores, smallest first for Hamming
distances), equal keys broken towards the lower index.  Keys are compared as
numbers, so -0.0 and +0.0 tie.  Keys must be finite.

Windows: the first ``n_sink`` and last ``n_local`` positions are always kept
and do not compete; ``k`` more are taken from [n_sink, n - n_local), so a row
yields k + n_sink + n_local distinct indices (the notes count the retrieval
budget separately from the fixed positions, with no overlap).  If k is at
least the size of the competition range, every index is returned.

Output: int64 indices in ascending order.
"""
from __future__ import annotations

import numpy as np


def topk(keys: np.ndarray, k: int, largest: bool = True, n_sink: int = 0,
         n_local: int = 0) -> np.ndarray:
    keys = np.asarray(keys)
    n = keys.shape[0]
    assert 0 <= n_sink and 0 <= n_local and n_sink + n_local <= n
    lo, hi = n_sink, n - n_local
    comp = keys[lo:hi].astype(np.float64)
    idx = np.arange(lo, hi)
    primary = -comp if largest else comp
    order = np.lexsort((idx, primary))          # last key is the primary sort key
    chosen = idx[order[:max(0, min(int(k), hi - lo))]]
    out = np.concatenate([np.arange(0, lo), np.sort(chosen), np.arange(hi, n)])
    return out.astype(np.int64)


def topk_rows(keys2d: np.ndarray, k: int, largest: bool = True, n_sink: int = 0,
              n_local: int = 0) -> np.ndarray:
    return np.stack([topk(r, k, largest, n_sink, n_local) for r in keys2d])
