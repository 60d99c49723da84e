"""Hamming score of packed binary signatures (HashAttention study notes,
sec. 2.2: the score of a cached key is minus the Hamming distance between its
signature and the query's, computed as the popcount of their XOR)."""
from __future__ import annotations

import numpy as np


def distances(sigs: np.ndarray, qsig) -> np.ndarray:
    """sigs uint32 [..., n], qsig uint32 broadcastable -> uint8 distances in [0, 32]."""
    x = np.bitwise_xor(np.asarray(sigs, np.uint32), np.asarray(qsig, np.uint32))
    return np.bitwise_count(x).astype(np.uint8)


def distances_heads(sigs: np.ndarray, qsig: np.ndarray) -> np.ndarray:
    return distances(sigs, np.asarray(qsig, np.uint32)[:, None])
