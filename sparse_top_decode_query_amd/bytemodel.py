"""Algorithmic byte and operation counts of the decode step's stages.

These are the bytes the method must move (what the roofline is priced on),
not what a kernel happens to move.  The formulas follow the pages' own
accounting:

  * Fathom summary, opening paragraphs: dense attention reads every cached
    K and V row; a 136-bit per-token scan index costs 17 bytes per token per
    KV head per layer, and the k winners' bf16 K/V rows are read afterwards.
  * OasisKV review, KV-cache background: M_KV = B * L * N_layer * 2 N_kv *
    d_h * s; its min/max summary is 1/16 of the KV cache (fp16 min and max
    per 16-token block).
  * HashAttention study notes, sec. 2.5: a 32-bit signature is 4 bytes per
    token per head, 1/64 of a 128-dim fp16 key; sec. 3.1 budget example:
    m retrieved plus the fixed sink/local positions.
"""
from __future__ import annotations


def kv_cache_bytes(batch: int, tokens: int, layers: int, kv_heads: int, head_dim: int,
                   elem_bytes: int = 2) -> int:
    """M_KV = B * L * N_layer * 2 * N_kv * d_h * s."""
    return batch * tokens * layers * 2 * kv_heads * head_dim * elem_bytes


def uniform_index_bytes(tokens: int, layers: int, kv_heads: int, bits_per_token: int) -> int:
    """A per-token scan index of ``bits_per_token`` bits per KV head and layer."""
    return tokens * layers * kv_heads * bits_per_token // 8


def plane_scan_read_bytes(n: int, depths) -> int:
    """Bytes the plane-prefix scan reads for one decode step of one layer.

    ``depths`` is one plan (sequence of per-channel depths) per KV head.  A
    channel read to depth t costs t plane bits per token, plus its 32-bit
    scale/offset word per 64-token block (A/16 bytes per token for A read
    channels)."""
    total = 0
    for dep in depths:
        bits = sum(int(t) for t in dep)
        active = sum(1 for t in dep if int(t) > 0)
        total += bits * n // 8 + active * (n // 64) * 4
    return total


def plane_scan_bytes(n: int, depths, score_bytes: int = 4) -> int:
    """Read bytes plus the fp32 score written per token per KV head."""
    return plane_scan_read_bytes(n, depths) + score_bytes * n * len(depths)


def plane_scan_bit_ops(n: int, depths) -> int:
    """One weighted accumulate per plane bit per token (the scan's inner work)."""
    return sum(sum(int(t) for t in dep) for dep in depths) * n


def summary_bytes_per_token(head_dim: int = 128, block: int = 16, elem_bytes: int = 2) -> float:
    """fp16 min and max vectors per block of ``block`` tokens, per token."""
    return 2 * head_dim * elem_bytes / block


def kv_bytes_per_token(head_dim: int = 128, elem_bytes: int = 2) -> int:
    return 2 * head_dim * elem_bytes


def minmax_scan_bytes(blocks: int, rows: int, head_dim: int = 128) -> int:
    """Summaries read (fp16 min + max per block) plus one fp32 score per block."""
    return rows * blocks * (2 * head_dim * 2 + 4)


def hamming_scan_bytes(n: int, heads: int) -> int:
    """4-byte signature read plus a 1-byte distance written per token-head."""
    return n * heads * (4 + 1)


def attend_bytes(rows_per_set: int, sets: int, head_dim: int = 128) -> int:
    """bf16 K and V rows read for every selected row of every set."""
    return rows_per_set * sets * 2 * head_dim * 2


def budget_fraction(n: int, m: int, fixed: int) -> float:
    """Share of the context read when m rows are retrieved plus ``fixed``
    always-kept positions (no overlap)."""
    return (m + fixed) / n
