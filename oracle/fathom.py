"""Bit-plane index and per-query read plan (Fathom summary page).

Sources (Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
Caches -- summary page):
  * paragraph on storing keys as channel-major bit planes: keys are quantised
    per channel to 4-bit uniform codes with an fp16 scale per 64-token block;
    each code bit becomes its own plane, planes are stored channel-major, and
    reading the first t planes of a channel is exactly the t-bit quantiser
    under the same block scale.
  * paragraph on per-query reverse water-filling: channel j adds q_j^2 times
    the key's calibrated variance to the score variance, each extra bit read
    cuts that channel's remaining error by about 4x, and a budget of B bits is
    spread over channels (0 to 4 bits each) by this marginal gain; the query
    heads under one KV head share one plan.

Readings taken where the page is silent:
  * the quantiser is asymmetric: offset = fp16(block min), scale =
    fp16((max - min) / 15), code = clamp(rint((x - offset) / scale), 0, 15),
    all in float32, code 0 when the scale is 0;
  * the index is built from the bf16 keys of the KV cache (widened exactly);
  * a t-bit prefix is reconstructed at the midpoint of its bin;
  * the GQA group's score is the sum of its heads' scores, i.e. one query
    qbar = sum of the group's query vectors, and the plan's channel weight is
    w_j = qbar_j^2 * var_j;
  * the marginal gain is exactly /4 per bit and ties are ordered by
    (gain descending, channel ascending, bit ascending);
  * the budget counts plane bits only (metadata is separate).

  * a growing cache's last, partly filled block is quantised over the
    tokens it holds (its scale and offset change as tokens arrive) and its
    absent tokens hold code 0; a block is final once its 64 tokens are in.

Layouts (shared with the GPU path by definition, not by code), for a row
capacity of n_cap tokens (a multiple of 64; n_cap = n for a full index):
  planes  uint32 [d][4][n_cap/32]  plane p holds code bit (3-p) (p=0 is the
                                   MSB); token i is bit (i & 31) of word (i >> 5)
  meta    uint32 [d][n_cap/64]     low half = fp16 scale bits, high half =
                                   fp16 offset bits, one word per 64-token block
"""
from __future__ import annotations

import numpy as np

BLOCK = 64          # tokens per quantisation block
BITS = 4            # code bits per channel


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# quantiser and plane packing (one KV head)
# --------------------------------------------------------------------------
def quantise_block(x: np.ndarray):
    """One 64-token block of one head: float32 keys [m][...] of the m >= 1
    tokens present -> codes uint8 [m][...], scale and offset float16 [...]
    (any trailing shape: channels, or blocks x channels)."""
    mn = x.min(axis=0)
    mx = x.max(axis=0)
    offset = mn.astype(np.float16)
    scale = ((mx - mn) / np.float32(15.0)).astype(np.float32).astype(np.float16)
    off32 = offset.astype(np.float32)[None]
    sc32 = scale.astype(np.float32)[None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint((x - off32) / sc32)
    r = np.where(sc32 == 0, np.float32(0), r)
    return np.clip(r, 0, 15).astype(np.uint8), scale, offset


def quantise(k_bf16: np.ndarray):
    """4-bit per-channel block quantiser of one head's keys.

    k_bf16: uint16 [n][d] (bf16 bits), any n >= 1.  Every 64-token block is
    quantised over the tokens it holds: a last, partly filled block (the open
    block of a growing cache) takes its scale and offset from its present
    tokens only, and is quantised again as tokens arrive until it is full.
    Returns codes uint8 [n][d], scale float16 [nb][d], offset float16 [nb][d]
    with nb = ceil(n / 64).
    """
    x = bf16_bits_to_f32(k_bf16)
    n, d = x.shape
    nf = n // BLOCK                       # full blocks, quantised side by side
    codes = np.zeros((n, d), np.uint8)
    scale = np.zeros((-(-n // BLOCK), d), np.float16)
    offset = np.zeros_like(scale)
    if nf:
        c, sc, off = quantise_block(x[:nf * BLOCK].reshape(nf, BLOCK, d).transpose(1, 0, 2))
        codes[:nf * BLOCK] = c.transpose(1, 0, 2).reshape(nf * BLOCK, d)
        scale[:nf], offset[:nf] = sc, off
    if n > nf * BLOCK:
        codes[nf * BLOCK:], scale[nf], offset[nf] = quantise_block(x[nf * BLOCK:])
    return codes, scale, offset


def pack_planes(codes: np.ndarray, n_cap: int | None = None) -> np.ndarray:
    """codes uint8 [n][d] -> planes uint32 [d][4][n_cap/32]; tokens from n
    up to the row capacity n_cap (default: n rounded up to 64) hold 0 bits."""
    n, d = codes.shape
    n_cap = -(-n // BLOCK) * BLOCK if n_cap is None else int(n_cap)
    assert n_cap % BLOCK == 0 and n_cap >= n
    planes = np.zeros((d, BITS, n_cap // 32), np.uint32)
    ct = np.zeros((d, n_cap), np.uint8)
    ct[:, :n] = codes.T                                                 # [d][n_cap]
    for p in range(BITS):
        bits = (ct >> (BITS - 1 - p)) & 1                               # [d][n]
        # byte b of a channel's bit string holds tokens 8b..8b+7, token 8b in bit 0;
        # four such bytes read little-endian form one 32-token word
        packed = np.packbits(bits, axis=1, bitorder="little")           # [d][n/8]
        planes[:, p, :] = packed.view("<u4")
    return planes


def pack_meta(scale: np.ndarray, offset: np.ndarray, nb_cap: int | None = None) -> np.ndarray:
    """scale/offset float16 [nb][d] -> meta uint32 [d][nb_cap] (blocks past
    nb hold 0)."""
    s = scale.view(np.uint16).astype(np.uint32)
    o = offset.view(np.uint16).astype(np.uint32)
    nb, d = s.shape
    nb_cap = nb if nb_cap is None else int(nb_cap)
    meta = np.zeros((d, nb_cap), np.uint32)
    meta[:, :nb] = (s | (o << 16)).T
    return meta


def unpack_meta(meta: np.ndarray):
    """meta uint32 [d][nb] -> (scale, offset) float16 [d][nb]."""
    s = (meta & 0xFFFF).astype(np.uint16).view(np.float16)
    o = (meta >> 16).astype(np.uint16).view(np.float16)
    return s, o


def plane_bits(planes_j: np.ndarray, p: int, n: int) -> np.ndarray:
    """Token bits (0/1 uint8 [n]) of plane p of one channel."""
    words = planes_j[p].astype("<u4")
    return np.unpackbits(words.view(np.uint8), bitorder="little")[:n]


def prefix_code(planes_j: np.ndarray, t: int, n: int) -> np.ndarray:
    """Value of the first t planes of one channel, read as a t-bit code."""
    c = np.zeros(n, np.int64)
    for p in range(t):
        c = (c << 1) | plane_bits(planes_j, p, n)
    return c


def ingest(k_bf16_heads: np.ndarray, n: int | None = None, n_cap: int | None = None):
    """Index of the first n tokens of every head (default: all of them).

    k_bf16_heads uint16 [G][>=n][d] -> planes uint32 [G][d][4][n_cap/32],
    meta uint32 [G][d][n_cap/64]; n_cap defaults to n rounded up to 64.  The
    result is what a growing index holds once its first n tokens have been
    appended, however the appends were split: closed blocks are final, the
    open block is quantised over its present tokens, and everything past
    token n is zero here (left as it was by the GPU append)."""
    n = k_bf16_heads.shape[1] if n is None else int(n)
    n_cap = -(-n // BLOCK) * BLOCK if n_cap is None else int(n_cap)
    planes, metas = [], []
    for kh in k_bf16_heads:
        codes, scale, offset = quantise(kh[:n])
        planes.append(pack_planes(codes, n_cap))
        metas.append(pack_meta(scale, offset, n_cap // BLOCK))
    return np.stack(planes), np.stack(metas)


# --------------------------------------------------------------------------
# read plan (one KV head)
# --------------------------------------------------------------------------
def group_query(q_grp: np.ndarray) -> np.ndarray:
    """qbar = sum of the group's query vectors, added in float32 in head order."""
    q_grp = np.asarray(q_grp, np.float32)
    acc = q_grp[0].copy()
    for h in range(1, q_grp.shape[0]):
        acc = (acc + q_grp[h]).astype(np.float32)
    return acc


def channel_weight(qbar: np.ndarray, var: np.ndarray) -> np.ndarray:
    """w_j = (qbar_j * qbar_j) * var_j, two float32 multiplies.

    A variance is never negative, so a weight that comes out negative or NaN
    (a negative or NaN variance handed in) is read as zero gain: that channel
    competes only for bits nobody else wants, in channel order."""
    qq = (qbar.astype(np.float32) * qbar.astype(np.float32)).astype(np.float32)
    w = (qq * np.asarray(var, np.float32)).astype(np.float32)
    return np.where(w > 0, w, np.float32(0)).astype(np.float32)


def plan(q_grp: np.ndarray, var: np.ndarray, budget: int):
    """Greedy marginal-gain bit allocation (reverse water-filling).

    Item (j, t) for t = 0..3 is the t-th extra bit of channel j; its gain is
    w_j * 4^-t (one float32 multiply by an exact power of two).  The first
    min(budget, 4d) items in the order (gain desc, j asc, t asc) are taken and
    depth_j counts the items taken from channel j.  Gains never grow with t
    and equal gains inside a channel go to the lower t, so the taken set is a
    prefix of every channel: a real read plan.

    Returns depth uint8 [d], qbar float32 [d].
    """
    qbar = group_query(q_grp)
    w = channel_weight(qbar, var)
    d = w.shape[0]
    items = []
    for j in range(d):
        for t in range(BITS):
            g = float(np.float32(w[j]) * np.float32(4.0 ** -t))
            items.append((-g, j, t))
    items.sort()
    depth = np.zeros(d, np.uint8)
    for _, j, _t in items[:max(0, min(int(budget), BITS * d))]:
        depth[j] += 1
    return depth, qbar


def plan_uniform(q_grp: np.ndarray, var: np.ndarray, n_channels: int):
    """Uniform-depth baseline plan: the n_channels channels of largest w_j
    (ties to the lower channel) read at all 4 bits."""
    qbar = group_query(q_grp)
    w = channel_weight(qbar, var)
    order = sorted(range(w.shape[0]), key=lambda j: (-float(w[j]), j))
    depth = np.zeros(w.shape[0], np.uint8)
    depth[order[:n_channels]] = BITS
    return depth, qbar


# --------------------------------------------------------------------------
# plane-prefix scan (one KV head)
# --------------------------------------------------------------------------
def dequant_prefix(planes_j, scale_j, offset_j, t: int, n: int) -> np.ndarray:
    """Keys of one channel rebuilt from its first t planes (float64 [n]):
    offset + scale * (bin midpoint of the t-bit prefix, in 4-bit code units)."""
    c = prefix_code(planes_j, t, n).astype(np.float64)
    step = float(2 ** (BITS - t))
    mid = c * step + (step - 1.0) / 2.0
    blk = np.arange(n) // BLOCK
    return offset_j.astype(np.float64)[blk] + scale_j.astype(np.float64)[blk] * mid


def scan(planes: np.ndarray, meta: np.ndarray, depth: np.ndarray, qbar: np.ndarray,
         n: int) -> np.ndarray:
    """Approximate scores s_i = sum over read channels of qbar_j * khat_ij
    (float64 [n]).  Unread channels contribute nothing and their metadata is
    not used."""
    scale, offset = unpack_meta(meta)
    s = np.zeros(n, np.float64)
    for j in range(planes.shape[0]):
        t = int(depth[j])
        if t == 0:
            continue
        s += float(qbar[j]) * dequant_prefix(planes[j], scale[j], offset[j], t, n)
    return s


def scan_heads(planes, meta, depth, qbar, n):
    return np.stack([scan(planes[g], meta[g], depth[g], qbar[g], n) for g in range(planes.shape[0])])


def plan_heads(q, var, Hgrp, budget=None, n_uniform=None):
    G = var.shape[0]
    deps, qbs = [], []
    for g in range(G):
        qg = q[g * Hgrp:(g + 1) * Hgrp]
        if n_uniform:
            dp, qb = plan_uniform(qg, var[g], n_uniform)
        else:
            dp, qb = plan(qg, var[g], budget)
        deps.append(dp)
        qbs.append(qb)
    return np.stack(deps), np.stack(qbs)
