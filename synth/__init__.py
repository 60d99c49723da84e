"""Seeded synthetic workloads for the sparse decode step.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic: no quantisation, no bit planes, no summaries, no
scoring, selection or attention.  Both the CPU oracle's tests and the GPU
path (tests, smoke run, bench) take their inputs from here, so the two sides
see the same bytes.

Every array is cut into independently seeded chunks (one chunk per head and
per 65,536 tokens), so any head or token range of a large workload can be
regenerated on its own, and the bytes do not depend on how many threads drew
them.

Shapes and value laws follow the settings the pages describe (the Fathom
summary's Qwen3-8B layer with 4-bit planes, the HashAttention notes' 32-bit
signatures with sink and local windows, and the OasisKV review's 16-token
min/max block summaries); the pages' real traces and benchmarks are not
available and these synthetic draws stand in for them.

bf16 data is returned as ``uint16`` bit patterns (round-to-nearest-even from
float32, done by torch on the CPU).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

D = 128                 # head dimension on every page's model
TOK_CHUNK = 65536       # tokens per independently seeded chunk

# Decode-step settings.  Sizes are those of the five workloads named for this
# path; the value laws are described in each generator below.
CONFIGS = {
    1: dict(kind="fathom", G=1, Hgrp=1, n=4096, budget=48, k=64, needles=0,
            boost_channels=8, boost=5.0, v_sigma="unit"),
    2: dict(kind="fathom", G=8, Hgrp=4, n=32768, budget=56, k=512, needles=16,
            boost_channels=8, boost=5.0, v_sigma="loguniform"),
    3: dict(kind="fathom", G=8, Hgrp=4, n=1 << 20, budget=56, k=512, needles=16,
            boost_channels=8, boost=5.0, v_sigma="loguniform",
            budgets=(47, 56, 92), uniform_channels=34),
    4: dict(kind="hamming", H=32, Hkv=8, n=131072, m=512, sink=128, local=128,
            planted=512, max_flips=4),
    5: dict(kind="minmax", R=64, G=8, Hgrp=4, n=16384, block=16, top_blocks=128,
            local_blocks=1),
}

SIGMA_LO, SIGMA_HI = 0.05, 4.0

# stream tags (arbitrary distinct integers)
_T_SIGMA, _T_SIGMA_V, _T_Q, _T_BOOST, _T_K, _T_V, _T_NEEDLE = 11, 12, 13, 14, 15, 16, 17
_T_SIG, _T_QSIG, _T_PLANT_POS, _T_PLANT_MASK = 21, 22, 23, 24
_T_ALIGN_POS, _T_ALIGN_T = 31, 32

# Layer "aligned": keys per KV head lifted along the group query, and the range
# of the lift in units of the bulk score's standard deviation.
ALIGNED_KEYS = 512
ALIGNED_LIFT = (3.0, 6.0)


def seed_of(cfg: int) -> int:
    return 1000 + cfg


def rng(*keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in keys])))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 (RNE) bit patterns as uint16 (torch CPU conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def log_uniform_sigma(g: np.random.Generator, shape) -> np.ndarray:
    u = g.uniform(math.log(SIGMA_LO), math.log(SIGMA_HI), size=shape)
    return np.exp(u).astype(np.float32)


def _normal_rows_bf16(keys, rows: int, sigma: np.ndarray | None) -> np.ndarray:
    """rows x D normal draws (scaled per channel by sigma) as bf16 bits."""
    x = rng(*keys).standard_normal((rows, D), dtype=np.float32)
    if sigma is not None:
        x *= sigma[None, :]
    return f32_to_bf16_bits(x)


def _fill_heads(out: np.ndarray, seed: int, tag: int, heads, sigmas) -> None:
    """out[h_i] <- normal rows for head heads[h_i], drawn chunk by chunk."""
    n = out.shape[1]
    jobs = []
    for hi, h in enumerate(heads):
        for c in range((n + TOK_CHUNK - 1) // TOK_CHUNK):
            jobs.append((hi, h, c))

    def run(job):
        hi, h, c = job
        lo = c * TOK_CHUNK
        rows = min(TOK_CHUNK, n - lo)
        sig = None if sigmas is None else sigmas[h]
        out[hi, lo:lo + rows] = _normal_rows_bf16((seed, tag, *np.atleast_1d(h), c), rows, sig)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(run, jobs))


# --------------------------------------------------------------------------
# Bit-plane (Fathom) workloads: configs 1-3
# --------------------------------------------------------------------------
def fathom_case(cfg: int, n: int | None = None, heads=None, with_values: bool = True,
                layer: str = "needles") -> dict:
    """One decode layer for the bit-plane index.

    Keys: bf16 N(0, sigma_j^2) per (KV head, channel), sigma log-uniform on
    [0.05, 4].  Queries: N(0, 1) per query head, with a set of 8 channels
    (drawn once per KV group) scaled by 5.  ``var`` is sigma^2: the key
    variance a calibration pass would report, handed to the read plan as an
    input.  Needles (configs 2-3): 16 distinct positions per KV head whose key
    is replaced by 3 * sqrt(sum_j sigma_j^2) * qsum / |qsum|, qsum being the sum
    of the group's query vectors, i.e. aligned with the query at three times
    the typical key norm.  Values: bf16 N(0,1) (config 1) or N(0, sigma'_j^2)
    with sigma' drawn independently from the same law (configs 2-3).

    ``layer="aligned"`` plants no needles.  Instead ALIGNED_KEYS = 512
    distinct positions per KV head (or n, if fewer) keep their normal draw k
    and add t * tau * qsum / |qsum|^2, with t uniform on [3, 6] per key and
    tau = sqrt(sum_j qsum_j^2 sigma_j^2) the standard deviation of qsum . k
    under the key law.  Their group score is the bulk's plus t standard
    deviations, and their norm stays near the bulk's, so which of them a scan
    ranks into the top k depends on how precisely it reads: a layer on which
    read plans of different depth give different attention mass, error and
    recall.  ``needle_pos`` then holds these positions.

    ``n`` overrides the token count (same per-chunk draws, so a shorter case
    is a prefix of the long one except for needle positions); ``heads``
    restricts the KV heads that are materialised (their bytes are identical to
    those in the full case).
    """
    assert layer in ("needles", "aligned")
    c = CONFIGS[cfg]
    assert c["kind"] == "fathom"
    seed = seed_of(cfg)
    G, Hgrp = c["G"], c["Hgrp"]
    n = c["n"] if n is None else int(n)
    heads = list(range(G)) if heads is None else [int(h) for h in heads]

    sigma = log_uniform_sigma(rng(seed, _T_SIGMA), (G, D))
    var = (sigma.astype(np.float32) * sigma.astype(np.float32)).astype(np.float32)

    q = np.empty((G * Hgrp, D), np.float32)
    for g in range(G):
        boost = rng(seed, _T_BOOST, g).choice(D, size=c["boost_channels"], replace=False)
        for h in range(Hgrp):
            qh = rng(seed, _T_Q, g * Hgrp + h).standard_normal(D, dtype=np.float32)
            qh[boost] *= np.float32(c["boost"])
            q[g * Hgrp + h] = qh

    K = np.empty((len(heads), n, D), np.uint16)
    _fill_heads(K, seed, _T_K, heads, sigma)

    if layer == "aligned":
        m = min(ALIGNED_KEYS, n)
        needle_pos = np.zeros((len(heads), m), np.int64)
        for hi, g in enumerate(heads):
            pos = np.sort(rng(seed, _T_ALIGN_POS, g, n).choice(n, size=m, replace=False))
            t = rng(seed, _T_ALIGN_T, g, n).uniform(*ALIGNED_LIFT, size=m)
            qsum = q[g * Hgrp:(g + 1) * Hgrp].astype(np.float64).sum(axis=0)
            tau = math.sqrt(float((qsum ** 2 * sigma[g].astype(np.float64) ** 2).sum()))
            lift = (t * tau / float(qsum @ qsum))[:, None] * qsum[None, :]
            K[hi, pos] = f32_to_bf16_bits((bf16_bits_to_f32(K[hi, pos]) + lift).astype(np.float32))
            needle_pos[hi] = pos
    elif c["needles"]:
        needle_pos = np.zeros((len(heads), c["needles"]), np.int64)
        for hi, g in enumerate(heads):
            pos = np.sort(rng(seed, _T_NEEDLE, g, n).choice(n, size=c["needles"], replace=False))
            qsum = q[g * Hgrp:(g + 1) * Hgrp].astype(np.float64).sum(axis=0)
            norm = 3.0 * math.sqrt(float((sigma[g].astype(np.float64) ** 2).sum()))
            vec = (norm * qsum / np.linalg.norm(qsum)).astype(np.float32)
            K[hi, pos] = f32_to_bf16_bits(vec[None, :])[0]
            needle_pos[hi] = pos
    else:
        needle_pos = np.zeros((len(heads), 0), np.int64)

    out = dict(cfg=cfg, G=G, Hgrp=Hgrp, n=n, d=D, heads=heads, sigma=sigma, var=var,
               q=q, K=K, needle_pos=needle_pos, budget=c["budget"], k=c["k"], layer=layer)
    if with_values:
        if c["v_sigma"] == "unit":
            vs = None
        else:
            vs = log_uniform_sigma(rng(seed, _T_SIGMA_V), (G, D))
        V = np.empty((len(heads), n, D), np.uint16)
        _fill_heads(V, seed, _T_V, heads, vs)
        out["V"] = V
    return out


# --------------------------------------------------------------------------
# Hamming-signature workload: config 4
# --------------------------------------------------------------------------
def hamming_case(cfg: int = 4, n: int | None = None, H: int | None = None,
                 with_kv: bool = True) -> dict:
    """32-bit signatures per (attention head, token), uniform random, except
    ``planted`` distinct positions per head in [sink, n - local) whose
    signature is the query signature with c bits flipped, c uniform on
    {0..4} and the flipped positions uniform.  Query signatures uniform.
    K/V: bf16 N(0,1) over ``Hkv`` KV heads; q: fp32 N(0,1) per query head.
    """
    c = CONFIGS[cfg]
    assert c["kind"] == "hamming"
    seed = seed_of(cfg)
    n = c["n"] if n is None else int(n)
    H = c["H"] if H is None else int(H)
    Hkv = min(c["Hkv"], H)
    sink, local = c["sink"], c["local"]
    planted = min(c["planted"], max(0, n - sink - local))

    qsig = rng(seed, _T_QSIG).integers(0, 1 << 32, size=c["H"], dtype=np.uint64).astype(np.uint32)[:H]
    sigs = np.empty((H, n), np.uint32)
    pos = np.zeros((H, planted), np.int64)
    flips = np.zeros((H, planted), np.int64)
    for h in range(H):
        for ch in range((n + TOK_CHUNK - 1) // TOK_CHUNK):
            lo = ch * TOK_CHUNK
            rows = min(TOK_CHUNK, n - lo)
            sigs[h, lo:lo + rows] = rng(seed, _T_SIG, h, ch).integers(
                0, 1 << 32, size=rows, dtype=np.uint64).astype(np.uint32)
        if planted:
            gp = rng(seed, _T_PLANT_POS, h, n)
            p = np.sort(gp.choice(n - sink - local, size=planted, replace=False) + sink)
            gm = rng(seed, _T_PLANT_MASK, h, n)
            cnt = gm.integers(0, c["max_flips"] + 1, size=planted)
            masks = np.zeros(planted, np.uint32)
            for i in range(planted):
                bits = gm.choice(32, size=int(cnt[i]), replace=False)
                for b in bits:
                    masks[i] |= np.uint32(1) << np.uint32(b)
            sigs[h, p] = qsig[h] ^ masks
            pos[h] = p
            flips[h] = cnt
    out = dict(cfg=cfg, H=H, Hkv=Hkv, n=n, d=D, sigs=sigs, qsig=qsig, planted_pos=pos,
               planted_flips=flips, m=c["m"], sink=sink, local=local)
    if with_kv:
        K = np.empty((Hkv, n, D), np.uint16)
        V = np.empty((Hkv, n, D), np.uint16)
        _fill_heads(K, seed, _T_K, list(range(Hkv)), None)
        _fill_heads(V, seed, _T_V, list(range(Hkv)), None)
        q = np.stack([rng(seed, _T_Q, h).standard_normal(D, dtype=np.float32) for h in range(H)])
        out.update(K=K, V=V, q=q)
    return out


# --------------------------------------------------------------------------
# Block-summary workload: config 5
# --------------------------------------------------------------------------
def minmax_case(cfg: int = 5, R: int | None = None, n: int | None = None,
                with_values: bool = True) -> dict:
    """R requests x G KV heads x n tokens.  Keys bf16 N(0, sigma_{r,g,j}^2)
    with sigma log-uniform on [0.05, 4]; values bf16 N(0,1); queries fp32
    N(0,1), Hgrp query heads per KV head."""
    c = CONFIGS[cfg]
    assert c["kind"] == "minmax"
    seed = seed_of(cfg)
    R = c["R"] if R is None else int(R)
    n = c["n"] if n is None else int(n)
    G, Hgrp = c["G"], c["Hgrp"]
    sigma = log_uniform_sigma(rng(seed, _T_SIGMA), (c["R"], G, D))[:R]
    heads = [(r, g) for r in range(R) for g in range(G)]
    sig_flat = {(r, g): sigma[r, g] for r, g in heads}

    K = np.empty((R * G, n, D), np.uint16)
    _fill_heads(K, seed, _T_K, heads, sig_flat)
    q = np.empty((R, G * Hgrp, D), np.float32)
    for r in range(R):
        for h in range(G * Hgrp):
            q[r, h] = rng(seed, _T_Q, r, h).standard_normal(D, dtype=np.float32)
    out = dict(cfg=cfg, R=R, G=G, Hgrp=Hgrp, n=n, d=D, block=c["block"],
               top_blocks=c["top_blocks"], local_blocks=c["local_blocks"],
               sigma=sigma, K=K.reshape(R, G, n, D), q=q)
    if with_values:
        V = np.empty((R * G, n, D), np.uint16)
        _fill_heads(V, seed, _T_V, heads, None)
        out["V"] = V.reshape(R, G, n, D)
    return out
