"""KV selection against a GPU-resident block pool (OasisKV review, core
method and method-steps sections).

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline use this module; the library never does.

Each (request, KV head) keeps a pool of S block slots on the GPU.  A decode
step predicts a set P of blocks (the top-K of the block scores under the draft
query).  Selection then:
  * keeps every resident block that is in P (a hit costs no transfer) and
    stamps its slot with the current step (the step it was last selected);
  * lists the predicted blocks that are not resident (the misses);
  * lists the slots whose block is not in P (eviction targets), least
    recently selected first;
  * pairs the i-th miss with the i-th target, for at most C pairs per KV
    head and step (the fetch cap), and writes each pair into the pool: the
    target slot now holds the missed block, stamped with the current step.
The pairs form the transfer plan of the step.

Readings taken where the pages are silent:
  * misses are taken best first: by block score descending, equal scores to
    the lower block id;
  * an empty slot (block id -1) is taken before any occupied one; occupied
    targets are ordered by their stamp ascending, equal stamps to the lower
    slot;
  * with more misses than the cap (or than targets), the remaining misses
    stay unfetched this step.
"""
from __future__ import annotations

import numpy as np


def select(pred, scores, resident, last_sel, step: int, cap: int):
    """One (request, KV head).

    pred      int [K]: predicted block ids (distinct; negative entries ignored)
    scores    float [nb]: block scores (rank the misses)
    resident  int [S]: block id per slot, -1 for an empty slot
    last_sel  int [S]: step at which each slot's block was last selected
    Returns (resident', last_sel', plan) with plan a list of (slot, block)
    pairs in the order they were made.
    """
    resident = [int(b) for b in resident]
    last_sel = [int(t) for t in last_sel]
    P = {int(b) for b in pred if int(b) >= 0}
    held = {b for b in resident if b >= 0}
    for s, b in enumerate(resident):
        if b >= 0 and b in P:
            last_sel[s] = int(step)
    misses = sorted(P - held, key=lambda b: (-float(scores[b]), b))
    targets = [s for s, b in enumerate(resident) if b < 0 or b not in P]
    targets.sort(key=lambda s: (resident[s] >= 0, last_sel[s] if resident[s] >= 0 else 0, s))
    plan = []
    for b, s in zip(misses[:max(0, int(cap))], targets):
        resident[s] = b
        last_sel[s] = int(step)
        plan.append((s, b))
    return resident, last_sel, plan


def select_rows(pred, scores, resident, last_sel, step: int, cap: int):
    """All rows: pred int [rows][K], scores [rows][nb], resident/last_sel
    [rows][S] -> (resident', last_sel', plan_slot [rows][cap],
    plan_block [rows][cap] (-1 padded), n_fetch [rows])."""
    rows, S = np.asarray(resident).shape
    res = np.empty((rows, S), np.int64)
    ls = np.empty((rows, S), np.int64)
    ps = np.full((rows, max(0, cap)), -1, np.int64)
    pb = np.full((rows, max(0, cap)), -1, np.int64)
    nf = np.zeros(rows, np.int64)
    for r in range(rows):
        res[r], ls[r], plan = select(pred[r], scores[r], resident[r], last_sel[r], step, cap)
        nf[r] = len(plan)
        for i, (s, b) in enumerate(plan):
            ps[r, i], pb[r, i] = s, b
    return res, ls, ps, pb, nf


def fetch(pool, host_blocks, plan):
    """Copy each planned block from the host-side cache into its slot.
    pool [S][...] and host_blocks [nb][...] (the same row shape) -> pool'."""
    pool = np.array(pool, copy=True)
    for s, b in plan:
        pool[s] = host_blocks[b]
    return pool
