"""Synthetic quality harness for the bit-plane decode step.

For one synthetic decode layer and several read plans, runs the library's
step -- plan + scan, block-max top-k, gather attention -- and compares it
with dense attention over every token:

* ``rel_err``: |o_sparse - o_dense| / |o_dense| per query head (L2 over d),
  mean and max over heads;
* ``mass``: the dense softmax weight that falls on the selected rows, per
  query head, mean and min over heads (the output error is at most
  2 (1 - mass) times the largest value-row norm);
* ``needle_recall``: share of the planted tokens among the selected rows;
* ``exact_topk_recall``: share of the k rows with the largest exact score
  q̄·k (float64, unquantised bf16 keys) that the step selects;
* ``scan_bytes``: the plan's scan bytes (planes, metadata, scores).

A reference row ``exact_topk`` attends over the exact top-k rows instead, the
error that selection alone would leave.

Two layers (``synth.fathom_case``): ``needles`` plants a few keys far above
every other score (the needle workloads of the Fathom summary's evaluation;
every plan finds them and they hold nearly all the attention), ``aligned``
lifts 512 keys per KV head by 3 to 6 standard deviations of the bulk score,
so that attention is spread over rows that a coarse read misranks and the
plans separate.  On a sweep of budgets and uniform plans the harness reports
equal-error bits (Fathom summary, equal-error bytes): for each measure, the
budget at which the water-filling curve reaches the uniform 34-channel
4-bit (136-bit) plan, interpolated linearly between budgets, and the scan
bytes at that point.

The dense reference is plain float64 torch on the GPU; it is measurement
tooling, not part of the library's path.

    python -m sparse_top_decode_query_amd.quality --config 2 --layer aligned --sweep
"""
from __future__ import annotations

import argparse
import json
import math


DEFAULT_BUDGETS = (47, 56, 92)
DEFAULT_UNIFORM_CHANNELS = 34
SWEEP_BUDGETS = (16, 24, 32, 40, 47, 56, 64, 72, 80, 92, 112, 128)
SWEEP_UNIFORM = (8, 16, 24, 34, 48)
# measure -> True when larger is better
MEASURES = {"mass_mean": True, "exact_topk_recall": True, "needle_recall": True,
            "rel_err_mean": False}


def dense_probs(q4, Kf, scale):
    """Softmax weights [h][n] of the query rows q4 [h][d] over every row of Kf."""
    z = (q4 @ Kf.T) * scale
    p = (z - z.max(dim=1, keepdim=True).values).exp()
    return p / p.sum(dim=1, keepdim=True)


def dense_attention(q4, Kf, Vf, scale):
    """Softmax attention of the query rows q4 [h][d] over every row of Kf/Vf
    [n][d] (torch tensors of one dtype, float64 here)."""
    return dense_probs(q4, Kf, scale) @ Vf


def set_recall(selected, reference) -> float:
    """Share of the reference positions (rows of int arrays) found in the
    selected rows of the same KV head."""
    hit = total = 0
    for sel, ref in zip(selected, reference):
        ref = set(int(x) for x in ref)
        hit += len(ref & set(int(x) for x in sel))
        total += len(ref)
    return hit / total if total else 1.0


def equal_error_bits(curve, target, higher_is_better):
    """First point at which a measure, known at increasing bit counts, reaches
    ``target``: ``curve`` is [(bits, value, scan_bytes)] sorted by bits.

    Between two budgets the measure is taken as linear in the bits, and so are
    the scan bytes.  Returns (bits, scan_bytes, exact) where exact is False
    when the first budget already reaches the target (its bits are then an
    upper bound), or None when no budget of the curve reaches it."""
    def reached(v):
        return v >= target if higher_is_better else v <= target
    for i, (b, v, nb) in enumerate(curve):
        if not reached(v):
            continue
        if i == 0:
            return float(b), float(nb), False
        b0, v0, nb0 = curve[i - 1]
        f = (target - v0) / (v - v0)
        return b0 + f * (b - b0), nb0 + f * (nb - nb0), True
    return None


def equal_error_report(res, uniform_name, uniform_bits_per_head):
    """Equal-error bits of the water-filling plans (rows named B<bits>) against
    one uniform plan, per measure, from an ``evaluate`` result."""
    rows = sorted(((int(name[1:]), row) for name, row in res["plans"].items()
                   if name.startswith("B")), key=lambda t: t[0])
    uni = res["plans"][uniform_name]
    out = {"against": uniform_name, "uniform_bits": uniform_bits_per_head,
           "uniform_scan_bytes": uni["scan_bytes"]}
    for m, hib in MEASURES.items():
        curve = [(b, row[m], row["scan_bytes"]) for b, row in rows]
        hit = equal_error_bits(curve, uni[m], hib)
        entry = {"uniform_value": uni[m]}
        if hit is None:
            entry.update(bits=None, saving=None)
        else:
            b, nb, exact = hit
            entry.update(bits=round(b, 2), scan_bytes=int(round(nb)), exact=exact,
                         saving=round(uniform_bits_per_head / b, 3),
                         byte_saving=round(uni["scan_bytes"] / nb, 3))
        out[m] = entry
    return out


def evaluate(K, V, q, var, index, needles, k, budgets=DEFAULT_BUDGETS,
             uniform_channels=DEFAULT_UNIFORM_CHANNELS):
    """Quality of each read plan on one resident layer.

    K, V: bf16 bits (int16) [G][n][128] on the device; q float32 [G*Hgrp][128];
    var float32 [G][128]; index the layer's PlaneIndex; needles int [G][m]
    (host) planted positions; k the rows selected per KV head; budgets the
    water-filling budgets; uniform_channels one channel count or several for
    the uniform 4-bit plans."""
    import torch

    from sparse_top_decode_query_amd import bytemodel, lib

    G, n, d = K.shape
    Hgrp = q.shape[0] // G
    dev = K.device
    scale = 1.0 / math.sqrt(d)

    def widen(bits):       # bf16 bits (int16) -> float64
        return (bits.to(torch.int32) << 16).view(torch.float32).to(torch.float64)

    # dense weights and outputs and the exact top-k rows, one KV head at a time
    dense = torch.empty(G * Hgrp, d, dtype=torch.float64, device=dev)
    probs = []
    exact_top = []
    for g in range(G):
        Kf, Vf = widen(K[g]), widen(V[g])
        q4 = q[g * Hgrp:(g + 1) * Hgrp].to(torch.float64)
        probs.append(dense_probs(q4, Kf, scale))
        dense[g * Hgrp:(g + 1) * Hgrp] = probs[-1] @ Vf
        s = Kf @ q4.sum(0)
        exact_top.append(torch.topk(s, k).indices.sort().values.to(torch.int32))
        del Kf, Vf, s
    exact_top = torch.stack(exact_top)
    exact_cpu = exact_top.cpu().numpy()

    q3, K4, V4 = q.view(1, G * Hgrp, d), K.view(1, G, n, d), V.view(1, G, n, d)

    def score(idx):
        out = lib.gather_attend(q3, K4, V4, idx.view(1, G, -1)).view(G * Hgrp, d).to(torch.float64)
        err = (out - dense).norm(dim=1) / dense.norm(dim=1)
        mass = torch.cat([probs[g][:, idx[g].long()].sum(dim=1) for g in range(G)])
        return {"rel_err_mean": round(float(err.mean()), 6), "rel_err_max": round(float(err.max()), 6),
                "mass_mean": round(float(mass.mean()), 6), "mass_min": round(float(mass.min()), 6)}

    res = {"n": n, "k": k, "kv_heads": G, "plans": {}}
    unis = (uniform_channels,) if isinstance(uniform_channels, int) else tuple(uniform_channels)
    plans = [(f"B{B}", B, None) for B in budgets] + [(f"uniform_{u}x4", 0, u) for u in unis]
    bm = torch.empty(G, n // 64, device=dev)
    for name, B, uni in plans:
        depth, qbar, scores = lib.fathom_plan_scan(index, q, var, B, n, block_max=bm,
                                                   uniform_channels=uni)
        idx = lib.topk_select_block_max(scores, bm, k)
        row = score(idx)
        sel = idx.cpu().numpy()
        row["needle_recall"] = round(set_recall(sel, needles), 6)
        row["exact_topk_recall"] = round(set_recall(sel, exact_cpu), 6)
        d_rows = depth.cpu().numpy()
        row["plan_bits"] = int(d_rows.astype(int).sum())
        row["scan_bytes"] = bytemodel.plane_scan_bytes(n, d_rows)
        res["plans"][name] = row
        del scores, idx
    ref = score(exact_top)
    ref["needle_recall"] = round(set_recall(exact_cpu, needles), 6)
    res["exact_topk"] = ref
    return res


def run(cfg: int = 2, n: int | None = None, budgets=None, uniform_channels=None, device="cuda",
        layer: str = "needles", sweep: bool = False):
    """Generate a bit-plane config's layer (``n`` overrides its length; layer
    "needles" or "aligned"), ingest it with the library and evaluate the
    plans on it.  ``sweep`` evaluates the sweep budgets and uniform plans and
    adds the equal-error report against the uniform 34 x 4 plan."""
    import numpy as np
    import torch

    import synth
    from sparse_top_decode_query_amd import lib

    case = synth.fathom_case(cfg, n=n, layer=layer)
    dev = torch.device(device)
    K = torch.from_numpy(case["K"].view(np.int16)).to(dev)
    V = torch.from_numpy(case["V"].view(np.int16)).to(dev)
    q = torch.from_numpy(case["q"]).to(dev)
    var = torch.from_numpy(case["var"]).to(dev)
    index = lib.fathom_ingest(K)
    if budgets is None:
        budgets = SWEEP_BUDGETS if sweep else DEFAULT_BUDGETS
    if uniform_channels is None:
        uniform_channels = SWEEP_UNIFORM if sweep else DEFAULT_UNIFORM_CHANNELS
    res = evaluate(K, V, q, var, index, case["needle_pos"], case["k"], budgets, uniform_channels)
    res["config"] = cfg
    res["layer"] = layer
    name = f"uniform_{DEFAULT_UNIFORM_CHANNELS}x4"
    if name in res["plans"] and any(p.startswith("B") for p in res["plans"]):
        res["equal_error"] = equal_error_report(res, name, 4 * DEFAULT_UNIFORM_CHANNELS)
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--config", type=int, default=2, choices=(1, 2, 3))
    ap.add_argument("--n", type=int, default=None, help="token count override")
    ap.add_argument("--budgets", type=int, nargs="+", default=None)
    ap.add_argument("--layer", default="needles", choices=("needles", "aligned"))
    ap.add_argument("--sweep", action="store_true",
                    help="sweep budgets and uniform plans; report equal-error bits")
    args = ap.parse_args(argv)
    print(json.dumps(run(args.config, n=args.n, budgets=args.budgets, layer=args.layer,
                         sweep=args.sweep), indent=1))


if __name__ == "__main__":
    main()
