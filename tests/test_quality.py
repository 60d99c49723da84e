"""The quality harness's own host-side pieces (CPU): its dense attention
against the oracle's attention over every row, and its recall count."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import attend
from sparse_top_decode_query_amd import quality


def test_dense_attention_matches_oracle_over_all_rows():
    rng = np.random.default_rng(7)
    n, d, h = 300, 128, 4
    Kb = synth.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32) * 2)
    Vb = synth.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32))
    q = rng.standard_normal((h, d)).astype(np.float32) * 3
    scale = 1.0 / math.sqrt(d)

    def widen(b):
        return torch.from_numpy((b.astype(np.uint32) << 16).view(np.float32).astype(np.float64))

    got = quality.dense_attention(torch.from_numpy(q.astype(np.float64)), widen(Kb), widen(Vb), scale)
    for i in range(h):
        ref = attend.attend_rows(q[i], Kb, Vb, scale)
        assert np.allclose(got[i].numpy(), ref, rtol=1e-12, atol=1e-14)


def test_set_recall_counts_per_head():
    sel = np.array([[0, 5, 9], [1, 2, 3]])
    ref = np.array([[5, 6], [3, 1]])
    assert quality.set_recall(sel, ref) == 0.75
    assert quality.set_recall(sel, np.zeros((2, 0), np.int64)) == 1.0


@pytest.mark.gpu
def test_quality_harness_recall_matches_oracle_plans():
    """The harness on the 32k-token layer: every plan finds every needle, and
    each plan's exact-top-k recall is the one the oracle's own plan, scan and
    top-k give (within a few swaps near the k-th score)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oracle import fathom
    print("[quality] config 2, plans B47 B56 B92 uniform 34x4", flush=True)
    res = quality.run(2)
    print(res, flush=True)
    case = synth.fathom_case(2)
    G, Hgrp, n, k = case["G"], case["Hgrp"], case["n"], case["k"]
    Kf = (case["K"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = [np.argsort(-(Kf[g] @ case["q"][g * Hgrp:(g + 1) * Hgrp].astype(np.float64).sum(0)),
                        kind="stable")[:k] for g in range(G)]
    planes, meta = fathom.ingest(case["K"])
    for name, (B, uni) in {"B47": (47, None), "B56": (56, None), "B92": (92, None),
                           "uniform_34x4": (None, 34)}.items():
        row = res["plans"][name]
        depth, qbar = fathom.plan_heads(case["q"], case["var"], Hgrp, budget=B, n_uniform=uni)
        sc = fathom.scan_heads(planes, meta, depth, qbar, n)
        sel = [np.argsort(-sc[g], kind="stable")[:k] for g in range(G)]
        assert row["plan_bits"] == int(np.asarray(depth).astype(int).sum())
        assert row["needle_recall"] == 1.0
        assert abs(row["exact_topk_recall"] - quality.set_recall(sel, exact)) <= 16 / (G * k)
        assert 0.0 <= row["rel_err_mean"] <= row["rel_err_max"] < 1.0
    assert res["exact_topk"]["needle_recall"] == 1.0


def test_mass_bounds_the_sparse_error():
    """|o_sparse - o_dense| <= 2 (1 - mass) max_i |v_i| for the renormalised
    attention over any subset (oracle attention over the subset)."""
    rng = np.random.default_rng(11)
    n, d = 500, 128
    Kb = synth.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32))
    Vb = synth.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32))
    q = rng.standard_normal(d).astype(np.float32) * 4
    scale = 1.0 / math.sqrt(d)
    Kf = torch.from_numpy((Kb.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    Vf = (Vb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    p = quality.dense_probs(torch.from_numpy(q.astype(np.float64))[None], Kf, scale)[0].numpy()
    assert abs(p.sum() - 1.0) < 1e-12
    dense = p @ Vf
    vmax = np.linalg.norm(Vf, axis=1).max()
    for m in (1, 10, 100, 499):
        sel = np.sort(rng.choice(n, m, replace=False))
        o = attend.attend_rows(q, Kb[sel], Vb[sel], scale)
        assert np.linalg.norm(o - dense) <= 2 * (1 - p[sel].sum()) * vmax + 1e-12


def test_equal_error_bits_interpolates_between_budgets():
    curve = [(16, 0.30, 1000), (32, 0.50, 2000), (64, 0.70, 4000)]
    b, nb, exact = quality.equal_error_bits(curve, 0.60, True)
    assert exact and b == pytest.approx(48.0) and nb == pytest.approx(3000.0)
    assert quality.equal_error_bits(curve, 0.25, True) == (16.0, 1000.0, False)
    assert quality.equal_error_bits(curve, 0.80, True) is None
    err = [(16, 0.9, 10), (32, 0.5, 20), (64, 0.1, 40)]
    b, nb, exact = quality.equal_error_bits(err, 0.3, False)
    assert exact and b == pytest.approx(48.0) and nb == pytest.approx(30.0)


def test_equal_error_report_against_uniform_plan():
    plans = {f"B{b}": {"mass_mean": m, "exact_topk_recall": r, "needle_recall": 1.0,
                       "rel_err_mean": e, "scan_bytes": 10 * b}
             for b, m, r, e in ((32, 0.40, 0.5, 0.8), (64, 0.50, 0.7, 0.6), (128, 0.60, 0.9, 0.4))}
    plans["uniform_34x4"] = {"mass_mean": 0.55, "exact_topk_recall": 0.8, "needle_recall": 1.0,
                             "rel_err_mean": 0.5, "scan_bytes": 1360}
    rep = quality.equal_error_report({"plans": plans}, "uniform_34x4", 136)
    assert rep["mass_mean"]["bits"] == pytest.approx(96.0)
    assert rep["exact_topk_recall"]["bits"] == pytest.approx(96.0)
    assert rep["rel_err_mean"]["bits"] == pytest.approx(96.0)
    assert rep["mass_mean"]["saving"] == pytest.approx(136 / 96, abs=1e-3)
    assert rep["mass_mean"]["byte_saving"] == pytest.approx(1360 / 960, abs=1e-3)
    assert rep["needle_recall"]["bits"] == 32.0 and rep["needle_recall"]["exact"] is False


def test_aligned_layer_lifts_keys_by_the_stated_deviations():
    """The aligned layer's planted keys score 3 to 6 bulk standard deviations
    above the bulk under the group query (float64, before bf16 rounding of the
    lift the score moves by exactly t tau), and every other row is the needle
    layer's row without its needles."""
    n = 8192
    a = synth.fathom_case(2, n=n, heads=[0, 3], with_values=False, layer="aligned")
    b = synth.fathom_case(2, n=n, heads=[0, 3], with_values=False)
    Hgrp = a["Hgrp"]
    for hi, g in enumerate(a["heads"]):
        pos = a["needle_pos"][hi]
        assert len(np.unique(pos)) == len(pos) == synth.ALIGNED_KEYS
        qs = a["q"][g * Hgrp:(g + 1) * Hgrp].astype(np.float64).sum(0)
        tau = math.sqrt(float((qs ** 2 * a["var"][g].astype(np.float64)).sum()))
        ka = synth.bf16_bits_to_f32(a["K"][hi]).astype(np.float64)
        kb = synth.bf16_bits_to_f32(b["K"][hi]).astype(np.float64)
        lift = (ka[pos] - kb[pos]) @ qs / tau
        ok = ~np.isin(pos, b["needle_pos"][hi])
        assert lift[ok].min() > 3.0 - 0.05 and lift[ok].max() < 6.0 + 0.05
        rest = np.setdiff1d(np.arange(n), np.union1d(pos, b["needle_pos"][hi]))
        assert np.array_equal(a["K"][hi][rest], b["K"][hi][rest])
        bulk = kb[rest] @ qs
        assert abs(bulk.std() / tau - 1.0) < 0.05


def test_aligned_layer_separates_the_plans_on_the_oracle():
    """On the aligned layer (32k tokens, 8 KV heads, k = 512) the oracle's
    plan, scan and top-k recall more of the exact top-k with more bits, and
    the water-filling plans reach the uniform 34 x 4 plan's recall between 56
    and 128 bits: the layer separates the plans."""
    from oracle import fathom
    case = synth.fathom_case(2, layer="aligned", with_values=False)
    G, Hgrp, n, k = case["G"], case["Hgrp"], case["n"], case["k"]
    Kf = synth.bf16_bits_to_f32(case["K"]).astype(np.float64)
    exact = [np.argsort(-(Kf[g] @ case["q"][g * Hgrp:(g + 1) * Hgrp].astype(np.float64).sum(0)),
                        kind="stable")[:k] for g in range(G)]
    planes, meta = fathom.ingest(case["K"])

    def recall(B=None, U=None):
        depth, qbar = fathom.plan_heads(case["q"], case["var"], Hgrp, budget=B, n_uniform=U)
        sc = fathom.scan_heads(planes, meta, depth, qbar, n)
        return quality.set_recall([np.argsort(-sc[g], kind="stable")[:k] for g in range(G)], exact)

    rb = {B: recall(B=B) for B in (32, 56, 92, 128)}
    ru = recall(U=34)
    assert rb[32] < rb[56] < rb[92] < rb[128]
    assert rb[56] < ru < rb[128]
    assert rb[128] - rb[32] > 0.2


@pytest.mark.gpu
def test_quality_aligned_sweep_matches_oracle_plans():
    """The sweep on the aligned layer (32k tokens): each plan's exact-top-k
    recall is the oracle's within a few swaps near the k-th score, the
    water-filling curve rises with bits, and its equal-recall bits against
    the uniform 136-bit plan are those the oracle's recalls give (within the
    few bits those swaps can move the interpolation)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oracle import fathom
    print("[quality] config 2 aligned layer, sweep", flush=True)
    res = quality.run(2, layer="aligned", sweep=True)
    print({k: v for k, v in res.items() if k != "plans"}, flush=True)
    case = synth.fathom_case(2, layer="aligned", with_values=False)
    G, Hgrp, n, k = case["G"], case["Hgrp"], case["n"], case["k"]
    Kf = synth.bf16_bits_to_f32(case["K"]).astype(np.float64)
    exact = [np.argsort(-(Kf[g] @ case["q"][g * Hgrp:(g + 1) * Hgrp].astype(np.float64).sum(0)),
                        kind="stable")[:k] for g in range(G)]
    planes, meta = fathom.ingest(case["K"])
    oracle_rec = {}
    for name, row in res["plans"].items():
        B = int(name[1:]) if name.startswith("B") else None
        U = None if B is not None else int(name.split("_")[1].split("x")[0])
        depth, qbar = fathom.plan_heads(case["q"], case["var"], Hgrp, budget=B, n_uniform=U)
        sc = fathom.scan_heads(planes, meta, depth, qbar, n)
        rec = quality.set_recall([np.argsort(-sc[g], kind="stable")[:k] for g in range(G)], exact)
        oracle_rec[name] = rec
        assert row["plan_bits"] == int(np.asarray(depth).astype(int).sum()), name
        assert abs(row["exact_topk_recall"] - rec) <= 16 / (G * k), name
    bs = sorted(int(p[1:]) for p in res["plans"] if p.startswith("B"))
    curve = [res["plans"][f"B{b}"]["exact_topk_recall"] for b in bs]
    assert curve[-1] - curve[0] > 0.2 and res["plans"]["B128"]["mass_mean"] > res["plans"]["B32"]["mass_mean"]
    ee = res["equal_error"]["exact_topk_recall"]
    ocurve = [(b, oracle_rec[f"B{b}"], 0) for b in bs]
    ob, _, _ = quality.equal_error_bits(ocurve, oracle_rec["uniform_34x4"], True)
    assert ee["bits"] is not None and abs(ee["bits"] - ob) <= 4.0
    assert ee["bits"] < 136
