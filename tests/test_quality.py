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
