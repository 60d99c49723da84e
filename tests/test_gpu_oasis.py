"""GPU parity for KV selection against a resident block pool (OasisKV
review, core method): oasis_select bit for bit against the oracle over chained
steps, oasis_fetch against the oracle's copy, and one selection step end to
end (draft-query block scan, top-K, selection, fetch, stacked attention of the
normal and draft queries) against float64 attention over the resident blocks."""
import math
import os
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import attend as o_attend
from oracle import oasis as o_oasis
from oracle import quest as o_quest
from oracle import select as o_select

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ATTN_ATOL = 2e-2


@pytest.fixture(scope="module")
def sdq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_top_decode_query_amd import lib
    lib.load()
    return lib


def _say(msg):
    print(f"[gpu-oasis] {msg}", flush=True)
    sys.stdout.flush()


def host(t):
    return t.cpu().numpy()


def _pool(sdq, resident, last_sel):
    resident, last_sel = np.asarray(resident), np.asarray(last_sel)
    pool = sdq.BlockPool(*resident.shape)
    pool.resident.copy_(torch.from_numpy(np.asarray(resident, np.int32)))
    pool.last_sel.copy_(torch.from_numpy(np.asarray(last_sel, np.int32)))
    return pool


def _check_step(sdq, pred, scores, resident, last_sel, step, cap):
    pred, resident, last_sel = np.asarray(pred), np.asarray(resident), np.asarray(last_sel)
    pool = _pool(sdq, resident, last_sel)
    ps, pb, nf, slots = sdq.oasis_select(torch.from_numpy(np.asarray(pred, np.int32)).cuda(),
                                         torch.from_numpy(np.asarray(scores, np.float32)).cuda(),
                                         pool, step, cap)
    torch.cuda.synchronize()
    r_res, r_ls, r_ps, r_pb, r_nf = o_oasis.select_rows(pred, scores, resident, last_sel, step, cap)
    assert np.array_equal(host(pool.resident), r_res)
    assert np.array_equal(host(pool.last_sel), r_ls)
    assert np.array_equal(host(ps), r_ps) and np.array_equal(host(pb), r_pb)
    assert np.array_equal(host(nf), r_nf)
    assert np.array_equal(host(slots), np.where(r_res >= 0, np.arange(r_res.shape[1])[None], -1))
    return r_res, r_ls


def test_oasis_select_worked_example_gpu(sdq):
    _say("oasis_select worked example")
    scores = np.zeros((1, 16), np.float32)
    scores[0, 4], scores[0, 6] = 1.0, 3.0
    for cap in (2, 1):
        _check_step(sdq, [[2, 4, 6]], scores, [[5, -1, 2, 9]], [[3, 0, 7, 1]], 10, cap)


@pytest.mark.parametrize("rows,nb,S,K", [(37, 1024, 129, 129), (5, 64, 17, 17), (3, 40000, 300, 1000),
                                         (9, 8, 8, 3)])
def test_oasis_select_chained_steps_bitexact(sdq, rows, nb, S, K):
    _say(f"oasis_select rows={rows} nb={nb} S={S} K={K}")
    g = np.random.default_rng(81 + nb)
    resident = np.full((rows, S), -1, np.int64)
    for r in range(rows):                     # start partly filled, distinct blocks
        m = int(g.integers(0, S + 1))
        resident[r, g.choice(S, m, replace=False)] = g.choice(nb, m, replace=False)
    last_sel = g.integers(0, 3, size=(rows, S))
    for step, cap in enumerate((0, 3, 16, 1024, 5, 2), start=3):
        scores = g.integers(0, 6, size=(rows, nb)).astype(np.float32)   # many ties
        pred = np.stack([g.choice(nb, min(K, nb), replace=False) for _ in range(rows)])
        resident, last_sel = _check_step(sdq, pred, scores, resident, last_sel, step, cap)


def test_oasis_select_edge_cases(sdq):
    """A block listed twice in the prediction is one miss; an empty prediction
    evicts nothing; a cap above the pool size fills every target."""
    _say("oasis_select edge cases")
    g = np.random.default_rng(84)
    nb, S = 50, 6
    scores = g.standard_normal((2, nb)).astype(np.float32)
    resident = np.array([[3, -1, 7, 9, -1, 20], [-1, -1, -1, -1, -1, -1]])
    last_sel = np.array([[1, 0, 2, 0, 0, 5], [0] * 6])
    pred = np.array([[7, 11, 11, 30, 3, 30], [4, 4, 4, 4, 4, 4]])
    for cap in (1, 2, 10):
        # the oracle's prediction is a set, so duplicates collapse there too
        _check_step(sdq, pred, scores, resident, last_sel, 4, cap)
    _check_step(sdq, np.zeros((2, 0), np.int64), scores, resident, last_sel, 4, 3)
    _check_step(sdq, np.array([[0, 1, 2, 4, 5, 6], [8, 9, 10, 11, 12, 13]]), scores, resident,
                last_sel, 4, 1000)


def test_oasis_fetch_matches_plan(sdq):
    _say("oasis_fetch")
    g = np.random.default_rng(82)
    rows, nb, S, bt = 3, 40, 9, 16
    Kh = torch.from_numpy(synth.f32_to_bf16_bits(g.standard_normal((rows, nb * bt, 128))).view(np.int16)).pin_memory()
    Vh = torch.from_numpy(synth.f32_to_bf16_bits(g.standard_normal((rows, nb * bt, 128))).view(np.int16)).pin_memory()
    Kp = torch.full((rows, S * bt, 128), 0x5A5A, dtype=torch.int16, device="cuda")
    Vp = Kp.clone()
    pool = sdq.BlockPool(rows, S)
    scores = torch.from_numpy(g.standard_normal((rows, nb)).astype(np.float32)).cuda()
    pred = torch.from_numpy(np.stack([g.choice(nb, 7, replace=False) for _ in range(rows)]).astype(np.int32)).cuda()
    ps, pb, nf, slots = sdq.oasis_select(pred, scores, pool, 1, 5)
    sdq.oasis_fetch(Kh, Vh, ps, pb, Kp, Vp, bt)
    torch.cuda.synchronize()
    for r in range(rows):
        plan = [(int(s), int(b)) for s, b in zip(host(ps)[r], host(pb)[r]) if s >= 0]
        assert len(plan) == 5
        for name, src, dst in (("K", Kh, Kp), ("V", Vh, Vp)):
            blocks = src[r].numpy().reshape(nb, bt, 128)
            ref = o_oasis.fetch(np.full((S, bt, 128), 0x5A5A, np.int16), blocks, plan)
            assert np.array_equal(host(dst[r]).reshape(S, bt, 128), ref), name


def test_oasis_selection_step_end_to_end(sdq):
    """Draft-query block scan -> top-16 blocks plus the local block -> selection
    against the pool -> fetch -> the normal and draft queries attend over the
    resident blocks in one call; two steps, the second with a small cap."""
    R, G, Hgrp, n, bt, k = 2, 2, 4, 1024, 16, 16
    nb, S = n // bt, k + 1
    g = np.random.default_rng(83)
    K = synth.f32_to_bf16_bits(g.standard_normal((R * G, n, 128)) * 1.5)
    V = synth.f32_to_bf16_bits(g.standard_normal((R * G, n, 128)))
    Kd = torch.from_numpy(K.view(np.int16)).cuda()
    Kh = torch.from_numpy(K.view(np.int16)).pin_memory()
    Vh = torch.from_numpy(V.view(np.int16)).pin_memory()
    bmin, bmax = sdq.minmax_summarize(Kd, bt)
    q = g.standard_normal((R, G * Hgrp, 128)).astype(np.float32)
    pool = sdq.BlockPool(R * G, S)
    Kp = torch.zeros((R * G, S * bt, 128), dtype=torch.int16, device="cuda")
    Vp = torch.zeros_like(Kp)
    resident = np.full((R * G, S), -1)
    last_sel = np.zeros((R * G, S), np.int64)
    mn, mx = zip(*[o_quest.summaries(K[rg], bt) for rg in range(R * G)])
    for step, cap in ((1, S), (2, 4)):
        _say(f"selection step {step}, cap {cap}")
        q_draft = (q + 0.3 * g.standard_normal(q.shape)).astype(np.float32)
        scores = sdq.minmax_block_scan(bmin, bmax, torch.from_numpy(q_draft.reshape(-1, 128)).cuda())
        pred = sdq.topk_select(scores, k, n_local=1)
        ps, pb, nf, slots = sdq.oasis_select(pred, scores, pool, step, cap)
        sdq.oasis_fetch(Kh, Vh, ps, pb, Kp, Vp, bt)
        qs = sdq.stacked_layout(torch.from_numpy(q).cuda(), torch.from_numpy(q_draft).cuda(), G)
        out_s = sdq.attend_stacked(qs, Kp.view(R, G, S * bt, 128), Vp.view(R, G, S * bt, 128),
                                   slots.view(R, G, S), bt)
        out, out_d = sdq.unstack_outputs(out_s, G)
        torch.cuda.synchronize()
        # selection parity on the GPU's own scores and top-K
        S_g, P_g = host(scores), host(pred)
        resident, last_sel, _, _, _ = o_oasis.select_rows(P_g, S_g, resident, last_sel, step, cap)
        assert np.array_equal(host(pool.resident), resident)
        # the top-K itself against the oracle's block scores
        for rg in range(R * G):
            ref_s = o_quest.block_scores(mn[rg], mx[rg], q_draft.reshape(R * G, Hgrp, 128)[rg])
            assert float(np.abs(S_g[rg] - ref_s).max()) <= 1e-3 * float(ref_s.max() - ref_s.min())
            assert np.array_equal(P_g[rg], o_select.topk(S_g[rg], k, n_local=1))
        O, Od = host(out), host(out_d)
        for r in range(R):
            for gg in range(G):
                rg = r * G + gg
                blocks = [b for b in resident[rg] if b >= 0]
                rows_ = np.concatenate([np.arange(b * bt, (b + 1) * bt) for b in blocks])
                for h in range(Hgrp):
                    hq = gg * Hgrp + h
                    for qq, oo in ((q, O), (q_draft, Od)):
                        ref = o_attend.attend_rows(qq[r, hq], K[rg, rows_], V[rg, rows_], 1 / math.sqrt(128))
                        assert float(np.abs(oo[r, hq] - ref).max()) <= ATTN_ATOL
