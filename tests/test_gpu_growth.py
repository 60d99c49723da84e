"""GPU parity for a growing cache: appends into the open block, scans of any
length n inside a fixed row capacity n_cap, and the calls that read
capacity-strided rows.  Every result is checked against the CPU oracle on the
same seeded inputs (bit for bit for indices, planes and summaries; scores
within 1e-3 of the row's score range; attention within 2e-2 max-abs)."""
import math
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import attend as o_attend
from oracle import fathom as o_fathom
from oracle import hamming as o_hamming
from oracle import quest as o_quest
from oracle import select as o_select

pytestmark = pytest.mark.gpu

SCORE_RTOL = 1e-3
ATTN_ATOL = 2e-2
SENTINEL = 0x5A5A5A5A


@pytest.fixture(scope="module")
def sdq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_top_decode_query_amd import lib
    lib.load()
    return lib


def _say(msg):
    print(f"[gpu-growth] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).cuda()
    return torch.from_numpy(a).cuda()


def host(t, dtype=None):
    x = t.cpu().numpy()
    return x.view(dtype) if dtype is not None else x


def _r64(n):
    return -(-n // 64) * 64


def _sentinel_index(sdq, G, n_cap):
    idx = sdq.plane_index_empty(G, n_cap)
    idx.planes.fill_(SENTINEL)
    idx.meta.fill_(SENTINEL)
    return idx


def _check_index(index, K, n, n_cap):
    """GPU index after appends up to n == oracle index of the first n tokens on
    every block touched so far; words past them still hold the sentinel."""
    P, M = host(index.planes, np.uint32), host(index.meta, np.uint32)
    rp, rm = o_fathom.ingest(K, n, n_cap)
    w, b = _r64(n) // 32, _r64(n) // 64
    assert np.array_equal(P[..., :w], rp[..., :w])
    assert np.array_equal(M[..., :b], rm[..., :b])
    assert np.all(P[..., w:] == SENTINEL) and np.all(M[..., b:] == SENTINEL)


# ---------------------------------------------------------------- append
def test_fathom_append_matches_prefix_index(sdq):
    G, n_cap = 2, 1024
    _say(f"fathom_append G={G} n_cap={n_cap}")
    K = synth.fathom_case(2, n=n_cap, heads=[0, 1], with_values=False)["K"]
    Kd = dev(K)
    index = _sentinel_index(sdq, G, n_cap)
    n = 0
    for step in (1, 62, 2, 63, 200, 1, 64, 631):
        sdq.fathom_append(Kd, n, step, index)
        n += step
        torch.cuda.synchronize()
        _check_index(index, K, n, n_cap)
    assert n == n_cap
    full = sdq.fathom_ingest(Kd)
    assert torch.equal(full.planes, index.planes) and torch.equal(full.meta, index.meta)
    # appending nothing changes nothing
    before = index.planes.clone()
    sdq.fathom_append(Kd, n_cap, 0, index)
    assert torch.equal(before, index.planes)


def test_fathom_append_token_by_token_closes_blocks(sdq):
    G, n_cap = 1, 256
    _say("fathom_append one token at a time")
    K = synth.fathom_case(2, n=n_cap, heads=[3], with_values=False)["K"]
    Kd = dev(K)
    index = _sentinel_index(sdq, G, n_cap)
    for n in range(1, 131):
        sdq.fathom_append(Kd, n - 1, 1, index)
        if n in (1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 130):
            torch.cuda.synchronize()
            _check_index(index, K, n, n_cap)


# ---------------------------------------------------------------- ragged scans
@pytest.mark.parametrize("n", [1, 63, 64, 65, 777, 1000, 1024])
def test_fathom_scan_ragged_n(sdq, n):
    G, Hgrp, n_cap, budget = 2, 4, 1024, 56
    _say(f"scan ragged n={n} n_cap={n_cap}")
    case = synth.fathom_case(2, n=n_cap, heads=[0, 1], with_values=False)
    K = case["K"]
    q = case["q"][:G * Hgrp]
    var = case["var"][:G]
    index = _sentinel_index(sdq, G, n_cap)
    sdq.fathom_append(dev(K), 0, n, index)
    n64 = _r64(n)
    bm = torch.full((G, n64 // 64), 7.0, device="cuda")
    depth, qbar, scores = sdq.fathom_plan_scan(index, dev(q), dev(var), budget, n, block_max=bm)
    s_sep = sdq.fathom_scan(index, depth, qbar, n)
    torch.cuda.synchronize()
    rd, rq = o_fathom.plan_heads(q, var, Hgrp, budget=budget)
    assert np.array_equal(host(depth), rd)
    rp, rm = o_fathom.ingest(K, n, n_cap)
    ref = o_fathom.scan_heads(rp, rm, rd, rq, n)
    S = host(scores)
    assert S.shape == (G, n64)
    assert torch.equal(scores, s_sep)
    for g in range(G):
        # score range; with a single token it is 0, so the scores' magnitude
        # stands in for it
        rng = max(float(ref[g].max() - ref[g].min()), float(np.abs(ref[g]).max()) if n == 1 else 0.0)
        assert float(np.abs(S[g, :n] - ref[g]).max()) <= SCORE_RTOL * rng + 1e-6
        assert np.all(np.isneginf(S[g, n:]))
        assert np.array_equal(host(bm)[g], S[g].reshape(-1, 64).max(axis=1))
    # the -inf pads compete like any key (ties to the lower index)
    for k in (4, 40):
        i_bm = host(sdq.topk_select_block_max(scores, bm, k))
        i_gen = host(sdq.topk_select(scores, k))
        for g in range(G):
            ref_i = o_select.topk(S[g], k)
            assert np.array_equal(i_bm[g], ref_i) and np.array_equal(i_gen[g], ref_i)


@pytest.mark.parametrize("n", [1, 100, 999])
def test_uniform_plan_scan_ragged_n(sdq, n):
    G, Hgrp, n_cap = 2, 4, 1024
    _say(f"uniform plan + scan ragged n={n}")
    case = synth.fathom_case(2, n=n_cap, heads=[0, 1], with_values=False)
    K, q, var = case["K"], case["q"][:G * Hgrp], case["var"][:G]
    index = _sentinel_index(sdq, G, n_cap)
    sdq.fathom_append(dev(K), 0, n, index)
    depth, qbar, scores = sdq.fathom_plan_scan(index, dev(q), dev(var), 0, n, uniform_channels=34)
    torch.cuda.synchronize()
    rd, rq = o_fathom.plan_heads(q, var, Hgrp, n_uniform=34)
    assert np.array_equal(host(depth), rd)
    rp, rm = o_fathom.ingest(K, n, n_cap)
    ref = o_fathom.scan_heads(rp, rm, rd, rq, n)
    S = host(scores)
    for g in range(G):
        rng = max(float(ref[g].max() - ref[g].min()), float(np.abs(ref[g]).max()) if n == 1 else 0.0)
        assert float(np.abs(S[g, :n] - ref[g]).max()) <= SCORE_RTOL * rng + 1e-6
        assert np.all(np.isneginf(S[g, n:]))


def test_decode_loop_on_growing_cache(sdq):
    """Several decode steps on one cache: append the new token, plan + scan the
    first n, top-k over the padded row with the last 64 positions kept as the
    local window (it covers the open block), attention over the first n rows."""
    G, Hgrp, n_cap, k, budget = 2, 4, 4096, 64, 56
    case = synth.fathom_case(2, n=n_cap, heads=[2, 5])
    K, V = case["K"], case["V"]
    q = case["q"].reshape(-1, Hgrp, 128)[[2, 5]].reshape(-1, 128)
    var = case["var"][[2, 5]]
    Kd, Vd = dev(K), dev(V)
    index = sdq.plane_index_empty(G, n_cap)
    n = 3000
    sdq.fathom_append(Kd, 0, n, index)
    for step in range(4):
        sdq.fathom_append(Kd, n, 1 + 30 * step, index)
        n += 1 + 30 * step
        _say(f"decode loop step {step}: n={n}")
        n64 = _r64(n)
        bm = torch.empty(G, n64 // 64, device="cuda")
        depth, qbar, scores = sdq.fathom_plan_scan(index, dev(q), dev(var), budget, n, block_max=bm)
        idx = sdq.topk_select_block_max(scores, bm, k, n_local=64)
        out = sdq.gather_attend(dev(q.reshape(1, G * Hgrp, 128)), Kd.view(1, G, n_cap, 128),
                                Vd.view(1, G, n_cap, 128), idx.view(1, G, -1), n=n)
        torch.cuda.synchronize()
        S, I, O = host(scores), host(idx), host(out)
        rp, rm = o_fathom.ingest(K, n, n_cap)
        rd, rq = o_fathom.plan_heads(q, var, Hgrp, budget=budget)
        ref = o_fathom.scan_heads(rp, rm, rd, rq, n)
        for g in range(G):
            # selection is exact on the GPU's own padded scores
            assert np.array_equal(I[g], o_select.topk(S[g], k, n_local=64))
            sel = I[g][I[g] < n]
            assert set(range(n64 - 64, n)) <= set(sel.tolist())
            rng = float(ref[g].max() - ref[g].min())
            comp = [i for i in I[g] if i < n64 - 64]
            order = np.lexsort((np.arange(n64 - 64), -ref[g][:n64 - 64]))
            kth = ref[g][order[k - 1]]
            for i in set(comp).symmetric_difference(order[:k].tolist()):
                assert abs(ref[g][i] - kth) <= SCORE_RTOL * rng
            for h in range(Hgrp):
                o_ref = o_attend.attend_rows(q[g * Hgrp + h], K[g, sel], V[g, sel], 1 / math.sqrt(128))
                assert float(np.abs(O[0, g * Hgrp + h] - o_ref).max()) <= ATTN_ATOL


# ---------------------------------------------------------------- capacity rows
def test_gather_attend_skips_rows_past_n(sdq):
    _say("gather_attend with n < n_cap")
    g = np.random.default_rng(61)
    R, Hq, Hkv, n, n_cap, m = 2, 8, 2, 700, 1024, 96
    K = synth.f32_to_bf16_bits(g.standard_normal((R, Hkv, n_cap, 128)))
    V = synth.f32_to_bf16_bits(g.standard_normal((R, Hkv, n_cap, 128)))
    K[:, :, n:] = synth.f32_to_bf16_bits(np.full((1,), 300.0, np.float32))[0]   # must never be read
    V[:, :, n:] = synth.f32_to_bf16_bits(np.full((1,), 1e4, np.float32))[0]
    q = g.standard_normal((R, Hq, 128)).astype(np.float32)
    idx = np.stack([np.stack([np.sort(g.choice(n_cap, m, replace=False)) for _ in range(Hkv)])
                    for _ in range(R)]).astype(np.int32)
    out = sdq.gather_attend(dev(q), dev(K), dev(V), dev(idx), n=n)
    torch.cuda.synchronize()
    O = host(out)
    for r in range(R):
        for h in range(Hq):
            sel = idx[r, h // 4]
            sel = sel[sel < n]
            ref = o_attend.attend_rows(q[r, h], K[r, h // 4, sel], V[r, h // 4, sel], 1 / math.sqrt(128))
            assert float(np.abs(O[r, h] - ref).max()) <= ATTN_ATOL


def test_hamming_scan_capacity_rows(sdq):
    _say("hamming_scan with n < n_cap")
    g = np.random.default_rng(62)
    for H, n, n_cap in ((4, 1000, 1024), (3, 17, 64), (2, 4096, 8192)):
        sigs = g.integers(0, 2 ** 32, size=(H, n_cap), dtype=np.uint32)
        qs = g.integers(0, 2 ** 32, size=H, dtype=np.uint32)
        dist = sdq.hamming_scan(dev(sigs), dev(qs), n=n)
        torch.cuda.synchronize()
        assert np.array_equal(host(dist), o_hamming.distances_heads(sigs[:, :n], qs))


def test_minmax_append_and_capacity_scan(sdq):
    RG, Hgrp, n_cap, block = 3, 4, 256, 16
    _say("minmax_append and minmax_block_scan with nb < nb_cap")
    g = np.random.default_rng(63)
    K = synth.f32_to_bf16_bits(g.standard_normal((RG, n_cap, 128)) * 2)
    Kd = dev(K)
    nb_cap = n_cap // block
    bmin = torch.full((RG, nb_cap, 128), 0x5A5A, dtype=torch.int16, device="cuda")
    bmax = bmin.clone()
    q = g.standard_normal((RG * Hgrp, 128)).astype(np.float32)
    n = 0
    for step in (1, 14, 2, 33, 100, 1, 105):
        sdq.minmax_append(Kd, n, step, bmin, bmax, block)
        n += step
        nb = -(-n // block)
        S = sdq.minmax_block_scan(bmin, bmax, dev(q), nb=nb)
        torch.cuda.synchronize()
        mn_g, mx_g = host(bmin, np.uint16), host(bmax, np.uint16)
        for rg in range(RG):
            mn, mx = o_quest.summaries(K[rg, :n], block)
            assert np.array_equal(mn_g[rg, :nb], mn.view(np.uint16))
            assert np.array_equal(mx_g[rg, :nb], mx.view(np.uint16))
            assert np.all(mn_g[rg, nb:] == 0x5A5A)
            ref = o_quest.block_scores(mn, mx, q[rg * Hgrp:(rg + 1) * Hgrp])
            rng = max(float(ref.max() - ref.min()), float(np.abs(ref).max()) if nb == 1 else 0.0)
            assert float(np.abs(host(S)[rg] - ref).max()) <= SCORE_RTOL * rng + 1e-6
    assert n == n_cap
    full_min, full_max = sdq.minmax_summarize(Kd, block)
    assert torch.equal(full_min, bmin) and torch.equal(full_max, bmax)


def test_fathom_gather_capacity_prefix(sdq):
    """Gather from a capacity row that holds n < n_cap tokens: the staged
    prefixes equal the oracle's index of the first n tokens (closed blocks
    final, the open block quantised over its present tokens), everything
    else keeps its sentinel, and the staged copy scores within tolerance of
    the oracle."""
    G, n_cap, n = 2, 2048, 1000
    _say(f"fathom_gather n={n} of n_cap={n_cap}")
    case = synth.fathom_case(2, n=n_cap, heads=[0, 1], with_values=False)
    index = sdq.plane_index_empty(G, n_cap)
    sdq.fathom_append(dev(case["K"]), 0, n, index)
    depth, qbar = sdq.fathom_plan(dev(case["q"][:8]), dev(case["var"][:2]), 56)
    ph, mh = index.planes.cpu().pin_memory(), index.meta.cpu().pin_memory()
    pd = torch.full_like(index.planes, SENTINEL)
    md = torch.full_like(index.meta, SENTINEL)
    sdq.fathom_gather(ph, mh, depth, pd, md, n=n)
    s_off = sdq.fathom_scan(index, depth, qbar, n, planes=pd, meta=md)
    s_on = sdq.fathom_scan(index, depth, qbar, n)
    torch.cuda.synchronize()
    rp, rm = o_fathom.ingest(case["K"], n, n_cap)
    rd, rq = o_fathom.plan_heads(case["q"][:8], case["var"][:2], 4, budget=56)
    d = host(depth)
    assert np.array_equal(d, rd)
    Pd, Md = host(pd, np.uint32), host(md, np.uint32)
    w, b = _r64(n) // 32, _r64(n) // 64
    for g in range(G):
        for j in range(128):
            t = int(d[g, j])
            assert np.array_equal(Pd[g, j, :t, :w], rp[g, j, :t, :w])
            assert np.all(Pd[g, j, :t, w:] == SENTINEL) and np.all(Pd[g, j, t:] == SENTINEL)
            if t:
                assert np.array_equal(Md[g, j, :b], rm[g, j, :b]) and np.all(Md[g, j, b:] == SENTINEL)
            else:
                assert np.all(Md[g, j] == SENTINEL)
    S = host(s_off)
    for g in range(G):
        ref = o_fathom.scan(rp[g], rm[g], rd[g], rq[g], n)
        rng = float(ref.max() - ref.min())
        assert float(np.abs(S[g, :n].astype(np.float64) - ref).max()) <= SCORE_RTOL * rng + 1e-6
        assert np.all(np.isneginf(S[g, n:]))
    assert torch.equal(s_off, s_on)
