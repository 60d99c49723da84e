"""GPU parity: every C-ABI entry point against the CPU oracle on the same
seeded inputs.  Integer and index results must match bit for bit; the
approximate scores within 1e-3 of the row's score range; the top-k set of the
end-to-end path may only differ by swaps within that tolerance of the k-th
score; attention within 2e-2 max-abs of the float64 oracle."""
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
from sparse_top_decode_query_amd import lib as sdq_lib

pytestmark = pytest.mark.gpu

SCORE_RTOL = 1e-3        # of the row's score range
ATTN_ATOL = 2e-2         # max-abs against float64


@pytest.fixture(scope="module")
def sdq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_top_decode_query_amd import lib
    lib.load()
    return lib


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
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


def _groups_of(bm):
    """Group maxima (sdq.GROUP_BLOCKS blocks a group, the last one shorter)
    of block maxima [rows][nb], as plain torch ops."""
    rows, nb = bm.shape
    gb = sdq_lib.GROUP_BLOCKS
    ng = (nb + gb - 1) // gb
    pad = torch.full((rows, ng * gb), float("-inf"), device=bm.device)
    pad[:, :nb] = bm
    return pad.view(rows, ng, gb).amax(-1)


def _assert_scores(gpu, ref):
    for g in range(ref.shape[0]):
        rng = float(ref[g].max() - ref[g].min())
        err = float(np.abs(gpu[g].astype(np.float64) - ref[g]).max())
        assert err <= SCORE_RTOL * rng + 1e-6, (g, err, rng)


def _assert_topk_set(sel_gpu, ref_scores, k, tol):
    """Sets equal up to swaps of tokens within tol of the k-th score."""
    order = np.lexsort((np.arange(len(ref_scores)), -ref_scores))
    kth = ref_scores[order[k - 1]]
    sel_ref = set(order[:k].tolist())
    sel = set(int(i) for i in sel_gpu if i >= 0)
    assert len(sel) == k
    for i in sel.symmetric_difference(sel_ref):
        assert abs(ref_scores[i] - kth) <= tol, (i, ref_scores[i], kth, tol)


# ---------------------------------------------------------------- ingest
@pytest.mark.parametrize("G,n", [(1, 4096), (3, 64 * 37), (2, 64)])
def test_fathom_ingest_bitexact(sdq, G, n):
    _say(f"ingest G={G} n={n}")
    case = synth.fathom_case(2, n=n, heads=list(range(G)), with_values=False)
    planes, meta = sdq.fathom_ingest(dev(case["K"]))
    torch.cuda.synchronize()
    rp, rm = o_fathom.ingest(case["K"])
    assert np.array_equal(host(planes, np.uint32), rp)
    assert np.array_equal(host(meta, np.uint32), rm)


def test_fathom_ingest_constant_and_tiny_blocks(sdq):
    _say("ingest degenerate blocks")
    n = 256
    k = np.zeros((1, n, 128), np.float32)
    k[0, :64] = 1.5                          # constant block: scale 0, codes 0
    k[0, 64:128] = np.linspace(-1e-6, 1e-6, 64)[:, None]   # subnormal-scale block
    g = np.random.default_rng(3)
    k[0, 128:] = g.standard_normal((128, 128)) * 30
    kb = synth.f32_to_bf16_bits(k)
    planes, meta = sdq.fathom_ingest(dev(kb))
    rp, rm = o_fathom.ingest(kb)
    assert np.array_equal(host(planes, np.uint32), rp)
    assert np.array_equal(host(meta, np.uint32), rm)


# ---------------------------------------------------------------- plan
@pytest.mark.parametrize("budget", [0, 1, 47, 48, 56, 92, 136, 511, 512, 700])
def test_fathom_plan_bitexact(sdq, budget):
    _say(f"plan budget={budget}")
    case = synth.fathom_case(2, n=64, with_values=False)
    q, var = case["q"], case["var"]
    depth, qbar = sdq.fathom_plan(dev(q), dev(var), budget)
    rd, rq = o_fathom.plan_heads(q, var, 4, budget=budget)
    assert np.array_equal(host(depth), rd)
    assert np.array_equal(host(qbar).view(np.uint32), rq.view(np.uint32))


def test_fathom_plan_ties_and_uniform(sdq):
    _say("plan ties / uniform")
    G = 5
    q = np.ones((G * 2, 128), np.float32)
    q[2:4, :64] = 2.0                       # head 1: two weight levels
    q[4:6] = 0.0                            # head 2: all weights zero
    q[6:8, ::3] = -3.0                      # head 3: negative entries
    var = np.ones((G, 128), np.float32)
    var[4] = np.random.default_rng(1).choice([0.25, 1.0, 4.0], 128).astype(np.float32)
    for budget in (1, 64, 65, 100, 128, 129, 300):
        depth, qbar = sdq.fathom_plan(dev(q), dev(var), budget)
        rd, rq = o_fathom.plan_heads(q, var, 2, budget=budget)
        assert np.array_equal(host(depth), rd), budget
    for nch in (0, 1, 34, 128):
        depth, _ = sdq.fathom_plan(dev(q), dev(var), 0, uniform_channels=nch)
        rd, _ = o_fathom.plan_heads(q, var, 2, n_uniform=nch) if nch else (np.zeros((G, 128), np.uint8), None)
        assert np.array_equal(host(depth), rd), nch


def test_fathom_plan_gain_extremes(sdq):
    """Gains in the subnormal range, mixed with normal ones, and exact powers of
    four that tie across channels and depths, against the oracle bit for bit."""
    _say("plan gain extremes")
    g = np.random.default_rng(5)
    G, Hgrp = 5, 2
    q = g.standard_normal((G * Hgrp, 128)).astype(np.float32)
    var = np.ones((G, 128), np.float32)
    q[0:2] *= np.float32(1e-5)
    var[0] = np.float32(1e-30)                                   # every gain subnormal
    var[1, :64] = np.float32(1e-30)                              # half subnormal, half normal
    q[4:6] = np.float32(0.5)                                     # qbar = 1 on head 2
    var[2] = (4.0 ** g.integers(-6, 6, 128)).astype(np.float32)  # gains are powers of four
    var[3] = np.exp(g.uniform(-40, 40, 128)).astype(np.float32)  # a wide exponent range
    q[8:10, :100] = 0.0                                          # head 4: few nonzero gains
    for budget in (1, 7, 56, 200, 511, 512):
        depth, qbar = sdq.fathom_plan(dev(q), dev(var), budget)
        rd, rq = o_fathom.plan_heads(q, var, Hgrp, budget=budget)
        assert np.array_equal(host(depth), rd), budget
    for nch in (1, 34, 100):
        depth, _ = sdq.fathom_plan(dev(q), dev(var), 0, uniform_channels=nch)
        rd, _ = o_fathom.plan_heads(q, var, Hgrp, n_uniform=nch)
        assert np.array_equal(host(depth), rd), nch


def test_fathom_plan_negative_and_nan_variance(sdq):
    """Negative, -0, NaN and -inf variances give zero gain on the GPU exactly
    as in the oracle (no out-of-range histogram bin), for the greedy and the
    uniform plan, alone and fused with the scan."""
    _say("plan with negative / NaN variances")
    g = np.random.default_rng(77)
    G, Hgrp = 4, 4
    q = g.standard_normal((G * Hgrp, 128)).astype(np.float32)
    var = g.uniform(0.01, 4, (G, 128)).astype(np.float32)
    var[0, [3, 40, 77]] = [-1.0, np.nan, -np.inf]
    var[1, :] = -2.0                                   # every gain bad: all ties at zero
    var[2, ::2] = np.float32(-0.0)
    var[3, 5] = np.nan
    q[12:16, 5] = 0.0                                  # 0 * NaN, too
    for B in (0, 1, 56, 300, 512):
        depth, _ = sdq.fathom_plan(dev(q), dev(var), B)
        rd, _ = o_fathom.plan_heads(q, var, Hgrp, budget=B)
        assert np.array_equal(host(depth), rd), B
    depth, _ = sdq.fathom_plan(dev(q), dev(var), 0, uniform_channels=34)
    assert np.array_equal(host(depth), o_fathom.plan_heads(q, var, Hgrp, n_uniform=34)[0])
    case = synth.fathom_case(2, n=4096, heads=list(range(G)), with_values=False)
    index = sdq.fathom_ingest(dev(case["K"]))
    d2, _, _ = sdq.fathom_plan_scan(index, dev(q), dev(var), 56, 4096)
    torch.cuda.synchronize()
    assert np.array_equal(host(d2), o_fathom.plan_heads(q, var, Hgrp, budget=56)[0])


def test_kernels_deterministic(sdq):
    """Every kernel of the step, run twice on the same inputs, gives the same
    bits (a race in LDS or a missing barrier would show up as a difference)."""
    _say("determinism: each kernel twice")
    G, n, k = 8, 65536, 512
    case = synth.fathom_case(2, n=n, heads=list(range(G)))
    Kd, Vd = dev(case["K"]), dev(case["V"])
    q, var = dev(case["q"]), dev(case["var"])
    index = sdq.fathom_ingest(Kd)

    def fathom_step():
        bm = torch.empty(G, n // 64, device="cuda")
        d, qb, s = sdq.fathom_plan_scan(index, q, var, 56, n, block_max=bm)
        i1 = sdq.topk_select_block_max(s, bm, k, 64, 64)
        i2 = sdq.topk_select(s, k, 16, 64)
        o = sdq.gather_attend(q.view(1, G * 4, 128), Kd.view(1, G, n, 128), Vd.view(1, G, n, 128),
                              i1[:, :k].contiguous().view(1, G, k))
        return [d, qb, s, bm, i1, i2, o]

    hc = synth.hamming_case(4)
    sig, qs = dev(hc["sigs"]), dev(hc["qsig"])

    def hamming_step():
        dist, idx = sdq.hamming_scan_topk(sig, qs, hc["m"], hc["sink"], hc["local"])
        return [dist, idx, sdq.topk_select(dist, hc["m"], hc["sink"], hc["local"])]

    mc = synth.minmax_case(5, R=4)
    Km = dev(mc["K"].reshape(-1, mc["n"], 128))

    def minmax_step():
        mn, mx = sdq.minmax_summarize(Km, 16)
        S = sdq.minmax_block_scan(mn, mx, dev(mc["q"].reshape(-1, 128)))
        return [mn, mx, S, sdq.topk_select(S, 128, 0, 1)]

    for step in (fathom_step, hamming_step, minmax_step):
        a = step()
        b = step()
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), step.__name__


# ---------------------------------------------------------------- scan
def _scan_case(sdq, G, n, budget, uniform=None):
    case = synth.fathom_case(2, n=n, heads=list(range(G)), with_values=False)
    q = case["q"][:G * 4]
    var = case["var"][:G]
    index = sdq.fathom_ingest(dev(case["K"]))
    depth, qbar = sdq.fathom_plan(dev(q), dev(var), budget, uniform_channels=uniform)
    bm = torch.empty(G, n // 64, device="cuda")
    gm = torch.empty(G, sdq.n_groups(n), device="cuda")
    scores = sdq.fathom_scan(index, depth, qbar, n, block_max=bm, group_max=gm)
    torch.cuda.synchronize()
    # block and group maxima are exactly the maxima of the written scores
    assert torch.equal(bm, scores.view(G, n // 64, 64).amax(-1))
    assert torch.equal(gm, _groups_of(bm))
    rp, rm = o_fathom.ingest(case["K"])
    rd, rq = o_fathom.plan_heads(q, var, 4, budget=budget, n_uniform=uniform)
    ref = o_fathom.scan_heads(rp, rm, rd, rq, n)
    return host(scores), ref, case


@pytest.mark.parametrize("G,n,budget", [(1, 4096, 48), (8, 8192, 56), (2, 64 * 37, 47),
                                        (1, 64, 92), (2, 4096, 512), (2, 4096, 1)])
def test_fathom_scan_parity(sdq, G, n, budget):
    _say(f"scan G={G} n={n} B={budget}")
    got, ref, _ = _scan_case(sdq, G, n, budget)
    _assert_scores(got, ref)


def test_fathom_scan_uniform_and_empty_plan(sdq):
    _say("scan uniform / empty plan")
    got, ref, _ = _scan_case(sdq, 2, 4096, 0, uniform=34)
    _assert_scores(got, ref)
    got, ref, _ = _scan_case(sdq, 1, 4096, 0)
    assert np.all(got == 0) and np.all(ref == 0)


@pytest.mark.parametrize("G,n,budget,uniform", [(8, 8192, 56, None), (2, 64 * 37, 47, None),
                                                (3, 4096, 92, None), (2, 4096, 0, 34),
                                                (1, 4096, 0, None), (2, 64, 512, None)])
def test_fathom_plan_scan_fused_equals_separate(sdq, G, n, budget, uniform):
    """The fused plan + scan gives bit-identical plan, scores and block maxima
    to fathom_plan followed by fathom_scan (same computation, one launch)."""
    _say(f"plan+scan fused G={G} n={n} B={budget} uniform={uniform}")
    case = synth.fathom_case(2, n=n, heads=list(range(G)), with_values=False)
    q, var = dev(case["q"][:G * 4]), dev(case["var"][:G])
    index = sdq.fathom_ingest(dev(case["K"]))
    depth, qbar = sdq.fathom_plan(q, var, budget, uniform_channels=uniform)
    bm = torch.empty(G, n // 64, device="cuda")
    scores = sdq.fathom_scan(index, depth, qbar, n, block_max=bm)
    bm2 = torch.full((G, n // 64), 7.0, device="cuda")
    gm2 = torch.full((G, sdq.n_groups(n)), 7.0, device="cuda")
    d2, q2, s2 = sdq.fathom_plan_scan(index, q, var, budget, n, block_max=bm2, uniform_channels=uniform,
                                      group_max=gm2)
    _, _, s3 = sdq.fathom_plan_scan(index, q, var, budget, n, uniform_channels=uniform, write_plan=False)
    torch.cuda.synchronize()
    assert torch.equal(d2, depth) and torch.equal(q2.view(torch.int32), qbar.view(torch.int32))
    assert torch.equal(s2.view(torch.int32), scores.view(torch.int32))
    assert torch.equal(s3.view(torch.int32), scores.view(torch.int32))
    assert torch.equal(bm2.view(torch.int32), bm.view(torch.int32))
    assert torch.equal(gm2, _groups_of(bm))


# ---------------------------------------------------------------- top-k
def _topk_ref(keys, k, n_sink, n_local, largest):
    rows = keys.shape[0]
    stride = k + n_sink + n_local
    out = np.full((rows, stride), -1, np.int64)
    for r in range(rows):
        sel = o_select.topk(keys[r], k, largest, n_sink, n_local)
        out[r, :len(sel)] = sel
    return out


@pytest.mark.parametrize("rows,n,k,ns,nl", [(3, 1, 1, 0, 0), (2, 100, 7, 0, 0), (4, 4096, 64, 0, 0),
                                            (2, 5000, 512, 3, 17), (1, 1000, 2000, 0, 0),
                                            (2, 70001, 512, 0, 0), (8, 1 << 20, 512, 0, 0),
                                            (2, 200000, 3000, 128, 128), (3, 300, 0, 5, 5),
                                            (8, 32768, 512, 0, 0), (3, 28672, 585, 0, 0), (2, 32788, 300, 10, 10),
                                            (2, 32809, 100, 20, 20), (3, 40000, 2000, 0, 0),
                                            (2, 16384, 16383, 0, 0), (1, 32768, 32768, 0, 0),
                                            (2, 1025, 1024, 0, 0), (4, 1500, 100, 0, 0),
                                            (3, 2048, 2047, 0, 0), (2, 3000, 64, 5, 7),
                                            (2, 6000, 700, 0, 0), (2, 12000, 1000, 64, 64),
                                            (2, 20000, 1, 0, 0), (3, 8192, 4000, 0, 0)])
def test_topk_f32_bitexact(sdq, rows, n, k, ns, nl):
    _say(f"topk f32 rows={rows} n={n} k={k}")
    g = np.random.default_rng(n + k)
    keys = (g.standard_normal((rows, n)) * 3).astype(np.float32)
    keys[:, ::7] = np.round(keys[:, ::7], 1)          # plenty of exact ties
    keys[0, : min(n, 50)] = 0.0
    if n > 3:
        keys[0, 1] = -0.0
    got = host(sdq.topk_select(dev(keys), k, ns, nl))
    assert np.array_equal(got, _topk_ref(keys, k, ns, nl, True))


def test_topk_f32_degenerate_rows(sdq):
    _say("topk degenerate rows")
    n = 100000
    keys = np.zeros((2, n), np.float32)            # every key tied: candidate overflow
    keys[1, 5000:] = 1.0
    got = host(sdq.topk_select(dev(keys), 700))
    assert np.array_equal(got, _topk_ref(keys, 700, 0, 0, True))
    keys = np.full((1, n), -2.5, np.float32)
    keys[0, 99999] = 7.0
    got = host(sdq.topk_select(dev(keys), 9000, 1, 1))
    assert np.array_equal(got, _topk_ref(keys, 9000, 1, 1, True))
    # rows held in registers (at most 32768 competing keys, ragged lengths
    # included): all tied, -inf pads, a single distinct key
    for n2 in (32768, 4096, 1500, 6000, 20001):
        keys = np.zeros((3, n2), np.float32)
        keys[1, n2 - 27:] = -np.inf
        keys[2, :] = 1.5
        keys[2, n2 // 2] = 9.0
        for k2 in (1, 512, n2 - 1):
            got = host(sdq.topk_select(dev(keys), k2, 0, 0))
            assert np.array_equal(got, _topk_ref(keys, k2, 0, 0, True)), (n2, k2)
    # rows split into 4096-key segments whose winners are united: keys drawn
    # from 50 values (ties inside and across segments), 7 and 8 segments
    rng = np.random.default_rng(7)
    for n2, k2 in ((32768, 512), (32768, 3), (28672, 585)):
        keys = rng.integers(0, 50, size=(3, n2)).astype(np.float32)
        keys[2, ::4096] = 60.0                     # each segment's first key above the rest
        got = host(sdq.topk_select(dev(keys), k2, 0, 0))
        assert np.array_equal(got, _topk_ref(keys, k2, 0, 0, True)), (n2, k2)


@pytest.mark.parametrize("rows,n,k,ns,nl", [(8, 1 << 20, 512, 0, 0), (2, 65536 + 128, 64, 64, 64),
                                            (3, 100032, 1563, 0, 0), (1, 131072, 4096, 0, 0),
                                            # windows and lengths that cut groups; a K just
                                            # within / beyond the whole groups (group path /
                                            # all block maxima)
                                            (2, 1 << 20, 512, 192, 64 * 21), (3, 64 * 4099, 300, 64, 0),
                                            (2, 64 * 800, 97, 64 * 7, 64 * 9), (2, 64 * 800, 99, 64, 64)])
def test_topk_block_max_bitexact(sdq, rows, n, k, ns, nl):
    _say(f"topk block-max rows={rows} n={n} k={k}")
    g = np.random.default_rng(n + 3 * k)
    keys = (g.standard_normal((rows, n)) * 3).astype(np.float32)
    keys[:, ::5] = np.round(keys[:, ::5], 1)
    kt = dev(keys)
    bm = kt.view(rows, n // 64, 64).amax(-1).contiguous()
    gm = _groups_of(bm)
    ref = _topk_ref(keys, k, ns, nl, True)
    assert np.array_equal(host(sdq.topk_select_block_max(kt, bm, k, ns, nl)), ref)
    assert np.array_equal(host(sdq.topk_select_block_max_split(kt, bm, k, ns, nl)), ref)
    assert np.array_equal(host(sdq.topk_select_block_max_split(kt, bm, k, ns, nl, group_max=gm)), ref)
    assert np.array_equal(host(sdq.topk_select(kt, k, ns, nl)), ref)


def test_topk_block_max_degenerate(sdq):
    """Ties and clustered maxima that overflow the candidate lists fall back
    to the exact row path."""
    _say("topk block-max degenerate rows")
    n = 1 << 17
    keys = np.zeros((3, n), np.float32)
    keys[1, ::64] = 1.0                          # every block has the same maximum
    keys[2, 64 * 100:64 * 164] = np.arange(64 * 64, dtype=np.float32)   # top keys in 64 blocks
    kt = dev(keys)
    bm = kt.view(3, n // 64, 64).amax(-1).contiguous()
    gm = _groups_of(bm)
    for k in (1, 512, 2048):
        ref = _topk_ref(keys, k, 0, 0, True)
        assert np.array_equal(host(sdq.topk_select_block_max(kt, bm, k)), ref), k
        assert np.array_equal(host(sdq.topk_select_block_max_split(kt, bm, k)), ref), k
        assert np.array_equal(host(sdq.topk_select_block_max_split(kt, bm, k, group_max=gm)), ref), k
        assert np.array_equal(host(sdq.topk_select(kt, k)), ref), k


def test_topk_block_max_split_groups_randomized(sdq):
    """Seeded random shapes for the split form with group maxima: lengths that
    cut groups, windows of any multiple of 64, k from 1 to the block count,
    and keys that are plain, heavily tied, or with the winners packed into
    one stretch of the row (which overflows a segment's share or needs many
    blocks of one group) -- each against the oracle."""
    _say("topk block-max split groups randomized")
    g = np.random.default_rng(2024)
    for case in range(12):
        rows = int(g.integers(1, 4))
        nb = int(g.integers(24, 4097))
        n = 64 * nb
        ns = 64 * int(g.integers(0, max(1, nb // 8)))
        nl = 64 * int(g.integers(0, max(1, nb // 8)))
        nbc = nb - ns // 64 - nl // 64
        k = int(g.integers(1, nbc + 1))
        keys = (g.standard_normal((rows, n)) * 2).astype(np.float32)
        kind = case % 3
        if kind == 1:
            keys = np.round(keys, 0).astype(np.float32)             # heavy ties
        elif kind == 2:
            a = int(g.integers(0, max(1, n - 8 * k)))
            keys[:, a:a + 4 * k] += 10.0                             # winners in one stretch
        kt = dev(keys)
        bm = kt.view(rows, nb, 64).amax(-1).contiguous()
        ref = _topk_ref(keys, k, ns, nl, True)
        got = host(sdq.topk_select_block_max_split(kt, bm, k, ns, nl, group_max=_groups_of(bm)))
        assert np.array_equal(got, ref), (case, rows, n, k, ns, nl, kind)
        got = host(sdq.topk_select_block_max_split(kt, bm, k, ns, nl))
        assert np.array_equal(got, ref), (case, rows, n, k, ns, nl, kind, "no groups")


def test_topk_block_max_split_wide_code_offsets(sdq):
    """The extremes of the segments' offset histograms (code offsets above
    code(thr)).  Row 0: the winners are packed into fewer than K blocks of a
    row of negative keys, so thr is far below zero while the K-th key is
    positive, more than 2^31 codes above it (the top bins).  Row 1: every key
    of the row is a distinct float one ulp from the next, shuffled, so the
    K-th key lies a few hundred codes above thr (the one-code bins).  Each
    against the oracle, with and without group maxima."""
    _say("topk block-max split wide code offsets")
    g = np.random.default_rng(77)
    ulp = np.finfo(np.float32).eps                      # one ulp in [1, 2)
    for n, k, ns, nl in ((1 << 16, 64, 0, 0), (1 << 18, 300, 128, 256), (64 * 1000, 17, 64, 64)):
        keys = np.empty((2, n), np.float32)
        keys[0] = (g.standard_normal(n) - 30.0).astype(np.float32)
        a = int(g.integers(ns, n - nl - 4 * k))
        keys[0, a:a + 4 * k] = np.abs(keys[0, a:a + 4 * k]) * 0.25   # 4k positive keys in k/16 blocks
        keys[1] = np.float32(1.5) + np.arange(n, dtype=np.float32) * ulp
        g.shuffle(keys[1])
        kt = dev(keys)
        bm = kt.view(2, n // 64, 64).amax(-1).contiguous()
        ref = _topk_ref(keys, k, ns, nl, True)
        got = host(sdq.topk_select_block_max_split(kt, bm, k, ns, nl, group_max=_groups_of(bm)))
        assert np.array_equal(got, ref), (n, k, ns, nl)
        got = host(sdq.topk_select_block_max_split(kt, bm, k, ns, nl))
        assert np.array_equal(got, ref), (n, k, ns, nl, "no groups")


def test_topk_block_max_split_workspace_reuse(sdq):
    """Calls in a row on one split workspace, fewer rows than it was sized
    for, rows that take the exact row path in between: every call is exact
    whatever the last call left in the workspace."""
    _say("topk block-max split workspace reuse")
    g = np.random.default_rng(404)
    n = 1 << 17
    ws = sdq.topk_bm_split_workspace(6, n)
    for rows, k, tied in ((6, 512, False), (2, 300, True), (5, 1, False), (1, 2048, True),
                          (6, 700, False), (3, 64, False)):
        keys = (g.standard_normal((rows, n)) * 2).astype(np.float32)
        if tied:
            keys[0] = 0.5                            # every block ties: row path
        kt = dev(keys)
        bm = kt.view(rows, n // 64, 64).amax(-1).contiguous()
        ref = _topk_ref(keys, k, 0, 0, True)
        got = host(sdq.topk_select_block_max_split(kt, bm, k, ws=ws))
        assert np.array_equal(got, ref), (rows, k, tied)
        got = host(sdq.topk_select_block_max_split(kt, bm, k, ws=ws, group_max=_groups_of(bm)))
        assert np.array_equal(got, ref), (rows, k, tied, "groups")


@pytest.mark.parametrize("rows,n,k,ns,nl,dist", [(32, 131072, 512, 128, 128, "binom"),
                                                 (3, 999, 40, 0, 0, "binom"),
                                                 (2, 50, 50, 0, 0, "binom"),
                                                 (1, 10000, 9000, 10, 10, "binom"),
                                                 # segmented path: unaligned rows, a partial last
                                                 # segment, k = 1, k = m - 1, all ties, all values
                                                 (4, 40001, 700, 3, 5, "binom"),
                                                 (2, 70000, 1, 0, 0, "binom"),
                                                 (2, 65536, 65535, 0, 0, "uniform"),
                                                 (3, 50000, 3000, 16, 0, "const"),
                                                 (2, 100000, 5000, 0, 100, "uniform")])
def test_topk_u8_bitexact(sdq, rows, n, k, ns, nl, dist):
    _say(f"topk u8 rows={rows} n={n} k={k} {dist}")
    g = np.random.default_rng(7 + n)
    if dist == "binom":
        keys = g.binomial(32, 0.5, size=(rows, n)).astype(np.uint8)
    elif dist == "uniform":
        keys = g.integers(0, 256, size=(rows, n)).astype(np.uint8)
    else:
        keys = np.full((rows, n), 9, np.uint8)
    got = host(sdq.topk_select(dev(keys), k, ns, nl))
    assert np.array_equal(got, _topk_ref(keys, k, ns, nl, False))


# ---------------------------------------------------------------- Hamming
def test_hamming_worked_example_gpu(sdq):
    _say("hamming worked example")
    sigs = np.array([[0b1011, 0b1001, 0b0110]], np.uint32)
    dist = host(sdq.hamming_scan(dev(sigs), dev(np.array([0b1011], np.uint32))))
    assert list(dist[0]) == [0, 1, 3]
    sel = host(sdq.topk_select(dev(dist), 2))
    assert list(sel[0]) == [0, 1]


@pytest.mark.parametrize("H,n", [(32, 131072), (3, 1000), (1, 17)])
def test_hamming_bitexact(sdq, H, n):
    _say(f"hamming H={H} n={n}")
    case = synth.hamming_case(4, n=max(n, 300), H=H, with_kv=False)
    sigs = np.ascontiguousarray(case["sigs"][:, :n])
    dist = host(sdq.hamming_scan(dev(sigs), dev(case["qsig"])))
    assert np.array_equal(dist, o_hamming.distances_heads(sigs, case["qsig"]))


@pytest.mark.parametrize("H,n,n_cap,k,ns,nl,kind", [
    (32, 131072, 131072, 512, 128, 128, "case"),      # the config 4 shape, segmented
    (3, 40001, 40017, 700, 3, 5, "case"),             # ragged n, odd capacity, unaligned rows
    (2, 65536, 70000, 1, 0, 0, "case"),               # capacity past n, k = 1
    (2, 70000, 70000, 5000, 0, 100, "const"),         # all distances tie
    (2, 50000, 50000, 0, 16, 16, "case"),             # windows only: the two-call path
    (3, 1000, 1024, 40, 0, 0, "case")])               # short rows: the two-call path
def test_hamming_scan_topk_equals_oracle_and_separate_calls(sdq, H, n, n_cap, k, ns, nl, kind):
    _say(f"hamming_scan_topk H={H} n={n} n_cap={n_cap} k={k} sink={ns} local={nl} {kind}")
    case = synth.hamming_case(4, n=n_cap, H=H, with_kv=False)
    sigs = case["sigs"].copy()
    if kind == "const":
        sigs[:] = case["qsig"][:, None] ^ np.uint32(0x0F0F)
    sig_d, q_d = dev(sigs), dev(case["qsig"])
    dist, idx = sdq.hamming_scan_topk(sig_d, q_d, k, ns, nl, n=n)
    dist2 = sdq.hamming_scan(sig_d, q_d, n=n)
    idx2 = sdq.topk_select(dist2, k, ns, nl)
    torch.cuda.synchronize()
    rdist = o_hamming.distances_heads(sigs[:, :n], case["qsig"])
    assert np.array_equal(host(dist), rdist)
    assert np.array_equal(host(idx), _topk_ref(rdist, k, ns, nl, False))
    assert np.array_equal(host(idx), host(idx2))


# ---------------------------------------------------------------- min/max summaries
def test_minmax_parity(sdq):
    _say("minmax summaries + block scores")
    case = synth.minmax_case(5, R=2, n=2048, with_values=False)
    R, G, n = case["R"], case["G"], case["n"]
    K = case["K"].reshape(R * G, n, 128)
    bmin, bmax = sdq.minmax_summarize(dev(K), 16)
    S = host(sdq.minmax_block_scan(bmin, bmax, dev(case["q"].reshape(R * G * 4, 128))))
    bm, bx = host(bmin, np.float16), host(bmax, np.float16)
    ref_S = np.zeros_like(S, dtype=np.float64)
    for rg in range(R * G):
        mn, mx = o_quest.summaries(K[rg], 16)
        assert np.array_equal(bm[rg].view(np.uint16), mn.view(np.uint16))
        assert np.array_equal(bx[rg].view(np.uint16), mx.view(np.uint16))
        r, g = divmod(rg, G)
        ref_S[rg] = o_quest.block_scores(mn, mx, case["q"][r, g * 4:(g + 1) * 4])
    _assert_scores(S, ref_S)


# ---------------------------------------------------------------- attention
def _rand_kv(g, R, Hkv, n):
    K = synth.f32_to_bf16_bits(g.standard_normal((R, Hkv, n, 128)) * 1.5)
    V = synth.f32_to_bf16_bits(g.standard_normal((R, Hkv, n, 128)))
    return K, V


@pytest.mark.parametrize("R,Hq,Hkv,n,m,per_qh,bt", [(1, 32, 8, 4096, 512, False, 1),
                                                    (1, 32, 8, 4096, 768, True, 1),
                                                    (2, 8, 2, 1024, 10, False, 16),
                                                    (1, 32, 8, 4096, 129, False, 16),
                                                    # >= 256 index sets: one workgroup per set
                                                    (32, 32, 8, 512, 100, False, 1),
                                                    (8, 32, 8, 1024, 300, True, 1),
                                                    (16, 16, 16, 512, 20, False, 16),
                                                    (1, 4, 4, 300, 300, False, 1),
                                                    (1, 8, 1, 2000, 65, False, 1),
                                                    (2, 8, 4, 700, 333, False, 1),      # 2 heads per set
                                                    (1, 32, 4, 2048, 1000, False, 1),   # 8 heads per set
                                                    (1, 8, 2, 999, 40, False, 3),       # 3-row blocks
                                                    (1, 8, 2, 3000, 2900, False, 1),    # 23 splits, ragged
                                                    (1, 32, 4, 2048, 400, False, 1),    # 8 heads, 8-wave sets
                                                    (1, 16, 4, 1024, 300, True, 1)])    # per head, 8-wave sets
def test_gather_attend_parity(sdq, R, Hq, Hkv, n, m, per_qh, bt):
    _say(f"attend R={R} Hq={Hq} Hkv={Hkv} n={n} m={m} per_qh={per_qh} bt={bt}")
    g = np.random.default_rng(n + m)
    K, V = _rand_kv(g, R, Hkv, n)
    q = g.standard_normal((R, Hq, 128)).astype(np.float32)
    Hsel = Hq if per_qh else Hkv
    units = n // bt
    idx = np.stack([np.stack([np.sort(g.choice(units, m, replace=False)) for _ in range(Hsel)])
                    for _ in range(R)]).astype(np.int32)
    out = host(sdq.gather_attend(dev(q), dev(K), dev(V), dev(idx), block_tokens=bt,
                                 per_query_head=per_qh))
    ref = o_attend.attend(q, K, V, idx, block_tokens=bt, per_query_head=per_qh)
    assert float(np.abs(out - ref).max()) <= ATTN_ATOL


def test_gather_attend_workspace_reuse(sdq):
    """Calls in a row on one workspace, with different split counts, stay
    exact (each call's partials overwrite the last call's)."""
    _say("attend workspace reuse")
    g = np.random.default_rng(21)
    n = 3000
    K, V = _rand_kv(g, 1, 2, n)
    Kd, Vd = dev(K), dev(V)
    ws = sdq.attend_workspace(1, 8, 2, False, 2900, 1)
    for m in (2900, 700, 2900, 129):
        q = g.standard_normal((1, 8, 128)).astype(np.float32)
        idx = np.stack([np.sort(g.choice(n, m, replace=False)) for _ in range(2)])[None].astype(np.int32)
        out = host(sdq.gather_attend(dev(q), Kd, Vd, dev(idx), ws=ws))
        ref = o_attend.attend(q, K, V, idx)
        assert float(np.abs(out - ref).max()) <= ATTN_ATOL, m


@pytest.mark.parametrize("R,Hq,Hkv,n,m,per_qh,bt", [(1, 32, 8, 8192, 512, False, 1),
                                                    (2, 8, 2, 4096, 40, False, 16),
                                                    (1, 8, 8, 3000, 300, True, 1)])
def test_gather_attend_host_kv_equals_device(sdq, R, Hq, Hkv, n, m, per_qh, bt):
    """K and V in pinned host memory, read in place over the host link: the
    same result as the device-resident call, and within tolerance of the
    oracle."""
    _say(f"attend host K/V R={R} Hq={Hq} Hkv={Hkv} n={n} m={m} per_qh={per_qh} bt={bt}")
    g = np.random.default_rng(77 + n)
    K, V = _rand_kv(g, R, Hkv, n)
    q = g.standard_normal((R, Hq, 128)).astype(np.float32)
    Hsel = Hq if per_qh else Hkv
    idx = np.stack([np.stack([np.sort(g.choice(n // bt, m, replace=False)) for _ in range(Hsel)])
                    for _ in range(R)]).astype(np.int32)
    Kh = torch.from_numpy(K.view(np.int16)).pin_memory()
    Vh = torch.from_numpy(V.view(np.int16)).pin_memory()
    out_h = host(sdq.gather_attend_host_kv(dev(q), Kh, Vh, dev(idx), block_tokens=bt, per_query_head=per_qh))
    out_d = host(sdq.gather_attend(dev(q), dev(K), dev(V), dev(idx), block_tokens=bt, per_query_head=per_qh))
    assert np.array_equal(out_h.view(np.uint32), out_d.view(np.uint32))
    ref = o_attend.attend(q, K, V, idx, block_tokens=bt, per_query_head=per_qh)
    assert float(np.abs(out_h - ref).max()) <= ATTN_ATOL
    with pytest.raises(sdq.SDQError):                       # device tensors are refused
        sdq.gather_attend_host_kv(dev(q), dev(K), dev(V), dev(idx))


def test_gather_attend_blocks_past_cache_end(sdq):
    """16-row blocks: rows of the last, partial block that lie past the cache
    end are skipped, as are blocks wholly past it and -1 padding."""
    _say("attend partial last block")
    g = np.random.default_rng(11)
    n = 1000                                   # block 62 holds rows 992..999 only
    K, V = _rand_kv(g, 1, 1, n)
    q = g.standard_normal((1, 4, 128)).astype(np.float32)
    blocks = [3, 17, 40, 62, 70, -1, 5]
    idx = np.array(blocks, np.int32)[None, None, :]
    out = host(sdq.gather_attend(dev(q), dev(K), dev(V), dev(idx), block_tokens=16))
    rows = [b * 16 + j for b in blocks if b >= 0 for j in range(16) if b * 16 + j < n]
    ref = o_attend.attend(q, K, V, np.array(rows, np.int64)[None, None, :])
    assert float(np.abs(out - ref).max()) <= ATTN_ATOL


def test_gather_attend_all_rows_equals_dense_and_padding(sdq):
    _say("attend k=n and padding")
    g = np.random.default_rng(5)
    n = 700
    K, V = _rand_kv(g, 1, 2, n)
    q = g.standard_normal((1, 4, 128)).astype(np.float32)
    idx = np.tile(np.arange(n, dtype=np.int32), (1, 2, 1))
    out = host(sdq.gather_attend(dev(q), dev(K), dev(V), dev(idx)))
    dense = np.zeros((1, 4, 128))
    for h in range(4):
        Kh = torch.from_numpy(o_attend.bf16_bits_to_f64(K[0, h // 2]))[None, None]
        Vh = torch.from_numpy(o_attend.bf16_bits_to_f64(V[0, h // 2]))[None, None]
        Qh = torch.from_numpy(q[0, h].astype(np.float64))[None, None, None]
        dense[0, h] = torch.nn.functional.scaled_dot_product_attention(Qh, Kh, Vh)[0, 0, 0].numpy()
    assert float(np.abs(out - dense).max()) <= ATTN_ATOL
    # -1 entries are padding; entries past the cache are skipped; all-padding gives zeros
    idx2 = np.full((1, 2, 10), -1, np.int32)
    idx2[0, 0, :3] = [5, 9, 100]
    idx2[0, 0, 3] = n + 5
    out2 = host(sdq.gather_attend(dev(q), dev(K), dev(V), dev(idx2)))
    ref2 = o_attend.attend(q, K, V, np.array([[[5, 9, 100], [5, 9, 100]]]))
    assert float(np.abs(out2[0, :2] - ref2[0, :2]).max()) <= ATTN_ATOL
    assert np.all(out2[0, 2:] == 0)


# ---------------------------------------------------------------- offload gather
def test_fathom_gather_copies_active_prefixes(sdq):
    """The staged copy holds the oracle's plane prefixes and metadata rows of
    the active channels and nothing else, and its scan is within tolerance
    of the oracle's scan (and identical to the scan of the resident index)."""
    _say("fathom gather (pinned host -> HBM)")
    G, n = 2, 8192
    case = synth.fathom_case(2, n=n, heads=[0, 1], with_values=False)
    index = sdq.fathom_ingest(dev(case["K"]))
    planes, meta = index.planes, index.meta
    depth, qbar = sdq.fathom_plan(dev(case["q"][:8]), dev(case["var"][:2]), 56)
    ph = planes.cpu().pin_memory()
    mh = meta.cpu().pin_memory()
    pd = torch.full_like(planes, 0x5A5A5A5A)
    md = torch.full_like(meta, 0x5A5A5A5A)
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ev.record()
    with torch.cuda.stream(side):
        side.wait_event(ev)
        sdq.fathom_gather(ph, mh, depth, pd, md, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    s_off = sdq.fathom_scan(index, depth, qbar, n, planes=pd, meta=md)
    s_on = sdq.fathom_scan(index, depth, qbar, n)
    torch.cuda.synchronize()
    rp, rm = o_fathom.ingest(case["K"])
    rd, rq = o_fathom.plan_heads(case["q"][:8], case["var"][:2], 4, budget=56)
    d = host(depth)
    assert np.array_equal(d, rd)
    Pd, Md = host(pd, np.uint32), host(md, np.uint32)
    for g in range(G):
        for j in range(128):
            t = int(d[g, j])
            assert np.array_equal(Pd[g, j, :t], rp[g, j, :t])
            assert np.all(Pd[g, j, t:] == 0x5A5A5A5A)
            if t:
                assert np.array_equal(Md[g, j], rm[g, j])
            else:
                assert np.all(Md[g, j] == 0x5A5A5A5A)
    _assert_scores(host(s_off), o_fathom.scan_heads(rp, rm, rd, rq, n))
    assert torch.equal(s_off, s_on)


# ---------------------------------------------------------------- end to end
def _fathom_step(sdq, case, budget, k, uniform=None):
    G, n = len(case["heads"]), case["n"]
    q = case["q"].reshape(-1, 4, 128)[case["heads"]].reshape(-1, 128)
    var = case["var"][case["heads"]]
    Kd, Vd = dev(case["K"]), dev(case["V"])
    index = sdq.fathom_ingest(Kd)
    planes, meta = index.planes, index.meta
    depth, qbar = sdq.fathom_plan(dev(q), dev(var), budget, uniform_channels=uniform)
    bm = torch.empty(G, n // 64, device="cuda")
    scores = sdq.fathom_scan(index, depth, qbar, n, block_max=bm)
    idx = sdq.topk_select_block_max(scores, bm, k)
    out = sdq.gather_attend(dev(q.reshape(1, G * 4, 128)), Kd.view(1, G, n, 128),
                            Vd.view(1, G, n, 128), idx.view(1, G, k))
    torch.cuda.synchronize()
    return dict(planes=planes, meta=meta, depth=host(depth), qbar=host(qbar), scores=host(scores),
                idx=host(idx), out=host(out), q=q, var=var)


@pytest.mark.parametrize("cfg,budget", [(1, 48), (2, 56)])
def test_end_to_end_step(sdq, cfg, budget):
    _say(f"end-to-end config {cfg}")
    case = synth.fathom_case(cfg)
    G, n, k, Hgrp = case["G"], case["n"], case["k"], case["Hgrp"]
    r = _fathom_step(sdq, case, budget, k) if Hgrp == 4 else None
    if Hgrp != 4:
        q = case["q"]
        Kd, Vd = dev(case["K"]), dev(case["V"])
        index = sdq.fathom_ingest(Kd)
        depth, qbar = sdq.fathom_plan(dev(q), dev(case["var"]), budget)
        scores = sdq.fathom_scan(index, depth, qbar, n)
        idx = sdq.topk_select(scores, k)
        out = sdq.gather_attend(dev(q.reshape(1, G, 128)), Kd.view(1, G, n, 128),
                                Vd.view(1, G, n, 128), idx.view(1, G, k))
        torch.cuda.synchronize()
        r = dict(depth=host(depth), qbar=host(qbar), scores=host(scores), idx=host(idx), out=host(out),
                 q=q, var=case["var"])
    rp, rm = o_fathom.ingest(case["K"])
    rd, rq = o_fathom.plan_heads(r["q"], r["var"], Hgrp, budget=budget)
    assert np.array_equal(r["depth"], rd)
    ref = o_fathom.scan_heads(rp, rm, rd, rq, n)
    _assert_scores(r["scores"], ref)
    for g in range(G):
        tol = SCORE_RTOL * float(ref[g].max() - ref[g].min())
        _assert_topk_set(r["idx"][g], ref[g], k, tol)
        # top-k alone is exact on the GPU's own scores
        assert np.array_equal(r["idx"][g], o_select.topk(r["scores"][g], k))
        if case["needle_pos"].shape[1]:
            assert set(case["needle_pos"][g].tolist()) <= set(r["idx"][g].tolist())
    # attention on the GPU's selected set, against float64
    ref_o = o_attend.attend(r["q"].reshape(1, -1, 128), case["K"][None], case["V"][None],
                            r["idx"][None])
    assert float(np.abs(r["out"] - ref_o).max()) <= ATTN_ATOL


def test_hamming_step_config4(sdq):
    _say("hamming step config 4")
    case = synth.hamming_case(4)
    H, n = case["H"], case["n"]
    dist = sdq.hamming_scan(dev(case["sigs"]), dev(case["qsig"]))
    idx = sdq.topk_select(dist, case["m"], case["sink"], case["local"])
    out = sdq.gather_attend(dev(case["q"][None]), dev(case["K"][None]), dev(case["V"][None]),
                            idx[None], per_query_head=True)
    torch.cuda.synchronize()
    rdist = o_hamming.distances_heads(case["sigs"], case["qsig"])
    assert np.array_equal(host(dist), rdist)
    ridx = np.stack([o_select.topk(rdist[h], case["m"], False, case["sink"], case["local"])
                     for h in range(H)])
    assert np.array_equal(host(idx), ridx)
    recall = np.mean([len(set(case["planted_pos"][h]) & set(ridx[h])) / case["m"] for h in range(H)])
    assert recall >= 0.99
    for h in (0, 17, 31):
        ref = o_attend.attend(case["q"][None, h:h + 1], case["K"][None, h // 4:h // 4 + 1],
                              case["V"][None, h // 4:h // 4 + 1], ridx[None, h:h + 1],
                              per_query_head=True)
        assert float(np.abs(host(out)[0, h] - ref[0, 0]).max()) <= ATTN_ATOL


def test_minmax_step_config5_sampled(sdq):
    """The batched block-summary step at full size (64 requests x 8 KV heads x
    16,384 tokens), checked on sampled (request, KV head) rows."""
    _say("minmax step config 5 (full size)")
    case = synth.minmax_case(5)
    R, G, n = case["R"], case["G"], case["n"]
    K = dev(case["K"].reshape(R * G, n, 128))
    V = dev(case["V"])
    bmin, bmax = sdq.minmax_summarize(K, 16)
    S = sdq.minmax_block_scan(bmin, bmax, dev(case["q"].reshape(-1, 128)))
    nb = n // 16
    idx = sdq.topk_select(S, case["top_blocks"], 0, 1)
    out = sdq.gather_attend(dev(case["q"]), K.view(R, G, n, 128), V, idx.view(R, G, -1),
                            block_tokens=16)
    torch.cuda.synchronize()
    S_h, idx_h, out_h = host(S), host(idx), host(out)
    assert idx_h.shape == (R * G, 129)
    for rg in (0, 77, 300, 511):
        r, g = divmod(rg, G)
        mn, mx = o_quest.summaries(case["K"][r, g], 16)
        ref = o_quest.block_scores(mn, mx, case["q"][r, g * 4:(g + 1) * 4])
        _assert_scores(S_h[rg:rg + 1], ref[None])
        tol = SCORE_RTOL * float(ref.max() - ref.min())
        _assert_topk_set(idx_h[rg, :128], ref[:nb - 1], 128, tol)
        assert idx_h[rg, 128] == nb - 1
        assert np.array_equal(idx_h[rg], o_select.topk(S_h[rg], 128, True, 0, 1))
        ref_o = o_attend.attend(case["q"][r:r + 1, g * 4:(g + 1) * 4], case["K"][r:r + 1, g:g + 1],
                                case["V"][r:r + 1, g:g + 1], idx_h[None, rg:rg + 1], block_tokens=16)
        assert float(np.abs(out_h[r, g * 4:(g + 1) * 4] - ref_o[0]).max()) <= ATTN_ATOL
