"""GPU parity at the largest sizes the entry points accept: a plane scan of
one KV head at n = 2^25 - 64 tokens (its planes fill the 31-bit offset range
of one buffer) and attention over a cache of 2^23 - 1 rows per head.  Inputs
are drawn on the GPU from seeded generators; parity is checked on sampled
64-token blocks and rows that the oracle computes one by one."""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import attend as o_attend
from oracle import fathom as o_fathom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sdq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_top_decode_query_amd import lib
    lib.load()
    return lib


def _say(msg):
    print(f"[gpu-limits] {msg}", flush=True)
    sys.stdout.flush()


def _bf16_keys(rows, seed, sigma):
    """bf16 bits (int16) [rows][128], N(0, sigma_j^2) per channel, drawn on the
    GPU in chunks from a seeded generator."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    out = torch.empty(rows, 128, dtype=torch.int16, device="cuda")
    sig = torch.from_numpy(sigma.astype(np.float32)).cuda()
    step = 1 << 22
    for a in range(0, rows, step):
        b = min(rows, a + step)
        x = torch.randn(b - a, 128, generator=gen, device="cuda") * sig
        out[a:b] = x.to(torch.bfloat16).view(torch.int16)
    return out


def test_fathom_scan_at_maximum_length(sdq):
    n = (1 << 25) - 64
    _say(f"plan + scan, one KV head, n={n}")
    g = np.random.default_rng(91)
    sigma = np.exp(g.uniform(np.log(0.05), np.log(4.0), 128))
    K = _bf16_keys(n, 91, sigma)
    index = sdq.fathom_ingest(K.view(1, n, 128))
    q = g.standard_normal((4, 128)).astype(np.float32)
    var = (sigma * sigma).astype(np.float32)[None]
    bm = torch.empty(1, n // 64, device="cuda")
    depth, qbar, scores = sdq.fathom_plan_scan(index, torch.from_numpy(q).cuda(), torch.from_numpy(var).cuda(),
                                               56, n, block_max=bm)
    torch.cuda.synchronize()
    rd, rq = o_fathom.plan_heads(q, var, 4, budget=56)
    assert np.array_equal(depth.cpu().numpy(), rd)
    blocks = np.unique(np.concatenate([[0, 1, n // 64 - 1, n // 64 - 2], g.integers(0, n // 64, 60)]))
    ref_all, got_all = [], []
    for b in blocks:
        kb = K[b * 64:(b + 1) * 64].cpu().numpy().view(np.uint16)
        rp, rm = o_fathom.ingest(kb[None])
        ref_all.append(o_fathom.scan_heads(rp, rm, rd, rq, 64)[0])
        got_all.append(scores[0, b * 64:(b + 1) * 64].cpu().numpy())
        assert float(bm[0, b]) == float(got_all[-1].max())
    ref_all, got_all = np.concatenate(ref_all), np.concatenate(got_all)
    rng = float(ref_all.max() - ref_all.min())
    assert float(np.abs(got_all - ref_all).max()) <= 1e-3 * rng
    del K, index, scores, bm
    torch.cuda.empty_cache()


def test_gather_attend_at_maximum_length(sdq):
    n = (1 << 23) - 1
    _say(f"gather_attend over n={n} rows per KV head")
    g = np.random.default_rng(92)
    K = _bf16_keys(n, 92, np.full(128, 1.5))
    V = _bf16_keys(n, 93, np.ones(128))
    q = g.standard_normal((1, 4, 128)).astype(np.float32)
    sel = np.unique(np.concatenate([[0, 1, n - 2, n - 1], g.integers(0, n, 500)]))[:512]
    idx = np.full((1, 1, 512), -1, np.int32)
    idx[0, 0, :len(sel)] = sel
    out = sdq.gather_attend(torch.from_numpy(q).cuda(), K.view(1, 1, n, 128), V.view(1, 1, n, 128),
                            torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    rows = torch.from_numpy(sel.astype(np.int64)).cuda()
    kr = K[rows].cpu().numpy().view(np.uint16)
    vr = V[rows].cpu().numpy().view(np.uint16)
    O = out.cpu().numpy()
    for h in range(4):
        ref = o_attend.attend_rows(q[0, h], kr, vr, 1 / math.sqrt(128))
        assert float(np.abs(O[0, h] - ref).max()) <= 2e-2
    del K, V
    torch.cuda.empty_cache()


def test_hamming_scan_topk_at_large_length(sdq):
    """2 rows of n = 2^25 + 12345 signatures (2049 segments per row, ragged
    tail): the distances equal the oracle's, and the selection is the unique
    one (every competition distance below the k-th, then the lowest-index
    ties), checked from the oracle's distances without a full sort."""
    from oracle import hamming as o_hamming
    H, n, k, ns, nl = 2, (1 << 25) + 12345, 2048, 64, 64
    _say(f"hamming_scan_topk H={H} n={n} k={k}")
    g = np.random.default_rng(94)
    sigs = g.integers(0, 1 << 32, size=(H, n), dtype=np.uint64).astype(np.uint32)
    qsig = g.integers(0, 1 << 32, size=H, dtype=np.uint64).astype(np.uint32)
    dist, idx = sdq.hamming_scan_topk(torch.from_numpy(sigs.view(np.int32)).cuda(),
                                      torch.from_numpy(qsig.view(np.int32)).cuda(), k, ns, nl)
    torch.cuda.synchronize()
    rd = o_hamming.distances_heads(sigs, qsig)
    assert np.array_equal(dist.cpu().numpy(), rd)
    got = idx.cpu().numpy()
    for h in range(H):
        comp = rd[h, ns:n - nl]
        cnt = np.bincount(comp, minlength=33)
        T = int(np.searchsorted(np.cumsum(cnt), k))      # smallest d with count(<= d) >= k
        below = int(cnt[:T].sum())
        ties = np.flatnonzero(comp == T)[:k - below] + ns
        want = np.sort(np.concatenate([np.arange(ns), np.flatnonzero(comp < T) + ns, ties,
                                       np.arange(n - nl, n)]))
        assert np.array_equal(got[h], want)
    del dist, idx
    torch.cuda.empty_cache()
