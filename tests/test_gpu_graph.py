"""Decode steps captured into a HIP graph and replayed: every replay must give
exactly the eager step's outputs.  The benchmark times its steps as graph
replays, so this is what makes those timings stand for the eager path.  Each
graph is replayed several times with other GPU work and host synchronisation
between the replays, and every replay is checked."""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sdq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_top_decode_query_amd import lib
    lib.load()
    return lib


def _say(msg):
    print(f"[gpu-graph] {msg}", flush=True)
    sys.stdout.flush()


def _check_replays(step, outputs, replays=3):
    """Runs step eagerly, captures it, replays it `replays` times with other
    work in between, and checks every replay against the eager outputs."""
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs]
    for t in outputs:
        t.fill_(0) if t.dtype.is_floating_point else t.fill_(-7)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    noise = torch.randn(1 << 20, device="cuda")
    for r in range(replays):
        for t in outputs:
            t.fill_(0) if t.dtype.is_floating_point else t.fill_(-7)
        g.replay()
        noise.mul_(1.0001).add_(0.5)              # eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(eager, outputs):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), r


def test_fathom_step_graph_replay(sdq):
    _say("bit-plane step: fused plan + scan, split block-max top-k, attention")
    G, n, k = 8, 65536, 512
    case = synth.fathom_case(2, n=n)
    K = torch.from_numpy(case["K"].view(np.int16)).cuda()
    V = torch.from_numpy(case["V"].view(np.int16)).cuda()
    q = torch.from_numpy(case["q"]).cuda()
    var = torch.from_numpy(case["var"]).cuda()
    index = sdq.fathom_ingest(K)
    scores = torch.empty(G, n, device="cuda")
    bm = torch.empty(G, n // 64, device="cuda")
    gm = torch.empty(G, sdq.n_groups(n), device="cuda")
    idx = torch.empty(G, k, dtype=torch.int32, device="cuda")
    out = torch.empty(1, G * 4, 128, device="cuda")
    ws = sdq.attend_workspace(1, G * 4, G, False, k, 1)
    ws_bm = sdq.topk_bm_split_workspace(G, n)

    def step():
        sdq.fathom_plan_scan(index, q, var, 56, n, scores=scores, block_max=bm, write_plan=False,
                             group_max=gm)
        sdq.topk_select_block_max_split(scores, bm, k, idx=idx, ws=ws_bm, group_max=gm)
        sdq.gather_attend(q.view(1, G * 4, 128), K.view(1, G, n, 128), V.view(1, G, n, 128),
                          idx.view(1, G, k), out=out, ws=ws)
    _check_replays(step, [scores, bm, gm, idx, out])


def test_hamming_step_graph_replay(sdq):
    _say("Hamming step: fused distances + top-k, per-query-head attention")
    h = synth.hamming_case(4)
    sigs = torch.from_numpy(h["sigs"].view(np.int32)).cuda()
    qsig = torch.from_numpy(h["qsig"].view(np.int32)).cuda()
    K = torch.from_numpy(h["K"].view(np.int16)).cuda()[None]
    V = torch.from_numpy(h["V"].view(np.int16)).cuda()[None]
    qh = torch.from_numpy(h["q"]).cuda()[None]
    m_tot = h["m"] + h["sink"] + h["local"]
    dist = torch.empty(h["H"], h["n"], dtype=torch.uint8, device="cuda")
    idx = torch.empty(h["H"], m_tot, dtype=torch.int32, device="cuda")
    out = torch.empty(1, h["H"], 128, device="cuda")
    ws_t = sdq.topk_workspace(h["H"], h["n"], h["m"], sdq.SDQ_KEY_U8_MIN)
    ws_a = sdq.attend_workspace(1, h["H"], h["Hkv"], True, m_tot, 1)

    def step():
        sdq.hamming_scan_topk(sigs, qsig, h["m"], h["sink"], h["local"], dist=dist, idx=idx, ws=ws_t)
        sdq.gather_attend(qh, K, V, idx[None], per_query_head=True, out=out, ws=ws_a)
    _check_replays(step, [dist, idx, out])


def test_minmax_step_graph_replay(sdq):
    _say("block-summary step: block scan, top-k + local block, 16-row attention")
    mm = synth.minmax_case(5, R=4)
    R, G, n = 4, mm["G"], mm["n"]
    Km = torch.from_numpy(mm["K"].reshape(R * G, n, 128).view(np.int16)).cuda()
    Vm = torch.from_numpy(mm["V"].view(np.int16)).cuda()
    qm = torch.from_numpy(mm["q"]).cuda()
    bmin, bmax = sdq.minmax_summarize(Km, 16)
    nb, kb = n // 16, mm["top_blocks"]
    S = torch.empty(R * G, nb, device="cuda")
    idx = torch.empty(R * G, kb + 1, dtype=torch.int32, device="cuda")
    out = torch.empty(R, G * mm["Hgrp"], 128, device="cuda")
    ws_t = sdq.topk_workspace(R * G, nb, kb, sdq.SDQ_KEY_F32_MAX)
    ws_a = sdq.attend_workspace(R, G * mm["Hgrp"], G, False, kb + 1, 16)

    def step():
        sdq.minmax_block_scan(bmin, bmax, qm.reshape(-1, 128), scores=S)
        sdq.topk_select(S, kb, 0, 1, idx=idx, ws=ws_t)
        sdq.gather_attend(qm, Km.view(R, G, n, 128), Vm, idx.view(R, G, -1), block_tokens=16,
                          out=out, ws=ws_a)
    _check_replays(step, [S, idx, out])
