"""topk_select_noalloc (the static-scratch variant of topk_select, for
callers that cannot allocate) against topk_select with a workspace: index
output bit for bit, on two calls in a row with the second one smaller, for
each selection path that uses scratch memory (float32 histogram path,
float32 block-max path, segmented uint8 path), plus a call too large for the
scratch, which is rejected before anything is launched."""
import sys

import numpy as np
import pytest
import torch

from oracle import select as o_select

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sdq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_top_decode_query_amd import lib
    lib.load()
    return lib


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _f32_rows(rows, n, seed, ties=False):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, n)).astype(np.float32)
    if ties:
        x = np.round(x * 4) / 4          # many equal keys
    return torch.from_numpy(x).cuda()


def _u8_rows(rows, n, seed):
    g = np.random.default_rng(seed)
    return torch.from_numpy(g.binomial(32, 0.5, (rows, n)).astype(np.uint8)).cuda()


# (rows, n, k, n_sink, n_local) pairs: the first call, then a smaller one
CASES = {
    "f32_block_max": [(8, 1 << 20, 512, 0, 0), (3, 1 << 17, 300, 64, 128)],
    "f32_histogram": [(6, 100000 + 37, 700, 5, 11), (2, 70000, 64, 0, 0)],
    "u8_segments": [(32, 131072, 512, 128, 128), (5, 40000, 100, 7, 9)],
    "small_rows": [(4, 4096, 64, 0, 0), (2, 300, 17, 3, 4)],
}


@pytest.mark.parametrize("kind", list(CASES))
def test_noalloc_equals_workspace_call(sdq, kind):
    for call, (rows, n, k, ns, nl) in enumerate(CASES[kind]):
        _say(f"{kind} call {call}: rows={rows} n={n} k={k} sink={ns} local={nl}")
        seed = 100 * call + len(kind)
        keys = _u8_rows(rows, n, seed) if kind.startswith("u8") else _f32_rows(rows, n, seed, call == 1)
        idx = torch.full((rows, k + ns + nl), -7, dtype=torch.int32, device="cuda")
        sdq.topk_select_noalloc(keys, k, ns, nl, idx=idx)
        ref = sdq.topk_select(keys, k, ns, nl)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref), (kind, call)
        # and the unique answer, on sampled rows
        K = keys.cpu().numpy()
        for r in sorted({0, rows - 1}):
            exp = o_select.topk(K[r], k, K.dtype == np.float32, ns, nl)
            assert np.array_equal(idx[r].cpu().numpy(), exp), (kind, call, r)


def test_noalloc_rejects_sizes_beyond_the_scratch(sdq):
    _say("too large for the static scratch")
    L = sdq.load()
    need = int(L.topk_select_workspace_bytes(512, 1 << 20, 512, sdq.SDQ_KEY_F32_MAX))
    assert need > (16 << 20)
    keys = torch.empty(1, device="cuda")
    idx = torch.empty(1, dtype=torch.int32, device="cuda")
    import ctypes
    rc = L.topk_select_noalloc(ctypes.c_void_p(keys.data_ptr()), sdq.SDQ_KEY_F32_MAX, 512, 1 << 20,
                               512, 0, 0, ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(0))
    assert rc == -1
    assert b"static scratch" in L.sdq_last_error()
