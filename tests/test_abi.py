"""C-ABI checks that need no GPU: the library loads, exports every function
include/sdq.h declares, and rejects invalid arguments with SDQ_EINVAL before
launching anything (the calls below never reach a HIP API)."""
import ctypes
import os
import re

import pytest

from sparse_top_decode_query_amd import lib as sdq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sdq.LIB_PATH), reason="libsdq.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, re.M)
    return sorted(set(names))


def test_header_matches_binding():
    assert _declared() == sorted(sdq.exported_symbols())


def test_library_exports_every_declared_symbol():
    L = sdq.load()
    for name in _declared():
        assert hasattr(L, name), name
    assert L.sdq_abi_version() == 3


def test_invalid_arguments_rejected_without_launch():
    L = sdq.load()
    p = ctypes.c_void_p(0x1000)       # never dereferenced: validation fails first
    null = ctypes.c_void_p(0)
    s = ctypes.c_void_p(0)
    EINVAL = -1
    assert L.fathom_scan(null, p, p, p, 8, 128, 4096, 4096, p, null, null, s) == EINVAL
    assert b"null" in L.sdq_last_error()
    assert L.fathom_scan(p, p, p, p, 8, 128, 4096, 4000, p, null, null, s) == EINVAL   # n_cap % 64
    assert L.fathom_scan(p, p, p, p, 8, 128, 4097, 4096, p, null, null, s) == EINVAL   # n > n_cap
    assert L.fathom_scan(p, p, p, p, 8, 128, 0, 4096, p, null, null, s) == EINVAL      # n < 1
    assert L.fathom_scan(p, p, p, p, 8, 128, 64, 1 << 25, p, null, null, s) == EINVAL  # n_cap >= 2^25
    assert L.fathom_scan(p, p, p, p, 8, 64, 4096, 4096, p, null, null, s) == EINVAL    # d != 128
    assert L.fathom_scan(p, p, p, p, 8, 128, 4096, 4096, ctypes.c_void_p(0x1004), null, null, s) == EINVAL  # align
    assert L.fathom_plan(p, p, 8, 4, 128, -1, p, p, s) == EINVAL             # negative budget
    assert L.fathom_plan_scan(p, p, 4, 56, 0, p, p, 8, 128, 4096, 4096, p, null, p, null, null, s) == EINVAL  # depth only
    assert L.fathom_plan_scan(p, p, 4, 56, 0, p, p, 8, 128, 4096, 4000, null, null, p, null, null, s) == EINVAL  # n_cap % 64
    assert L.fathom_plan_scan(p, p, 4, 129, 1, p, p, 8, 128, 4096, 4096, null, null, p, null, null, s) == EINVAL  # > d channels
    assert L.fathom_plan_uniform(p, p, 8, 4, 128, 129, p, p, s) == EINVAL    # > d channels
    assert L.fathom_ingest(p, 0, 4096, 128, p, p, s) == EINVAL               # G < 1
    assert L.fathom_append(p, 8, 128, 4096, 4000, 97, p, p, s) == EINVAL     # past n_cap
    assert L.fathom_append(p, 8, 128, 4000, 0, 1, p, p, s) == EINVAL         # n_cap % 64
    assert L.fathom_append(p, 8, 128, 4096, -1, 1, p, p, s) == EINVAL        # n_old < 0
    assert L.fathom_append(null, 8, 128, 4096, 0, 1, p, p, s) == EINVAL
    assert L.fathom_append(ctypes.c_void_p(0x1008), 8, 128, 4096, 0, 1, p, p, s) == EINVAL  # align
    assert L.fathom_append(p, 8, 128, 4096, 100, 0, p, p, s) == 0            # nothing to do
    assert L.minmax_append(p, 8, 128, 4096, 0, 1, 0, p, p, s) == EINVAL      # block < 1
    assert L.minmax_append(p, 8, 128, 4001, 0, 1, 16, p, p, s) == EINVAL     # n_cap % block
    assert L.minmax_append(p, 8, 128, 4096, 4096, 1, 16, p, p, s) == EINVAL  # past n_cap
    assert L.fathom_gather(p, p, p, 8, 128, 4097, 4096, p, p, s) == EINVAL   # n > n_cap
    assert L.topk_select(p, 7, 1, 10, 2, 0, 0, p, p, 256, s) == EINVAL       # key type
    assert L.topk_select(p, 0, 1, 10, 2, 6, 5, p, p, 256, s) == EINVAL       # windows > n
    assert L.topk_select(p, 0, 8, 1 << 20, 512, 0, 0, p, null, 0, s) == EINVAL   # no workspace
    assert L.topk_select_noalloc(p, 0, 512, 1 << 20, 512, 0, 0, p, s) == EINVAL  # beyond the scratch
    assert b"static scratch" in L.sdq_last_error()
    assert L.topk_select_noalloc(p, 7, 1, 10, 2, 0, 0, p, s) == EINVAL             # key type
    ws_bm = L.topk_select_block_max_split_workspace_bytes(8, 1 << 20)
    assert L.topk_select_block_max_split(p, p, null, 8, 1 << 20, 512, 0, 0, p, null, ws_bm, s) == EINVAL  # no ws
    assert L.topk_select_block_max_split(p, p, null, 8, 1 << 20, 512, 0, 0, p, p, ws_bm - 1, s) == EINVAL  # short
    assert b"workspace" in L.sdq_last_error()
    assert L.topk_select_block_max_split(p, null, null, 8, 1 << 20, 512, 0, 0, p, p, ws_bm, s) == EINVAL  # bm
    assert L.topk_select_block_max_split(p, p, null, 8, 1000, 512, 0, 0, p, p, ws_bm, s) == EINVAL  # n % 64
    assert L.topk_select_block_max_split(p, p, null, 8, 1 << 21, 512, 0, 0, p, p, 1 << 30, s) == EINVAL  # > 2^20
    assert L.hamming_scan(p, p, 0, 10, 10, p, s) == EINVAL
    assert L.hamming_scan(p, p, 4, 11, 10, p, s) == EINVAL                   # n > n_cap
    assert L.hamming_scan_topk(p, p, 4, 11, 10, 2, 0, 0, p, p, p, 256, s) == EINVAL   # n > n_cap
    assert L.hamming_scan_topk(p, p, 4, 10, 10, 2, 6, 5, p, p, p, 256, s) == EINVAL   # windows > n
    assert L.hamming_scan_topk(p, p, 8, 1 << 20, 1 << 20, 512, 0, 0, p, p, null, 0, s) == EINVAL  # ws
    assert L.minmax_block_scan(p, p, p, 1, 4, 0, 8, 128, p, s) == EINVAL
    assert L.minmax_block_scan(p, p, p, 1, 4, 9, 8, 128, p, s) == EINVAL     # nb > nb_cap
    assert L.gather_attend(p, p, p, p, 1, 32, 6, 0, 100, 100, 8, 1, 128, 1.0, p, p, 1 << 20, s) == EINVAL
    assert L.gather_attend(p, p, p, p, 1, 32, 8, 0, 2000, 2000, 1024, 1, 128, 1.0, p, p, 0, s) == EINVAL  # ws
    assert L.gather_attend(p, p, p, p, 1, 32, 8, 0, 1 << 23, 1 << 23, 512, 1, 128, 1.0, p, p, 1 << 20,
                           s) == EINVAL
    assert L.gather_attend(p, p, p, p, 1, 32, 8, 0, 2001, 2000, 8, 1, 128, 1.0, p, p, 1 << 20, s) == EINVAL
    assert L.gather_attend(ctypes.c_void_p(0x1004), p, p, p, 1, 32, 8, 0, 2000, 2000, 8, 1, 128, 1.0, p, p,
                           1 << 20, s) == EINVAL                                 # q misaligned
    assert b"aligned" in L.sdq_last_error()
    assert L.oasis_select(p, 1025, p, 64, 4, p, p, 16, 0, 2, p, p, p, null, s) == EINVAL    # K
    assert L.oasis_select(p, 16, p, 64, 4, p, p, 0, 0, 2, p, p, p, null, s) == EINVAL       # S
    assert L.oasis_select(p, 16, p, 70000, 4, p, p, 16, 0, 2, p, p, p, null, s) == EINVAL   # nb
    assert L.oasis_select(p, 16, p, 64, 4, p, p, 16, 0, -1, p, p, p, null, s) == EINVAL     # cap
    assert L.oasis_select(p, 16, p, 64, 0, p, p, 16, 0, 2, p, p, p, null, s) == EINVAL      # rows
    assert L.oasis_select(p, 16, p, 64, 4, null, p, 16, 0, 2, p, p, p, null, s) == EINVAL
    assert L.oasis_fetch(p, p, p, p, 4, 2, 8, 16, 64, p, p, 8, s) == EINVAL                 # d
    assert L.oasis_fetch(p, p, p, p, 0, 2, 8, 16, 128, p, p, 8, s) == EINVAL                # rows
    assert L.oasis_fetch(p, p, p, p, 4, 2, 8, 16, 128, ctypes.c_void_p(0x1008), p, 8, s) == EINVAL  # align


def test_workspace_sizes():
    L = sdq.load()
    assert L.topk_select_workspace_bytes(8, 1 << 20, 512, 0) >= 8 * 8192 * 8
    assert L.topk_select_workspace_bytes(0, 10, 1, 0) == 0
    assert L.topk_select_block_max_split_workspace_bytes(8, 1 << 20) >= 8 * 8 * 512 * 8
    assert L.topk_select_block_max_split_workspace_bytes(0, 1 << 20) == 0
    ws = L.gather_attend_workspace_bytes(1, 32, 8, 0, 512, 1, 128)
    # 8 sets split in 4 parts of 128 rows: a partial per query head and part
    assert ws == 32 * 4 * 130 * 4
    # sets of up to 128 rows take one workgroup each: no partials
    assert L.gather_attend_workspace_bytes(1, 32, 8, 0, 128, 1, 128) == 0
    # 512 sets of 129 16-row blocks: one workgroup per set, no partials
    assert L.gather_attend_workspace_bytes(64, 32, 8, 0, 129, 16, 128) == 0
    # sets longer than 4096 rows are always split
    assert L.gather_attend_workspace_bytes(64, 32, 8, 0, 5000, 1, 128) == 64 * 32 * 2 * 130 * 4
    assert L.gather_attend_workspace_bytes(1, 32, 8, 0, 512, 1, 64) == 0
