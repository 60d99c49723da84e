"""ctypes binding of libsdq.so (declarations in include/sdq.h).

Argument marshalling only: every function checks that the torch tensors it
is handed live on the GPU, are contiguous and have the element size and
shape the C entry point will assume, then passes raw device pointers and the
current (or given) HIP stream.  All arithmetic runs in the library's HIP
kernels; there is no fallback.  Output tensors may be passed in, otherwise
they are allocated with torch.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsdq.so")

SDQ_KEY_F32_MAX = 0
SDQ_KEY_U8_MIN = 1
GROUP_BLOCKS = 8            # SDQ_GROUP_BLOCKS: 64-token blocks per group maximum
D = 128

_lib = None

_c_int, _c_size, _vp, _f = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_SIGS = {
    "sdq_last_error": ([], ctypes.c_char_p),
    "sdq_abi_version": ([], _c_int),
    "fathom_ingest": ([_vp, _c_int, _c_int, _c_int, _vp, _vp, _vp], _c_int),
    "fathom_append": ([_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp], _c_int),
    "minmax_summarize": ([_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp], _c_int),
    "minmax_append": ([_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp], _c_int),
    "fathom_plan": ([_vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp], _c_int),
    "fathom_plan_uniform": ([_vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp], _c_int),
    "fathom_gather": ([_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp], _c_int),
    "fathom_scan": ([_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp], _c_int),
    "fathom_plan_scan": ([_vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp,
                          _vp, _vp, _vp, _vp, _vp], _c_int),
    "topk_select_block_max": ([_vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp], _c_int),
    "topk_select_block_max_split": ([_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_size,
                                     _vp], _c_int),
    "topk_select_block_max_split_workspace_bytes": ([_c_int, _c_int], _c_size),
    "topk_select_workspace_bytes": ([_c_int, _c_int, _c_int, _c_int], _c_size),
    "topk_select": ([_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_size, _vp], _c_int),
    "topk_select_noalloc": ([_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp], _c_int),
    "hamming_scan": ([_vp, _vp, _c_int, _c_int, _c_int, _vp, _vp], _c_int),
    "hamming_scan_topk": ([_vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _c_size,
                           _vp], _c_int),
    "minmax_block_scan": ([_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp], _c_int),
    "gather_attend_workspace_bytes": ([_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int], _c_size),
    "gather_attend": ([_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                       _c_int, _f, _vp, _vp, _c_size, _vp], _c_int),
    "oasis_select": ([_vp, _c_int, _vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp,
                      _vp, _vp], _c_int),
    "oasis_fetch": ([_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_int, _vp],
                    _c_int),
    "gather_attend_host_kv": ([_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                               _c_int, _c_int, _f, _vp, _vp, _c_size, _vp], _c_int),
}


class SDQError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Load libsdq.so (torch's HIP runtime is loaded first and shared)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise SDQError(f"{path} is not built: run `python -m sparse_top_decode_query_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def exported_symbols():
    return list(_SIGS)


def _check(rc: int, name: str) -> None:
    if rc != 0:
        msg = load().sdq_last_error().decode(errors="replace")
        raise SDQError(f"{name} failed ({rc}): {msg}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return _vp(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, elem: int, numel: int | None = None) -> _vp:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SDQError(f"{name} must be a CUDA/HIP tensor")
    if not t.is_contiguous():
        raise SDQError(f"{name} must be contiguous")
    if t.element_size() != elem:
        raise SDQError(f"{name} must have {elem}-byte elements, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise SDQError(f"{name} has {t.numel()} elements, expected {numel}")
    return _vp(t.data_ptr())


def _out(t, shape, dtype, device, name, elem):
    if t is None:
        t = torch.empty(shape, dtype=dtype, device=device)
    n = 1
    for s in shape:
        n *= s
    _dev(t, name, elem, n)
    return t


# ------------------------------------------------------------------ ingest
class PlaneIndex:
    """The bit-plane index of one layer: planes uint32 [G][128][4][n_cap/32]
    and meta uint32 [G][128][n_cap/64], rows of n_cap tokens (n_cap = n for
    an index built in one go)."""

    def __init__(self, planes, meta):
        self.planes, self.meta = planes, meta

    @property
    def n_cap(self) -> int:
        return self.planes.shape[-1] * 32

    def __iter__(self):
        return iter((self.planes, self.meta))


def _round64(n: int) -> int:
    return -(-int(n) // 64) * 64


def plane_index_empty(G, n_cap, device="cuda"):
    """An index of row capacity n_cap (a multiple of 64) for fathom_append."""
    if n_cap % 64:
        raise SDQError("n_cap must be a multiple of 64")
    return PlaneIndex(torch.zeros(G, D, 4, n_cap // 32, dtype=torch.int32, device=device),
                      torch.zeros(G, D, n_cap // 64, dtype=torch.int32, device=device))


def _index_sizes(planes, meta, G, d):
    if planes.dim() != 4 or planes.shape[:3] != (G, d, 4):
        raise SDQError("planes must be [G][128][4][n_cap/32]")
    n_cap = planes.shape[3] * 32
    _dev(planes, "planes", 4, G * d * 4 * (n_cap // 32))
    _dev(meta, "meta", 4, G * d * (n_cap // 64))
    return n_cap


def fathom_append(keys, n_old, n_new, index, stream=None):
    """keys bf16 [G][n_cap][128] (the key cache, first n_old + n_new tokens
    valid) -> index updated in place over the blocks the new tokens touch."""
    G, n_cap, d = keys.shape
    _dev(keys, "keys", 2)
    if _index_sizes(index.planes, index.meta, G, d) != n_cap:
        raise SDQError("keys and index have different row capacities")
    _check(load().fathom_append(_vp(keys.data_ptr()), G, d, n_cap, int(n_old), int(n_new),
                                _vp(index.planes.data_ptr()), _vp(index.meta.data_ptr()),
                                _stream(stream)), "fathom_append")
    return index


def fathom_ingest(keys, planes=None, meta=None, stream=None):
    """keys bf16 [G][n][128] -> PlaneIndex(planes, meta)."""
    G, n, d = keys.shape
    _dev(keys, "keys", 2)
    planes = _out(planes, (G, d, 4, n // 32), torch.int32, keys.device, "planes", 4)
    meta = _out(meta, (G, d, n // 64), torch.int32, keys.device, "meta", 4)
    _check(load().fathom_ingest(_vp(keys.data_ptr()), G, n, d, _vp(planes.data_ptr()),
                                _vp(meta.data_ptr()), _stream(stream)), "fathom_ingest")
    return PlaneIndex(planes, meta)


def minmax_append(keys, n_old, n_new, bmin, bmax, block=16, stream=None):
    """keys bf16 [RG][n_cap][128] -> bmin, bmax fp16 bits [RG][n_cap/block][128]
    updated in place over the blocks the new tokens touch."""
    RG, n_cap, d = keys.shape
    _dev(keys, "keys", 2)
    _dev(bmin, "bmin", 2, RG * (n_cap // block) * d)
    _dev(bmax, "bmax", 2, RG * (n_cap // block) * d)
    _check(load().minmax_append(_vp(keys.data_ptr()), RG, d, n_cap, int(n_old), int(n_new), block,
                                _vp(bmin.data_ptr()), _vp(bmax.data_ptr()), _stream(stream)),
           "minmax_append")
    return bmin, bmax


def minmax_summarize(keys, block=16, bmin=None, bmax=None, stream=None):
    """keys bf16 [RG][n][128] -> (bmin, bmax) fp16 bits [RG][n/block][128]."""
    RG, n, d = keys.shape
    _dev(keys, "keys", 2)
    nb = n // block
    bmin = _out(bmin, (RG, nb, d), torch.int16, keys.device, "bmin", 2)
    bmax = _out(bmax, (RG, nb, d), torch.int16, keys.device, "bmax", 2)
    _check(load().minmax_summarize(_vp(keys.data_ptr()), RG, n, d, block, _vp(bmin.data_ptr()),
                                   _vp(bmax.data_ptr()), _stream(stream)), "minmax_summarize")
    return bmin, bmax


# ------------------------------------------------------------------ decode step
def fathom_plan(q, key_var, budget_bits, depth=None, qbar=None, uniform_channels=None,
                stream=None):
    """q float32 [G*H_grp][128], key_var float32 [G][128] -> (depth uint8 [G][128], qbar float32 [G][128]).
    With ``uniform_channels`` set, builds the uniform-depth baseline plan instead."""
    G, d = key_var.shape
    rows = q.shape[0]
    if rows % G:
        raise SDQError("q rows must be a multiple of G")
    Hgrp = rows // G
    _dev(q, "q", 4, rows * d)
    _dev(key_var, "key_var", 4, G * d)
    depth = _out(depth, (G, d), torch.uint8, q.device, "depth", 1)
    qbar = _out(qbar, (G, d), torch.float32, q.device, "qbar", 4)
    args = (_vp(q.data_ptr()), _vp(key_var.data_ptr()), G, Hgrp, d)
    outs = (_vp(depth.data_ptr()), _vp(qbar.data_ptr()), _stream(stream))
    if uniform_channels is None:
        _check(load().fathom_plan(*args, int(budget_bits), *outs), "fathom_plan")
    else:
        _check(load().fathom_plan_uniform(*args, int(uniform_channels), *outs), "fathom_plan_uniform")
    return depth, qbar


def fathom_gather(planes_host, meta_host, depth, planes_dev, meta_dev, n=None, stream=None):
    """Copy the plan's active plane prefixes (the first n tokens, default all
    n_cap of a row) from pinned host tensors to device tensors."""
    G, d, four, nw = planes_host.shape
    n_cap = nw * 32
    n = n_cap if n is None else int(n)
    for t, nm in ((planes_host, "planes_host"), (meta_host, "meta_host")):
        if t.is_cuda or not t.is_pinned() or not t.is_contiguous():
            raise SDQError(f"{nm} must be a contiguous pinned host tensor")
    if meta_host.numel() != G * d * (n_cap // 64):
        raise SDQError("meta_host has the wrong size")
    _dev(depth, "depth", 1, G * d)
    _dev(planes_dev, "planes_dev", 4, planes_host.numel())
    _dev(meta_dev, "meta_dev", 4, meta_host.numel())
    _check(load().fathom_gather(_vp(planes_host.data_ptr()), _vp(meta_host.data_ptr()),
                                _vp(depth.data_ptr()), G, d, n, n_cap, _vp(planes_dev.data_ptr()),
                                _vp(meta_dev.data_ptr()), _stream(stream)), "fathom_gather")


def n_groups(n):
    """Group maxima per row for n tokens (SDQ_GROUP_BLOCKS blocks of 64)."""
    return (_round64(n) // 64 + GROUP_BLOCKS - 1) // GROUP_BLOCKS


def _maxima(block_max, group_max, G, n64):
    bm = gm = _vp(0)
    if block_max is not None:
        bm = _dev(block_max, "block_max", 4, G * (n64 // 64))
    if group_max is not None:
        gm = _dev(group_max, "group_max", 4, G * n_groups(n64))
    return bm, gm


def fathom_scan(index, depth, qbar, n, scores=None, block_max=None, planes=None, meta=None,
                stream=None, group_max=None):
    """index: PlaneIndex (``planes``/``meta`` override its HBM buffers, e.g. a
    staging copy filled by fathom_gather); the first n tokens of its rows are
    scored -> scores float32 [G][n64], n64 = n rounded up to 64 (tokens past n
    score -inf); also fills ``block_max`` float32 [G][n64/64] and
    ``group_max`` float32 [G][n_groups(n)] if given."""
    G, d = depth.shape
    planes = index.planes if planes is None else planes
    meta = index.meta if meta is None else meta
    n_cap = _index_sizes(planes, meta, G, d)
    n64 = _round64(n)
    _dev(depth, "depth", 1, G * d)
    _dev(qbar, "qbar", 4, G * d)
    scores = _out(scores, (G, n64), torch.float32, planes.device, "scores", 4)
    bm, gm = _maxima(block_max, group_max, G, n64)
    _check(load().fathom_scan(_vp(planes.data_ptr()), _vp(meta.data_ptr()), _vp(depth.data_ptr()),
                              _vp(qbar.data_ptr()), G, d, int(n), n_cap, _vp(scores.data_ptr()), bm,
                              gm, _stream(stream)), "fathom_scan")
    return scores


def fathom_plan_scan(index, q, key_var, budget_bits, n, depth=None, qbar=None, scores=None,
                     block_max=None, planes=None, meta=None, uniform_channels=None, stream=None,
                     write_plan=True, group_max=None):
    """fathom_plan (or the uniform plan with ``uniform_channels``) and fathom_scan in one
    launch -> (depth, qbar, scores); depth/qbar are None when ``write_plan`` is False."""
    G, d = key_var.shape
    rows = q.shape[0]
    if rows % G:
        raise SDQError("q rows must be a multiple of G")
    planes = index.planes if planes is None else planes
    meta = index.meta if meta is None else meta
    _dev(q, "q", 4, rows * d)
    _dev(key_var, "key_var", 4, G * d)
    n_cap = _index_sizes(planes, meta, G, d)
    n64 = _round64(n)
    if write_plan:
        depth = _out(depth, (G, d), torch.uint8, q.device, "depth", 1)
        qbar = _out(qbar, (G, d), torch.float32, q.device, "qbar", 4)
        dp, qp = _vp(depth.data_ptr()), _vp(qbar.data_ptr())
    else:
        depth = qbar = None
        dp = qp = _vp(0)
    scores = _out(scores, (G, n64), torch.float32, q.device, "scores", 4)
    bm, gm = _maxima(block_max, group_max, G, n64)
    uniform = uniform_channels is not None
    budget = int(uniform_channels) if uniform else int(budget_bits)
    _check(load().fathom_plan_scan(_vp(q.data_ptr()), _vp(key_var.data_ptr()), rows // G, budget,
                                   int(uniform), _vp(planes.data_ptr()), _vp(meta.data_ptr()), G, d,
                                   int(n), n_cap, dp, qp, _vp(scores.data_ptr()), bm, gm,
                                   _stream(stream)),
           "fathom_plan_scan")
    return depth, qbar, scores


def topk_select_block_max(keys, block_max, k, n_sink=0, n_local=0, idx=None, stream=None):
    """float32 keys [rows][n] with their 64-key block maxima [rows][n/64] ->
    idx int32 [rows][k + n_sink + n_local] (as topk_select)."""
    rows, n = keys.shape
    _dev(keys, "keys", 4, rows * n)
    _dev(block_max, "block_max", 4, rows * (n // 64))
    idx = _out(idx, (rows, k + n_sink + n_local), torch.int32, keys.device, "idx", 4)
    _check(load().topk_select_block_max(_vp(keys.data_ptr()), _vp(block_max.data_ptr()), rows, n,
                                        int(k), int(n_sink), int(n_local), _vp(idx.data_ptr()),
                                        _stream(stream)), "topk_select_block_max")
    return idx


def topk_bm_split_workspace(rows, n, device="cuda"):
    nbytes = int(load().topk_select_block_max_split_workspace_bytes(rows, n))
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def topk_select_block_max_split(keys, block_max, k, n_sink=0, n_local=0, idx=None, ws=None,
                                stream=None, group_max=None):
    """topk_select_block_max with each row's candidate gather spread over
    several workgroups; ``group_max`` [rows][n_groups(n)] (as fathom_scan
    writes it) lets each workgroup read only its share of the block maxima;
    ws from topk_bm_split_workspace (allocated here if not given)."""
    rows, n = keys.shape
    _dev(keys, "keys", 4, rows * n)
    _dev(block_max, "block_max", 4, rows * (n // 64))
    gm = _vp(0)
    if group_max is not None:
        gm = _dev(group_max, "group_max", 4, rows * n_groups(n))
    idx = _out(idx, (rows, k + n_sink + n_local), torch.int32, keys.device, "idx", 4)
    if ws is None:
        ws = topk_bm_split_workspace(rows, n, keys.device)
    _dev(ws, "ws", 1)
    _check(load().topk_select_block_max_split(_vp(keys.data_ptr()), _vp(block_max.data_ptr()), gm,
                                              rows, n, int(k), int(n_sink), int(n_local),
                                              _vp(idx.data_ptr()), _vp(ws.data_ptr()), ws.numel(),
                                              _stream(stream)), "topk_select_block_max_split")
    return idx


def topk_workspace(rows, n, k, key_type, device="cuda"):
    nbytes = int(load().topk_select_workspace_bytes(rows, n, k, key_type))
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def topk_select(keys, k, n_sink=0, n_local=0, idx=None, ws=None, stream=None):
    """keys float32 (largest first) or uint8 (smallest first) [rows][n] ->
    idx int32 [rows][k + n_sink + n_local], ascending, -1 padded."""
    rows, n = keys.shape
    if keys.dtype == torch.float32:
        kt = SDQ_KEY_F32_MAX
        _dev(keys, "keys", 4, rows * n)
    elif keys.dtype == torch.uint8:
        kt = SDQ_KEY_U8_MIN
        _dev(keys, "keys", 1, rows * n)
    else:
        raise SDQError("keys must be float32 or uint8")
    idx = _out(idx, (rows, k + n_sink + n_local), torch.int32, keys.device, "idx", 4)
    need = int(load().topk_select_workspace_bytes(rows, n, k, kt))
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=keys.device)
    _dev(ws, "ws", 1)
    _check(load().topk_select(_vp(keys.data_ptr()), kt, rows, n, int(k), int(n_sink), int(n_local),
                              _vp(idx.data_ptr()), _vp(ws.data_ptr()), ws.numel(), _stream(stream)),
           "topk_select")
    return idx


def topk_select_noalloc(keys, k, n_sink=0, n_local=0, idx=None, stream=None):
    """topk_select on the library's static scratch (no workspace argument):
    keys float32 (largest first) or uint8 (smallest first) [rows][n] ->
    idx int32 [rows][k + n_sink + n_local].  Pass ``idx`` to allocate nothing
    at all; calls that overlap on one GPU share the scratch and race."""
    rows, n = keys.shape
    if keys.dtype == torch.float32:
        kt = SDQ_KEY_F32_MAX
        _dev(keys, "keys", 4, rows * n)
    elif keys.dtype == torch.uint8:
        kt = SDQ_KEY_U8_MIN
        _dev(keys, "keys", 1, rows * n)
    else:
        raise SDQError("keys must be float32 or uint8")
    idx = _out(idx, (rows, k + n_sink + n_local), torch.int32, keys.device, "idx", 4)
    _check(load().topk_select_noalloc(_vp(keys.data_ptr()), kt, rows, n, int(k), int(n_sink),
                                      int(n_local), _vp(idx.data_ptr()), _stream(stream)),
           "topk_select_noalloc")
    return idx


def hamming_scan(sigs, qsig, dist=None, n=None, stream=None):
    """sigs uint32 [H][n_cap] (the first n scored, default all), qsig uint32 [H]
    -> dist uint8 [H][n]."""
    H, n_cap = sigs.shape
    n = n_cap if n is None else int(n)
    _dev(sigs, "sigs", 4, H * n_cap)
    _dev(qsig, "qsig", 4, H)
    dist = _out(dist, (H, n), torch.uint8, sigs.device, "dist", 1)
    _check(load().hamming_scan(_vp(sigs.data_ptr()), _vp(qsig.data_ptr()), H, n, n_cap,
                               _vp(dist.data_ptr()), _stream(stream)), "hamming_scan")
    return dist


def hamming_scan_topk(sigs, qsig, k, n_sink=0, n_local=0, dist=None, idx=None, ws=None, n=None,
                      stream=None):
    """hamming_scan then the top-k smallest distances per row, in one call:
    sigs uint32 [H][n_cap] (the first n scored), qsig uint32 [H] ->
    (dist uint8 [H][n], idx int32 [H][n_sink + k + n_local])."""
    H, n_cap = sigs.shape
    n = n_cap if n is None else int(n)
    _dev(sigs, "sigs", 4, H * n_cap)
    _dev(qsig, "qsig", 4, H)
    dist = _out(dist, (H, n), torch.uint8, sigs.device, "dist", 1)
    idx = _out(idx, (H, int(n_sink) + int(k) + int(n_local)), torch.int32, sigs.device, "idx", 4)
    if ws is None:
        ws = topk_workspace(H, n, k, SDQ_KEY_U8_MIN, sigs.device)
    _dev(ws, "ws", 1)
    _check(load().hamming_scan_topk(_vp(sigs.data_ptr()), _vp(qsig.data_ptr()), H, n, n_cap, int(k),
                                    int(n_sink), int(n_local), _vp(dist.data_ptr()),
                                    _vp(idx.data_ptr()), _vp(ws.data_ptr()), ws.numel(),
                                    _stream(stream)), "hamming_scan_topk")
    return dist, idx


def minmax_block_scan(bmin, bmax, q, scores=None, nb=None, stream=None):
    """bmin, bmax fp16 bits [RG][nb_cap][128] (the first nb blocks scored,
    default all), q float32 [RG*H_grp][128] -> scores float32 [RG][nb]."""
    RG, nb_cap, d = bmin.shape
    nb = nb_cap if nb is None else int(nb)
    _dev(bmin, "bmin", 2, RG * nb_cap * d)
    _dev(bmax, "bmax", 2, RG * nb_cap * d)
    rows = q.numel() // d
    if rows % RG:
        raise SDQError("q rows must be a multiple of RG")
    _dev(q, "q", 4, rows * d)
    scores = _out(scores, (RG, nb), torch.float32, bmin.device, "scores", 4)
    _check(load().minmax_block_scan(_vp(bmin.data_ptr()), _vp(bmax.data_ptr()), _vp(q.data_ptr()),
                                    RG, rows // RG, nb, nb_cap, d, _vp(scores.data_ptr()),
                                    _stream(stream)),
           "minmax_block_scan")
    return scores


def attend_workspace(R, Hq, Hkv, per_query_head, n_idx, block_tokens, device="cuda"):
    nbytes = int(load().gather_attend_workspace_bytes(R, Hq, Hkv, int(per_query_head), n_idx,
                                                      block_tokens, D))
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def gather_attend_host_kv(q, K_host, V_host, idx, block_tokens=1, per_query_head=False,
                          softmax_scale=None, out=None, ws=None, n=None, stream=None):
    """As gather_attend, with K and V pinned host tensors (bf16 bits as int16/uint16)
    read in place over the host link."""
    R, Hq, d = q.shape
    _, Hkv, n_cap, _ = K_host.shape
    n = n_cap if n is None else int(n)
    n_idx = idx.shape[-1]
    Hsel = Hq if per_query_head else Hkv
    for t, nm in ((K_host, "K_host"), (V_host, "V_host")):
        if t.is_cuda or not t.is_pinned() or not t.is_contiguous() or t.element_size() != 2:
            raise SDQError(f"{nm} must be a contiguous pinned host tensor of 2-byte elements")
        if t.numel() != R * Hkv * n_cap * d:
            raise SDQError(f"{nm} has the wrong size")
    _dev(q, "q", 4, R * Hq * d)
    _dev(idx, "idx", 4, R * Hsel * n_idx)
    out = _out(out, (R, Hq, d), torch.float32, q.device, "out", 4)
    if ws is None:
        ws = attend_workspace(R, Hq, Hkv, per_query_head, n_idx, block_tokens, q.device)
    _dev(ws, "ws", 1)
    scale = (1.0 / d ** 0.5) if softmax_scale is None else float(softmax_scale)
    _check(load().gather_attend_host_kv(_vp(q.data_ptr()), _vp(K_host.data_ptr()),
                                        _vp(V_host.data_ptr()), _vp(idx.data_ptr()), R, Hq, Hkv,
                                        int(bool(per_query_head)), n, n_cap, n_idx, int(block_tokens), d,
                                        scale, _vp(out.data_ptr()), _vp(ws.data_ptr()), ws.numel(),
                                        _stream(stream)), "gather_attend_host_kv")
    return out


def gather_attend(q, K, V, idx, block_tokens=1, per_query_head=False, softmax_scale=None,
                  out=None, ws=None, n=None, stream=None):
    """q float32 [R][Hq][128]; K, V bf16 [R][Hkv][n_cap][128] with the first n
    rows valid (default all); idx int32 [R][Hsel][n_idx] -> out float32 [R][Hq][128]."""
    R, Hq, d = q.shape
    _, Hkv, n_cap, _ = K.shape
    n = n_cap if n is None else int(n)
    n_idx = idx.shape[-1]
    Hsel = Hq if per_query_head else Hkv
    _dev(q, "q", 4, R * Hq * d)
    _dev(K, "K", 2, R * Hkv * n_cap * d)
    _dev(V, "V", 2, R * Hkv * n_cap * d)
    _dev(idx, "idx", 4, R * Hsel * n_idx)
    out = _out(out, (R, Hq, d), torch.float32, q.device, "out", 4)
    if ws is None:
        ws = attend_workspace(R, Hq, Hkv, per_query_head, n_idx, block_tokens, q.device)
    _dev(ws, "ws", 1)
    scale = (1.0 / d ** 0.5) if softmax_scale is None else float(softmax_scale)
    _check(load().gather_attend(_vp(q.data_ptr()), _vp(K.data_ptr()), _vp(V.data_ptr()),
                                _vp(idx.data_ptr()), R, Hq, Hkv, int(bool(per_query_head)), n, n_cap, n_idx,
                                int(block_tokens), d, scale, _vp(out.data_ptr()), _vp(ws.data_ptr()),
                                ws.numel(), _stream(stream)), "gather_attend")
    return out


# ------------------------------------------------------------------ resident pool
class BlockPool:
    """A GPU-resident block pool per row (request x KV head): the block id held
    by each of S slots (-1 = empty) and the step at which it was last
    selected."""

    def __init__(self, rows, S, device="cuda"):
        self.resident = torch.full((rows, S), -1, dtype=torch.int32, device=device)
        self.last_sel = torch.zeros((rows, S), dtype=torch.int32, device=device)


def oasis_select(pred, block_scores, pool, step, cap, plan_slot=None, plan_block=None,
                 n_fetch=None, slots=None, stream=None):
    """pred int32 [rows][K] (predicted block ids), block_scores float32
    [rows][nb]; pool (BlockPool) updated in place -> (plan_slot, plan_block
    int32 [rows][cap], n_fetch int32 [rows], slots int32 [rows][S])."""
    rows, K = pred.shape
    nb = block_scores.shape[1]
    S = pool.resident.shape[1]
    _dev(pred, "pred", 4, rows * K)
    _dev(block_scores, "block_scores", 4, rows * nb)
    _dev(pool.resident, "resident", 4, rows * S)
    _dev(pool.last_sel, "last_sel", 4, rows * S)
    dv = pred.device
    plan_slot = _out(plan_slot, (rows, cap), torch.int32, dv, "plan_slot", 4)
    plan_block = _out(plan_block, (rows, cap), torch.int32, dv, "plan_block", 4)
    n_fetch = _out(n_fetch, (rows,), torch.int32, dv, "n_fetch", 4)
    slots = _out(slots, (rows, S), torch.int32, dv, "slots", 4)
    _check(load().oasis_select(_vp(pred.data_ptr()), K, _vp(block_scores.data_ptr()), nb, rows,
                               _vp(pool.resident.data_ptr()), _vp(pool.last_sel.data_ptr()), S,
                               int(step), int(cap), _vp(plan_slot.data_ptr()), _vp(plan_block.data_ptr()),
                               _vp(n_fetch.data_ptr()), _vp(slots.data_ptr()), _stream(stream)),
           "oasis_select")
    return plan_slot, plan_block, n_fetch, slots


def oasis_fetch(K_host, V_host, plan_slot, plan_block, K_pool, V_pool, block_tokens=16, stream=None):
    """K_host, V_host pinned bf16 [rows][nb*bt][128]; K_pool, V_pool device bf16
    [rows][S*bt][128]: copies the planned blocks into their slots."""
    if K_host.dim() != 3:
        raise SDQError("K_host must be [rows][nb*block_tokens][128]")
    rows, n_host, _ = K_host.shape
    for t, nm in ((K_host, "K_host"), (V_host, "V_host")):
        if t.is_cuda or not t.is_pinned() or not t.is_contiguous() or t.element_size() != 2:
            raise SDQError(f"{nm} must be a contiguous pinned host tensor of 2-byte elements")
        if t.shape != (rows, n_host, D):
            raise SDQError(f"{nm} must be [rows][nb*block_tokens][128]")
    if n_host % block_tokens:
        raise SDQError("host rows must hold whole blocks")
    nb = n_host // block_tokens
    S = K_pool.shape[1] // block_tokens
    cap = plan_slot.shape[1]
    _dev(K_pool, "K_pool", 2, rows * S * block_tokens * D)
    _dev(V_pool, "V_pool", 2, rows * S * block_tokens * D)
    _dev(plan_slot, "plan_slot", 4, rows * cap)
    _dev(plan_block, "plan_block", 4, rows * cap)
    _check(load().oasis_fetch(_vp(K_host.data_ptr()), _vp(V_host.data_ptr()), _vp(plan_slot.data_ptr()),
                              _vp(plan_block.data_ptr()), rows, cap, nb, int(block_tokens), D,
                              _vp(K_pool.data_ptr()), _vp(V_pool.data_ptr()), S, _stream(stream)),
           "oasis_fetch")


def attend_stacked(q_stacked, K_pool, V_pool, slots, block_tokens=16, out=None, ws=None,
                   stream=None):
    """The normal and draft queries of each KV head attend over the same
    resident blocks in one gather_attend call, so each block is read once for
    both.  q_stacked float32 [R][Hkv*2*grp][128], per KV head its grp normal
    query rows followed by its grp draft rows; K_pool, V_pool bf16
    [R][Hkv][S*bt][128]; slots int32 [R][Hkv][S] -> out float32 in q_stacked's
    layout (unstack_outputs splits it)."""
    return gather_attend(q_stacked, K_pool, V_pool, slots, block_tokens=block_tokens, out=out,
                         ws=ws, stream=stream)


def stacked_layout(q, q_draft, Hkv):
    """q, q_draft [R][Hq][128] -> q_stacked [R][2*Hq][128] for attend_stacked."""
    R, Hq, d = q.shape
    grp = Hq // Hkv
    return torch.cat([q.view(R, Hkv, grp, d), q_draft.view(R, Hkv, grp, d)], dim=2).reshape(R, 2 * Hq, d)


def unstack_outputs(out, Hkv):
    """attend_stacked's output -> (out, out_draft) [R][Hq][128]."""
    R, H2, d = out.shape
    grp = H2 // (2 * Hkv)
    o = out.view(R, Hkv, 2 * grp, d)
    return o[:, :, :grp].reshape(R, Hkv * grp, d), o[:, :, grp:].reshape(R, Hkv * grp, d)
