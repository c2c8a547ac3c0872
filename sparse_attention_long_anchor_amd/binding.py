"""ctypes binding of libkascade_mi355x.so (argument marshalling only).

Names follow the C ABI (include/kascade.h): decode_anchor, decode_reuse,
prefill_anchor, prefill_reuse, decode_dense, prefill_dense, topk_count,
prefill_offsets, workspace_size.
Tensors must already live on the GPU in the documented layouts; outputs may be
passed in (preallocated) or are allocated with torch.empty on the inputs'
device. Work is enqueued on torch's current stream of that device.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "libkascade_mi355x.so")

OP_DECODE_ANCHOR, OP_DECODE_REUSE, OP_PREFILL_ANCHOR, OP_PREFILL_REUSE = 0, 1, 2, 3
OP_DECODE_DENSE, OP_PREFILL_DENSE = 4, 5
DTYPE_F32, DTYPE_BF16, DTYPE_F16 = 0, 1, 2


class KasError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__(f"{where}: status {status}: {text}")
        self.status = status


class KasDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("seq_len", ctypes.c_int64),
        ("topk_pct", ctypes.c_int32),
        ("tile", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("kv_batch_stride", ctypes.c_int64),
        ("kv_head_stride", ctypes.c_int64),
        ("pool_scope", ctypes.c_int32),
        ("pool_op", ctypes.c_int32),
        ("query_head_map", ctypes.c_int32),
        ("q_batch_stride", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64),
        ("q_token_stride", ctypes.c_int64),
        ("o_batch_stride", ctypes.c_int64),
        ("o_head_stride", ctypes.c_int64),
        ("o_token_stride", ctypes.c_int64),
        ("anchor_dense_output", ctypes.c_int32),
    ]


class KasKvCache(ctypes.Structure):
    _fields_ = [
        ("seq_lens", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("page_stride", ctypes.c_int64),
        ("page_head_stride", ctypes.c_int64),
    ]


_lib = None


def lib_path() -> str:
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise ImportError(f"HIP library {_LIB} is not built; run "
                              "`python -m sparse_attention_long_anchor_amd.build`")
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        st = ctypes.c_int
        dp = ctypes.POINTER(KasDesc)
        L.kas_topk_count.argtypes = [ctypes.c_int64, ctypes.c_int32]
        L.kas_topk_count.restype = ctypes.c_int64
        L.kas_prefill_index_offsets.argtypes = [dp, P, ctypes.POINTER(ctypes.c_int64)]
        L.kas_workspace_size.argtypes = [dp, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.kas_decode_anchor.argtypes = [dp, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kas_decode_reuse.argtypes = [dp, P, P, P, P, ctypes.c_int32, P, P, P, ctypes.c_size_t, P]
        L.kas_prefill_anchor.argtypes = [dp, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kas_prefill_reuse.argtypes = [dp, P, P, P, P, ctypes.c_int32, P, P, P, ctypes.c_size_t, P]
        L.kas_decode_dense.argtypes = [dp, P, P, P, P, P, ctypes.c_size_t, P]
        L.kas_decode_reuse_noalloc.argtypes = [dp, P, P, P, P, ctypes.c_int32, P, P, P]
        cp = ctypes.POINTER(KasKvCache)
        L.kas_workspace_size_kv.argtypes = [dp, cp, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.kas_decode_anchor_kv.argtypes = [dp, cp, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kas_decode_reuse_kv.argtypes = [dp, cp, P, P, P, P, ctypes.c_int32, P, P, P, ctypes.c_size_t, P]
        L.kas_decode_dense_kv.argtypes = [dp, cp, P, P, P, P, P, ctypes.c_size_t, P]
        L.kas_prefill_anchor_kv.argtypes = [dp, cp, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kas_prefill_reuse_kv.argtypes = [dp, cp, P, P, P, P, ctypes.c_int32, P, P, P, ctypes.c_size_t, P]
        L.kas_prefill_dense_kv.argtypes = [dp, cp, P, P, P, P, P, ctypes.c_size_t, P]
        L.kas_workspace_size_refine.argtypes = [dp, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]
        L.kas_decode_refine.argtypes = [dp, P, P, P, P, ctypes.c_int32, ctypes.c_int64, P, P, P, P,
                                        ctypes.c_size_t, P]
        L.kas_workspace_size_refine_kv.argtypes = [dp, cp, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]
        L.kas_decode_refine_kv.argtypes = [dp, cp, P, P, P, P, ctypes.c_int32, ctypes.c_int64, P, P, P, P, P,
                                           ctypes.c_size_t, P]
        L.kas_prefill_dense.argtypes = [dp, P, P, P, P, P, ctypes.c_size_t, P]
        L.kas_set_option.argtypes = [ctypes.c_int32, ctypes.c_int64]
        L.kas_get_option.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]
        L.kas_status_string.argtypes = [st]
        L.kas_status_string.restype = ctypes.c_char_p
        L.kas_last_error.restype = ctypes.c_char_p
        L.kas_profile_enable.argtypes = [ctypes.c_int32]
        L.kas_profile_query.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64)]
        L.kas_profile_names.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
        for n in ("kas_prefill_index_offsets", "kas_workspace_size", "kas_decode_anchor",
                  "kas_decode_reuse", "kas_prefill_anchor", "kas_prefill_reuse",
                  "kas_decode_dense", "kas_prefill_dense", "kas_workspace_size_kv",
                  "kas_decode_anchor_kv", "kas_decode_reuse_kv", "kas_decode_dense_kv",
                  "kas_workspace_size_refine", "kas_decode_refine", "kas_prefill_anchor_kv",
                  "kas_prefill_reuse_kv", "kas_prefill_dense_kv", "kas_workspace_size_refine_kv",
                  "kas_decode_refine_kv", "kas_profile_enable", "kas_profile_reset", "kas_profile_query",
                  "kas_profile_names", "kas_set_option", "kas_get_option", "kas_decode_reuse_noalloc"):
            getattr(L, n).restype = st
        _lib = L
    return _lib


def _check(rc: int, where: str) -> None:
    if rc != 0:
        L = _load()
        raise KasError(rc, where, L.kas_last_error().decode())


OPT_DECODE_SPLIT_ROWS, OPT_DECODE_SELECT_ONE_PASS, OPT_PREFILL_POOL_MB, OPT_PREFILL_SELECT_CAP = 0, 1, 2, 3


def set_option(option: int, value: int) -> None:
    """Process-wide tuning option (kas_set_option); -1 restores the default."""
    _check(_load().kas_set_option(option, value), "set_option")


def get_option(option: int) -> int:
    v = ctypes.c_int64(0)
    _check(_load().kas_get_option(option, ctypes.byref(v)), "get_option")
    return int(v.value)


def make_desc(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, seq_len: int,
              topk_pct: int, dtype: torch.dtype, tile: int = 32, softmax_scale: float = 0.0,
              kv_batch_stride: int = 0, kv_head_stride: int = 0, pool_scope: int = 0,
              pool_op: int = 0, query_head_map: int = 0, q_strides=(0, 0, 0),
              o_strides=(0, 0, 0), anchor_dense_output: int = 0) -> KasDesc:
    if dtype == torch.bfloat16:
        dt = DTYPE_BF16
    elif dtype == torch.float16:
        dt = DTYPE_F16
    elif dtype == torch.float32:
        dt = DTYPE_F32
    else:
        raise KasError(2, "make_desc", f"dtype {dtype} not supported")
    return KasDesc(batch, n_q_heads, n_kv_heads, head_dim, seq_len, topk_pct, tile, dt,
                   softmax_scale, kv_batch_stride, kv_head_stride, pool_scope, pool_op, query_head_map,
                   *q_strides, *o_strides, anchor_dense_output)


def topk_count(n: int, pct: int) -> int:
    return int(_load().kas_topk_count(n, pct))


def decode_k(n: int, pct: int) -> int:
    return max(1, topk_count(n, pct)) if n >= 1 else 0


def prefill_offsets(desc: KasDesc) -> np.ndarray:
    L = _load()
    total = ctypes.c_int64(0)
    _check(L.kas_prefill_index_offsets(ctypes.byref(desc), None, ctypes.byref(total)), "prefill_offsets")
    off = np.zeros(desc.seq_len // desc.tile + 1, dtype=np.int64)
    _check(L.kas_prefill_index_offsets(ctypes.byref(desc), off.ctypes.data_as(ctypes.c_void_p),
                                       ctypes.byref(total)), "prefill_offsets")
    return off


def workspace_size(desc: KasDesc, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_load().kas_workspace_size(ctypes.byref(desc), op, ctypes.byref(n)), "workspace_size")
    return int(n.value)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ws(desc: KasDesc, op: int, ws: Optional[torch.Tensor], device) -> torch.Tensor:
    need = workspace_size(desc, op)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return ws


def _row_strides(t: torch.Tensor, name: str):
    """(batch, head, token) element strides of q or o ([B, H, D] or [B, H, N, D],
    head_dim contiguous); a dimension of size 1 passes 0 (its stride is unused)."""
    if t.stride(-1) != 1:
        raise KasError(1, name, f"{name} must have a contiguous last (head_dim) dimension")
    dims = list(zip(t.shape[:-1], t.stride()[:-1])) + ([] if t.dim() == 4 else [(1, 0)])
    return tuple(0 if n == 1 else st for n, st in dims)


def _check_tensors(where: str, q, k, v, o=None, **ints) -> None:
    """q, k, v (and o) share dtype and device; index-like arguments are
    contiguous int32 tensors on that device."""
    for name, t in (("k", k), ("v", v), ("o", o)):
        if t is None:
            continue
        if t.dtype != q.dtype:
            raise KasError(1, where, f"{name} has dtype {t.dtype}, q has {q.dtype}")
        if t.device != q.device:
            raise KasError(1, where, f"{name} is on {t.device}, q on {q.device}")
    for name, t in ints.items():
        if t is None:
            continue
        if t.dtype != torch.int32 or t.device != q.device or not t.is_contiguous():
            raise KasError(1, where, f"{name} must be a contiguous int32 tensor on {q.device}")
    if q.device.type != "cuda":
        raise KasError(1, where, "tensors must live on the GPU")


def _new_out(q: torch.Tensor) -> torch.Tensor:
    return torch.empty(q.shape, dtype=q.dtype, device=q.device)


def _desc_from(q: torch.Tensor, k: torch.Tensor, pct: int, prefill: bool, scale: float,
               tile: int = 32, pool_scope: int = 0, pool_op: int = 0, query_head_map: int = 0,
               o: Optional[torch.Tensor] = None, anchor_dense_output: int = 0) -> KasDesc:
    if prefill:
        B, Hq, N, D = q.shape
    else:
        B, Hq, D = q.shape
        N = k.shape[2]
    Hkv = k.shape[1]
    if k.stride(3) != 1 or k.stride(2) != D:
        raise KasError(1, "desc", "k/v rows must be contiguous [.., N, D]")
    return make_desc(B, Hq, Hkv, D, N, pct, q.dtype, tile=tile, softmax_scale=scale,
                     kv_batch_stride=k.stride(0), kv_head_stride=k.stride(1),
                     pool_scope=pool_scope, pool_op=pool_op, query_head_map=query_head_map,
                     q_strides=_row_strides(q, "q"), o_strides=_row_strides(q if o is None else o, "o"),
                     anchor_dense_output=anchor_dense_output)


def _cache(q, k, seq_lens, block_table, seq_len):
    """(descriptor overrides, KasKvCache or None) of a varlen / paged decode cache.
    Paged: k, v are page pools [num_pages, Hkv, P, D]; block_table [B, max_pages];
    seq_len is the longest sequence the call may see."""
    if seq_lens is None and block_table is None:
        return None, None
    c = KasKvCache(None if seq_lens is None else seq_lens.data_ptr(),
                   None if block_table is None else block_table.data_ptr(), 0, 0, 0, 0, 0)
    over = None
    if block_table is not None:
        if seq_len is None:
            raise KasError(1, "cache", "a paged cache needs seq_len (the longest sequence)")
        if k.stride(3) != 1 or k.stride(2) != k.shape[3]:
            raise KasError(1, "cache", "page rows must be contiguous [.., P, D]")
        c.page_size, c.max_pages, c.num_pages = k.shape[2], block_table.shape[1], k.shape[0]
        c.page_stride, c.page_head_stride = k.stride(0), k.stride(1)
        over = dict(seq_len=int(seq_len), n_kv_heads=k.shape[1], head_dim=k.shape[3])
    return over, c


def _decode_desc(q, k, pct, scale, over, o, **kw) -> KasDesc:
    if over is None:
        return _desc_from(q, k, pct, False, scale, o=o, **kw)
    B, Hq, D = q.shape
    return make_desc(B, Hq, over["n_kv_heads"], over["head_dim"], over["seq_len"], pct, q.dtype,
                     softmax_scale=scale, q_strides=_row_strides(q, "q"), o_strides=_row_strides(o, "o"), **kw)


def _ws_kv(desc, cache, op, ws, device):
    if cache is None:
        return _ws(desc, op, ws, device)
    n = ctypes.c_size_t(0)
    _check(_load().kas_workspace_size_kv(ctypes.byref(desc), ctypes.byref(cache), op, ctypes.byref(n)),
           "workspace_size")
    if ws is None:
        ws = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=device)
    return ws


def decode_anchor(q, k, v, pct: int, scale: float = 0.0, idx_out=None, o=None, ws=None,
                  pool_scope: int = 0, pool_op: int = 0, seq_lens=None, block_table=None,
                  seq_len=None, dense_output: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """q [B,Hq,D], k/v [B,Hkv,N,D] -> (idx int32 [B,Hs,kd], o [B,Hq,D]); Hs = Hkv, or 1
    with pool_scope=1 (one set pooled over all heads). seq_lens (device int32 [B])
    gives each sequence's length; block_table (device int32 [B, max_pages]) makes
    k, v page pools [num_pages, Hkv, P, D] (then seq_len = the longest sequence).
    q and o may be strided views with a contiguous head_dim. dense_output: o is
    dense attention over all keys (the sets are selected as usual)."""
    o = _new_out(q) if o is None else o
    _check_tensors("decode_anchor", q, k, v, o, idx_out=idx_out, seq_lens=seq_lens, block_table=block_table)
    over, cache = _cache(q, k, seq_lens, block_table, seq_len)
    desc = _decode_desc(q, k, pct, scale, over, o, pool_scope=pool_scope, pool_op=pool_op,
                        anchor_dense_output=int(dense_output))
    if k.stride() != v.stride():
        raise KasError(1, "decode_anchor", "k and v must share strides")
    kd = decode_k(desc.seq_len, pct)
    if idx_out is None:
        hs = 1 if pool_scope else desc.n_kv_heads
        idx_out = torch.empty((desc.batch, hs, kd), dtype=torch.int32, device=q.device)
    ws = _ws_kv(desc, cache, OP_DECODE_ANCHOR, ws, q.device)
    if cache is None:
        rc = _load().kas_decode_anchor(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(idx_out),
                                       _ptr(o), _ptr(ws), ws.numel(), _stream(q))
    else:
        rc = _load().kas_decode_anchor_kv(ctypes.byref(desc), ctypes.byref(cache), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(idx_out), _ptr(o), _ptr(ws), ws.numel(), _stream(q))
    _check(rc, "decode_anchor")
    return idx_out, o


def decode_reuse(q, k, v, anchor_idx, head_map, pct: int, scale: float = 0.0, o=None, ws=None,
                 query_head_map: bool = False, seq_lens=None, block_table=None, seq_len=None) -> torch.Tensor:
    """anchor_idx [B,Hkv_a,kd] int32 (device), head_map int32 [Hkv] (device) or None;
    with query_head_map, head_map holds one entry per query head [Hq]. Cache
    arguments as in decode_anchor."""
    o = _new_out(q) if o is None else o
    _check_tensors("decode_reuse", q, k, v, o, anchor_idx=anchor_idx, head_map=head_map, seq_lens=seq_lens,
                   block_table=block_table)
    over, cache = _cache(q, k, seq_lens, block_table, seq_len)
    desc = _decode_desc(q, k, pct, scale, over, o, query_head_map=int(query_head_map))
    if k.stride() != v.stride():
        raise KasError(1, "decode_reuse", "k and v must share strides")
    ws = _ws_kv(desc, cache, OP_DECODE_REUSE, ws, q.device)
    if cache is None:
        rc = _load().kas_decode_reuse(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(anchor_idx),
                                      anchor_idx.shape[1], _ptr(head_map), _ptr(o), _ptr(ws), ws.numel(),
                                      _stream(q))
    else:
        rc = _load().kas_decode_reuse_kv(ctypes.byref(desc), ctypes.byref(cache), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(anchor_idx), anchor_idx.shape[1], _ptr(head_map), _ptr(o),
                                         _ptr(ws), ws.numel(), _stream(q))
    _check(rc, "decode_reuse")
    return o


NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_reuse_noalloc(q, k, v, anchor_idx, head_map, pct: int, scale: float = 0.0, o=None) -> torch.Tensor:
    """decode_reuse without a workspace (kas_decode_reuse_noalloc: the library's
    static per-GPU scratch buffer; pass o to allocate nothing at all)."""
    o = _new_out(q) if o is None else o
    _check_tensors("decode_reuse_noalloc", q, k, v, o, anchor_idx=anchor_idx, head_map=head_map)
    desc = _desc_from(q, k, pct, False, scale, o=o)
    if k.stride() != v.stride():
        raise KasError(1, "decode_reuse_noalloc", "k and v must share strides")
    _check(_load().kas_decode_reuse_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(anchor_idx),
                                            anchor_idx.shape[1], _ptr(head_map), _ptr(o), _stream(q)),
           "decode_reuse_noalloc")
    return o


def _prefill_desc(q, k, pct, scale, seq_lens, block_table, o, **kw):
    """(descriptor, KasKvCache or None) of a prefill call. With block_table
    (device int32 [B, max_pages]), k and v are page pools [num_pages, Hkv, P, D]
    and the prompt length N comes from q [B, Hq, N, D]."""
    if block_table is None:
        desc = _desc_from(q, k, pct, True, scale, o=o, **kw)
        cache = None if seq_lens is None else KasKvCache(seq_lens.data_ptr(), None, 0, 0, 0, 0, 0)
        return desc, cache
    over, cache = _cache(q, k, seq_lens, block_table, q.shape[2])
    B, Hq, N, D = q.shape
    desc = make_desc(B, Hq, over["n_kv_heads"], over["head_dim"], N, pct, q.dtype, softmax_scale=scale,
                     q_strides=_row_strides(q, "q"), o_strides=_row_strides(o, "o"), **kw)
    return desc, cache


def prefill_anchor(q, k, v, pct: int, scale: float = 0.0, idx_out=None, o=None, ws=None,
                   pool_scope: int = 0, pool_op: int = 0, seq_lens=None,
                   block_table=None, dense_output: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """q [B,Hq,N,D], k/v [B,Hkv,N,D] bf16 or fp16 -> (idx int32 [B,Hs,total] CSR,
    o [B,Hq,N,D]); Hs as in decode_anchor. seq_lens (device int32 [B]) gives each
    prompt's length; block_table (device int32 [B, max_pages]) makes k, v page
    pools [num_pages, Hkv, P, D]. q and o may be strided views (for example the
    [B,N,Hq,D] projection output transposed) with a contiguous head_dim.
    dense_output: o is dense causal attention (the sets are selected as usual)."""
    o = _new_out(q) if o is None else o
    _check_tensors("prefill_anchor", q, k, v, o, idx_out=idx_out, seq_lens=seq_lens, block_table=block_table)
    desc, c = _prefill_desc(q, k, pct, scale, seq_lens, block_table, o, pool_scope=pool_scope, pool_op=pool_op,
                            anchor_dense_output=int(dense_output))
    if k.stride() != v.stride():
        raise KasError(1, "prefill_anchor", "k and v must share strides")
    total = int(prefill_offsets(desc)[-1])
    if idx_out is None:
        hs = 1 if pool_scope else desc.n_kv_heads
        idx_out = torch.empty((desc.batch, hs, max(total, 1)), dtype=torch.int32,
                              device=q.device)
    ws = _ws_kv(desc, c, OP_PREFILL_ANCHOR, ws, q.device)
    if c is None:
        rc = _load().kas_prefill_anchor(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(idx_out),
                                        _ptr(o), _ptr(ws), ws.numel(), _stream(q))
    else:
        rc = _load().kas_prefill_anchor_kv(ctypes.byref(desc), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(idx_out), _ptr(o), _ptr(ws), ws.numel(), _stream(q))
    _check(rc, "prefill_anchor")
    return idx_out, o


def prefill_reuse(q, k, v, anchor_idx, head_map, pct: int, scale: float = 0.0, o=None, ws=None,
                  query_head_map: bool = False, seq_lens=None, block_table=None) -> torch.Tensor:
    """head_map as in decode_reuse; cache arguments and strides as in prefill_anchor."""
    o = _new_out(q) if o is None else o
    _check_tensors("prefill_reuse", q, k, v, o, anchor_idx=anchor_idx, head_map=head_map, seq_lens=seq_lens,
                   block_table=block_table)
    desc, c = _prefill_desc(q, k, pct, scale, seq_lens, block_table, o, query_head_map=int(query_head_map))
    if k.stride() != v.stride():
        raise KasError(1, "prefill_reuse", "k and v must share strides")
    ws = _ws_kv(desc, c, OP_PREFILL_REUSE, ws, q.device)
    if c is None:
        rc = _load().kas_prefill_reuse(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(anchor_idx),
                                       anchor_idx.shape[1], _ptr(head_map), _ptr(o), _ptr(ws), ws.numel(),
                                       _stream(q))
    else:
        rc = _load().kas_prefill_reuse_kv(ctypes.byref(desc), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(anchor_idx), anchor_idx.shape[1], _ptr(head_map), _ptr(o),
                                          _ptr(ws), ws.numel(), _stream(q))
    _check(rc, "prefill_reuse")
    return o


def decode_dense(q, k, v, scale: float = 0.0, o=None, ws=None, seq_lens=None, block_table=None,
                 seq_len=None) -> torch.Tensor:
    """Dense decode attention over all keys: q [B,Hq,D], k/v [B,Hkv,N,D] -> o [B,Hq,D].
    Cache arguments as in decode_anchor."""
    o = _new_out(q) if o is None else o
    _check_tensors("decode_dense", q, k, v, o, seq_lens=seq_lens, block_table=block_table)
    over, cache = _cache(q, k, seq_lens, block_table, seq_len)
    desc = _decode_desc(q, k, 100, scale, over, o)
    if k.stride() != v.stride():
        raise KasError(1, "decode_dense", "k and v must share strides")
    ws = _ws_kv(desc, cache, OP_DECODE_DENSE, ws, q.device)
    if cache is None:
        rc = _load().kas_decode_dense(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(ws),
                                      ws.numel(), _stream(q))
    else:
        rc = _load().kas_decode_dense_kv(ctypes.byref(desc), ctypes.byref(cache), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(o), _ptr(ws), ws.numel(), _stream(q))
    _check(rc, "decode_dense")
    return o


def prefill_dense(q, k, v, scale: float = 0.0, o=None, seq_lens=None, block_table=None,
                  ws=None) -> torch.Tensor:
    """Dense causal attention: q [B,Hq,N,D], k/v [B,Hkv,N,D] bf16 or fp16 -> o [B,Hq,N,D].
    Cache arguments as in prefill_anchor (only a paged call needs a workspace)."""
    o = _new_out(q) if o is None else o
    _check_tensors("prefill_dense", q, k, v, o, seq_lens=seq_lens, block_table=block_table)
    desc, c = _prefill_desc(q, k, 100, scale, seq_lens, block_table, o)
    if k.stride() != v.stride():
        raise KasError(1, "prefill_dense", "k and v must share strides")
    if c is None:
        rc = _load().kas_prefill_dense(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), None, 0, _stream(q))
    else:
        if block_table is not None:
            ws = _ws_kv(desc, c, OP_PREFILL_DENSE, ws, q.device)
        rc = _load().kas_prefill_dense_kv(ctypes.byref(desc), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                          _ptr(ws), 0 if ws is None else ws.numel(), _stream(q))
    _check(rc, "prefill_dense")
    return o


def decode_refine(q, k, v, pool_idx, head_map, pct: int, scale: float = 0.0, idx_out=None, o=None,
                  ws=None, query_head_map: bool = False, seq_lens=None, pool_lens=None, block_table=None,
                  seq_len=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Refined layer of proposal-refined reuse: pool_idx [B, Hkv_p, n_pool] int32 (an anchor
    set at a larger percentage), head_map [Hkv] or None -> (idx int32 [B, Hs, kappa],
    o [B, Hq, D]) with kappa this layer's own k for pct and Hs = Hkv (Hq with
    query_head_map, head_map then [Hq]). seq_lens / block_table as in decode_anchor;
    pool_lens [B] int32: valid entries of each sequence's pool rows."""
    o = _new_out(q) if o is None else o
    _check_tensors("decode_refine", q, k, v, o, pool_idx=pool_idx, head_map=head_map, idx_out=idx_out,
                   seq_lens=seq_lens, pool_lens=pool_lens, block_table=block_table)
    over, cache = _cache(q, k, seq_lens, block_table, seq_len)
    desc = _decode_desc(q, k, pct, scale, over, o, query_head_map=int(query_head_map))
    if k.stride() != v.stride():
        raise KasError(1, "decode_refine", "k and v must share strides")
    n_pool = pool_idx.shape[2]
    kappa = decode_k(desc.seq_len, pct)
    sets = desc.n_q_heads if query_head_map else desc.n_kv_heads
    if idx_out is None:
        idx_out = torch.empty((desc.batch, sets, kappa), dtype=torch.int32, device=q.device)
    L = _load()
    cref = None if cache is None else ctypes.byref(cache)
    if ws is None:
        n = ctypes.c_size_t(0)
        _check(L.kas_workspace_size_refine_kv(ctypes.byref(desc), cref, n_pool, ctypes.byref(n)), "workspace_size")
        ws = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=q.device)
    _check(L.kas_decode_refine_kv(ctypes.byref(desc), cref, _ptr(q), _ptr(k), _ptr(v), _ptr(pool_idx),
                                  pool_idx.shape[1], n_pool, _ptr(pool_lens), _ptr(head_map), _ptr(idx_out),
                                  _ptr(o), _ptr(ws), ws.numel(), _stream(q)),
           "decode_refine")
    return idx_out, o


def profile_enable(on: bool = True) -> None:
    _check(_load().kas_profile_enable(1 if on else 0), "profile_enable")


def profile_reset() -> None:
    _check(_load().kas_profile_reset(), "profile_reset")


def profile_query(kernel: str) -> Tuple[float, int]:
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    _check(_load().kas_profile_query(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)), "profile_query")
    return ms.value, n.value


def profile_names():
    buf = ctypes.create_string_buffer(1024)
    _check(_load().kas_profile_names(buf, 1024), "profile_names")
    return buf.value.decode().split(",")
