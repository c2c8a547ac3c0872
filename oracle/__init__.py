"""ctypes front end of the CPU oracle (kascade_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg. The product library never imports or calls it.

All inputs are numpy float32 arrays (bf16 values are exactly representable);
all floating outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kascade_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkascade_oracle.so")
_lib = None

_i32, _i64, _dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
_fp = ctypes.POINTER(ctypes.c_float)
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O3, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_topk_count.argtypes = [_i64, _i32]
        L.orc_topk_count.restype = _i64
        L.orc_prefill_offsets.argtypes = [_i64, _i32, _i32, _lp]
        L.orc_prefill_offsets.restype = _i64
        L.orc_dense_attention.argtypes = [_fp, _fp, _fp, _dp, _i32, _i32, _i32, _i64, _i64,
                                          _i32, _i32, _dbl]
        L.orc_decode_anchor.argtypes = [_fp, _fp, _fp, _i32, _i32, _i32, _i64, _i32, _i32, _dbl,
                                        _ip, _dp, _dp]
        L.orc_decode_reuse.argtypes = [_fp, _fp, _fp, _i32, _i32, _i32, _i64, _i32, _dbl,
                                       _ip, _i32, _i64, _ip, _dp]
        L.orc_prefill_pooled.argtypes = [_fp, _fp, _i32, _i32, _i32, _i64, _i32, _i32, _dbl,
                                         _i64, _i64, _i64, _i64, _i64, _dp]
        L.orc_prefill_anchor.argtypes = [_fp, _fp, _fp, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                         _dbl, _i64, _i64, _ip, _dp]
        L.orc_prefill_reuse.argtypes = [_fp, _fp, _fp, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                        _dbl, _i64, _i64, _ip, _i32, _ip, _dp]
        L.orc_decode_anchor_v.argtypes = [_fp, _fp, _fp, _i32, _i32, _i32, _i64, _i32, _i32, _dbl,
                                          _i32, _i32, _ip, _dp, _dp]
        L.orc_prefill_pooled_v.argtypes = [_fp, _fp, _i32, _i32, _i32, _i64, _i32, _i32, _dbl,
                                           _i64, _i64, _i32, _i32, _i64, _i64, _i64, _dp]
        L.orc_prefill_anchor_v.argtypes = [_fp, _fp, _fp, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                           _dbl, _i64, _i64, _i32, _i32, _ip, _dp]
        L.orc_decode_reuse_q.argtypes = L.orc_decode_reuse.argtypes
        L.orc_decode_refine.argtypes = [_fp, _fp, _fp, _i32, _i32, _i32, _i64, _i32, _dbl,
                                        _ip, _i32, _i64, _ip, _i64, _ip, _dp]
        L.orc_decode_refine.restype = ctypes.c_int
        L.orc_prefill_reuse_q.argtypes = L.orc_prefill_reuse.argtypes
        for name in ("orc_decode_reuse_q", "orc_prefill_reuse_q",
                     "orc_dense_attention", "orc_decode_anchor", "orc_decode_reuse",
                     "orc_prefill_pooled", "orc_prefill_anchor", "orc_prefill_reuse",
                     "orc_decode_anchor_v", "orc_prefill_pooled_v", "orc_prefill_anchor_v"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float32 or not a.flags.c_contiguous:
        a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _i32a(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def topk_count(n: int, pct: int) -> int:
    return int(lib().orc_topk_count(n, pct))


def decode_k(n: int, pct: int) -> int:
    return max(1, topk_count(n, pct)) if n >= 1 else 0


def prefill_offsets(n: int, tile: int, pct: int) -> np.ndarray:
    T = (n + tile - 1) // tile
    off = np.zeros(T + 1, dtype=np.int64)
    lib().orc_prefill_offsets(n, tile, pct, _ptr(off, _lp))
    return off


def dense_attention(q, k, v, causal: bool, scale: float = 0.0) -> np.ndarray:
    """q [B,Hq,Nq,D], k/v [B,Hkv,Nk,D] -> o [B,Hq,Nq,D] (float64)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    o = np.zeros((B, Hq, Nq, D), dtype=np.float64)
    _check(lib().orc_dense_attention(_ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), _ptr(o, _dp),
                                     B, Hq, Hkv, Nq, Nk, D, int(causal), scale), "dense")
    return o


def decode_anchor(q, k, v, pct: int, scale: float = 0.0, want_pooled: bool = False,
                  pool_scope: int = 0, pool_op: int = 0
                  ) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """q [B,Hq,D], k/v [B,Hkv,N,D] -> (idx int32 [B,Hs,kk], o [B,Hq,D], pooled [B,Hs,N]).

    pool_scope 0: one set per KV head (its group's heads pooled), Hs = Hkv;
    1: one set per batch row pooled over all heads, Hs = 1. pool_op 0: sum,
    1: maximum."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Hq, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    Hs = 1 if pool_scope else Hkv
    kk = decode_k(N, pct)
    idx = np.zeros((B, Hs, kk), dtype=np.int32)
    o = np.zeros((B, Hq, D), dtype=np.float64)
    pooled = np.zeros((B, Hs, N), dtype=np.float64) if want_pooled else None
    pp = _ptr(pooled, _dp) if want_pooled else None
    if pool_scope == 0 and pool_op == 0:
        rc = lib().orc_decode_anchor(_ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), B, Hq, Hkv, N, D,
                                     pct, scale, _ptr(idx, _ip), _ptr(o, _dp), pp)
    else:
        rc = lib().orc_decode_anchor_v(_ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), B, Hq, Hkv, N, D,
                                       pct, scale, pool_scope, pool_op, _ptr(idx, _ip), _ptr(o, _dp), pp)
    _check(rc, "decode_anchor")
    return idx, o, pooled


def decode_reuse(q, k, v, anchor_idx, head_map, scale: float = 0.0,
                 query_head_map: bool = False) -> np.ndarray:
    """head_map: [Hkv] anchor set per KV head, or [Hq] per query head with
    query_head_map=True."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    anchor_idx, head_map = _i32a(anchor_idx), _i32a(head_map)
    B, Hq, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    Hkv_a, kk = anchor_idx.shape[1], anchor_idx.shape[2]
    assert head_map.shape == ((Hq,) if query_head_map else (Hkv,))
    o = np.zeros((B, Hq, D), dtype=np.float64)
    fn = lib().orc_decode_reuse_q if query_head_map else lib().orc_decode_reuse
    _check(fn(_ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), B, Hq, Hkv, N, D, scale, _ptr(anchor_idx, _ip),
              Hkv_a, kk, _ptr(head_map, _ip), _ptr(o, _dp)), "decode_reuse")
    return o


def decode_refine(q, k, v, pool_idx, head_map, kappa: int, scale: float = 0.0
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Refined layer of proposal-refined reuse: pool_idx [B, Hkv_p, n_pool] (ascending
    keys), head_map [Hkv] -> (idx int32 [B, Hkv, kappa], o [B, Hq, D])."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    pool_idx, head_map = _i32a(pool_idx), _i32a(head_map)
    B, Hq, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    idx = np.zeros((B, Hkv, kappa), dtype=np.int32)
    o = np.zeros((B, Hq, D), dtype=np.float64)
    _check(lib().orc_decode_refine(_ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), B, Hq, Hkv, N, D, scale,
                                   _ptr(pool_idx, _ip), pool_idx.shape[1], pool_idx.shape[2],
                                   _ptr(head_map, _ip), kappa, _ptr(idx, _ip), _ptr(o, _dp)), "decode_refine")
    return idx, o


def prefill_anchor(q_rows, k, v, pct: int, tile: int = 32, t0: int = 0, t1: Optional[int] = None,
                   scale: float = 0.0, pool_scope: int = 0, pool_op: int = 0
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """q_rows [B,Hq,R,D] = query rows of tiles [t0,t1); k/v [B,Hkv,N,D].

    Returns (idx int32 [B,Hs,off[t1]-off[t0]], o float64 [B,Hq,R,D]); Hs and
    the pooling variants as in decode_anchor."""
    q_rows, k, v = _f32(q_rows), _f32(k), _f32(v)
    B, Hq, R, D = q_rows.shape
    Hkv, N = k.shape[1], k.shape[2]
    Hs = 1 if pool_scope else Hkv
    T = (N + tile - 1) // tile
    t1 = T if t1 is None else t1
    off = prefill_offsets(N, tile, pct)
    assert R == min(N, tile * t1) - tile * t0, "q_rows must hold exactly the tile range"
    idx = np.zeros((B, Hs, int(off[t1] - off[t0])), dtype=np.int32)
    o = np.zeros((B, Hq, R, D), dtype=np.float64)
    if pool_scope == 0 and pool_op == 0:
        rc = lib().orc_prefill_anchor(_ptr(q_rows, _fp), _ptr(k, _fp), _ptr(v, _fp), B, Hq, Hkv, N,
                                      D, tile, pct, scale, t0, t1, _ptr(idx, _ip), _ptr(o, _dp))
    else:
        rc = lib().orc_prefill_anchor_v(_ptr(q_rows, _fp), _ptr(k, _fp), _ptr(v, _fp), B, Hq, Hkv, N,
                                        D, tile, pct, scale, t0, t1, pool_scope, pool_op,
                                        _ptr(idx, _ip), _ptr(o, _dp))
    _check(rc, "prefill_anchor")
    return idx, o


def prefill_pooled(q_rows, k, b: int, t: int, g: int, tile: int = 32, t0: int = 0,
                   t1: Optional[int] = None, scale: float = 0.0, pool_scope: int = 0,
                   pool_op: int = 0) -> np.ndarray:
    """Pooled scores of set g of tile t (g = 0 when pool_scope is 1)."""
    q_rows, k = _f32(q_rows), _f32(k)
    B, Hq, R, D = q_rows.shape
    Hkv, N = k.shape[1], k.shape[2]
    T = (N + tile - 1) // tile
    t1 = T if t1 is None else t1
    P = np.zeros(min(N, tile * (t + 1)), dtype=np.float64)
    if pool_scope == 0 and pool_op == 0:
        rc = lib().orc_prefill_pooled(_ptr(q_rows, _fp), _ptr(k, _fp), B, Hq, Hkv, N, D, tile,
                                      scale, t0, t1, b, t, g, _ptr(P, _dp))
    else:
        rc = lib().orc_prefill_pooled_v(_ptr(q_rows, _fp), _ptr(k, _fp), B, Hq, Hkv, N, D, tile,
                                        scale, t0, t1, pool_scope, pool_op, b, t, g, _ptr(P, _dp))
    _check(rc, "prefill_pooled")
    return P


def prefill_reuse(q_rows, k, v, anchor_idx, head_map, pct: int, tile: int = 32, t0: int = 0,
                  t1: Optional[int] = None, scale: float = 0.0, query_head_map: bool = False) -> np.ndarray:
    """anchor_idx: the anchor's FULL CSR array [B, Hkv_a, total]; head_map as in decode_reuse."""
    q_rows, k, v = _f32(q_rows), _f32(k), _f32(v)
    anchor_idx, head_map = _i32a(anchor_idx), _i32a(head_map)
    B, Hq, R, D = q_rows.shape
    Hkv, N = k.shape[1], k.shape[2]
    assert head_map.shape == ((Hq,) if query_head_map else (Hkv,))
    T = (N + tile - 1) // tile
    t1 = T if t1 is None else t1
    o = np.zeros((B, Hq, R, D), dtype=np.float64)
    fn = lib().orc_prefill_reuse_q if query_head_map else lib().orc_prefill_reuse
    _check(fn(_ptr(q_rows, _fp), _ptr(k, _fp), _ptr(v, _fp), B, Hq, Hkv, N, D, tile, pct, scale, t0, t1,
              _ptr(anchor_idx, _ip), anchor_idx.shape[1], _ptr(head_map, _ip), _ptr(o, _dp)),
           "prefill_reuse")
    return o
