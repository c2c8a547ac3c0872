"""GPU parity over shapes drawn at random once, from a seeded generator, so
every run checks the same cases. Each case runs the anchor and a reuse layer
through the C ABI and checks them against the CPU oracle with the same helpers
and tolerances as the fixed-shape tests: index sets equal except near ties,
outputs within the dtype's tolerance, k = N against dense attention.

Decode: B 1-3, 1-4 KV heads, 1-8 query heads per KV head, D 64 or 128,
N 1-12000 keys (a third of the cases below 300), 1-100 %, fp32, bf16 or
fp16. Prefill: B 1-2, 1-2 KV heads, 1-8 query heads per KV head, D 64 or 128,
1-24 tiles, 1-100 %, bf16 or fp16. Varlen and paged caches (the same
helpers as the fixed kv-cache tests): per-sequence lengths drawn in [1, N]
with one sequence at full length, page sizes 16-1024 (bf16 and fp16; a
paged fp32 cache is unsupported), every sequence against the oracle and
the paged calls against the contiguous ones. Selection variants: pooling
over all heads and max-pooling, decode and prefill; proposal-refined
decode reuse with a pool of 1-100 % drawn at or above the refined layer's
share.
"""
import numpy as np
import pytest
import torch

import inputgen
import oracle
from parity_util import TOL, max_abs
from test_gpu_decode import _check_anchor, _check_reuse
from test_gpu_kvcache import _check_prefill_paged, _check_prefill_varlen, _check_varlen
from test_gpu_prefill import _check_reuse_tiles, _check_tiles
from test_gpu_variants import _check_decode as _check_decode_variant
from test_gpu_variants import _check_prefill_tiles as _check_prefill_variant
from test_gpu_variants import _check_refine

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _decode_cases(n, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.integers(1, 300)) if i % 3 == 0 else int(rng.integers(300, 12001))
        out.append((int(rng.integers(1, 4)), int(rng.choice([1, 2, 4])), int(rng.choice([1, 2, 4, 8])),
                    int(rng.choice([64, 128])), N, int(rng.integers(1, 101)),
                    str(rng.choice(["bf16", "f16", "f32"])), int(rng.integers(0, 1000))))
    return out


def _prefill_cases(n, seed=20261204):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 3)), int(rng.choice([1, 2])), int(rng.choice([1, 2, 4, 8])),
             int(rng.choice([64, 128])), int(rng.integers(1, 25)), int(rng.integers(1, 101)),
             str(rng.choice(["bf16", "f16"])), int(rng.integers(0, 1000))) for _ in range(n)]


def _kv_cases(n, phase, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dec = phase == "decode"
        dt = str(rng.choice(["bf16", "f16", "f32"] if dec else ["bf16", "f16"]))
        paged = dt != "f32" and rng.random() < 0.75
        P = int(rng.choice([16, 32, 64, 128, 256, 1024])) if paged else 0
        N = int(rng.integers(1, 9001)) if dec else 32 * int(rng.integers(1, 25))
        out.append((int(rng.integers(1, 5)), int(rng.choice([1, 2, 4])), int(rng.choice([1, 2, 4, 8])),
                    int(rng.choice([64, 128])), N, int(rng.integers(1, 101)), dt, P, int(rng.integers(0, 1000))))
    return out


DECODE_CASES = _decode_cases(40)
PREFILL_CASES = _prefill_cases(40)
KV_DECODE_CASES = _kv_cases(20, "decode", 20261205)
KV_PREFILL_CASES = _kv_cases(12, "prefill", 20261206)
# (pool_scope, pool_op) other than the default (0, 0), drawn per case
VARIANT_DECODE_CASES = [c + (v,) for c, v in zip(_decode_cases(12, seed=20261207),
                        np.random.default_rng(7).integers(0, 3, 12).tolist())]
VARIANT_PREFILL_CASES = [c + (v,) for c, v in zip(_prefill_cases(12, seed=20261208),
                         np.random.default_rng(8).integers(0, 3, 12).tolist())]
VARIANTS = [(0, 1), (1, 0), (1, 1)]
REFINE_CASES = [c + (int(np.random.default_rng(c[7]).integers(c[5], 101)),) for c in _decode_cases(16, seed=20261209)]


def _id(c):
    return "B{}_Hkv{}_G{}_D{}_N{}_pct{}_{}_w{}".format(*c)


def _kv_id(c):
    return "B{}_Hkv{}_G{}_D{}_N{}_pct{}_{}_P{}_w{}".format(*c)


def _lengths(B, N, wid, step=1):
    """Per-sequence lengths in [1, N] (multiples of `step`), the first at N."""
    L = np.random.default_rng(wid).integers(1, N // step + 1, B) * step
    L[0] = N
    return L.astype(np.int32)


def _kas():
    import sparse_attention_long_anchor_amd as kas
    return kas


def _np(t):
    return t.detach().float().cpu().numpy()


@pytest.mark.parametrize("case", DECODE_CASES, ids=[_id(c) for c in DECODE_CASES])
def test_decode_random_shapes(case):
    B, Hkv, G, D, N, pct, dt, wid = case
    label = f"random decode B{B} Hkv{Hkv} G{G} D{D} N{N} {dt} pct{pct} wid{wid}"
    w = inputgen.custom("decode", B, Hkv * G, Hkv, D, N, dt, wid=wid, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    idx, o = _check_anchor(w, q, k, v, pct, label)
    if oracle.decode_k(N, pct) == N:
        dense = oracle.dense_attention(_np(q)[:, :, None, :], _np(k), _np(v), causal=False)[:, :, 0, :]
        assert max_abs(_np(o), dense) <= TOL[dt]
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.random.default_rng(wid).integers(0, Hkv, Hkv).astype(np.int32)
    _check_reuse(w, q2, k2, v2, idx, hm, pct, label)


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[_id((c[0], c[1], c[2], c[3], 32 * c[4], c[5], c[6], c[7])) for c in PREFILL_CASES])
def test_prefill_random_shapes(case):
    B, Hkv, G, D, T, pct, dt, wid = case
    N = 32 * T
    label = f"random prefill B{B} Hkv{Hkv} G{G} D{D} N{N} {dt} pct{pct} wid{wid}"
    print(f"[prefill anchor] {label}", flush=True)
    kas = _kas()
    w = inputgen.custom("prefill", B, Hkv * G, Hkv, D, N, dt, wid=wid, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    gidx, go = kas.prefill_anchor(q, k, v, pct)
    torch.cuda.synchronize()
    _check_tiles(w, q, k, v, pct, gidx, go, range(T), label)
    if pct == 100:
        dense = oracle.dense_attention(_np(q), _np(k), _np(v), causal=True)
        assert max_abs(_np(go), dense) <= TOL[dt]
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.random.default_rng(wid).integers(0, Hkv, Hkv).astype(np.int32)
    print(f"[prefill reuse] {label}", flush=True)
    o2 = kas.prefill_reuse(q2, k2, v2, gidx, torch.as_tensor(hm, device=DEV), pct)
    torch.cuda.synchronize()
    _check_reuse_tiles(w, q2, k2, v2, pct, gidx, hm, o2, range(T), label)


@pytest.mark.parametrize("case", KV_DECODE_CASES, ids=[_kv_id(c) for c in KV_DECODE_CASES])
def test_decode_varlen_paged_random_shapes(case):
    B, Hkv, G, D, N, pct, dt, P, wid = case
    label = f"random decode varlen B{B} Hkv{Hkv} G{G} D{D} N{N} {dt} pct{pct} P{P} wid{wid}"
    w = inputgen.custom("decode", B, Hkv * G, Hkv, D, N, dt, wid=wid, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    _check_varlen(w, q, k, v, _lengths(B, N, wid), pct, label, P or None)


@pytest.mark.parametrize("case", KV_PREFILL_CASES, ids=[_kv_id(c) for c in KV_PREFILL_CASES])
def test_prefill_varlen_paged_random_shapes(case):
    B, Hkv, G, D, N, pct, dt, P, wid = case
    label = f"random prefill varlen B{B} Hkv{Hkv} G{G} D{D} N{N} {dt} pct{pct} P{P} wid{wid}"
    w = inputgen.custom("prefill", B, Hkv * G, Hkv, D, N, dt, wid=wid, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    lens = _lengths(B, N, wid)
    ref = _check_prefill_varlen(w, q, k, v, lens, pct, label)
    if P:
        _check_prefill_paged(w, q, k, v, lens, pct, P, ref)


@pytest.mark.parametrize("case", VARIANT_DECODE_CASES, ids=[_id(c[:8]) + f"_v{c[8]}" for c in VARIANT_DECODE_CASES])
def test_decode_variant_random_shapes(case):
    B, Hkv, G, D, N, pct, dt, wid, vi = case
    scope, op = VARIANTS[vi]
    label = f"random decode variant B{B} Hkv{Hkv} G{G} D{D} N{N} {dt} pct{pct} scope{scope} op{op} wid{wid}"
    w = inputgen.custom("decode", B, Hkv * G, Hkv, D, N, dt, wid=wid, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    idx = _check_decode_variant(w, q, k, v, pct, scope, op, label)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    kas = _kas()
    if scope:
        o2 = kas.decode_reuse(q2, k2, v2, idx, None, pct)
        hm = np.zeros(Hkv, np.int32)
    else:
        hm = np.random.default_rng(wid).integers(0, Hkv, Hkv).astype(np.int32)
        o2 = kas.decode_reuse(q2, k2, v2, idx, torch.as_tensor(hm, device=DEV), pct)
    torch.cuda.synchronize()
    ref = oracle.decode_reuse(_np(q2), _np(k2), _np(v2), idx.cpu().numpy(), hm)
    assert max_abs(_np(o2), ref) <= TOL[dt]


@pytest.mark.parametrize("case", VARIANT_PREFILL_CASES,
                         ids=[_id((c[0], c[1], c[2], c[3], 32 * c[4], c[5], "bf16", c[7])) + f"_v{c[8]}"
                              for c in VARIANT_PREFILL_CASES])
def test_prefill_variant_random_shapes(case):
    B, Hkv, G, D, T, pct, _, wid, vi = case
    scope, op = VARIANTS[vi]
    N = 32 * T
    label = f"random prefill variant B{B} Hkv{Hkv} G{G} D{D} N{N} pct{pct} scope{scope} op{op} wid{wid}"
    print(f"[prefill anchor] {label}", flush=True)
    kas = _kas()
    w = inputgen.custom("prefill", B, Hkv * G, Hkv, D, N, "bf16", wid=wid, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    gidx, go = kas.prefill_anchor(q, k, v, pct, pool_scope=scope, pool_op=op)
    torch.cuda.synchronize()
    _check_prefill_variant(w, q, k, v, pct, scope, op, gidx, go, range(T), label)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.zeros(Hkv, np.int32) if scope else np.random.default_rng(wid).integers(0, Hkv, Hkv).astype(np.int32)
    o2 = kas.prefill_reuse(q2, k2, v2, gidx, None if scope else torch.as_tensor(hm, device=DEV), pct)
    torch.cuda.synchronize()
    ref = oracle.prefill_reuse(_np(q2), _np(k2), _np(v2), gidx.cpu().numpy(), hm, pct)
    assert max_abs(_np(o2), ref) <= TOL["bf16"]


@pytest.mark.parametrize("case", REFINE_CASES, ids=[_id(c[:8]) + f"_pool{c[8]}" for c in REFINE_CASES])
def test_decode_refine_random_shapes(case):
    B, Hkv, G, D, N, pct, dt, wid, ppct = case
    label = f"random decode refine B{B} Hkv{Hkv} G{G} D{D} N{N} {dt} pct{pct} pool{ppct} wid{wid}"
    print(f"[decode refine] {label}", flush=True)
    kas = _kas()
    w = inputgen.custom("decode", B, Hkv * G, Hkv, D, N, dt, wid=wid, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    pool, _ = kas.decode_anchor(q, k, v, ppct)                      # the proposal layer
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.random.default_rng(wid).integers(0, Hkv, Hkv).astype(np.int32)
    _check_refine(w, q2, k2, v2, pool, hm, pct, label)
