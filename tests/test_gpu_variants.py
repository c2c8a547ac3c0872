"""GPU parity of the anchor selection variants against the oracle, through
the C ABI: pooling over all query heads (one set shared by every KV head, the
README's all-heads-pooled strategy) and max-pooling instead of the sum, in
decode and prefill, with reuse layers reading the shared sets; and reuse
layers whose head map has one entry per query head.

Index sets must match the oracle's exactly except inside the near-tie band
(relative 1e-4 of the oracle's k-th pooled score, using the oracle's pooled
scores of the same variant); outputs within 2e-2 (bf16) / 1e-4 (fp32).
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import inputgen
import oracle
from parity_util import TOL, assert_index_set, max_abs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
VARIANTS = [(0, 1), (1, 0), (1, 1)]          # (pool_scope, pool_op); (0, 0) is the default path
VIDS = ["group_max", "all_sum", "all_max"]


def _kas():
    import sparse_attention_long_anchor_amd as kas
    return kas


def _np(t):
    return t.detach().float().cpu().numpy()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check_decode(w, q, k, v, pct, scope, op, label):
    kas = _kas()
    _say(f"[decode anchor {VIDS[VARIANTS.index((scope, op))]}] {label}: B={w.batch} Hq={w.n_q_heads} "
         f"Hkv={w.n_kv_heads} N={w.seq_len} {w.dtype}")
    idx, o = kas.decode_anchor(q, k, v, pct, pool_scope=scope, pool_op=op)
    torch.cuda.synchronize()
    Hs = 1 if scope else w.n_kv_heads
    assert tuple(idx.shape) == (w.batch, Hs, oracle.decode_k(w.seq_len, pct))
    qn, kn, vn = _np(q), _np(k), _np(v)
    oidx, oo, pooled = oracle.decode_anchor(qn, kn, vn, pct, want_pooled=True, pool_scope=scope, pool_op=op)
    kk = oracle.decode_k(w.seq_len, pct)
    gidx = idx.cpu().numpy()
    swaps = 0
    for b in range(w.batch):
        for s in range(Hs):
            swaps += assert_index_set(gidx[b, s], oidx[b, s], pooled[b, s], kk, where=f"{label} b{b} s{s}")
    hm = np.zeros(w.n_kv_heads, np.int32) if scope else np.arange(w.n_kv_heads, dtype=np.int32)
    o_same = oracle.decode_reuse(qn, kn, vn, gidx, hm)
    err_same, err_e2e = max_abs(_np(o), o_same), max_abs(_np(o), oo)
    tol = TOL[w.dtype]
    _say(f"    near-tie swaps={swaps} max|o-o_oracle(same set)|={err_same:.3g} max|o-o_oracle|={err_e2e:.3g}")
    assert err_same <= tol and err_e2e <= tol
    return idx


DECODE_SHAPES = [
    # (label, B, Hq, Hkv, D, N, dtype, pct)
    ("f32_d64_g4", 1, 8, 2, 64, 2048, "f32", 10),
    ("bf16_d128_g4_ragged", 2, 32, 8, 128, 5037, "bf16", 10),
    ("bf16_d64_g1", 2, 4, 4, 64, 3001, "bf16", 10),
    ("bf16_d128_g8", 1, 16, 2, 128, 4099, "bf16", 10),
    ("bf16_n17", 1, 8, 2, 128, 17, "bf16", 30),
]


@pytest.mark.parametrize("variant", VARIANTS, ids=VIDS)
@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=[s[0] for s in DECODE_SHAPES])
def test_decode_variant_anchor_then_reuse(shape, variant):
    kas = _kas()
    label, B, Hq, Hkv, D, N, dt, pct = shape
    scope, op = variant
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    idx = _check_decode(w, q, k, v, pct, scope, op, label)
    # a reuse layer reads the shared set (no head map) or a mapped per-head set
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    if scope:
        o2 = kas.decode_reuse(q2, k2, v2, idx, None, pct)
        hm = np.zeros(Hkv, np.int32)
    else:
        hm = np.random.default_rng(2).integers(0, Hkv, Hkv).astype(np.int32)
        o2 = kas.decode_reuse(q2, k2, v2, idx, torch.as_tensor(hm, device=DEV), pct)
    torch.cuda.synchronize()
    ref = oracle.decode_reuse(_np(q2), _np(k2), _np(v2), idx.cpu().numpy(), hm)
    err = max_abs(_np(o2), ref)
    _say(f"    reuse max|o-o_oracle|={err:.3g}")
    assert err <= TOL[dt]


@pytest.mark.parametrize("variant", [(1, 0), (0, 1)], ids=["all_sum", "group_max"])
def test_decode_variant_full_size(variant):
    w = inputgen.WORKLOADS["llama8b_decode_128k"]
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    _check_decode(w, q, k, v, w.topk_pct, variant[0], variant[1], w.name)


def _check_prefill_tiles(w, q, k, v, pct, scope, op, gidx, go, tiles, label):
    N, B, Hkv = w.seq_len, w.batch, w.n_kv_heads
    Hs = 1 if scope else Hkv
    off = oracle.prefill_offsets(N, 32, pct)
    kn, vn = _np(k), _np(v)
    gi = gidx.cpu().numpy()
    assert gi.shape[1] == Hs
    hm = np.zeros(Hkv, np.int32) if scope else np.arange(Hkv, dtype=np.int32)
    worst_set, worst_e2e, swaps = 0.0, 0.0, 0
    for t in tiles:
        qr = _np(q[:, :, 32 * t: 32 * t + 32])
        oidx, oo = oracle.prefill_anchor(qr, kn, vn, pct, t0=t, t1=t + 1, pool_scope=scope, pool_op=op)
        kt = int(off[t + 1] - off[t])
        for b in range(B):
            for s in range(Hs):
                gs = gi[b, s, off[t]:off[t + 1]]
                if not np.array_equal(gs, oidx[b, s]):
                    P = oracle.prefill_pooled(qr, kn, b, t, s, t0=t, t1=t + 1, pool_scope=scope,
                                              pool_op=op)[: 32 * t]
                    swaps += assert_index_set(gs, oidx[b, s], P, kt, where=f"{label} b{b} t{t} s{s}")
        o_same = oracle.prefill_reuse(qr, kn, vn, gi, hm, pct, t0=t, t1=t + 1)
        gor = _np(go[:, :, 32 * t: 32 * t + 32])
        worst_set = max(worst_set, max_abs(gor, o_same))
        worst_e2e = max(worst_e2e, max_abs(gor, oo))
    _say(f"    tiles={list(tiles)[:8]}{'...' if len(tiles) > 8 else ''} near-tie swaps={swaps} "
         f"max|o-o_oracle(same set)|={worst_set:.3g} max|o-o_oracle|={worst_e2e:.3g}")
    assert worst_set <= TOL["bf16"] and worst_e2e <= TOL["bf16"]


PREFILL_SHAPES = [
    # (label, B, Hq, Hkv, D, N, pct)
    ("d128_g4_n256", 1, 8, 2, 128, 256, 10),
    ("d128_g4_b2_n1184", 2, 8, 2, 128, 1184, 10),
    ("d64_g1_n640", 1, 2, 2, 64, 640, 10),
    ("d128_g8_n384_pct25", 1, 16, 2, 128, 384, 25),
    ("d128_g4_n32_single_tile", 1, 8, 2, 128, 32, 10),
]


@pytest.mark.parametrize("variant", VARIANTS, ids=VIDS)
@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=[s[0] for s in PREFILL_SHAPES])
def test_prefill_variant_anchor_then_reuse(shape, variant):
    kas = _kas()
    label, B, Hq, Hkv, D, N, pct = shape
    scope, op = variant
    w = inputgen.custom("prefill", B, Hq, Hkv, D, N, "bf16", wid=zlib.crc32(label.encode()) % 1000,
                        topk_pct=pct)
    _say(f"[prefill anchor {VIDS[VARIANTS.index(variant)]}] {label}: B={B} Hq={Hq} Hkv={Hkv} D={D} N={N}")
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    gidx, go = kas.prefill_anchor(q, k, v, pct, pool_scope=scope, pool_op=op)
    torch.cuda.synchronize()
    _check_prefill_tiles(w, q, k, v, pct, scope, op, gidx, go, range(N // 32), label)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.zeros(Hkv, np.int32)
    o2 = kas.prefill_reuse(q2, k2, v2, gidx, None if scope else torch.as_tensor(hm, device=DEV), pct)
    torch.cuda.synchronize()
    ref = oracle.prefill_reuse(_np(q2), _np(k2), _np(v2), gidx.cpu().numpy(), hm, pct)
    err = max_abs(_np(o2), ref)
    _say(f"    reuse max|o-o_oracle|={err:.3g}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("variant", [(1, 0), (0, 1)], ids=["all_sum", "group_max"])
def test_prefill_variant_full_size_sampled_tiles(variant):
    kas = _kas()
    w = inputgen.WORKLOADS["qwen8b_prefill_32k"]
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    _say(f"[prefill anchor {variant}] {w.name}: N={w.seq_len}")
    gidx, go = kas.prefill_anchor(q, k, v, w.topk_pct, pool_scope=variant[0], pool_op=variant[1])
    torch.cuda.synchronize()
    _check_prefill_tiles(w, q, k, v, w.topk_pct, variant[0], variant[1], gidx, go, (1, 37, 500, 1023), w.name)


# ---------------------------------------------------------------- per-query-head maps

QMAP_DECODE = [
    # (label, B, Hq, Hkv, D, N, dtype, pct)
    ("f32_d64_g4", 1, 8, 2, 64, 2048, "f32", 10),
    ("bf16_d128_g4_ragged", 2, 32, 8, 128, 5037, "bf16", 10),
    ("bf16_d128_g8", 1, 16, 2, 128, 4099, "bf16", 10),
    ("f16_d64_g2", 2, 8, 4, 64, 3001, "f16", 25),
]


@pytest.mark.parametrize("shape", QMAP_DECODE, ids=[s[0] for s in QMAP_DECODE])
def test_decode_reuse_query_head_map(shape):
    kas = _kas()
    label, B, Hq, Hkv, D, N, dt, pct = shape
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    idx, _ = kas.decode_anchor(q, k, v, pct)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    qm = np.random.default_rng(7).integers(0, Hkv, Hq).astype(np.int32)
    o = kas.decode_reuse(q2, k2, v2, idx, torch.as_tensor(qm, device=DEV), pct, query_head_map=True)
    torch.cuda.synchronize()
    ref = oracle.decode_reuse(_np(q2), _np(k2), _np(v2), idx.cpu().numpy(), qm, query_head_map=True)
    err = max_abs(_np(o), ref)
    _say(f"[decode reuse, map per query head] {label}: qmap={qm.tolist()} max|o-o_oracle|={err:.3g}")
    assert err <= TOL[dt]


QMAP_PREFILL = [
    # (label, B, Hq, Hkv, D, N, dtype, pct)
    ("bf16_d128_g4_n256", 1, 8, 2, 128, 256, "bf16", 10),
    ("bf16_d128_g4_b2_n1184", 2, 8, 2, 128, 1184, "bf16", 10),
    ("bf16_d64_g2_n640", 1, 4, 2, 64, 640, "bf16", 25),
    ("f16_d128_g8_n384", 1, 16, 2, 128, 384, "f16", 10),
]


@pytest.mark.parametrize("shape", QMAP_PREFILL, ids=[s[0] for s in QMAP_PREFILL])
def test_prefill_reuse_query_head_map(shape):
    kas = _kas()
    label, B, Hq, Hkv, D, N, dt, pct = shape
    w = inputgen.custom("prefill", B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    idx, _ = kas.prefill_anchor(q, k, v, pct)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    qm = np.random.default_rng(8).integers(0, Hkv, Hq).astype(np.int32)
    o = kas.prefill_reuse(q2, k2, v2, idx, torch.as_tensor(qm, device=DEV), pct, query_head_map=True)
    torch.cuda.synchronize()
    ref = oracle.prefill_reuse(_np(q2), _np(k2), _np(v2), idx.cpu().numpy(), qm, pct, query_head_map=True)
    err = max_abs(_np(o), ref)
    _say(f"[prefill reuse, map per query head] {label}: max|o-o_oracle|={err:.3g}")
    assert err <= TOL[dt]


def test_reuse_query_head_map_full_size():
    kas = _kas()
    w = inputgen.WORKLOADS["llama8b_decode_128k"]
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    idx, _ = kas.decode_anchor(q, k, v, w.topk_pct)
    del q, k, v
    q, k, v = inputgen.layer_inputs(w, 1, DEV, pos)
    qm = np.random.default_rng(9).integers(0, w.n_kv_heads, w.n_q_heads).astype(np.int32)
    o = kas.decode_reuse(q, k, v, idx, torch.as_tensor(qm, device=DEV), w.topk_pct, query_head_map=True)
    torch.cuda.synchronize()
    ref = oracle.decode_reuse(_np(q), _np(k), _np(v), idx.cpu().numpy(), qm, query_head_map=True)
    err = max_abs(_np(o), ref)
    _say(f"[decode reuse, map per query head] {w.name}: max|o-o_oracle|={err:.3g}")
    assert err <= TOL["bf16"]
    del q, k, v
    wp = inputgen.WORKLOADS["qwen8b_prefill_32k"]
    posp = inputgen.heavy_positions(wp)
    q, k, v = inputgen.layer_inputs(wp, 0, DEV, posp)
    pidx, _ = kas.prefill_anchor(q, k, v, wp.topk_pct)
    q, k, v = inputgen.layer_inputs(wp, 1, DEV, posp)
    qm = np.random.default_rng(10).integers(0, wp.n_kv_heads, wp.n_q_heads).astype(np.int32)
    o = kas.prefill_reuse(q, k, v, pidx, torch.as_tensor(qm, device=DEV), wp.topk_pct, query_head_map=True)
    torch.cuda.synchronize()
    worst = 0.0
    for t in (1, 500, 1023):
        qr = _np(q[:, :, 32 * t: 32 * t + 32])
        ref = oracle.prefill_reuse(qr, _np(k), _np(v), pidx.cpu().numpy(), qm, wp.topk_pct, t0=t, t1=t + 1,
                                   query_head_map=True)
        worst = max(worst, max_abs(_np(o[:, :, 32 * t: 32 * t + 32]), ref))
    _say(f"[prefill reuse, map per query head] {wp.name}: tiles (1, 500, 1023) max|o-o_oracle|={worst:.3g}")
    assert worst <= TOL["bf16"]


# ---------------------------------------------------------------- proposal-refined reuse

REFINE = [
    # (label, B, Hq, Hkv, D, N, dtype, pct, pool pct)
    ("bf16_d128_g4_ragged", 2, 32, 8, 128, 5037, "bf16", 10, 40),
    ("f32_d64_g4", 1, 8, 2, 64, 2048, "f32", 10, 40),
    ("f16_d128_g8", 1, 16, 2, 128, 4099, "f16", 10, 20),
    ("bf16_d64_g1_small", 2, 4, 4, 64, 300, "bf16", 5, 100),
    ("f16_d64_g2_b3", 3, 8, 4, 64, 7001, "f16", 10, 30),
]


def _check_refine(w, q2, k2, v2, pool, hm, pct, label):
    kas = _kas()
    idx, o = kas.decode_refine(q2, k2, v2, pool, torch.as_tensor(hm, device=DEV), pct)
    torch.cuda.synchronize()
    qn, kn, vn = _np(q2), _np(k2), _np(v2)
    pn = pool.cpu().numpy()
    kappa = oracle.decode_k(w.seq_len, pct)
    oidx, oo = oracle.decode_refine(qn, kn, vn, pn, hm, kappa)
    gi = idx.cpu().numpy()
    G = w.n_q_heads // w.n_kv_heads
    swaps = 0
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            if np.array_equal(gi[b, g], oidx[b, g]):
                continue
            # near ties: the pool-restricted pooled scores (float64, torch), indexed by key
            keys = pn[b, hm[g]]
            s = torch.from_numpy(qn[b, g * G:(g + 1) * G]).double() @ torch.from_numpy(kn[b, g, keys]).double().T
            P = torch.softmax(s / np.sqrt(w.head_dim), -1).sum(0).numpy()
            full = np.zeros(w.seq_len)
            full[keys] = P
            swaps += assert_index_set(gi[b, g], oidx[b, g], full, kappa, where=f"{label} b{b} g{g}")
    o_same = oracle.decode_reuse(qn, kn, vn, gi, np.arange(w.n_kv_heads, dtype=np.int32))
    err_same, err = max_abs(_np(o), o_same), max_abs(_np(o), oo)
    _say(f"[decode refine] {label}: pool {pn.shape[-1]} -> kappa {kappa}, near-tie swaps={swaps} "
         f"max|o-o_oracle(same set)|={err_same:.3g} max|o-o_oracle|={err:.3g}")
    assert err_same <= TOL[w.dtype] and err <= TOL[w.dtype]
    return idx, o


@pytest.mark.parametrize("case", REFINE, ids=[c[0] for c in REFINE])
def test_decode_refine(case):
    kas = _kas()
    label, B, Hq, Hkv, D, N, dt, pct, ppct = case
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    pool, _ = kas.decode_anchor(q, k, v, ppct)                      # the proposal layer
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.random.default_rng(6).integers(0, Hkv, Hkv).astype(np.int32)
    idx, o = _check_refine(w, q2, k2, v2, pool, hm, pct, label)
    if dt != "f32":
        _check_refine_paged(w, q2, k2, v2, pool, hm, pct, idx, o, P=64 if N > 1000 else 16)
    if ppct == 100:
        # the pool is every key: the refined layer selects what an anchor on it selects
        aidx, _ = kas.decode_anchor(q2, k2, v2, pct)
        ident = np.arange(Hkv, dtype=np.int32)
        idx2, _ = kas.decode_refine(q2, k2, v2, pool, torch.as_tensor(ident, device=DEV), pct)
        torch.cuda.synchronize()
        assert torch.equal(idx2, aidx)


def _check_refine_paged(w, q2, k2, v2, pool, hm, pct, idx, o, P):
    """The refined layer over a paged copy of the cache: the same sets and
    the same output, bit for bit."""
    kas = _kas()
    from test_gpu_kvcache import _paged
    kp, vp, bt = _paged(k2, v2, P, seed=P)
    idx_p, o_p = kas.decode_refine(q2, kp, vp, pool, torch.as_tensor(hm, device=DEV), pct, block_table=bt,
                                   seq_len=w.seq_len)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx), "paged refined sets differ from the contiguous cache's"
    assert torch.equal(o_p, o), "paged refined output differs from the contiguous cache's"
    _say(f"    paged (P = {P}): sets and output bit-identical to the contiguous cache")


def test_decode_refine_full_size():
    kas = _kas()
    w = inputgen.WORKLOADS["llama8b_decode_128k"]
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    pool, _ = kas.decode_anchor(q, k, v, 4 * w.topk_pct)
    del q, k, v
    q, k, v = inputgen.layer_inputs(w, 1, DEV, pos)
    hm = inputgen.head_maps(w)[1]
    idx, o = _check_refine(w, q, k, v, pool, hm, w.topk_pct, w.name)
    _check_refine_paged(w, q, k, v, pool, hm, w.topk_pct, idx, o, P=256)


REFINE_QMAP = [
    # (label, B, Hq, Hkv, D, N, dtype, pct, pool pct)
    ("bf16_d128_g4", 2, 16, 4, 128, 3001, "bf16", 10, 40),
    ("f16_d64_g2", 1, 8, 4, 64, 1500, "f16", 5, 25),
]


@pytest.mark.parametrize("case", REFINE_QMAP, ids=[c[0] for c in REFINE_QMAP])
def test_decode_refine_query_head_map(case):
    """One refined set per query head: query head h refines within pool
    head_map[h] by its own softmax. The oracle's refined layer over K and V
    expanded to one head per query head (groups of one) defines it."""
    kas = _kas()
    label, B, Hq, Hkv, D, N, dt, pct, ppct = case
    G = Hq // Hkv
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000 + 7, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    pool, _ = kas.decode_anchor(q, k, v, ppct)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.random.default_rng(8).integers(0, Hkv, Hq).astype(np.int32)
    hmt = torch.as_tensor(hm, device=DEV)
    idx, o = kas.decode_refine(q2, k2, v2, pool, hmt, pct, query_head_map=True)
    torch.cuda.synchronize()
    assert idx.shape == (B, Hq, oracle.decode_k(N, pct))
    qn, kn, vn, pn = _np(q2), _np(k2), _np(v2), pool.cpu().numpy()
    ke, ve = np.repeat(kn, G, axis=1), np.repeat(vn, G, axis=1)
    kappa = oracle.decode_k(N, pct)
    oidx, oo = oracle.decode_refine(qn, ke, ve, pn, hm, kappa)
    gi = idx.cpu().numpy()
    swaps = 0
    for b in range(B):
        for h in range(Hq):
            if np.array_equal(gi[b, h], oidx[b, h]):
                continue
            keys = pn[b, hm[h]]
            s = torch.from_numpy(qn[b, h]).double() @ torch.from_numpy(kn[b, h // G, keys]).double().T
            full = np.zeros(N)
            full[keys] = torch.softmax(s / np.sqrt(D), -1).numpy()
            swaps += assert_index_set(gi[b, h], oidx[b, h], full, kappa, where=f"{label} b{b} h{h}")
    o_same = oracle.decode_reuse(qn, ke, ve, gi, np.arange(Hq, dtype=np.int32))
    err_same, err = max_abs(_np(o), o_same), max_abs(_np(o), oo)
    _say(f"[decode refine, per query head] {label}: near-tie swaps={swaps} "
         f"max|o-o_oracle(same set)|={err_same:.3g} max|o-o_oracle|={err:.3g}")
    assert err_same <= TOL[dt] and err <= TOL[dt]
    from test_gpu_kvcache import _paged
    kp, vp, bt = _paged(k2, v2, 64, seed=9)
    idx_p, o_p = kas.decode_refine(q2, kp, vp, pool, hmt, pct, query_head_map=True, block_table=bt, seq_len=N)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx) and torch.equal(o_p, o)


REFINE_VARLEN = [
    # (label, B, Hq, Hkv, D, N, dtype, pct, pool pct, lengths)
    ("bf16_d128_g4", 3, 8, 2, 128, 4099, "bf16", 10, 40, (4099, 1777, 300)),
    ("f16_d64_g2_short", 4, 8, 4, 64, 2048, "f16", 5, 20, (2048, 1, 33, 1200)),
]


@pytest.mark.parametrize("case", REFINE_VARLEN, ids=[c[0] for c in REFINE_VARLEN])
def test_decode_refine_varlen(case):
    """Sequences of different lengths, with pools from a varlen anchor call:
    sequence b refines within its pool_b valid pool entries and keeps
    kappa_b = min(k(L_b), pool_b) keys, as the oracle's refined layer on that
    sequence alone. A paged copy gives the same bits."""
    kas = _kas()
    label, B, Hq, Hkv, D, N, dt, pct, ppct, lens = case
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000 + 11, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    L = np.array(lens, dtype=np.int32)
    tl = torch.as_tensor(L, device=DEV)
    pool, _ = kas.decode_anchor(q, k, v, ppct, seq_lens=tl)
    plen = np.array([oracle.decode_k(int(x), ppct) for x in L], dtype=np.int32)
    tp = torch.as_tensor(plen, device=DEV)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.random.default_rng(12).integers(0, Hkv, Hkv).astype(np.int32)
    hmt = torch.as_tensor(hm, device=DEV)
    idx, o = kas.decode_refine(q2, k2, v2, pool, hmt, pct, seq_lens=tl, pool_lens=tp)
    torch.cuda.synchronize()
    qn, kn, vn, pn, gi = _np(q2), _np(k2), _np(v2), pool.cpu().numpy(), idx.cpu().numpy()
    G = Hq // Hkv
    worst_same, worst, swaps = 0.0, 0.0, 0
    for b in range(B):
        n, pb = int(L[b]), int(plen[b])
        kappa = min(oracle.decode_k(n, pct), pb)
        kb, vb = kn[b:b + 1, :, :n], vn[b:b + 1, :, :n]
        pool_b = np.ascontiguousarray(pn[b:b + 1, :, :pb])
        oidx, oo = oracle.decode_refine(qn[b:b + 1], kb, vb, pool_b, hm, kappa)
        for g in range(Hkv):
            got = gi[b, g, :kappa]
            if np.array_equal(got, oidx[0, g]):
                continue
            keys = pool_b[0, hm[g]]
            s = torch.from_numpy(qn[b, g * G:(g + 1) * G]).double() @ torch.from_numpy(kn[b, g, keys]).double().T
            full = np.zeros(n)
            full[keys] = torch.softmax(s / np.sqrt(D), -1).sum(0).numpy()
            swaps += assert_index_set(got, oidx[0, g], full, kappa, where=f"{label} b{b} g{g}")
        o_same = oracle.decode_reuse(qn[b:b + 1], kb, vb, np.ascontiguousarray(gi[b:b + 1, :, :kappa]),
                                     np.arange(Hkv, dtype=np.int32))
        worst_same = max(worst_same, max_abs(_np(o[b:b + 1]), o_same))
        worst = max(worst, max_abs(_np(o[b:b + 1]), oo))
    _say(f"[decode refine, varlen] {label}: lengths {list(L)} pools {list(plen)} near-tie swaps={swaps} "
         f"max|o-o_oracle(same set)|={worst_same:.3g} max|o-o_oracle|={worst:.3g}")
    assert worst_same <= TOL[dt] and worst <= TOL[dt]
    from test_gpu_kvcache import _paged
    kp, vp, bt = _paged(k2, v2, 16, seed=13)
    idx_p, o_p = kas.decode_refine(q2, kp, vp, pool, hmt, pct, seq_lens=tl, pool_lens=tp, block_table=bt,
                                   seq_len=N)
    torch.cuda.synchronize()
    for b in range(B):
        kappa = min(oracle.decode_k(int(L[b]), pct), int(plen[b]))
        assert torch.equal(idx_p[b, :, :kappa], idx[b, :, :kappa])
    assert torch.equal(o_p, o)


def test_decode_refine_full_lengths_equal_plain_call():
    """Lengths of N for every sequence and full pools take the per-sequence
    path; the sets and outputs are those of the plain call, bit for bit."""
    kas = _kas()
    B, Hq, Hkv, D, N, pct = 2, 32, 8, 128, 5000, 10
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, "bf16", wid=314, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    pool, _ = kas.decode_anchor(q, k, v, 4 * pct)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = torch.as_tensor(np.random.default_rng(15).integers(0, Hkv, Hkv).astype(np.int32), device=DEV)
    idx, o = kas.decode_refine(q2, k2, v2, pool, hm, pct)
    tl = torch.full((B,), N, dtype=torch.int32, device=DEV)
    tp = torch.full((B,), pool.shape[2], dtype=torch.int32, device=DEV)
    idx_v, o_v = kas.decode_refine(q2, k2, v2, pool, hm, pct, seq_lens=tl, pool_lens=tp)
    idx_l, o_l = kas.decode_refine(q2, k2, v2, pool, hm, pct, pool_lens=tp)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_v) and torch.equal(o, o_v)
    assert torch.equal(idx, idx_l) and torch.equal(o, o_l)
