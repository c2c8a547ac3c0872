"""GPU parity of decode and prefill over varlen and paged KV caches (the
README announces paged and varlen kernels), through the C ABI.

Each sequence b of a varlen batch is checked against the oracle run on its
own contiguous keys [0, seq_lens[b]); keys past a sequence's end hold random
values that must not matter. A paged cache holds the same rows scattered over
a shuffled page pool; its index sets, reuse and dense outputs must equal the
contiguous varlen results bit for bit (the same kernels over the same rows),
and its anchor output (which reads K again instead of stored logits) must
match the oracle. Prefill over a paged cache copies the pages into a
contiguous cache first, so all of its results must equal the contiguous
ones bit for bit.
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


def _kas():
    import sparse_attention_long_anchor_amd as kas
    return kas


def _np(t):
    return t.detach().float().cpu().numpy()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _paged(k, v, P, seed):
    """Scatter contiguous k, v [B, Hkv, N, D] into page pools [num_pages, Hkv, P, D]
    (shuffled page ids, spare pages filled with noise) and a block table."""
    B, Hkv, N, D = k.shape
    per = (N + P - 1) // P
    npages = B * per + 3
    rng = np.random.default_rng(seed)
    ids = rng.permutation(npages)[: B * per].reshape(B, per).astype(np.int32)
    kp = torch.randn((npages, Hkv, P, D), device=DEV).to(k.dtype)
    vp = torch.randn((npages, Hkv, P, D), device=DEV).to(v.dtype)
    for b in range(B):
        for i in range(per):
            n = min(P, N - i * P)
            kp[ids[b, i], :, :n] = k[b, :, i * P: i * P + n]
            vp[ids[b, i], :, :n] = v[b, :, i * P: i * P + n]
    return kp, vp, torch.as_tensor(ids, device=DEV)


def _lens(B, N, seed, must=()):
    rng = np.random.default_rng(seed)
    L = rng.integers(1, N + 1, B)
    for i, x in enumerate(must):
        L[i] = x
    return L.astype(np.int32)


def _check_varlen(w, q, k, v, lens, pct, label, P=None):
    kas = _kas()
    B, Hkv = w.batch, w.n_kv_heads
    tl = torch.as_tensor(lens, device=DEV)
    _say(f"[decode varlen{' paged P=%d' % P if P else ''}] {label}: lens={lens.tolist()} pct={pct}")
    idx, o = kas.decode_anchor(q, k, v, pct, seq_lens=tl)
    o_dense = kas.decode_dense(q, k, v, seq_lens=tl)
    q2 = torch.flip(q, dims=[1]).contiguous()                 # a reuse layer: other queries, same cache
    hm = np.random.default_rng(3).integers(0, Hkv, Hkv).astype(np.int32)
    o_reuse = kas.decode_reuse(q2, k, v, idx, torch.as_tensor(hm, device=DEV), pct, seq_lens=tl)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    qn, kn, vn = _np(q), _np(k), _np(v)
    q2n = _np(q2)
    tol = TOL[w.dtype]
    worst = [0.0, 0.0, 0.0]
    swaps = 0
    for b in range(B):
        n = int(lens[b])
        kk = oracle.decode_k(n, pct)
        sl = (slice(b, b + 1), slice(None), slice(0, n))
        oidx, oo, pooled = oracle.decode_anchor(qn[b:b + 1], kn[sl], vn[sl], pct, want_pooled=True)
        for g in range(Hkv):
            swaps += assert_index_set(gi[b, g, :kk], oidx[0, g], pooled[0, g], kk, where=f"{label} b{b} g{g}")
        own = gi[b:b + 1, :, :kk]
        o_same = oracle.decode_reuse(qn[b:b + 1], kn[sl], vn[sl], own, np.arange(Hkv, dtype=np.int32))
        worst[0] = max(worst[0], max_abs(_np(o[b:b + 1]), o_same), max_abs(_np(o[b:b + 1]), oo))
        ref_r = oracle.decode_reuse(q2n[b:b + 1], kn[sl], vn[sl], own, hm)
        worst[1] = max(worst[1], max_abs(_np(o_reuse[b:b + 1]), ref_r))
        ref_d = oracle.dense_attention(qn[b:b + 1, :, None, :], kn[sl], vn[sl], causal=False)[:, :, 0, :]
        worst[2] = max(worst[2], max_abs(_np(o_dense[b:b + 1]), ref_d))
    _say(f"    near-tie swaps={swaps} max|o-o_oracle| anchor={worst[0]:.3g} reuse={worst[1]:.3g} "
         f"dense={worst[2]:.3g} tol={tol}")
    assert max(worst) <= tol
    if P is None:
        return idx, o, o_reuse, o_dense
    # the same calls on a paged copy of the cache
    kp, vp, bt = _paged(k, v, P, seed=P + B)
    idx_p, o_p = kas.decode_anchor(q, kp, vp, pct, seq_lens=tl, block_table=bt, seq_len=w.seq_len)
    od_p = kas.decode_dense(q, kp, vp, seq_lens=tl, block_table=bt, seq_len=w.seq_len)
    or_p = kas.decode_reuse(q2, kp, vp, idx, torch.as_tensor(hm, device=DEV), pct, seq_lens=tl,
                            block_table=bt, seq_len=w.seq_len)
    torch.cuda.synchronize()
    for b in range(B):
        kk = oracle.decode_k(int(lens[b]), pct)
        assert torch.equal(idx_p[b, :, :kk], idx[b, :, :kk]), f"paged index sets differ (b{b})"
    assert torch.equal(or_p, o_reuse), "paged reuse differs from the contiguous cache"
    assert torch.equal(od_p, o_dense), "paged dense differs from the contiguous cache"
    err = max_abs(_np(o_p), _np(o))
    _say(f"    paged: sets, reuse and dense bit-identical; anchor output vs contiguous {err:.3g}")
    assert err <= tol
    return idx, o, o_reuse, o_dense


VARLEN = [
    # (label, B, Hq, Hkv, D, N, dtype, pct, forced lengths, page size)
    ("bf16_d128_g4", 4, 32, 8, 128, 5037, "bf16", 10, (5037, 1, 16), 64),
    ("bf16_d64_g1", 3, 4, 4, 64, 3001, "bf16", 10, (17,), 16),
    ("f16_d128_g8", 2, 16, 2, 128, 4099, "f16", 25, (4099,), 1024),
    ("f32_d64_g4", 3, 8, 2, 64, 2048, "f32", 10, (2048, 300), None),
    ("bf16_many_splits", 2, 8, 2, 128, 40000, "bf16", 50, (40000, 23457), 32),
]


@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
def test_decode_varlen_and_paged(case):
    label, B, Hq, Hkv, D, N, dt, pct, must, P = case
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    _check_varlen(w, q, k, v, _lens(B, N, 5, must), pct, label, P)


def test_decode_paged_full_length_equals_dense_cache():
    """All sequences full length: the paged calls give the contiguous calls' results."""
    kas = _kas()
    w = inputgen.custom("decode", 2, 8, 2, 128, 3000, "bf16", wid=55)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    idx, o = kas.decode_anchor(q, k, v, 10)
    kp, vp, bt = _paged(k, v, 128, seed=9)
    idx_p, o_p = kas.decode_anchor(q, kp, vp, 10, block_table=bt, seq_len=3000)
    od = kas.decode_dense(q, k, v)
    od_p = kas.decode_dense(q, kp, vp, block_table=bt, seq_len=3000)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_p)
    assert torch.equal(od, od_p)
    assert max_abs(_np(o), _np(o_p)) <= TOL["bf16"]


def test_decode_varlen_paged_full_size():
    w = inputgen.WORKLOADS["llama8b_decode_128k"]
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    lens = np.array([131072, 100000, 65536, 4097], np.int32)
    _check_varlen(w, q, k, v, lens, w.topk_pct, w.name, P=256)


# ---------------------------------------------------------------- varlen prefill

def _check_prefill_varlen(w, q, k, v, lens, pct, label, tiles=None):
    kas = _kas()
    B, Hkv = w.batch, w.n_kv_heads
    tl = torch.as_tensor(lens, device=DEV)
    _say(f"[prefill varlen] {label}: lens={lens.tolist()} pct={pct}")
    idx, o = kas.prefill_anchor(q, k, v, pct, seq_lens=tl)
    hm = np.random.default_rng(2).integers(0, Hkv, Hkv).astype(np.int32)
    q2 = torch.flip(q, dims=[1]).contiguous()
    o_r = kas.prefill_reuse(q2, k, v, idx, torch.as_tensor(hm, device=DEV), pct, seq_lens=tl)
    o_d = kas.prefill_dense(q, k, v, seq_lens=tl)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    tol = TOL[w.dtype]
    worst = [0.0, 0.0, 0.0]
    swaps = 0
    for b in range(B):
        n = int(lens[b])
        T = n // 32
        off = oracle.prefill_offsets(n, 32, pct)
        kb, vb = _np(k[b:b + 1, :, :n]), _np(v[b:b + 1, :, :n])
        for t in (range(T) if tiles is None else [x for x in tiles if x < T]):
            qr = _np(q[b:b + 1, :, 32 * t: 32 * t + 32])
            oidx, oo = oracle.prefill_anchor(qr, kb, vb, pct, t0=t, t1=t + 1)
            for g in range(Hkv):
                gs = gi[b, g, off[t]:off[t + 1]]
                if not np.array_equal(gs, oidx[0, g]):
                    P = oracle.prefill_pooled(qr, kb, 0, t, g, t0=t, t1=t + 1)[: 32 * t]
                    swaps += assert_index_set(gs, oidx[0, g], P, int(off[t + 1] - off[t]), where=f"{label} b{b} t{t}")
            worst[0] = max(worst[0], max_abs(_np(o[b:b + 1, :, 32 * t: 32 * t + 32]), oo))
            q2r = _np(q2[b:b + 1, :, 32 * t: 32 * t + 32])
            own = np.ascontiguousarray(gi[b:b + 1, :, : off[-1]])   # this sequence's tiles' sets
            ref = oracle.prefill_reuse(q2r, kb, vb, own, hm, pct, t0=t, t1=t + 1)
            worst[1] = max(worst[1], max_abs(_np(o_r[b:b + 1, :, 32 * t: 32 * t + 32]), ref))
            refd = oracle.dense_attention(qr, _np(k[b:b + 1, :, :32 * t + 32]), _np(v[b:b + 1, :, :32 * t + 32]),
                                          causal=True)
            worst[2] = max(worst[2], max_abs(_np(o_d[b:b + 1, :, 32 * t: 32 * t + 32]), refd))
    _say(f"    near-tie swaps={swaps} max|o-o_oracle| anchor={worst[0]:.3g} reuse={worst[1]:.3g} "
         f"dense={worst[2]:.3g} tol={tol}")
    assert max(worst) <= tol
    return idx, o, o_r, o_d, q2, hm


def _check_prefill_paged(w, q, k, v, lens, pct, P, ref):
    """The prefill calls on a paged copy of the cache equal the contiguous ones
    (ref = their results) bit for bit on every tile inside the prompts. Block
    table entries of pages past a prompt's last whole tile hold ids far out of
    range: the calls must not need them."""
    kas = _kas()
    idx, o, o_r, o_d, q2, hm = ref
    B, Hkv = w.batch, w.n_kv_heads
    kp, vp, bt = _paged(k, v, P, seed=P + 7 * B)
    tl = None if lens is None else torch.as_tensor(lens, device=DEV)
    tiles = [w.seq_len // 32] * B if lens is None else [max(int(n), 32) // 32 for n in lens]
    for b in range(B):
        bt[b, (32 * tiles[b] + P - 1) // P:] = 1 << 30
    _say(f"[prefill paged P={P}] {w.name}: lens={None if lens is None else lens.tolist()} "
         f"pool={tuple(kp.shape)}")
    idx_p, o_p = kas.prefill_anchor(q, kp, vp, pct, seq_lens=tl, block_table=bt)
    or_p = kas.prefill_reuse(q2, kp, vp, idx, torch.as_tensor(hm, device=DEV), pct, seq_lens=tl, block_table=bt)
    od_p = kas.prefill_dense(q, kp, vp, seq_lens=tl, block_table=bt)
    # a head map per query head (each query head reads its KV head's rows)
    qm = torch.as_tensor(np.repeat(hm, w.n_q_heads // Hkv), device=DEV)
    oq = kas.prefill_reuse(q2, k, v, idx, qm, pct, query_head_map=True, seq_lens=tl)
    oq_p = kas.prefill_reuse(q2, kp, vp, idx, qm, pct, query_head_map=True, seq_lens=tl, block_table=bt)
    torch.cuda.synchronize()
    off = oracle.prefill_offsets(w.seq_len, 32, pct)
    for b in range(B):
        rows, sets = 32 * tiles[b], int(off[tiles[b]])
        assert torch.equal(idx_p[b, :, :sets], idx[b, :, :sets]), f"paged index sets differ (b{b})"
        for name, x, y in (("anchor", o_p, o), ("reuse", or_p, o_r), ("dense", od_p, o_d),
                           ("reuse, query-head map", oq_p, oq)):
            assert torch.equal(x[b, :, :rows], y[b, :, :rows]), f"paged {name} output differs (b{b})"
    _say("    paged: sets, anchor, reuse (both map kinds) and dense outputs bit-identical to the contiguous cache")


PREFILL_VARLEN = [
    # (label, B, Hq, Hkv, D, N, dtype, pct, lens)
    ("bf16_d128_g4", 3, 8, 2, 128, 640, "bf16", 10, (640, 96, 32)),
    ("f16_d64_g2", 2, 4, 2, 64, 1184, "f16", 25, (1184, 608)),
    ("bf16_d128_g8_anchor_pairs", 2, 16, 2, 128, 384, "bf16", 10, (352, 64)),
]


@pytest.mark.parametrize("case", PREFILL_VARLEN, ids=[c[0] for c in PREFILL_VARLEN])
def test_prefill_varlen(case):
    label, B, Hq, Hkv, D, N, dt, pct, lens = case
    w = inputgen.custom("prefill", B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    _check_prefill_varlen(w, q, k, v, np.array(lens, np.int32), pct, label)


PREFILL_PAGED = [
    # (label, B, Hq, Hkv, D, N, dtype, pct, lens or None, page size)
    ("bf16_d128_g4_P16_varlen", 3, 8, 2, 128, 640, "bf16", 10, (640, 96, 32), 16),
    ("f16_d64_g2_P64_varlen", 2, 4, 2, 64, 1184, "f16", 25, (1184, 608), 64),
    ("bf16_d128_g8_P32", 2, 16, 2, 128, 384, "bf16", 10, None, 32),
    ("bf16_d64_g1_P1024", 1, 4, 4, 64, 2080, "bf16", 10, None, 1024),
    ("f16_d128_g2_P128_varlen", 3, 8, 4, 128, 800, "f16", 20, (800, 33, 500), 128),
]


@pytest.mark.parametrize("case", PREFILL_PAGED, ids=[c[0] for c in PREFILL_PAGED])
def test_prefill_paged(case):
    """Paged prefill: every prompt against the oracle (through the contiguous
    calls) and the paged calls bit-identical to the contiguous ones."""
    label, B, Hq, Hkv, D, N, dt, pct, lens, P = case
    w = inputgen.custom("prefill", B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    L = np.array(lens if lens else [N] * B, np.int32)
    ref = _check_prefill_varlen(w, q, k, v, L, pct, label)
    if lens is None:      # full-length prompts: also the calls without lengths
        kas = _kas()
        idx, o = kas.prefill_anchor(q, k, v, pct)
        assert torch.equal(idx, ref[0]) and torch.equal(o, ref[1])
        ref = (idx, o, kas.prefill_reuse(ref[4], k, v, idx, torch.as_tensor(ref[5], device=DEV), pct),
               kas.prefill_dense(q, k, v), ref[4], ref[5])
    _check_prefill_paged(w, q, k, v, None if lens is None else L, pct, P, ref)


def test_prefill_varlen_full_size_sampled_tiles():
    import dataclasses
    w = dataclasses.replace(inputgen.WORKLOADS["qwen8b_prefill_32k"], batch=2)
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    lens = np.array([32768, 8192], np.int32)
    ref = _check_prefill_varlen(w, q, k, v, lens, w.topk_pct, w.name, tiles=(1, 37, 255, 500, 1023))
    _check_prefill_paged(w, q, k, v, lens, w.topk_pct, 256, ref)
