"""Pins of the CPU oracle to things other than itself (closed forms, library
routines on special cases, invariants, brute force, hand-worked examples).

The oracle follows the Kascade README (abstract: exact Top-k of post-softmax
scores in anchor layers, head-aware reuse, tile-level operations) and the
textbook attention definition from the I/O-complexity-of-attention abstract.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import inputgen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def _sdpa(q, k, v, causal, mask=None):
    """torch's scaled_dot_product_attention on CPU in float64, GQA by repeating KV heads."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64))
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64))
    G = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(G, dim=1)
    vt = vt.repeat_interleave(G, dim=1)
    if mask is not None:
        return torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=torch.from_numpy(mask)).numpy()
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal).numpy()


# ---------------------------------------------------------------- k rule

def test_k_rule_golden():
    g = json.load(open(os.path.join(GOLDEN, "k_rule.json")))
    for row in g["decode"]:
        assert oracle.decode_k(row["n"], row["pct"]) == row["k"], row
    for row in g["prefill_offsets"]:
        off = oracle.prefill_offsets(row["n"], row["tile"], row["pct"])
        assert off.tolist() == row["offsets"], row


# ---------------------------------------------------------------- dense

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 4, 2, 7, 7, 16), (2, 6, 3, 1, 33, 8), (1, 8, 2, 40, 40, 64)])
def test_dense_matches_torch_sdpa(shape, causal):
    B, Hq, Hkv, Nq, Nk, D = shape
    if causal and Nq != Nk and Nq != 1:
        pytest.skip("causal alignment only defined for Nq == Nk here")
    q, k, v = _rand((B, Hq, Nq, D), 1), _rand((B, Hkv, Nk, D), 2), _rand((B, Hkv, Nk, D), 3)
    o = oracle.dense_attention(q, k, v, causal=causal)
    ref = _sdpa(q, k, v, causal and Nq == Nk)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_dense_equal_keys_is_mean_of_visible_values():
    # identical keys -> uniform weights -> prefix means (closed form)
    B, Hq, Hkv, N, D = 1, 2, 1, 9, 4
    q = _rand((B, Hq, N, D), 4)
    k = np.repeat(_rand((B, Hkv, 1, D), 5), N, axis=2)
    v = _rand((B, Hkv, N, D), 6)
    o = oracle.dense_attention(q, k, v, causal=True)
    for i in range(N):
        np.testing.assert_allclose(o[0, :, i], np.broadcast_to(v[0, 0, : i + 1].astype(np.float64).mean(0), (Hq, D)),
                                   rtol=0, atol=1e-12)


# ---------------------------------------------------------------- decode

def _decode_case(B=2, Hq=8, Hkv=2, N=300, D=32, seed=0):
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, "f32", wid=seed, n_heavy=8)
    q, k, v = inputgen.layer_inputs(w, 0)
    return q.numpy(), k.numpy(), v.numpy()


def test_decode_worked_example():
    """Hand-worked: D=1, keys ln1..ln4, two heads q=+1/-1, 50 % -> k=2.

    head 0 softmax = [1,2,3,4]/10; head 1 softmax = [12,6,4,3]/25;
    pooled = [0.58, 0.44, 0.46, 0.52] -> set {0, 3};
    V = [1,2,3,4] -> head 0: (0.1*1 + 0.4*4)/0.5 = 3.4; head 1: (12*1+3*4)/15 = 1.6.
    """
    q = np.array([[[1.0], [-1.0]]], dtype=np.float32)           # [1, 2, 1]
    k = np.log(np.arange(1, 5, dtype=np.float64)).astype(np.float32).reshape(1, 1, 4, 1)
    v = np.arange(1, 5, dtype=np.float32).reshape(1, 1, 4, 1)
    idx, o, pooled = oracle.decode_anchor(q, k, v, pct=50, want_pooled=True)
    assert idx.tolist() == [[[0, 3]]]
    np.testing.assert_allclose(pooled[0, 0], [0.58, 0.44, 0.46, 0.52], rtol=1e-6)
    np.testing.assert_allclose(o[0, :, 0], [3.4, 1.6], rtol=1e-6)
    # dense outputs for reference: head 0 = 3.0, head 1 = (12+12+12+12)/25 = 1.92
    od = oracle.dense_attention(q[:, :, None, :], k, v, causal=False)
    np.testing.assert_allclose(od[0, :, 0, 0], [3.0, 1.92], rtol=1e-6)


def test_decode_full_k_equals_dense():
    q, k, v = _decode_case()
    idx, o, _ = oracle.decode_anchor(q, k, v, pct=100)
    N = k.shape[2]
    assert (idx == np.arange(N)).all()
    ref = _sdpa(q[:, :, None, :], k, v, causal=False)[:, :, 0]
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_decode_pooled_mass_and_single_head_softmax():
    q, k, v = _decode_case()
    B, Hq, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    G = Hq // Hkv
    _, _, P = oracle.decode_anchor(q, k, v, pct=10, want_pooled=True)
    np.testing.assert_allclose(P.sum(-1), np.full((B, Hkv), float(G)), rtol=1e-12)
    # G = 1: pooled score is exactly the head's softmax (torch, float64)
    q1 = q[:, :Hkv].copy()
    _, _, P1 = oracle.decode_anchor(q1, k, v, pct=10, want_pooled=True)
    logits = torch.einsum("bhd,bhnd->bhn", torch.from_numpy(q1).double(), torch.from_numpy(k).double())
    ref = torch.softmax(logits / math.sqrt(D), dim=-1).numpy()
    np.testing.assert_allclose(P1, ref, rtol=1e-12, atol=1e-15)
    # identical heads inside a group: pooled = G * that head's softmax
    qg = np.repeat(q1, G, axis=1)
    _, _, Pg = oracle.decode_anchor(qg, k, v, pct=10, want_pooled=True)
    np.testing.assert_allclose(Pg, G * ref, rtol=1e-12, atol=1e-15)


def _assert_topk_property(P, S, k):
    """S is the exact Top-k of P (compared in float32) with lowest-index ties."""
    S = np.asarray(S)
    assert len(S) == k and (np.diff(S) > 0).all()
    Pf = P.astype(np.float32)
    chosen = np.zeros(len(P), dtype=bool)
    chosen[S] = True
    if k == 0 or chosen.all():
        return
    worst_in = Pf[chosen].min()
    best_out = Pf[~chosen].max()
    assert worst_in >= best_out
    if worst_in == best_out:
        tie_in = np.flatnonzero(chosen & (Pf == worst_in))
        tie_out = np.flatnonzero(~chosen & (Pf == worst_in))
        assert tie_in.max() < tie_out.min()


def test_decode_selection_is_topk_with_low_index_ties():
    q, k, v = _decode_case(N=517)
    # plant exact ties: copy one heavy row to several positions
    k[:, :, 100:110] = k[:, :, 5:6]
    idx, _, P = oracle.decode_anchor(q, k, v, pct=10, want_pooled=True)
    kk = oracle.decode_k(517, 10)
    for b in range(q.shape[0]):
        for g in range(k.shape[1]):
            _assert_topk_property(P[b, g], idx[b, g], kk)


def test_decode_tie_break_cuts_through_tie_group():
    # 6 keys; key 0 largest, keys 1..5 identical -> k=3 must pick {0,1,2}
    D = 4
    q = np.ones((1, 1, D), np.float32)
    k = np.zeros((1, 1, 6, D), np.float32)
    k[0, 0, 0] = 1.0
    v = np.arange(6 * D, dtype=np.float32).reshape(1, 1, 6, D)
    idx, _, _ = oracle.decode_anchor(q, k, v, pct=50)
    assert idx.tolist() == [[[0, 1, 2]]]


def test_decode_selection_brute_force_tiny():
    # exhaustive search over all k-subsets for the max pooled mass
    rng = np.random.default_rng(7)
    for trial in range(5):
        N, D, G = 11, 4, 3
        q = rng.standard_normal((1, G, D)).astype(np.float32)
        k = rng.standard_normal((1, 1, N, D)).astype(np.float32)
        v = rng.standard_normal((1, 1, N, D)).astype(np.float32)
        pct = 30
        kk = oracle.decode_k(N, pct)
        idx, _, P = oracle.decode_anchor(q, k, v, pct=pct, want_pooled=True)
        best = max(itertools.combinations(range(N), kk), key=lambda s: sum(P[0, 0, list(s)]))
        assert sorted(best) == idx[0, 0].tolist()


def test_decode_reuse_matches_sdpa_over_gathered_keys():
    q, k, v = _decode_case(B=2, Hq=8, Hkv=4, N=200)
    rng = np.random.default_rng(3)
    kk = 17
    anchor = np.sort(np.stack([np.stack([rng.choice(200, kk, replace=False) for _ in range(3)])
                               for _ in range(2)]), axis=-1).astype(np.int32)   # Hkv_a = 3
    head_map = np.array([2, 0, 0, 1], np.int32)
    o = oracle.decode_reuse(q, k, v, anchor, head_map)
    G = 2
    for b in range(2):
        for h in range(8):
            g = h // G
            S = anchor[b, head_map[g]]
            ref = _sdpa(q[b:b + 1, h:h + 1, None, :], k[b:b + 1, g:g + 1, S], v[b:b + 1, g:g + 1, S], False)
            np.testing.assert_allclose(o[b, h], ref[0, 0, 0], rtol=0, atol=1e-12)


def test_decode_identity_reuse_reproduces_anchor():
    q, k, v = _decode_case()
    idx, o_anchor, _ = oracle.decode_anchor(q, k, v, pct=10)
    o_reuse = oracle.decode_reuse(q, k, v, idx, np.arange(k.shape[1], dtype=np.int32))
    np.testing.assert_allclose(o_reuse, o_anchor, rtol=0, atol=1e-13)


def test_decode_head_map_permutation_invariance():
    q, k, v = _decode_case(B=1, Hq=8, Hkv=4, N=256)
    idx, _, _ = oracle.decode_anchor(q, k, v, pct=10)
    head_map = np.array([3, 3, 1, 0], np.int32)
    o = oracle.decode_reuse(q, k, v, idx, head_map)
    perm = np.array([2, 0, 3, 1])                      # anchor head a lands at slot inv[a]
    inv = np.argsort(perm)
    idx_p = idx[:, perm]
    o_p = oracle.decode_reuse(q, k, v, idx_p, inv[head_map].astype(np.int32))
    np.testing.assert_array_equal(o, o_p)


# ---------------------------------------------------------------- prefill

def _prefill_case(B=1, Hq=4, Hkv=2, N=160, D=16, seed=0):
    w = inputgen.custom("prefill", B, Hq, Hkv, D, N, "f32", wid=seed, n_heavy=4)
    q, k, v = inputgen.layer_inputs(w, 0)
    return q.numpy(), k.numpy(), v.numpy()


def test_prefill_worked_example():
    """Hand-worked: D=1, q=1, all keys 0 except key 5 = ln 2 (weight 2), V_j = j.

    Tile 1 pooled score of key j<32: H = sum_{i=32..63} 1/(i+1) * w_j with
    w_5 = 2 -> key 5 first, then exact ties among the others -> lowest indices
    {0, 1}. Row i of tile 1 attends over {0,1,5} + [32, i]:
        o_i = (0 + 1 + 2*5 + sum_{j=32..i} j) / (1 + 1 + 2 + (i-31)).
    Tile 0 row i is dense causal: o_i = (sum_{j<=i} j + [i>=5]*5) / (i + 1 + [i>=5]).
    """
    N = 64
    q = np.ones((1, 1, N, 1), np.float32)
    k = np.zeros((1, 1, N, 1), np.float32)
    k[0, 0, 5, 0] = np.float32(math.log(2.0))
    v = np.arange(N, dtype=np.float32).reshape(1, 1, N, 1)
    idx, o = oracle.prefill_anchor(q, k, v, pct=10)
    assert idx.tolist() == [[[0, 1, 5]]]
    exp_o = []
    for i in range(N):
        if i < 32:
            extra = 1 if i >= 5 else 0
            exp_o.append((i * (i + 1) / 2 + 5 * extra) / (i + 1 + extra))
        else:
            exp_o.append((0 + 1 + 10 + sum(range(32, i + 1))) / (4 + (i - 31)))
    np.testing.assert_allclose(o[0, 0, :, 0], exp_o, rtol=1e-6)
    P = oracle.prefill_pooled(q, k, 0, 1, 0)
    H = sum(1.0 / (i + 2) for i in range(32, 64))   # row i: l_i = (i+1) - 1 + 2
    np.testing.assert_allclose(P[5], 2 * H, rtol=1e-6)
    np.testing.assert_allclose(P[[0, 31]], [H, H], rtol=1e-6)


def test_prefill_full_k_equals_causal_dense():
    q, k, v = _prefill_case(N=128 + 17)   # ragged last tile
    _, o = oracle.prefill_anchor(q, k, v, pct=100)
    ref = _sdpa(q, k, v, causal=True)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_prefill_tile0_is_dense_and_sets_precede_tile():
    q, k, v = _prefill_case(N=160)
    idx, o = oracle.prefill_anchor(q, k, v, pct=10)
    ref = _sdpa(q, k, v, causal=True)
    np.testing.assert_allclose(o[:, :, :32], ref[:, :, :32], rtol=0, atol=1e-12)
    off = oracle.prefill_offsets(160, 32, 10)
    for t in range(1, 5):
        seg = idx[..., off[t]:off[t + 1]]
        assert (seg >= 0).all() and (seg < 32 * t).all()
        assert (np.diff(seg, axis=-1) > 0).all()


def test_prefill_pooled_mass_and_single_head_softmax():
    q, k, v = _prefill_case(B=1, Hq=2, Hkv=2, N=96 + 5)
    D = q.shape[-1]
    for t in range(4):
        rows = min(101, 32 * (t + 1)) - 32 * t
        for g in range(2):
            P = oracle.prefill_pooled(q, k, 0, t, g)
            np.testing.assert_allclose(P.sum(), rows * 1.0, rtol=1e-12)    # G = 1
            # torch: masked softmax of each row, summed over the tile's rows
            qt = torch.from_numpy(q[0, g, 32 * t: 32 * t + rows]).double()
            kt = torch.from_numpy(k[0, g, : 32 * t + rows]).double()
            s = qt @ kt.T / math.sqrt(D)
            mask = torch.arange(32 * t + rows)[None, :] > torch.arange(32 * t, 32 * t + rows)[:, None]
            s = s.masked_fill(mask, float("-inf"))
            ref = torch.softmax(s, dim=-1).sum(0).numpy()
            np.testing.assert_allclose(P, ref, rtol=1e-12, atol=1e-15)


def test_prefill_pooled_group_mass():
    q, k, v = _prefill_case(B=1, Hq=8, Hkv=2, N=128)
    for t in (1, 3):
        P = oracle.prefill_pooled(q, k, 0, t, 1)
        np.testing.assert_allclose(P.sum(), 32 * 4, rtol=1e-12)


def _torch_tile_pooled(q, k, b, t, heads, op, tile=32):
    """Pooled scores of tile t from torch (float64): each query head's causal
    softmax, with query head h reading KV head h // G (the KV heads expanded by
    repeat_interleave, as Hugging Face's repeat_kv does), then summed (op 0) or
    maxed (op 1) over the tile's rows and the given heads."""
    D, N = q.shape[-1], k.shape[2]
    G = q.shape[1] // k.shape[1]
    kx = torch.from_numpy(k).double().repeat_interleave(G, dim=1)
    i0, i1 = tile * t, min(N, tile * (t + 1))
    rows = torch.arange(i0, i1)
    mask = torch.arange(i1)[None, :] > rows[:, None]
    acc = None
    for h in heads:
        s = torch.from_numpy(q[b, h, i0:i1]).double() @ kx[b, h, :i1].T / math.sqrt(D)
        p = torch.softmax(s.masked_fill(mask, float("-inf")), dim=-1)
        p = p.max(0).values if op else p.sum(0)
        acc = p if acc is None else (torch.maximum(acc, p) if op else acc + p)
    return acc.numpy()


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 4), (6, 3)])
def test_prefill_pooled_grouped_heads_match_torch(Hq, Hkv):
    """Pooling across several KV heads with G > 1: KV head g pools query heads
    g*G .. g*G + G - 1 (consecutive heads share a KV head), over every row of
    the tile, for both scopes and both operators; the sets are the stable Top-k
    of the torch-pooled scores, compared in float32."""
    N, B = 101, 2
    q, k, v = _prefill_case(B=B, Hq=Hq, Hkv=Hkv, N=N, seed=31 + Hkv)
    G = Hq // Hkv
    T = (N + 31) // 32
    off = oracle.prefill_offsets(N, 32, 25)
    for scope, op in itertools.product((0, 1), (0, 1)):
        groups = [list(range(Hq))] if scope else [list(range(g * G, g * G + G)) for g in range(Hkv)]
        idx, _ = oracle.prefill_anchor(q, k, v, pct=25, pool_scope=scope, pool_op=op)
        for b in range(B):
            for t in range(T):
                for s, heads in enumerate(groups):
                    ref = _torch_tile_pooled(q, k, b, t, heads, op)
                    P = oracle.prefill_pooled(q, k, b, t, s, pool_scope=scope, pool_op=op)
                    np.testing.assert_allclose(P, ref, rtol=1e-12, atol=1e-15,
                                               err_msg=f"scope {scope} op {op} b {b} t {t} set {s}")
                    kt = int(off[t + 1] - off[t])
                    cand = ref[: 32 * t]
                    order = sorted(range(32 * t), key=lambda j: (-np.float32(cand[j]), j))
                    assert idx[b, s, off[t]:off[t + 1]].tolist() == sorted(order[:kt]), (scope, op, b, t, s)


def test_prefill_selection_is_topk():
    q, k, v = _prefill_case(B=2, Hq=4, Hkv=2, N=192)
    k[:, :, 40:48] = k[:, :, 7:8]       # exact ties among candidates
    idx, _ = oracle.prefill_anchor(q, k, v, pct=10)
    off = oracle.prefill_offsets(192, 32, 10)
    for b in range(2):
        for g in range(2):
            for t in range(1, 6):
                P = oracle.prefill_pooled(q, k, b, t, g)[: 32 * t]
                _assert_topk_property(P, idx[b, g, off[t]:off[t + 1]], off[t + 1] - off[t])


def test_prefill_reuse_matches_sdpa_with_mask():
    q, k, v = _prefill_case(B=1, Hq=4, Hkv=2, N=128)
    rng = np.random.default_rng(5)
    off = oracle.prefill_offsets(128, 32, 25)
    Hkv_a = 3
    anchor = np.zeros((1, Hkv_a, off[-1]), np.int32)
    for a in range(Hkv_a):
        for t in range(4):
            kt = off[t + 1] - off[t]
            anchor[0, a, off[t]:off[t + 1]] = np.sort(rng.choice(32 * t, kt, replace=False)) if kt else []
    head_map = np.array([2, 0], np.int32)
    o = oracle.prefill_reuse(q, k, v, anchor, head_map, pct=25)
    G = 2
    for h in range(4):
        g = h // G
        for t in range(4):
            S = anchor[0, head_map[g], off[t]:off[t + 1]]
            keys = np.concatenate([S, np.arange(32 * t, 32 * t + 32)])
            mask = np.zeros((32, len(keys)), bool)
            mask[:, : len(S)] = True
            mask[:, len(S):] = np.tril(np.ones((32, 32), bool))
            ref = _sdpa(q[:, h:h + 1, 32 * t:32 * t + 32], k[:, g:g + 1, keys], v[:, g:g + 1, keys],
                        False, mask=mask)
            np.testing.assert_allclose(o[0, h, 32 * t:32 * t + 32], ref[0, 0], rtol=0, atol=1e-12)


def test_prefill_identity_reuse_reproduces_anchor():
    q, k, v = _prefill_case(B=1, Hq=4, Hkv=2, N=160)
    idx, o_a = oracle.prefill_anchor(q, k, v, pct=10)
    o_r = oracle.prefill_reuse(q, k, v, idx, np.arange(2, dtype=np.int32), pct=10)
    np.testing.assert_allclose(o_r, o_a, rtol=0, atol=1e-13)


def test_prefill_tile_range_matches_full():
    q, k, v = _prefill_case(B=1, Hq=4, Hkv=2, N=192)
    idx, o = oracle.prefill_anchor(q, k, v, pct=10)
    off = oracle.prefill_offsets(192, 32, 10)
    idx_r, o_r = oracle.prefill_anchor(q[:, :, 64:128], k, v, pct=10, t0=2, t1=4)
    np.testing.assert_array_equal(idx_r, idx[..., off[2]:off[4]])
    np.testing.assert_array_equal(o_r, o[:, :, 64:128])


# ---------------------------------------------------------------- pooling variants
# Pooling scope (the README's strategies: post-softmax pooling per KV-head
# group, or over all heads) and operator (sum, or max-pooling).

def _two_head_logits():
    """Probabilities of three live keys for two heads, chosen so that sum and
    max pooling disagree: A = [0.6, 0.35, 0.05], B = [~0, 0.45, 0.55].
    sum = [0.6, 0.8, 0.6] -> key 1 first; max = [0.6, 0.45, 0.55] -> key 0."""
    pa = np.log([0.6, 0.35, 0.05])
    pb = np.array([-40.0, math.log(0.45), math.log(0.55)])   # e^-40 / (1 + e^-40) ~ 4e-18
    return pa, pb


def test_decode_pool_variants_worked_example():
    pa, pb = _two_head_logits()      # rounded to float32 on input: values to ~1e-7
    D = 3
    k1 = np.eye(3, dtype=np.float32).reshape(1, 1, 3, 3)               # key j = e_j
    v1 = (np.arange(1, 4, dtype=np.float32)[:, None] * np.array([1, 10, 100], np.float32)).reshape(1, 1, 3, 3)
    q = (np.stack([pa, pb]) * math.sqrt(D)).astype(np.float32)[None]   # logits = q . e_j / sqrt(3)
    # one KV head with both query heads: group scope = all heads scope
    for scope in (0, 1):
        idx, o, P = oracle.decode_anchor(q, k1, v1, pct=33, want_pooled=True, pool_scope=scope)
        assert idx.tolist() == [[[1]]]
        np.testing.assert_allclose(P[0, 0], [0.6, 0.8, 0.6], rtol=1e-6)
        np.testing.assert_allclose(o[0, :], np.repeat(v1[0, 0, 1][None], 2, 0), rtol=1e-6)
        idx, o, P = oracle.decode_anchor(q, k1, v1, pct=33, want_pooled=True, pool_scope=scope, pool_op=1)
        assert idx.tolist() == [[[0]]]
        np.testing.assert_allclose(P[0, 0], [0.6, 0.45, 0.55], rtol=1e-6)
        np.testing.assert_allclose(o[0, :], np.repeat(v1[0, 0, 0][None], 2, 0), rtol=1e-6)
    # two KV heads with one query head each: per-head sets differ from the shared one
    k2 = np.repeat(k1, 2, axis=1)
    v2 = np.concatenate([v1, 2 * v1], axis=1)
    idx, o, _ = oracle.decode_anchor(q, k2, v2, pct=33)
    assert idx.tolist() == [[[0], [2]]]
    np.testing.assert_allclose(o[0], [v2[0, 0, 0], v2[0, 1, 2]], rtol=1e-6)
    idx, o, P = oracle.decode_anchor(q, k2, v2, pct=33, want_pooled=True, pool_scope=1)
    assert idx.tolist() == [[[1]]]
    np.testing.assert_allclose(P[0, 0], [0.6, 0.8, 0.6], rtol=1e-6)
    np.testing.assert_allclose(o[0], [v2[0, 0, 1], v2[0, 1, 1]], rtol=1e-6)
    idx, _, _ = oracle.decode_anchor(q, k2, v2, pct=33, pool_scope=1, pool_op=1)
    assert idx.tolist() == [[[0]]]


def test_decode_pool_variant_invariants():
    q, k, v = _decode_case(B=2, Hq=8, Hkv=2, N=257)
    Hq = q.shape[1]
    _, _, Pg = oracle.decode_anchor(q, k, v, pct=10, want_pooled=True)
    _, _, Pa = oracle.decode_anchor(q, k, v, pct=10, want_pooled=True, pool_scope=1)
    _, _, Pm = oracle.decode_anchor(q, k, v, pct=10, want_pooled=True, pool_scope=1, pool_op=1)
    _, _, Pgm = oracle.decode_anchor(q, k, v, pct=10, want_pooled=True, pool_op=1)
    assert Pa.shape == (2, 1, 257) and Pgm.shape == Pg.shape
    np.testing.assert_allclose(Pa.sum(-1), np.full((2, 1), float(Hq)), rtol=1e-12)
    # all-heads sum = sum of the group sums; max lies between sum / heads and sum
    np.testing.assert_allclose(Pa[:, 0], Pg.sum(1), rtol=1e-12)
    assert (Pm <= Pa * (1 + 1e-12)).all() and (Pm * Hq >= Pa * (1 - 1e-12)).all()
    assert (Pgm <= Pg * (1 + 1e-12)).all() and (Pgm * 4 >= Pg * (1 - 1e-12)).all()
    assert (Pm <= 1.0).all() and (Pm[:, 0] >= Pgm.max(1) * (1 - 1e-12)).all()


def test_decode_pool_variants_brute_force_tiny():
    """Softmax per head (torch, float64), pooled, then a full stable sort."""
    for seed, (Hq, Hkv, N) in enumerate([(4, 2, 40), (8, 4, 65), (2, 1, 33)]):
        q, k, v = _decode_case(B=1, Hq=Hq, Hkv=Hkv, N=N, seed=seed + 11)
        G = Hq // Hkv
        qt, kt = torch.from_numpy(q).double(), torch.from_numpy(k).double()
        kr = kt.repeat_interleave(G, dim=1)
        p = torch.softmax(torch.einsum("bhd,bhnd->bhn", qt, kr) / math.sqrt(q.shape[-1]), -1)[0].numpy()
        for scope, op in itertools.product((0, 1), (0, 1)):
            groups = [list(range(Hq))] if scope else [list(range(g * G, g * G + G)) for g in range(Hkv)]
            idx, _, _ = oracle.decode_anchor(q, k, v, pct=25, pool_scope=scope, pool_op=op)
            kk = oracle.decode_k(N, 25)
            for s, heads in enumerate(groups):
                P = p[heads].max(0) if op else p[heads].sum(0)
                order = sorted(range(N), key=lambda j: (-np.float32(P[j]), j))
                assert idx[0, s].tolist() == sorted(order[:kk]), (seed, scope, op, s)


def test_prefill_pool_variants_worked_example():
    """Tile 1 of a 64-row prompt (k_1 = 1 at 4 %): every row of both heads
    sees keys 0..2 with the probabilities of _two_head_logits; every other
    key gets logit -50. sum over rows and heads = 32 * [0.6, 0.8, 0.6] -> key
    1; max = [0.6, 0.45, 0.55] -> key 0."""
    pa, pb = _two_head_logits()
    N, D = 64, 4
    k = np.zeros((1, 1, N, D), np.float32)
    k[0, 0, :3, :3] = np.eye(3)
    k[0, 0, 3:, 3] = -1.0                               # dead keys
    q = np.zeros((1, 2, N, D), np.float32)
    q[0, 0, :, :3] = 2 * pa                             # scale 1/sqrt(4) = 1/2
    q[0, 1, :, :3] = 2 * pb
    q[0, :, :, 3] = 100.0                               # dead keys: logit -50
    v = np.arange(N * D, dtype=np.float32).reshape(1, 1, N, D)
    assert oracle.topk_count(32, 4) == 1
    for scope in (0, 1):
        idx, _ = oracle.prefill_anchor(q, k, v, pct=4, pool_scope=scope)
        assert idx.tolist() == [[[1]]]
        P = oracle.prefill_pooled(q, k, 0, 1, 0, pool_scope=scope)
        np.testing.assert_allclose(P[:3], [19.2, 25.6, 19.2], rtol=1e-6)
        idx, _ = oracle.prefill_anchor(q, k, v, pct=4, pool_scope=scope, pool_op=1)
        assert idx.tolist() == [[[0]]]
        P = oracle.prefill_pooled(q, k, 0, 1, 0, pool_scope=scope, pool_op=1)
        np.testing.assert_allclose(P[:3], [0.6, 0.45, 0.55], rtol=1e-6)
    # two KV heads, one query head each
    k2 = np.repeat(k, 2, axis=1)
    v2 = np.repeat(v, 2, axis=1)
    idx, _ = oracle.prefill_anchor(q, k2, v2, pct=4)
    assert idx.tolist() == [[[0], [2]]]
    idx, o = oracle.prefill_anchor(q, k2, v2, pct=4, pool_scope=1)
    assert idx.tolist() == [[[1]]]
    # row 40 of head 1 attends over {1} + [32, 40]: the dead keys vanish, only key 1 counts
    np.testing.assert_allclose(o[0, 1, 40], v2[0, 1, 1], rtol=1e-6)


def test_prefill_pool_variant_invariants():
    q, k, v = _prefill_case(B=1, Hq=8, Hkv=2, N=128)
    Hq = 8
    for t in range(4):
        Pa = oracle.prefill_pooled(q, k, 0, t, 0, pool_scope=1)
        Pg = sum(oracle.prefill_pooled(q, k, 0, t, g) for g in range(2))
        np.testing.assert_allclose(Pa.sum(), 32.0 * Hq, rtol=1e-12)
        np.testing.assert_allclose(Pa, Pg, rtol=1e-12, atol=1e-15)
        Pm = oracle.prefill_pooled(q, k, 0, t, 0, pool_scope=1, pool_op=1)
        assert (Pm <= Pa * (1 + 1e-12) + 1e-300).all()
        assert (Pm * 32 * Hq >= Pa * (1 - 1e-12)).all() and (Pm <= 1.0).all()
    # one KV head: all-heads scope is the group scope
    q1, k1, v1 = _prefill_case(B=1, Hq=4, Hkv=1, N=96, seed=3)
    for op in (0, 1):
        a = oracle.prefill_anchor(q1, k1, v1, pct=10, pool_op=op)
        b = oracle.prefill_anchor(q1, k1, v1, pct=10, pool_op=op, pool_scope=1)
        assert (a[0] == b[0]).all() and np.array_equal(a[1], b[1])


def test_prefill_shared_set_output_matches_reuse():
    """The all-heads anchor's output equals a reuse pass over its shared set."""
    q, k, v = _prefill_case(B=1, Hq=4, Hkv=2, N=128, seed=5)
    for op in (0, 1):
        idx, o = oracle.prefill_anchor(q, k, v, pct=10, pool_scope=1, pool_op=op)
        o2 = oracle.prefill_reuse(q, k, v, idx, np.zeros(2, np.int32), pct=10)
        np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- per-query-head maps

def test_query_head_map_worked_example():
    """Two query heads sharing one KV head read different single-key sets:
    each output is exactly that key's V row (a softmax over one key)."""
    q, k, v = _decode_case(B=1, Hq=2, Hkv=1, N=50, seed=9)
    sets = np.array([[[7], [31]]], np.int32)                 # anchor sets of 2 anchor KV heads
    o = oracle.decode_reuse(q, k, v, sets, np.array([1, 0], np.int32), query_head_map=True)
    np.testing.assert_allclose(o[0], [v[0, 0, 31], v[0, 0, 7]], rtol=0, atol=1e-15)
    # prefill: tile 1 rows of head 0 over {3} + diagonal, head 1 over {20} + diagonal
    qp, kp, vp = _prefill_case(B=1, Hq=2, Hkv=1, N=64, seed=9)
    off = oracle.prefill_offsets(64, 32, 4)                  # k_1 = 1
    psets = np.array([[[3], [20]]], np.int32)
    assert off[-1] == 1
    op = oracle.prefill_reuse(qp, kp, vp, psets, np.array([0, 1], np.int32), pct=4, query_head_map=True)
    for h, j in ((0, 3), (1, 20)):
        keys = [j] + list(range(32, 33))                     # row 32: set + diagonal key 32
        qd, kd, vd = (x.astype(np.float64) for x in (qp[0, h, 32], kp[0, 0], vp[0, 0]))
        s_ = np.array([qd @ kd[x] for x in keys]) / math.sqrt(qp.shape[-1])
        w_ = np.exp(s_ - s_.max())
        np.testing.assert_allclose(op[0, h, 32], (w_[:, None] * vd[keys]).sum(0) / w_.sum(), rtol=1e-12)


def test_query_head_map_reduces_to_kv_head_map():
    q, k, v = _decode_case(B=2, Hq=8, Hkv=2, N=300, seed=4)
    idx, _, _ = oracle.decode_anchor(q, k, v, pct=10)
    hm = np.array([1, 0], np.int32)
    a = oracle.decode_reuse(q, k, v, idx, hm)
    b = oracle.decode_reuse(q, k, v, idx, np.repeat(hm, 4), query_head_map=True)
    assert np.array_equal(a, b)
    qp, kp, vp = _prefill_case(B=1, Hq=4, Hkv=2, N=128, seed=4)
    pidx, _ = oracle.prefill_anchor(qp, kp, vp, pct=10)
    a = oracle.prefill_reuse(qp, kp, vp, pidx, hm, pct=10)
    b = oracle.prefill_reuse(qp, kp, vp, pidx, np.repeat(hm, 2), pct=10, query_head_map=True)
    assert np.array_equal(a, b)
    # a query head reading another head's set: its output is the KV-head-map
    # output of a layer whose map sends its KV head to that set
    qm = np.array([0, 1, 1, 1, 0, 0, 1, 0], np.int32)
    c = oracle.decode_reuse(q, k, v, idx, qm, query_head_map=True)
    for h in range(8):
        ref = oracle.decode_reuse(q, k, v, idx, np.full(2, qm[h], np.int32))
        np.testing.assert_array_equal(c[:, h], ref[:, h])


# ---------------------------------------------------------------- proposal-refined reuse

def test_refine_worked_example():
    """Pool {0, 1, 2} of 4 keys; key 3 (outside the pool) has a huge logit for
    head A, which must not enter the pool's softmax. Within the pool the heads'
    probabilities are A = [0.6, 0.35, 0.05], B = [~0, 0.45, 0.55]; summed,
    key 1 wins (kappa 1) and both heads then attend over key 1 alone."""
    pa, pb = _two_head_logits()
    D = 4
    k = np.zeros((1, 1, 4, D), np.float32)
    k[0, 0, :3, :3] = np.eye(3)
    k[0, 0, 3, 3] = 1.0
    q = np.zeros((1, 2, D), np.float32)
    q[0, 0, :3], q[0, 1, :3] = 2 * pa, 2 * pb          # scale 1/sqrt(4)
    q[0, 0, 3] = 60.0                                   # head A: key 3 dominates the full row
    v = np.arange(4 * D, dtype=np.float32).reshape(1, 1, 4, D)
    idx, o = oracle.decode_refine(q, k, v, np.array([[[0, 1, 2]]], np.int32), np.zeros(1, np.int32), 1)
    assert idx.tolist() == [[[1]]]
    np.testing.assert_allclose(o[0], np.repeat(v[0, 0, 1][None], 2, 0), rtol=0, atol=1e-12)


def test_refine_reduces_to_reuse_and_anchor():
    q, k, v = _decode_case(B=2, Hq=8, Hkv=2, N=300, seed=12)
    N = 300
    pool, _, _ = oracle.decode_anchor(q, k, v, pct=40)
    hm = np.array([1, 0], np.int32)
    n_pool = pool.shape[-1]
    # kappa = whole pool: the refined set is the pool, the output a reuse over it
    idx, o = oracle.decode_refine(q, k, v, pool, hm, n_pool)
    assert np.array_equal(idx, pool[:, hm])
    np.testing.assert_array_equal(o, oracle.decode_reuse(q, k, v, pool, hm))
    # pool = every key: the refined set is this layer's own anchor selection
    every = np.broadcast_to(np.arange(N, dtype=np.int32), (2, 2, N)).copy()
    kk = oracle.decode_k(N, 10)
    idx, o = oracle.decode_refine(q, k, v, every, np.arange(2, dtype=np.int32), kk)
    aidx, ao, _ = oracle.decode_anchor(q, k, v, pct=10)
    assert np.array_equal(idx, aidx)
    np.testing.assert_allclose(o, ao, rtol=0, atol=1e-14)


def test_refine_brute_force_tiny():
    for seed, (Hq, Hkv, N, pct_pool, kappa) in enumerate([(4, 2, 60, 50, 7), (8, 2, 97, 30, 5), (2, 1, 40, 75, 11)]):
        q, k, v = _decode_case(B=1, Hq=Hq, Hkv=Hkv, N=N, seed=seed + 31)
        G = Hq // Hkv
        pool, _, _ = oracle.decode_anchor(q, k, v, pct=pct_pool)
        hm = np.random.default_rng(seed).integers(0, Hkv, Hkv).astype(np.int32)
        idx, _ = oracle.decode_refine(q, k, v, pool, hm, kappa)
        qt, kt = torch.from_numpy(q).double(), torch.from_numpy(k).double()
        for g in range(Hkv):
            keys = pool[0, hm[g]]
            s = qt[0, g * G:(g + 1) * G] @ kt[0, g, keys].T / math.sqrt(q.shape[-1])
            P = torch.softmax(s, -1).sum(0).numpy()
            order = sorted(range(len(keys)), key=lambda a: (-np.float32(P[a]), a))
            assert idx[0, g].tolist() == sorted(keys[order[:kappa]].tolist()), (seed, g)
