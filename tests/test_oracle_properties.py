"""Property-based pins of the oracle (hypothesis, CPU): over random small
shapes, percentages and inputs, including inputs drawn from a handful of
values so that exact ties are common, what the oracle computes must agree
with definitions outside it:

- the pooled scores (Kascade README "Abstract": exact post-softmax scores,
  pooled over the query heads that share a KV head and, in prefill, over the
  rows of a query tile) against torch's softmax in float64, with the KV heads
  expanded by repeat_interleave (query head h on KV head h / G);
- the index sets against a brute-force stable sort of those scores rounded
  to float32 (larger first, ties to the lower key), the count from the
  published k rule;
- the outputs against torch's scaled_dot_product_attention (float64) over
  the selected keys (prefill: plus the tile's causal diagonal keys);
- k = N reducing to dense attention, and reuse with the identity map
  reproducing the anchor's output.

Shapes stay tiny (the oracle takes any prefill tile size; 4 and 8 here) so
the whole module runs in seconds.
"""
import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _draw(rng, shape, tied):
    if tied:
        # a few values only: equal scores (and equal pooled scores) are common
        return rng.choice(np.array([-1.0, -0.5, 0.0, 0.5, 1.0], dtype=np.float32), size=shape)
    return rng.standard_normal(shape).astype(np.float32)


def _stable_topk(p32, k):
    """The k keys of p32 (float32 values) with the largest values, ties to the
    lower key, in ascending key order."""
    order = sorted(range(len(p32)), key=lambda j: (-float(p32[j]), j))
    return np.array(sorted(order[:k]), dtype=np.int64)


def _sdpa(q, k, v, mask=None):
    """softmax(q k^T / sqrt(d)) v in float64 through torch; q [R, D], k/v [M, D]."""
    qt = torch.from_numpy(q).double()[None, None]
    kt = torch.from_numpy(k).double()[None, None]
    vt = torch.from_numpy(v).double()[None, None]
    am = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am)[0, 0].numpy()


decode_cases = st.tuples(
    st.integers(0, 2**31 - 1),          # seed
    st.integers(1, 2),                  # B
    st.sampled_from([1, 2]),            # Hkv
    st.sampled_from([1, 2, 4]),         # G
    st.sampled_from([4, 8, 16]),        # D
    st.integers(1, 48),                 # N
    st.integers(1, 100),                # pct
    st.booleans(),                      # tied inputs
)


@SETTINGS
@given(decode_cases)
def test_decode_anchor_properties(case):
    seed, B, Hkv, G, D, N, pct, tied = case
    Hq = Hkv * G
    rng = np.random.default_rng(seed)
    q, k, v = _draw(rng, (B, Hq, D), tied), _draw(rng, (B, Hkv, N, D), tied), _draw(rng, (B, Hkv, N, D), False)
    idx, o, pooled = oracle.decode_anchor(q, k, v, pct, want_pooled=True)
    kk = oracle.decode_k(N, pct)
    assert kk == max(1, min(N, (pct * N + 50) // 100))
    ke = torch.from_numpy(k).double().repeat_interleave(G, dim=1)
    s = torch.einsum("bhd,bhnd->bhn", torch.from_numpy(q).double(), ke) / np.sqrt(D)
    p = torch.softmax(s, dim=-1).view(B, Hkv, G, N).sum(2).numpy()
    np.testing.assert_allclose(pooled, p, rtol=1e-12, atol=1e-15)
    for b in range(B):
        for g in range(Hkv):
            sel = _stable_topk(p[b, g].astype(np.float32), kk)
            np.testing.assert_array_equal(idx[b, g], sel)
            for r in range(G):
                h = g * G + r
                ref = _sdpa(q[b, h][None], k[b, g, sel], v[b, g, sel])[0]
                np.testing.assert_allclose(o[b, h], ref, rtol=1e-10, atol=1e-12)
    # reuse of the anchor's own sets with the identity map is the anchor's output
    o2 = oracle.decode_reuse(q, k, v, idx, np.arange(Hkv, dtype=np.int32))
    np.testing.assert_array_equal(o2, o)
    if kk == N:
        dense = oracle.dense_attention(q[:, :, None, :], k, v, causal=False)[:, :, 0, :]
        np.testing.assert_allclose(o, dense, rtol=1e-10, atol=1e-12)


prefill_cases = st.tuples(
    st.integers(0, 2**31 - 1),          # seed
    st.sampled_from([1, 2]),            # Hkv
    st.sampled_from([1, 2, 4]),         # G
    st.sampled_from([4, 8]),            # D
    st.sampled_from([4, 8]),            # tile
    st.integers(1, 8),                  # tiles
    st.integers(1, 100),                # pct
    st.booleans(),                      # tied inputs
)


@SETTINGS
@given(prefill_cases)
def test_prefill_anchor_properties(case):
    seed, Hkv, G, D, tile, T, pct, tied = case
    Hq, N = Hkv * G, tile * T
    rng = np.random.default_rng(seed)
    q, k, v = _draw(rng, (1, Hq, N, D), tied), _draw(rng, (1, Hkv, N, D), tied), _draw(rng, (1, Hkv, N, D), False)
    idx, o = oracle.prefill_anchor(q, k, v, pct, tile=tile)
    off = oracle.prefill_offsets(N, tile, pct)
    ke = torch.from_numpy(k[0]).double().repeat_interleave(G, dim=0)        # [Hq, N, D]
    s = torch.einsum("hid,hjd->hij", torch.from_numpy(q[0]).double(), ke) / np.sqrt(D)
    causal = torch.ones(N, N, dtype=torch.bool).tril()
    prob = torch.softmax(s.masked_fill(~causal, float("-inf")), dim=-1)    # [Hq, N, N] causal rows
    for t in range(T):
        rows = slice(tile * t, tile * t + tile)
        kt = int(off[t + 1] - off[t])
        assert kt == min(tile * t, (pct * tile * t + 50) // 100)
        for g in range(Hkv):
            # pooled over the tile's rows and the group's heads, keys before the tile
            P = prob[g * G:(g + 1) * G, rows, :tile * t].sum(dim=(0, 1)).numpy()
            sel = _stable_topk(P.astype(np.float32), kt) if t else np.zeros(0, dtype=np.int64)
            np.testing.assert_array_equal(idx[0, g, off[t]:off[t + 1]], sel)
            # each row attends over the set plus its causal diagonal keys
            for r in range(G):
                h = g * G + r
                keys = np.concatenate([sel, np.arange(tile * t, tile * t + tile)])
                mask = np.zeros((tile, len(keys)), dtype=bool)
                mask[:, :len(sel)] = True
                mask[:, len(sel):] = np.tril(np.ones((tile, tile), dtype=bool))
                ref = _sdpa(q[0, h, rows], k[0, g, keys], v[0, g, keys], mask)
                np.testing.assert_allclose(o[0, h, rows], ref, rtol=1e-10, atol=1e-12)
    if pct == 100:
        dense = oracle.dense_attention(q, k, v, causal=True)
        np.testing.assert_allclose(o, dense, rtol=1e-10, atol=1e-12)
