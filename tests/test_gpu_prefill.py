"""GPU parity of the prefill path (anchor and reuse, 32-query tiles) against the
CPU oracle, through the C ABI. Small prompts are checked on every tile; the
full-size prompts on a sample of tiles the oracle can compute one by one."""
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


def _check_tiles(w, q, k, v, pct, gidx, go, tiles, label):
    """Compare the GPU index sets and output rows of `tiles` with the oracle."""
    N, B, Hkv = w.seq_len, w.batch, w.n_kv_heads
    off = oracle.prefill_offsets(N, 32, pct)
    kn, vn = _np(k), _np(v)
    gidx_np = gidx.cpu().numpy()
    worst_set, worst_e2e, swaps = 0.0, 0.0, 0
    for t in tiles:
        qr = _np(q[:, :, 32 * t: 32 * t + 32])
        oidx, oo = oracle.prefill_anchor(qr, kn, vn, pct, t0=t, t1=t + 1)
        kt = int(off[t + 1] - off[t])
        for b in range(B):
            for g in range(Hkv):
                gs = gidx_np[b, g, off[t]:off[t + 1]]
                os_ = oidx[b, g]
                if not np.array_equal(gs, os_):
                    P = oracle.prefill_pooled(qr, kn, b, t, g, t0=t, t1=t + 1)[: 32 * t]
                    swaps += assert_index_set(gs, os_, P, kt, where=f"{label} b{b} t{t} g{g}")
                else:
                    assert len(gs) == kt
        # attention over the GPU's own sets (isolates the attention arithmetic)
        o_same = oracle.prefill_reuse(qr, kn, vn, gidx_np, np.arange(Hkv, dtype=np.int32), pct,
                                      t0=t, t1=t + 1)
        gor = _np(go[:, :, 32 * t: 32 * t + 32])
        worst_set = max(worst_set, max_abs(gor, o_same))
        worst_e2e = max(worst_e2e, max_abs(gor, oo))
    _say(f"    tiles={list(tiles)} near-tie swaps={swaps} max|o-o_oracle(same set)|={worst_set:.3g} "
         f"max|o-o_oracle|={worst_e2e:.3g}")
    assert worst_set <= TOL[w.dtype]
    assert worst_e2e <= TOL[w.dtype]


def _check_reuse_tiles(w, q, k, v, pct, anchor_idx, head_map, go, tiles, label):
    kn, vn = _np(k), _np(v)
    aidx = anchor_idx.cpu().numpy()
    worst = 0.0
    for t in tiles:
        qr = _np(q[:, :, 32 * t: 32 * t + 32])
        ref = oracle.prefill_reuse(qr, kn, vn, aidx, head_map, pct, t0=t, t1=t + 1)
        worst = max(worst, max_abs(_np(go[:, :, 32 * t: 32 * t + 32]), ref))
    _say(f"    reuse head_map={list(head_map)} tiles={list(tiles)} max|o-o_oracle|={worst:.3g}")
    assert worst <= TOL[w.dtype]


SHAPES = [
    # (label, B, Hq, Hkv, D, N, pct)
    ("d128_g4_n256", 1, 8, 2, 128, 256, 10),
    ("d128_g4_b2_n1184", 2, 8, 2, 128, 1184, 10),
    ("d64_g1_n640", 1, 2, 2, 64, 640, 10),
    ("d128_g2_n512_pct25", 1, 4, 2, 128, 512, 25),
    ("d128_g8_n384", 1, 16, 2, 128, 384, 10),
    ("d128_g4_n32_single_tile", 1, 8, 2, 128, 32, 10),
    ("d128_g4_n448_pct1", 1, 8, 2, 128, 448, 1),
    ("d128_g4_n320_full", 1, 8, 2, 128, 320, 100),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_prefill_anchor_then_reuse(shape):
    kas = _kas()
    label, B, Hq, Hkv, D, N, pct = shape
    w = inputgen.custom("prefill", B, Hq, Hkv, D, N, "bf16", wid=zlib.crc32(label.encode()) % 1000,
                        topk_pct=pct)
    _say(f"[prefill anchor] {label}: B={B} Hq={Hq} Hkv={Hkv} D={D} N={N} pct={pct}")
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    gidx, go = kas.prefill_anchor(q, k, v, pct)
    torch.cuda.synchronize()
    T = N // 32
    _check_tiles(w, q, k, v, pct, gidx, go, range(T), label)
    if pct == 100:
        dense = oracle.dense_attention(_np(q), _np(k), _np(v), causal=True)
        err = max_abs(_np(go), dense)
        _say(f"    pct=100 vs dense causal: {err:.3g}")
        assert err <= TOL["bf16"]
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.random.default_rng(3).integers(0, Hkv, Hkv).astype(np.int32)
    _say(f"[prefill reuse] {label}")
    o2 = kas.prefill_reuse(q2, k2, v2, gidx, torch.as_tensor(hm, device=DEV), pct)
    torch.cuda.synchronize()
    _check_reuse_tiles(w, q2, k2, v2, pct, gidx, hm, o2, range(T), label)


# Oracle-checked tiles: first and last tiles, both members of several tile
# pairs (2p, 2p+1) of the statistics and pooling kernels, and tiles that land
# on different XCDs and in different groups of 64 workgroups of the
# XCD-local order (the attention kernel takes tile T - 1 - order(j)).
@pytest.mark.parametrize("name,tiles", [
    ("qwen8b_prefill_32k", (1, 2, 3, 37, 64, 65, 500, 511, 700, 1022, 1023)),
    ("llama8b_prefill_128k", (1, 2, 3, 63, 64, 776, 777, 1500, 2048, 2049, 3001, 4094, 4095)),
])
def test_full_size_prefill_sampled_tiles(name, tiles):
    kas = _kas()
    w = inputgen.WORKLOADS[name]
    pos = inputgen.heavy_positions(w)
    maps = inputgen.head_maps(w)
    _say(f"[prefill anchor] {name}: N={w.seq_len} sampled tiles {tiles}")
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    gidx, go = kas.prefill_anchor(q, k, v, w.topk_pct)
    torch.cuda.synchronize()
    _check_tiles(w, q, k, v, w.topk_pct, gidx, go, tiles, name)
    # structural checks on every tile: sizes, order, range
    off = oracle.prefill_offsets(w.seq_len, 32, w.topk_pct)
    gi = gidx.cpu().numpy()
    tile_of = np.repeat(np.arange(len(off) - 1), np.diff(off))
    assert (gi >= 0).all() and (gi < 32 * tile_of[None, None, :]).all()
    seg_start = np.zeros(gi.shape[-1], bool)
    seg_start[off[:-1][np.diff(off) > 0]] = True
    d = np.diff(gi, axis=-1)
    assert ((d > 0) | seg_start[None, None, 1:]).all()
    del q, k, v, go
    q, k, v = inputgen.layer_inputs(w, 1, DEV, pos)
    _say(f"[prefill reuse] {name} layer1")
    o2 = kas.prefill_reuse(q, k, v, gidx, torch.as_tensor(maps[1], device=DEV), w.topk_pct)
    torch.cuda.synchronize()
    _check_reuse_tiles(w, q, k, v, w.topk_pct, gidx, maps[1], o2, tiles, name)


def test_prefill_deterministic_and_identity_reuse():
    kas = _kas()
    w = inputgen.custom("prefill", 1, 8, 2, 128, 640, "bf16", wid=21)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    i1, o1 = kas.prefill_anchor(q, k, v, 10)
    i2, o2 = kas.prefill_anchor(q, k, v, 10)
    o3 = kas.prefill_reuse(q, k, v, i1, None, 10)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(o1, o2)
    assert torch.equal(o1, o3)


def test_prefill_scores_far_above_first_block():
    """Row statistics keep a per-lane reference from the first key block; a
    later key whose score exceeds it by more than 2^64 in probability takes
    the rescaling path. Plant such a key and compare with the oracle."""
    kas = _kas()
    B, Hq, Hkv, D, N, pct = 1, 8, 2, 128, 640, 10
    w = inputgen.custom("prefill", B, Hq, Hkv, D, N, "bf16", wid=51, sinks=False)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    u = torch.randn(D, generator=torch.Generator().manual_seed(5)).to(DEV)
    u = u / u.norm()
    q[:, :, 320:] = (11.0 * u).to(torch.bfloat16)          # same direction for late queries
    k[:, :, 300] = (70.0 * u).to(torch.bfloat16)           # base-2 score ~ 70*11/sqrt(128)*log2(e) ~ 98
    _say("[prefill anchor] planted key 300 with a score far above the first block's")
    gidx, go = kas.prefill_anchor(q, k, v, pct)
    torch.cuda.synchronize()
    _check_tiles(w, q, k, v, pct, gidx, go, range(N // 32), "far_scores")


def test_prefill_select_without_lds_candidates(kas_options):
    """A select cap of 0 (KAS_OPT_PREFILL_SELECT_CAP) sends every tile's selection through the
    in-place histogram passes over the pooled row (the path a first-digit bin
    too large for LDS takes); the index sets and outputs are bit-identical."""
    kas = _kas()
    w = inputgen.custom("prefill", 1, 8, 2, 128, 2048, "bf16", wid=62)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    gidx, go = kas.prefill_anchor(q, k, v, 10)
    kas_options(kas.OPT_PREFILL_SELECT_CAP, 0)
    gidx2, go2 = kas.prefill_anchor(q, k, v, 10)
    torch.cuda.synchronize()
    assert torch.equal(gidx, gidx2) and torch.equal(go, go2)
    _check_tiles(w, q, k, v, 10, gidx2, go2, (1, 17, 40, 63), "select_in_place")


def test_prefill_pooling_in_tile_ranges(kas_options):
    """A small pooled-score budget splits pooling and selection into many
    tile ranges; the index sets and outputs are bit-identical to one range."""
    kas = _kas()
    w = inputgen.custom("prefill", 1, 8, 2, 128, 2048, "bf16", wid=61)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    gidx, go = kas.prefill_anchor(q, k, v, 10)
    kas_options(kas.OPT_PREFILL_POOL_MB, 1)            # ~262K floats per range
    gidx2, go2 = kas.prefill_anchor(q, k, v, 10)
    torch.cuda.synchronize()
    assert torch.equal(gidx, gidx2) and torch.equal(go, go2)
    _check_tiles(w, q, k, v, 10, gidx2, go2, (1, 17, 40, 63), "pool_ranges")
