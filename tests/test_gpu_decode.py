"""GPU parity of the decode path (anchor and reuse) against the CPU oracle,
through the C ABI."""
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


def _check_anchor(w, q, k, v, pct, label):
    kas = _kas()
    _say(f"[decode anchor] {label}: B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} D={w.head_dim} "
         f"N={w.seq_len} {w.dtype} pct={pct}")
    idx, o = kas.decode_anchor(q, k, v, pct)
    torch.cuda.synchronize()
    qn, kn, vn = _np(q), _np(k), _np(v)
    oidx, oo, pooled = oracle.decode_anchor(qn, kn, vn, pct, want_pooled=True)
    kk = oracle.decode_k(w.seq_len, pct)
    gidx = idx.cpu().numpy()
    swaps = 0
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            swaps += assert_index_set(gidx[b, g], oidx[b, g], pooled[b, g], kk, where=f"{label} b{b} g{g}")
    tol = TOL[w.dtype]
    # attention over the GPU's own set (isolates the attention arithmetic)
    o_same = oracle.decode_reuse(qn, kn, vn, gidx, np.arange(w.n_kv_heads, dtype=np.int32))
    err_same = max_abs(_np(o), o_same)
    err_e2e = max_abs(_np(o), oo)
    _say(f"    near-tie swaps={swaps} max|o-o_oracle(same set)|={err_same:.3g} "
         f"max|o-o_oracle|={err_e2e:.3g} tol={tol}")
    assert err_same <= tol
    assert err_e2e <= tol
    return idx, o


def _check_reuse(w, q, k, v, anchor_idx, head_map, pct, label):
    kas = _kas()
    _say(f"[decode reuse] {label}: head_map={list(head_map)}")
    hm = torch.as_tensor(head_map, dtype=torch.int32, device=DEV)
    o = kas.decode_reuse(q, k, v, anchor_idx, hm, pct)
    torch.cuda.synchronize()
    ref = oracle.decode_reuse(_np(q), _np(k), _np(v), anchor_idx.cpu().numpy(), head_map)
    err = max_abs(_np(o), ref)
    _say(f"    max|o-o_oracle|={err:.3g} tol={TOL[w.dtype]}")
    assert err <= TOL[w.dtype]
    return o


SHAPES = [
    # (label, B, Hq, Hkv, D, N, dtype, pct)
    ("f32_d64_g4", 1, 8, 2, 64, 2048, "f32", 10),
    ("f32_d128_g4", 1, 8, 2, 128, 1500, "f32", 10),
    ("bf16_d128_g4_ragged", 2, 32, 8, 128, 5037, "bf16", 10),
    ("bf16_d64_g1", 2, 4, 4, 64, 3001, "bf16", 10),
    ("bf16_d128_g2", 3, 4, 2, 128, 777, "bf16", 7),
    ("bf16_d128_g8", 1, 16, 2, 128, 4099, "bf16", 10),
    ("bf16_n1", 1, 8, 2, 128, 1, "bf16", 10),
    ("bf16_n7", 1, 8, 2, 128, 7, "bf16", 10),
    ("bf16_n17_full", 1, 8, 2, 128, 17, "bf16", 100),
    ("bf16_full_k", 1, 8, 2, 128, 600, "bf16", 100),
    ("bf16_k_many_splits", 1, 8, 2, 128, 40000, "bf16", 50),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_decode_anchor_then_reuse(shape):
    label, B, Hq, Hkv, D, N, dt, pct = shape
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    idx, _ = _check_anchor(w, q, k, v, pct, label)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.random.default_rng(1).integers(0, Hkv, Hkv).astype(np.int32)
    _check_reuse(w, q2, k2, v2, idx, hm, pct, label)


def test_tiny_workload_both_layers():
    w = inputgen.WORKLOADS["tiny_decode_2k"]
    maps = inputgen.head_maps(w)
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    idx, _ = _check_anchor(w, q, k, v, w.topk_pct, w.name + " layer0")
    q, k, v = inputgen.layer_inputs(w, 1, DEV, pos)
    _check_reuse(w, q, k, v, idx, maps[1], w.topk_pct, w.name + " layer1")


@pytest.mark.parametrize("name", ["llama8b_decode_32k", "llama8b_decode_128k"])
def test_full_size_workload_anchor_and_reuse(name):
    w = inputgen.WORKLOADS[name]
    maps = inputgen.head_maps(w)
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    idx, _ = _check_anchor(w, q, k, v, w.topk_pct, w.name + " layer0")
    del q, k, v
    q, k, v = inputgen.layer_inputs(w, 1, DEV, pos)
    _check_reuse(w, q, k, v, idx, maps[1], w.topk_pct, w.name + " layer1")


def test_exact_ties_take_lowest_indices():
    kas = _kas()
    B, Hq, Hkv, D, N, pct = 1, 8, 2, 128, 1000, 10     # k = 100
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, "bf16", wid=7, n_heavy=0, sinks=False)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    qf = q.float().view(B, Hkv, 4, D).mean(2)
    heavy = (16.0 * qf / qf.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    pos = torch.arange(300, 450, device=DEV)             # 150 identical heavy rows
    k[:, :, pos] = heavy[:, :, None, :]
    idx, o = kas.decode_anchor(q, k, v, pct)
    torch.cuda.synchronize()
    oidx, _, pooled = oracle.decode_anchor(_np(q), _np(k), _np(v), pct, want_pooled=True)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    assert (oidx == np.arange(300, 400)).all()


@pytest.mark.parametrize("case", ["random_n3000", "random_n40000", "all_tied_n70000"])
def test_select_paths_agree(case, kas_options):
    """The chunked selection (per-chunk candidates of the first digit's bin,
    digits 2 and 3 resolved per row) and the one-workgroup-per-row kernel
    (KAS_OPT_DECODE_SELECT_ONE_PASS 0 and 1; the default takes the one-pass
    kernel for rows of at most 8192 keys) give identical index sets and
    outputs, equal to the oracle's. With every score tied the first digit's
    bin holds all N scores, more than either kernel's LDS candidate list
    takes: the one-pass kernel then sweeps the row in every pass, the chunked
    resolve step reads the chunks' lists in every pass (a random row takes the
    LDS paths); the kept keys are then the k lowest indices."""
    kas = _kas()
    B, Hq, Hkv, D, pct = 1, 8, 2, 128, 10
    N = int(case.split("_n")[1])
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, "bf16", wid=23)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    if case.startswith("all_tied"):
        k = torch.zeros_like(k)
    _say(f"[decode select paths] {case}")
    idx0, o0 = kas.decode_anchor(q, k, v, pct)
    kas_options(kas.OPT_DECODE_SELECT_ONE_PASS, 0)
    idx1, o1 = kas.decode_anchor(q, k, v, pct)
    kas_options(kas.OPT_DECODE_SELECT_ONE_PASS, 1)
    idx2, o2 = kas.decode_anchor(q, k, v, pct)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2) and torch.equal(o1, o2)
    assert torch.equal(idx0, idx1) and torch.equal(o0, o1)
    oidx, oo, _ = oracle.decode_anchor(_np(q), _np(k), _np(v), pct)
    np.testing.assert_array_equal(idx1.cpu().numpy(), oidx)
    assert max_abs(_np(o1), oo) <= TOL["bf16"]
    if case.startswith("all_tied"):
        kk = idx1.shape[-1]
        assert (idx1.cpu().numpy() == np.arange(kk)).all()


def test_deterministic_and_strided_cache():
    kas = _kas()
    B, Hq, Hkv, D, N, pct = 2, 32, 8, 128, 3000, 10
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, "bf16", wid=11)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    idx1, o1 = kas.decode_anchor(q, k, v, pct)
    idx2, o2 = kas.decode_anchor(q, k, v, pct)
    # the same cache inside a larger allocation (capacity 4096 tokens)
    kc = torch.zeros((B, Hkv, 4096, D), dtype=k.dtype, device=DEV)
    vc = torch.zeros_like(kc)
    kc[:, :, :N] = k
    vc[:, :, :N] = v
    idx3, o3 = kas.decode_anchor(q, kc[:, :, :N], vc[:, :, :N], pct)
    hm = torch.arange(Hkv, dtype=torch.int32, device=DEV)
    o4 = kas.decode_reuse(q, kc[:, :, :N], vc[:, :, :N], idx1, hm, pct)
    o5 = kas.decode_reuse(q, k, v, idx1, None, pct)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2) and torch.equal(o1, o2)
    assert torch.equal(idx1, idx3) and torch.equal(o1, o3)
    assert torch.equal(o4, o5)
    # identity reuse over the anchor's own set reproduces the anchor output
    assert max_abs(_np(o4), _np(o1)) <= TOL["bf16"]


def test_workspace_contents_do_not_matter():
    """A workspace full of stale bytes, reused across calls and shapes, gives
    the same bits as a fresh one."""
    kas = _kas()
    B, Hq, Hkv, D, N, pct = 2, 32, 8, 128, 20000, 10
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, "bf16", wid=31)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    idx, _ = kas.decode_anchor(q, k, v, pct)
    d = kas.make_desc(B, Hq, Hkv, D, N, pct, torch.bfloat16)
    need = kas.workspace_size(d, kas.OP_DECODE_REUSE)
    hm = torch.arange(Hkv, dtype=torch.int32, device=DEV)
    ref = kas.decode_reuse(q, k, v, idx, hm, pct, ws=torch.zeros(need, dtype=torch.uint8, device=DEV))
    ref1 = kas.decode_reuse(q[:1], k[:1], v[:1], idx[:1], hm, pct,
                            ws=torch.zeros(need, dtype=torch.uint8, device=DEV))
    for fill in (0xFF, 0x00, 0x5A):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        o1 = kas.decode_reuse(q, k, v, idx, hm, pct, ws=ws)
        o2 = kas.decode_reuse(q, k, v, idx, hm, pct, ws=ws)
        # a smaller problem through the same workspace, then the first again
        o3 = kas.decode_reuse(q[:1], k[:1], v[:1], idx[:1], hm, pct, ws=ws)
        o4 = kas.decode_reuse(q, k, v, idx, hm, pct, ws=ws)
        torch.cuda.synchronize()
        _say(f"    workspace fill 0x{fill:02x}: bitwise equal to a fresh workspace")
        assert torch.equal(o1, ref) and torch.equal(o2, ref) and torch.equal(o4, ref)
        assert torch.equal(o3, ref1)
    err = max_abs(_np(ref), oracle.decode_reuse(_np(q), _np(k), _np(v), idx.cpu().numpy(),
                                                np.arange(Hkv, dtype=np.int32)))
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("rows", [16, 2048], ids=["split16", "split_max"])
def test_split_variants(rows, kas_options):
    """Many splits (a merge over hundreds of partials) and the largest split
    both match the oracle."""
    kas = _kas()
    kas_options(kas.OPT_DECODE_SPLIT_ROWS, rows)
    env = {"split_rows": rows}
    B, Hq, Hkv, D, N, pct = 1, 32, 8, 128, 30000, 10
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, "bf16", wid=41)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    label = ",".join(f"{a}={b}" for a, b in env.items())
    idx, _ = _check_anchor(w, q, k, v, pct, label)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    _check_reuse(w, q2, k2, v2, idx, np.arange(Hkv, dtype=np.int32)[::-1].copy(), pct, label)
