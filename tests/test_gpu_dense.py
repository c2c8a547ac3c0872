"""GPU parity of the dense baselines (decode over every key, causal prefill)
against the oracle's dense attention, through the C ABI.

The dense calls are the comparison the pages quote Kascade's speed-ups
against (Kascade README, "Abstract"); what they compute is the textbook
softmax(Q K^T / sqrt(d)) V ("I/O complexity of attention", abstract), which
the oracle's dense_attention follows and the oracle tests pin. Besides the
oracle, each dense result must equal, bit for bit, the sparse path run with
the full key list (decode reuse with every key, prefill reuse at pct 100):
the same kernels with an index set that names every key in order.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import inputgen
import oracle
from parity_util import TOL, max_abs

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


DECODE_SHAPES = [
    # (label, B, Hq, Hkv, D, N, dtype)
    ("f32_d64_g4", 1, 8, 2, 64, 2048, "f32"),
    ("f32_d128_g4_ragged", 1, 8, 2, 128, 1500, "f32"),
    ("bf16_d128_g4_ragged", 2, 32, 8, 128, 5037, "bf16"),
    ("bf16_d64_g1", 2, 4, 4, 64, 3001, "bf16"),
    ("bf16_d128_g2", 3, 4, 2, 128, 777, "bf16"),
    ("bf16_d128_g8", 1, 16, 2, 128, 4099, "bf16"),
    ("bf16_n1", 1, 8, 2, 128, 1, "bf16"),
    ("bf16_n17", 1, 8, 2, 128, 17, "bf16"),
    ("bf16_many_splits", 1, 8, 2, 128, 40000, "bf16"),
]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=[s[0] for s in DECODE_SHAPES])
def test_decode_dense(shape):
    kas = _kas()
    label, B, Hq, Hkv, D, N, dt = shape
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000, topk_pct=10)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    _say(f"[decode dense] {label}: B={B} Hq={Hq} Hkv={Hkv} D={D} N={N} {dt}")
    o = kas.decode_dense(q, k, v)
    # the sparse gather with every key, in order, per (b, KV head)
    every = torch.arange(N, dtype=torch.int32, device=DEV).expand(B, Hkv, N).contiguous()
    o_sparse = kas.decode_reuse(q, k, v, every, None, 100)
    torch.cuda.synchronize()
    ref = oracle.dense_attention(_np(q)[:, :, None, :], _np(k), _np(v), causal=False)[:, :, 0, :]
    err = max_abs(_np(o), ref)
    _say(f"    max|o-o_oracle|={err:.3g} tol={TOL[dt]}")
    assert err <= TOL[dt]
    assert torch.equal(o, o_sparse)


def test_decode_dense_full_size():
    """Every head of the 128K, batch-4 decode workload against the oracle."""
    kas = _kas()
    w = inputgen.WORKLOADS["llama8b_decode_128k"]
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 3, DEV, pos)
    _say(f"[decode dense] {w.name} layer 3: B={w.batch} N={w.seq_len}")
    o = kas.decode_dense(q, k, v)
    torch.cuda.synchronize()
    ref = oracle.dense_attention(_np(q)[:, :, None, :], _np(k), _np(v), causal=False)[:, :, 0, :]
    err = max_abs(_np(o), ref)
    _say(f"    max|o-o_oracle|={err:.3g}")
    assert err <= TOL["bf16"]


PREFILL_SHAPES = [
    # (label, B, Hq, Hkv, D, N)
    ("d128_g4_n32", 1, 8, 2, 128, 32),
    ("d128_g4_n256", 1, 32, 8, 128, 256),
    ("d64_g2_b2_n1184", 2, 4, 2, 64, 1184),
    ("d128_g8_n96", 1, 16, 2, 128, 96),
    ("d128_g1_n160", 1, 2, 2, 128, 160),
    ("d128_g4_n2080", 1, 8, 2, 128, 2080),
]


def _full_sets(B, Hkv, N):
    """CSR index sets naming every key before each tile (what pct 100 selects)."""
    T = N // 32
    row = np.concatenate([np.arange(32 * t, dtype=np.int32) for t in range(T)])
    assert row.size == int(oracle.prefill_offsets(N, 32, 100)[-1])
    if row.size == 0:                # one tile: no sets, but the call wants a buffer
        row = np.zeros(1, np.int32)
    return torch.as_tensor(np.broadcast_to(row, (B, Hkv, row.size)).copy(), device=DEV)


@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=[s[0] for s in PREFILL_SHAPES])
def test_prefill_dense(shape):
    kas = _kas()
    label, B, Hq, Hkv, D, N = shape
    w = inputgen.custom("prefill", B, Hq, Hkv, D, N, "bf16", wid=zlib.crc32(label.encode()) % 1000)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    _say(f"[prefill dense] {label}: B={B} Hq={Hq} Hkv={Hkv} D={D} N={N}")
    o = kas.prefill_dense(q, k, v)
    o_sparse = kas.prefill_reuse(q, k, v, _full_sets(B, Hkv, N), None, 100)
    torch.cuda.synchronize()
    ref = oracle.dense_attention(_np(q), _np(k), _np(v), causal=True)
    err = max_abs(_np(o), ref)
    _say(f"    max|o-o_oracle|={err:.3g} tol={TOL['bf16']}")
    assert err <= TOL["bf16"]
    assert torch.equal(o, o_sparse)


@pytest.mark.parametrize("name,rows", [
    ("qwen8b_prefill_32k", (0, 31, 32, 1000, 16415, 32767)),
    ("llama8b_prefill_128k", (0, 33, 65535, 100000, 131071)),
])
def test_prefill_dense_full_size_sampled_rows(name, rows):
    """Whole-prompt launch; rows checked one by one (row i over keys [0, i])."""
    kas = _kas()
    w = inputgen.WORKLOADS[name]
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    _say(f"[prefill dense] {name}: N={w.seq_len} sampled rows {rows}")
    o = kas.prefill_dense(q, k, v)
    torch.cuda.synchronize()
    worst = 0.0
    for i in rows:
        qi = _np(q[:, :, i:i + 1, :])
        ki, vi = _np(k[:, :, :i + 1, :]), _np(v[:, :, :i + 1, :])
        ref = oracle.dense_attention(qi, ki, vi, causal=True)
        worst = max(worst, max_abs(_np(o[:, :, i:i + 1, :]), ref))
    _say(f"    max|o-o_oracle| over sampled rows={worst:.3g}")
    assert worst <= TOL["bf16"]
    assert torch.isfinite(o.float()).all()


# ---------------------------------------------------------------- anchor layers with a dense output

ANCHOR_DENSE = [
    # (label, phase, B, Hq, Hkv, D, N, dtype, varlen, page size)
    ("decode_bf16_g4", "decode", 2, 32, 8, 128, 5037, "bf16", False, None),
    ("decode_f32_d64", "decode", 1, 8, 2, 64, 2048, "f32", False, None),
    ("decode_f16_varlen_paged", "decode", 3, 8, 2, 128, 3001, "f16", True, 64),
    ("prefill_bf16_g4", "prefill", 1, 8, 2, 128, 640, "bf16", False, None),
    ("prefill_f16_varlen", "prefill", 2, 8, 4, 64, 352, "f16", True, None),
    ("prefill_bf16_paged", "prefill", 1, 8, 2, 128, 512, "bf16", False, 32),
]


@pytest.mark.parametrize("case", ANCHOR_DENSE, ids=[c[0] for c in ANCHOR_DENSE])
def test_anchor_dense_output(case):
    """kas_desc_t.anchor_dense_output = 1: the anchor call selects exactly the
    sets it selects without the flag (bit for bit) and writes the dense
    attention of the dense call (bit for bit), which the oracle's dense
    attention checks as well."""
    kas = _kas()
    label, phase, B, Hq, Hkv, D, N, dt, varlen, P = case
    w = inputgen.custom(phase, B, Hq, Hkv, D, N, dt, wid=zlib.crc32(label.encode()) % 1000 + 3, topk_pct=10)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    kc, vc = k, v                     # the contiguous cache, for the oracle
    kw = {}
    lens = None
    if varlen:
        lens = np.array([N, N // 2, 96][:B] if phase == "decode" else [N, 96][:B], dtype=np.int32)
        kw["seq_lens"] = torch.as_tensor(lens, device=DEV)
    if P is not None:
        from test_gpu_kvcache import _paged
        k, v, bt = _paged(k, v, P, seed=P)
        kw["block_table"] = bt
        if phase == "decode":
            kw["seq_len"] = N
    _say(f"[anchor dense output] {label}")
    if phase == "decode":
        idx, _ = kas.decode_anchor(q, k, v, 10, **kw)
        idx_d, o_d = kas.decode_anchor(q, k, v, 10, dense_output=True, **kw)
        o_ref = kas.decode_dense(q, k, v, **kw)
    else:
        idx, _ = kas.prefill_anchor(q, k, v, 10, **kw)
        idx_d, o_d = kas.prefill_anchor(q, k, v, 10, dense_output=True, **kw)
        o_ref = kas.prefill_dense(q, k, v, **kw)
    torch.cuda.synchronize()
    if varlen and phase == "decode":
        for b in range(B):
            kb = oracle.decode_k(int(lens[b]), 10)
            assert torch.equal(idx[b, :, :kb], idx_d[b, :, :kb])
    elif varlen:
        off = oracle.prefill_offsets(N, 32, 10)
        for b in range(B):
            used = off[int(lens[b]) // 32]
            assert torch.equal(idx[b, :, :used], idx_d[b, :, :used])
    else:
        assert torch.equal(idx, idx_d)
    if varlen and phase == "prefill":
        for b in range(B):
            n = int(lens[b])
            assert torch.equal(o_d[b, :, :n], o_ref[b, :, :n])
    else:
        assert torch.equal(o_d, o_ref)
    # and against the oracle's dense attention (first sequence, its own keys)
    qn, kn, vn = _np(q[:1]), _np(kc[:1]), _np(vc[:1])
    if phase == "decode":
        ref = oracle.dense_attention(qn[:, :, None, :], kn, vn, causal=False)[:, :, 0, :]
    else:
        ref = oracle.dense_attention(qn, kn, vn, causal=True)
    err = max_abs(_np(o_d[:1]), ref)
    _say(f"    sets bit-identical, output bit-identical to the dense call; max|o-o_oracle dense|={err:.3g}")
    assert err <= TOL[dt]
