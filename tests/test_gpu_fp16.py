"""GPU parity of the fp16 paths against the oracle, through the C ABI.

The README's own kernels run fp16 only (README notes); here bf16 and fp16 go
through the same kernels with the matrix instructions, packing and stores of
the element type. Inputs are the same seeded recipe rounded once to fp16 (the
oracle reads them exactly as fp32); index sets must match the oracle's as for
bf16, outputs within the fp16 tolerance.
"""
import zlib

import numpy as np
import pytest
import torch

import inputgen
import oracle
from parity_util import TOL, max_abs
from test_gpu_decode import _check_anchor, _check_reuse, _np, _say
from test_gpu_prefill import _check_reuse_tiles, _check_tiles

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _kas():
    import sparse_attention_long_anchor_amd as kas
    return kas


DECODE_SHAPES = [
    # (label, B, Hq, Hkv, D, N, pct)
    ("f16_d128_g4_ragged", 2, 32, 8, 128, 5037, 10),
    ("f16_d64_g1", 2, 4, 4, 64, 3001, 10),
    ("f16_d128_g8", 1, 16, 2, 128, 4099, 10),
    ("f16_n7", 1, 8, 2, 128, 7, 10),
    ("f16_many_splits", 1, 8, 2, 128, 40000, 50),
]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=[s[0] for s in DECODE_SHAPES])
def test_decode_fp16_anchor_reuse_dense(shape):
    kas = _kas()
    label, B, Hq, Hkv, D, N, pct = shape
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, "f16", wid=zlib.crc32(label.encode()) % 1000, topk_pct=pct)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    assert q.dtype == torch.float16
    idx, _ = _check_anchor(w, q, k, v, pct, label)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.random.default_rng(5).integers(0, Hkv, Hkv).astype(np.int32)
    _check_reuse(w, q2, k2, v2, idx, hm, pct, label)
    o = kas.decode_dense(q2, k2, v2)
    torch.cuda.synchronize()
    ref = oracle.dense_attention(_np(q2)[:, :, None, :], _np(k2), _np(v2), causal=False)[:, :, 0, :]
    err = max_abs(_np(o), ref)
    _say(f"    dense max|o-o_oracle|={err:.3g}")
    assert err <= TOL["f16"]


def test_decode_fp16_full_size():
    w0 = inputgen.WORKLOADS["llama8b_decode_128k"]
    import dataclasses
    w = dataclasses.replace(w0, dtype="f16")
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    idx, _ = _check_anchor(w, q, k, v, w.topk_pct, w.name + " fp16 layer0")
    del q, k, v
    q, k, v = inputgen.layer_inputs(w, 1, DEV, pos)
    _check_reuse(w, q, k, v, idx, inputgen.head_maps(w)[1], w.topk_pct, w.name + " fp16 layer1")


PREFILL_SHAPES = [
    # (label, B, Hq, Hkv, D, N, pct)
    ("f16_d128_g4_n256", 1, 8, 2, 128, 256, 10),
    ("f16_d128_g4_b2_n1184", 2, 8, 2, 128, 1184, 10),
    ("f16_d64_g1_n640", 1, 2, 2, 64, 640, 10),
    ("f16_d128_g8_n384", 1, 16, 2, 128, 384, 25),
    ("f16_d128_g4_n32", 1, 8, 2, 128, 32, 10),
]


@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=[s[0] for s in PREFILL_SHAPES])
def test_prefill_fp16_anchor_reuse_dense(shape):
    kas = _kas()
    label, B, Hq, Hkv, D, N, pct = shape
    w = inputgen.custom("prefill", B, Hq, Hkv, D, N, "f16", wid=zlib.crc32(label.encode()) % 1000, topk_pct=pct)
    _say(f"[prefill anchor fp16] {label}: B={B} Hq={Hq} Hkv={Hkv} D={D} N={N}")
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    gidx, go = kas.prefill_anchor(q, k, v, pct)
    torch.cuda.synchronize()
    _check_tiles(w, q, k, v, pct, gidx, go, range(N // 32), label)
    q2, k2, v2 = inputgen.layer_inputs(w, 1, DEV)
    hm = np.random.default_rng(4).integers(0, Hkv, Hkv).astype(np.int32)
    o2 = kas.prefill_reuse(q2, k2, v2, gidx, torch.as_tensor(hm, device=DEV), pct)
    torch.cuda.synchronize()
    _check_reuse_tiles(w, q2, k2, v2, pct, gidx, hm, o2, range(N // 32), label)
    o3 = kas.prefill_dense(q2, k2, v2)
    torch.cuda.synchronize()
    err = max_abs(_np(o3), oracle.dense_attention(_np(q2), _np(k2), _np(v2), causal=True))
    _say(f"    dense max|o-o_oracle|={err:.3g}")
    assert err <= TOL["f16"]


def test_prefill_fp16_scores_far_above_first_block():
    """fp16 probabilities overflow at 65504: a row whose later scores exceed its
    first block's maximum by far must rescale before packing (the lazy
    reference); the output must stay finite and match the oracle."""
    kas = _kas()
    w = inputgen.custom("prefill", 1, 8, 2, 128, 320, "f16", wid=77)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    k[:, :, 200:232] = (k[:, :, 200:232].float() * 6.0).to(torch.float16)    # large logits in block 6
    q = (q.float() * 2.0).to(torch.float16)
    o = kas.prefill_dense(q, k, v)
    gidx, go = kas.prefill_anchor(q, k, v, 50)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(go.float()).all()
    err = max_abs(_np(o), oracle.dense_attention(_np(q), _np(k), _np(v), causal=True))
    _say(f"    dense max|o-o_oracle|={err:.3g}")
    assert err <= TOL["f16"]
    _check_tiles(w, q, k, v, 50, gidx, go, range(10), "f16_far_scores")


def test_prefill_fp16_full_size_sampled_tiles():
    import dataclasses
    kas = _kas()
    w = dataclasses.replace(inputgen.WORKLOADS["qwen8b_prefill_32k"], dtype="f16")
    pos = inputgen.heavy_positions(w)
    q, k, v = inputgen.layer_inputs(w, 0, DEV, pos)
    _say(f"[prefill anchor fp16] {w.name}: N={w.seq_len}")
    gidx, go = kas.prefill_anchor(q, k, v, w.topk_pct)
    torch.cuda.synchronize()
    _check_tiles(w, q, k, v, w.topk_pct, gidx, go, (1, 37, 500, 1023), w.name + " fp16")
