"""q and o passed as strided views through the C ABI (kas_desc_t q_*_stride /
o_*_stride): every call must give exactly the bits of the same call on
contiguous copies, and leave the memory around a strided o untouched.

Prefill takes the common projection layout [B, N, Hq, D] seen as
[B, Hq, N, D] (token stride Hq * D, head stride D); decode takes q and o as
every other head of a wider buffer (head stride 2 * D) with a padded batch
stride.
"""
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


def _bnhd_view(x):
    """A [B, Hq, N, D] view of a [B, N, Hq, D] copy of x."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


def _strided_out(shape, dtype):
    """A [B, Hq, N, D] view of a [B, N, Hq, D] buffer filled with a sentinel."""
    B, Hq, N, D = shape
    buf = torch.full((B, N, Hq, D), 7.0, dtype=dtype, device=DEV)
    return buf, buf.transpose(1, 2)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_prefill_strided_q_and_o(dt):
    kas = _kas()
    B, Hq, Hkv, D, N, pct = 2, 8, 2, 128, 352, 10
    w = inputgen.custom("prefill", B, Hq, Hkv, D, N, dt, wid=77)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    q1, k1, v1 = inputgen.layer_inputs(w, 1, DEV)
    qs, q1s = _bnhd_view(q), _bnhd_view(q1)
    assert qs.stride() == (N * Hq * D, D, Hq * D, 1)
    print(f"[strides] prefill {dt}: q/o as [B,N,Hq,D] views", flush=True)
    idx, o = kas.prefill_anchor(q, k, v, pct)
    hm = torch.tensor([1, 0], dtype=torch.int32, device=DEV)
    o_r = kas.prefill_reuse(q1, k1, v1, idx, hm, pct)
    o_d = kas.prefill_dense(q, k, v)
    buf_a, oa = _strided_out(q.shape, q.dtype)
    idx_s, _ = kas.prefill_anchor(qs, k, v, pct, o=oa)
    buf_r, orr = _strided_out(q.shape, q.dtype)
    kas.prefill_reuse(q1s, k1, v1, idx_s, hm, pct, o=orr)
    buf_d, od = _strided_out(q.shape, q.dtype)
    kas.prefill_dense(qs, k, v, o=od)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_s)
    assert torch.equal(o, oa) and torch.equal(o_r, orr) and torch.equal(o_d, od)
    # the views cover their buffers completely: no sentinel survives
    for buf in (buf_a, buf_r, buf_d):
        assert not (buf == 7.0).all(dim=-1).any()
    # and the contiguous result itself matches the oracle on two tiles
    off = oracle.prefill_offsets(N, 32, pct)
    f = _np
    for t in (3, 10):
        rows = slice(32 * t, 32 * t + 32)
        ref = oracle.prefill_reuse(f(q[:, :, rows]), f(k), f(v), idx.cpu().numpy()[:, :, :off[-1]],
                                   np.arange(Hkv, dtype=np.int32), pct, t0=t, t1=t + 1)
        assert max_abs(f(o[:, :, rows]), ref) <= TOL[dt]


def test_decode_strided_q_and_o():
    kas = _kas()
    B, Hq, Hkv, D, N, pct = 2, 32, 8, 128, 5000, 10
    w = inputgen.custom("decode", B, Hq, Hkv, D, N, "bf16", wid=78)
    q, k, v = inputgen.layer_inputs(w, 0, DEV)
    q1, k1, v1 = inputgen.layer_inputs(w, 1, DEV)

    def wide(x):
        # every other head of a [B + 1, 2 Hq, D] buffer (padded batch stride)
        buf = torch.zeros((B + 1, 2 * Hq, D), dtype=x.dtype, device=DEV)
        buf[:B, ::2] = x
        return buf[:B, ::2]

    def wide_out():
        buf = torch.full((B + 1, 2 * Hq, D), 7.0, dtype=q.dtype, device=DEV)
        return buf, buf[:B, ::2]

    qs, q1s = wide(q), wide(q1)
    assert qs.stride() == (2 * Hq * D, 2 * D, 1)
    print("[strides] decode: q/o every other head of a wider buffer", flush=True)
    idx, o = kas.decode_anchor(q, k, v, pct)
    hm = torch.arange(Hkv, dtype=torch.int32, device=DEV).flip(0).contiguous()
    o_r = kas.decode_reuse(q1, k1, v1, idx, hm, pct)
    o_d = kas.decode_dense(q, k, v)
    pool = kas.decode_anchor(q, k, v, 4 * pct)[0]
    ridx, o_f = kas.decode_refine(q1, k1, v1, pool, hm, pct)
    bufs = []
    ba, oa = wide_out()
    idx_s, _ = kas.decode_anchor(qs, k, v, pct, o=oa)
    br, orr = wide_out()
    kas.decode_reuse(q1s, k1, v1, idx_s, hm, pct, o=orr)
    bd, od = wide_out()
    kas.decode_dense(qs, k, v, o=od)
    bf, of = wide_out()
    ridx_s, _ = kas.decode_refine(q1s, k1, v1, pool, hm, pct, o=of)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_s) and torch.equal(ridx, ridx_s)
    assert torch.equal(o, oa) and torch.equal(o_r, orr) and torch.equal(o_d, od) and torch.equal(o_f, of)
    for buf in (ba, br, bd, bf):
        # the skipped heads and the padding batch row keep the sentinel
        assert (buf[:, 1::2] == 7.0).all() and (buf[B] == 7.0).all()
    ref = oracle.decode_reuse(_np(q1), _np(k1), _np(v1), idx.cpu().numpy(), hm.cpu().numpy())
    assert max_abs(_np(orr), ref) <= TOL["bf16"]
