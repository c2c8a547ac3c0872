"""The library's calls inside a captured HIP graph (torch.cuda.graph).

Every call only enqueues kernels on the caller's stream: no allocation, no
synchronisation and no memset node (counters and histograms are cleared by
the kernels themselves), so an anchor layer and the reuse layers after it
can be captured once and replayed. Each replay here runs after eager work of
its own on the same buffers (outputs reset, the same calls run eagerly on
other inputs), and must equal the eager result bit for bit. The eager result
itself is checked against the oracle elsewhere; here the reference is the
library's own eager call on the same inputs.
"""
import sys

import numpy as np
import pytest
import torch

import inputgen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _kas():
    import sparse_attention_long_anchor_amd as kas
    return kas


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _reset(outs):
    """Fixed contents for every output (entries a call leaves unspecified,
    such as index slots past a shorter sequence's count, keep them)."""
    for t in outs:
        if t.dtype == torch.int32:
            t.fill_(-1)
        else:
            t.zero_()


def _replay_and_compare(run, run_other, outs, reps=3):
    """run() enqueues the calls writing into outs; run_other() is the same
    calls on other inputs. The graph of run() is replayed reps times, each
    after the outputs were reset and run_other() ran eagerly, then
    synchronised; every replay must reproduce the eager outputs of run()."""
    _reset(outs)
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                # warm-up on the capture stream
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(reps):
        _reset(outs)
        run_other()
        torch.cuda.synchronize()
        assert not all(torch.equal(t, x) for t, x in zip(outs, ref)), "the eager work left the outputs unchanged"
        g.replay()
        torch.cuda.synchronize()
        for i, (t, x) in enumerate(zip(outs, ref)):
            assert torch.equal(t, x), f"replay {r}: output {i} differs from the eager call"
    _say(f"    {reps} replays equal to the eager calls")


def test_decode_anchor_and_reuse_in_a_graph():
    kas = _kas()
    w = inputgen.custom("decode", 2, 32, 8, 128, 9000, "bf16", wid=31, n_layers=3, anchors=(0,))
    maps = inputgen.head_maps(w)
    (q0, k0, v0), (q1, k1, v1), (q2, k2, v2) = (inputgen.layer_inputs(w, l, DEV) for l in range(3))
    hm1, hm2 = (torch.as_tensor(maps[l], device=DEV) for l in (1, 2))
    kd = kas.decode_k(w.seq_len, w.topk_pct)
    idx = torch.empty((w.batch, w.n_kv_heads, kd), dtype=torch.int32, device=DEV)
    o0, o1, o2 = (torch.empty_like(q0) for _ in range(3))
    d = kas.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.topk_pct, torch.bfloat16)
    ws_a = torch.empty(kas.workspace_size(d, kas.OP_DECODE_ANCHOR), dtype=torch.uint8, device=DEV)
    ws_r = torch.empty(kas.workspace_size(d, kas.OP_DECODE_REUSE), dtype=torch.uint8, device=DEV)
    _say(f"[graph decode] B={w.batch} N={w.seq_len} k={kd}: anchor + 2 reuse layers")

    def run(qa=q0):
        kas.decode_anchor(qa, k0, v0, w.topk_pct, idx_out=idx, o=o0, ws=ws_a)
        kas.decode_reuse(q1, k1, v1, idx, hm1, w.topk_pct, o=o1, ws=ws_r)
        kas.decode_reuse(q2, k2, v2, idx, hm2, w.topk_pct, o=o2, ws=ws_r)

    qx = torch.flip(q0, dims=[1]).contiguous()
    _replay_and_compare(run, lambda: run(qx), [idx, o0, o1, o2])


def test_prefill_anchor_and_reuse_in_a_graph():
    kas = _kas()
    w = inputgen.custom("prefill", 1, 8, 2, 128, 1024, "bf16", wid=32, n_layers=2, anchors=(0,))
    maps = inputgen.head_maps(w)
    (q0, k0, v0), (q1, k1, v1) = (inputgen.layer_inputs(w, l, DEV) for l in range(2))
    hm1 = torch.as_tensor(maps[1], device=DEV)
    d = kas.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.topk_pct, torch.bfloat16)
    total = int(kas.prefill_offsets(d)[-1])
    idx = torch.empty((w.batch, w.n_kv_heads, total), dtype=torch.int32, device=DEV)
    o0, o1, od = (torch.empty_like(q0) for _ in range(3))
    ws_a = torch.empty(kas.workspace_size(d, kas.OP_PREFILL_ANCHOR), dtype=torch.uint8, device=DEV)
    ws_r = torch.empty(max(256, kas.workspace_size(d, kas.OP_PREFILL_REUSE)), dtype=torch.uint8, device=DEV)
    _say(f"[graph prefill] N={w.seq_len}: anchor + reuse + dense")

    def run(qa=q0):
        kas.prefill_anchor(qa, k0, v0, w.topk_pct, idx_out=idx, o=o0, ws=ws_a)
        kas.prefill_reuse(q1, k1, v1, idx, hm1, w.topk_pct, o=o1, ws=ws_r)
        kas.prefill_dense(qa, k0, v0, o=od)

    qx = torch.flip(q0, dims=[1]).contiguous()
    _replay_and_compare(run, lambda: run(qx), [idx, o0, o1, od])


def test_paged_calls_in_a_graph():
    """The paged decode translation pass and the paged prefill page copy are
    capturable too."""
    kas = _kas()
    from test_gpu_kvcache import _paged
    wd = inputgen.custom("decode", 2, 8, 2, 128, 3000, "bf16", wid=33)
    q, k, v = inputgen.layer_inputs(wd, 0, DEV)
    kp, vp, bt = _paged(k, v, 64, seed=5)
    lens = torch.as_tensor(np.array([3000, 1777], np.int32), device=DEV)
    kd = kas.decode_k(wd.seq_len, wd.topk_pct)
    idx = torch.empty((wd.batch, wd.n_kv_heads, kd), dtype=torch.int32, device=DEV)
    o, orr = torch.empty_like(q), torch.empty_like(q)
    over, cache = kas.binding._cache(q, kp, lens, bt, wd.seq_len)
    dd = kas.binding._decode_desc(q, kp, wd.topk_pct, 0.0, over, o)
    ws_a = kas.binding._ws_kv(dd, cache, kas.OP_DECODE_ANCHOR, None, DEV)
    ws_r = kas.binding._ws_kv(dd, cache, kas.OP_DECODE_REUSE, None, DEV)
    hm = torch.as_tensor(np.array([1, 0], np.int32), device=DEV)
    wp = inputgen.custom("prefill", 2, 8, 2, 128, 512, "bf16", wid=34)
    pq, pk, pv = inputgen.layer_inputs(wp, 0, DEV)
    pkp, pvp, pbt = _paged(pk, pv, 32, seed=6)
    plens = torch.as_tensor(np.array([512, 320], np.int32), device=DEV)
    po = torch.empty_like(pq)
    pdesc, pcache = kas.binding._prefill_desc(pq, pkp, 100, 0.0, plens, pbt, pq)
    ws_p = kas.binding._ws_kv(pdesc, pcache, kas.OP_PREFILL_DENSE, None, DEV)
    _say("[graph paged] decode anchor + reuse (P 64), prefill dense (P 32), varlen")

    def run(qa=q, pqa=pq):
        kas.decode_anchor(qa, kp, vp, wd.topk_pct, idx_out=idx, o=o, ws=ws_a, seq_lens=lens, block_table=bt,
                          seq_len=wd.seq_len)
        kas.decode_reuse(qa, kp, vp, idx, hm, wd.topk_pct, o=orr, ws=ws_r, seq_lens=lens, block_table=bt,
                         seq_len=wd.seq_len)
        kas.prefill_dense(pqa, pkp, pvp, o=po, seq_lens=plens, block_table=pbt, ws=ws_p)

    qx, pqx = torch.flip(q, dims=[1]).contiguous(), torch.flip(pq, dims=[1]).contiguous()
    # entries the calls leave unspecified (index slots past the shorter
    # sequence's count, rows past the shorter prompt) keep the reset values
    _replay_and_compare(run, lambda: run(qx, pqx), [idx, o, orr, po])
