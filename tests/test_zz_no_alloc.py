"""kas_decode_reuse_noalloc through the C ABI: the same decode reuse layer as
kas_decode_reuse with a caller workspace, but with its split partials in the
library's static per-GPU buffer. Two calls in a row (the second smaller,
reading what the first left in the buffer) must each give exactly the bits of
the workspace call, and match the oracle."""
import numpy as np
import pytest
import torch

import inputgen
import oracle
from parity_util import TOL, max_abs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np(t):
    return t.detach().float().cpu().numpy()


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_reuse_matches_workspace_call(order):
    import sparse_attention_long_anchor_amd as kas
    shapes = [(4, 32, 8, 128, 32768, "bf16"), (1, 8, 2, 64, 3000, "bf16")]
    if order == "small_then_large":
        shapes = shapes[::-1]
    for i, (B, Hq, Hkv, D, N, dt) in enumerate(shapes):
        w = inputgen.custom("decode", B, Hq, Hkv, D, N, dt, wid=120 + i)
        q, k, v = inputgen.layer_inputs(w, 0, DEV)
        q1, k1, v1 = inputgen.layer_inputs(w, 1, DEV)
        print(f"[noalloc] call {i + 1}: B={B} Hq={Hq} Hkv={Hkv} D={D} N={N}", flush=True)
        idx, _ = kas.decode_anchor(q, k, v, 10)
        hm = torch.as_tensor(np.arange(Hkv, dtype=np.int32)[::-1].copy(), device=DEV)
        ref = kas.decode_reuse(q1, k1, v1, idx, hm, 10)
        o = torch.full_like(q1, 3.0)
        got = kas.decode_reuse_noalloc(q1, k1, v1, idx, hm, 10, o=o)
        torch.cuda.synchronize()
        assert got.data_ptr() == o.data_ptr()
        assert torch.equal(got, ref)
        err = max_abs(_np(got), oracle.decode_reuse(_np(q1), _np(k1), _np(v1), idx.cpu().numpy(), hm.cpu().numpy()))
        assert err <= TOL[dt]


def test_noalloc_rejects_calls_beyond_its_buffer():
    import sparse_attention_long_anchor_amd as kas
    # 1024 sequences x 64 query heads of split partials need more than the buffer
    q = torch.zeros((1024, 64, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((1, 8, 64, 128), dtype=torch.bfloat16, device=DEV).expand(1024, 8, 64, 128)
    idx = torch.zeros((1024, 8, 6), dtype=torch.int32, device=DEV)
    d = kas.make_desc(1024, 64, 8, 128, 64, 10, torch.bfloat16)
    assert kas.workspace_size(d, kas.OP_DECODE_REUSE) > kas.NOALLOC_SCRATCH_BYTES
    with pytest.raises(kas.KasError) as e:
        kas.decode_reuse_noalloc(q, k, k, idx, None, 10)
    assert e.value.status == 2 and "static buffer" in str(e.value)
