"""Seeded synthetic inputs for the Kascade sparse-attention hot path.

This module is shared by the test harness, the benchmark and the CPU
oracle's tests. It only draws random tensors and plants structure in them;
it computes nothing the method computes (no softmax, no pooling, no
selection, no attention).

Workloads (shapes follow the Llama-3.1-8B / Qwen3-8B attention geometry the
Kascade README evaluates, page "microsoft/kascade", sections "Running
Evaluations" and "Kernel Benchmarks"):

  tiny_decode_2k        2 layers, B 1, Hq 8 / Hkv 2, D 64, N 2048, fp32
  llama8b_decode_32k    32 layers, anchors {0,2,8,13,22}, B 1, Hq 32 / Hkv 8,
                        D 128, N 32768, bf16
  llama8b_decode_128k   as above with B 4, N 131072
  qwen8b_prefill_32k    36 layers, anchors {0,3,9,17,27}, B 1, Hq 32 / Hkv 8,
                        D 128, N 32768, bf16, tile 32
  llama8b_prefill_128k  32 layers, anchors {0,2,8,13,22}, N 131072, tile 32

Value recipe (per layer): Q, K, V ~ N(0, 1) in fp32 from a torch generator
seeded with 1000 * workload_id + layer. For every (batch, KV head) a set of
heavy key positions (1 % of N, 16 for the tiny workload) drawn from [4, N)
gets K_j <- K_j + 4 * u, and (except for the tiny workload) the four sink
positions 0..3 get K_j <- K_j + 16 * u, where u is the unit vector of the mean
of the group's query vectors (decode: its G query heads; prefill: all prompt
queries of its G heads). The heavy set of layer l+1 keeps a random 80 % of
layer l's set and draws the rest fresh. Planting happens in fp32, followed by
one round-to-nearest-even cast to the storage dtype. Head maps are drawn per
reuse layer uniformly over the anchor's KV heads. Positions and head maps come
from numpy's default_rng(workload_id).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # seed namespace
    phase: str               # "decode" or "prefill"
    n_layers: int
    anchors: tuple
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    dtype: str               # "f32", "bf16" or "f16"
    topk_pct: int = 10
    tile: int = 32
    n_heavy: int = 0         # per (batch, KV head, layer)
    sinks: bool = True
    heavy_scale: float = 4.0
    sink_scale: float = 16.0
    overlap: float = 0.8

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self):
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.dtype]


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_decode_2k", 0, "decode", 2, (0,), 1, 8, 2, 64, 2048, "f32",
                 n_heavy=16, sinks=False),
        Workload("llama8b_decode_32k", 1, "decode", 32, (0, 2, 8, 13, 22), 1, 32, 8, 128,
                 32768, "bf16", n_heavy=328),
        Workload("llama8b_decode_128k", 2, "decode", 32, (0, 2, 8, 13, 22), 4, 32, 8, 128,
                 131072, "bf16", n_heavy=1311),
        Workload("qwen8b_prefill_32k", 3, "prefill", 36, (0, 3, 9, 17, 27), 1, 32, 8, 128,
                 32768, "bf16", n_heavy=328),
        Workload("llama8b_prefill_128k", 4, "prefill", 32, (0, 2, 8, 13, 22), 1, 32, 8, 128,
                 131072, "bf16", n_heavy=1311),
    ]
}


def custom(phase: str, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
           seq_len: int, dtype: str, *, wid: int = 100, n_heavy: Optional[int] = None,
           sinks: bool = True, topk_pct: int = 10, n_layers: int = 2,
           anchors: Sequence[int] = (0,)) -> Workload:
    """A workload of arbitrary shape with the same value recipe (for tests)."""
    if n_heavy is None:
        n_heavy = max(1, round(0.01 * seq_len))
    n_heavy = min(n_heavy, max(0, seq_len - 4))
    return Workload(f"custom_{phase}_{wid}", wid, phase, n_layers, tuple(anchors), batch,
                    n_q_heads, n_kv_heads, head_dim, seq_len, dtype, topk_pct=topk_pct,
                    n_heavy=n_heavy, sinks=sinks)


def heavy_positions(w: Workload) -> List[np.ndarray]:
    """Per layer, int64 [B, Hkv, n_heavy] heavy key positions in [4, N)."""
    rng = np.random.default_rng(w.wid)
    lo, n = 4, w.seq_len
    pool = max(0, n - lo)
    h = min(w.n_heavy, pool)
    out = []
    prev = None
    for _layer in range(w.n_layers):
        cur = np.zeros((w.batch, w.n_kv_heads, h), dtype=np.int64)
        for b in range(w.batch):
            for g in range(w.n_kv_heads):
                if h == 0:
                    continue
                if prev is None:
                    cur[b, g] = lo + rng.choice(pool, size=h, replace=False)
                else:
                    keep_n = int(round(w.overlap * h))
                    keep = rng.choice(prev[b, g], size=keep_n, replace=False)
                    taken = np.zeros(pool, dtype=bool)
                    taken[keep - lo] = True
                    free = np.flatnonzero(~taken)
                    fresh = lo + rng.choice(free, size=h - keep_n, replace=False)
                    cur[b, g] = np.concatenate([keep, fresh])
        out.append(cur)
        prev = cur
    return out


def head_maps(w: Workload) -> List[Optional[np.ndarray]]:
    """Per layer: None for anchor layers, else int32 [Hkv] map to anchor KV heads."""
    rng = np.random.default_rng(10_000 + w.wid)
    maps: List[Optional[np.ndarray]] = []
    for layer in range(w.n_layers):
        if layer in w.anchors:
            maps.append(None)
        else:
            maps.append(rng.integers(0, w.n_kv_heads, size=w.n_kv_heads).astype(np.int32))
    return maps


def _plant(k: torch.Tensor, q_group_mean: torch.Tensor, pos: np.ndarray, w: Workload) -> None:
    """k: fp32 [B, Hkv, N, D]; q_group_mean: fp32 [B, Hkv, D]."""
    u = q_group_mean / q_group_mean.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    B, Hkv = k.shape[0], k.shape[1]
    if pos.shape[-1] > 0:
        idx = torch.as_tensor(pos, device=k.device)
        for b in range(B):
            for g in range(Hkv):
                k[b, g, idx[b, g]] += w.heavy_scale * u[b, g]
    if w.sinks:
        ns = min(4, w.seq_len)
        k[:, :, :ns, :] += w.sink_scale * u[:, :, None, :]


def layer_inputs(w: Workload, layer: int, device="cpu", positions=None):
    """Q, K, V for one layer, already cast to the workload's dtype.

    decode : Q [B, Hq, D],    K/V [B, Hkv, N, D]
    prefill: Q [B, Hq, N, D], K/V [B, Hkv, N, D]
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 * w.wid + layer)
    B, Hq, Hkv, D, N = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seq_len
    G = Hq // Hkv
    if w.phase == "decode":
        q = torch.randn((B, Hq, D), generator=gen, device=device, dtype=torch.float32)
        qmean = q.view(B, Hkv, G, D).mean(dim=2)
    else:
        q = torch.randn((B, Hq, N, D), generator=gen, device=device, dtype=torch.float32)
        qmean = q.view(B, Hkv, G, N, D).mean(dim=(2, 3))
    k = torch.randn((B, Hkv, N, D), generator=gen, device=device, dtype=torch.float32)
    v = torch.randn((B, Hkv, N, D), generator=gen, device=device, dtype=torch.float32)
    if positions is None:
        positions = heavy_positions(w)
    _plant(k, qmean, positions[layer], w)
    dt = w.torch_dtype
    return q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous()


def anchor_of(w: Workload, layer: int) -> int:
    """The anchor layer whose indices a layer uses (itself if an anchor).

    Reading taken: a reuse layer uses the nearest anchor at or before it.
    """
    best = None
    for a in sorted(w.anchors):
        if a <= layer:
            best = a
    if best is None:
        raise ValueError(f"layer {layer} precedes every anchor {w.anchors}")
    return best
