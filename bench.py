#!/usr/bin/env python3
"""Benchmark of the Kascade sparse-attention hot path on one MI355X.

One step = one decode step of the 32-layer Llama-3.1-8B-shaped schedule at
131072 context (batch 4, anchors {0,2,8,13,22}, Top-k 10 %) followed by one
prefill of the 32-layer Llama-3.1-8B-shaped schedule at 131072 tokens (tile 32,
Top-k 10 %). Every layer has its own synthetic, seeded Q/K/V resident in HBM
before timing starts; anchor layers write their index sets, reuse layers read
the nearest preceding anchor's sets through their head map.

Prints one JSON line. `value` is the decode step's algorithmic HBM throughput
(GB/s over all layers); per-layer microseconds, prefill TFLOP/s, the roofline
of the dominant kernel (device time from HIP events recorded by the library
around each launch during the timed steps) and the CPU oracle baseline are
reported alongside. After the timed steps, the same layers run through the
library's dense attention (every key; causal in prefill), the comparison the
pages state their speed-ups against, and the speed-up of the Kascade step over
the dense step is reported as well (outside the timed region).
"""
import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn μs/layer + HBM GB/s at 128K ctx, Top-k 10%; prefill attn TFLOP/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic work

def decode_work(w, k):
    """Algorithmic bytes of one decode layer call and of its main kernels."""
    B, Hq, Hkv, D, N, G = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.group
    s = 2 if w.dtype == "bf16" else 4
    qo = 2 * B * Hq * D * s
    reuse = B * Hkv * k * 2 * D * s + B * Hkv * k * 4 + qo
    anchor = B * Hkv * N * D * s + B * Hkv * k * D * s + B * Hkv * k * 4 + qo
    kern = {
        "decode_attn": B * Hkv * k * (2 * D * s + 4) + B * Hq * D * s,
        "decode_attn_anchor": B * Hkv * k * (D * s + 4 + 4 * G),
        "decode_score": B * Hkv * N * D * s + B * Hq * D * s,
    }
    return reuse, anchor, kern


def dense_work(wd, wp):
    """Algorithmic work of one dense layer: decode bytes (all of K and V, Q,
    O), prefill flops (causal Q.K^T and P.V)."""
    s = 2 if wd.dtype == "bf16" else 4
    dec = wd.batch * wd.n_kv_heads * wd.seq_len * 2 * wd.head_dim * s + 2 * wd.batch * wd.n_q_heads * wd.head_dim * s
    pre = 2 * wp.head_dim * wp.n_q_heads * wp.batch * wp.seq_len * (wp.seq_len + 1)
    return dec, pre


def prefill_work(w, offsets):
    B, Hq, D, N = w.batch, w.n_q_heads, w.head_dim, w.seq_len
    T = N // 32
    sum_k = int(offsets[-1])
    stats = D * Hq * B * N * (N + 1)                       # causal Q.K^T, 2 flop / MAC
    pool = 2 * D * Hq * B * 1024 * T * (T - 1) // 2        # Q.K^T over keys before each tile
    attn = 4 * D * Hq * B * (32 * sum_k + 528 * T)         # Q.K^T + P.V over set + diagonal
    return {"prefill_stats": stats, "prefill_pool": pool, "prefill_attn": attn}


# ---------------------------------------------------------------- setup

def build_decode(w, dev, torch, inputgen, kas):
    pos = inputgen.heavy_positions(w)
    maps = inputgen.head_maps(w)
    layers = []
    for l in range(w.n_layers):
        q, k, v = inputgen.layer_inputs(w, l, dev, pos)
        hm = None if maps[l] is None else torch.as_tensor(maps[l], device=dev)
        layers.append((q, k, v, hm))
    kd = kas.decode_k(w.seq_len, w.topk_pct)
    idx = {a: torch.empty((w.batch, w.n_kv_heads, kd), dtype=torch.int32, device=dev) for a in w.anchors}
    o = torch.empty_like(layers[0][0])
    d = kas.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.topk_pct, w.torch_dtype)
    ws_a = torch.empty(kas.workspace_size(d, kas.OP_DECODE_ANCHOR), dtype=torch.uint8, device=dev)
    ws_r = torch.empty(kas.workspace_size(d, kas.OP_DECODE_REUSE), dtype=torch.uint8, device=dev)
    return layers, idx, o, ws_a, ws_r, kd


def run_decode_step(w, st, inputgen, kas, events=None):
    layers, idx, o, ws_a, ws_r, _ = st
    for l, (q, k, v, hm) in enumerate(layers):
        if events is not None:
            events[l][0].record()
        if l in w.anchors:
            kas.decode_anchor(q, k, v, w.topk_pct, idx_out=idx[l], o=o, ws=ws_a)
        else:
            kas.decode_reuse(q, k, v, idx[inputgen.anchor_of(w, l)], hm, w.topk_pct, o=o, ws=ws_r)
        if events is not None:
            events[l][1].record()


def build_prefill(w, dev, torch, inputgen, kas):
    pos = inputgen.heavy_positions(w)
    maps = inputgen.head_maps(w)
    layers = []
    for l in range(w.n_layers):
        q, k, v = inputgen.layer_inputs(w, l, dev, pos)
        hm = None if maps[l] is None else torch.as_tensor(maps[l], device=dev)
        layers.append((q, k, v, hm))
    d = kas.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.topk_pct, w.torch_dtype)
    off = kas.prefill_offsets(d)
    idx = {a: torch.empty((w.batch, w.n_kv_heads, int(off[-1])), dtype=torch.int32, device=dev)
           for a in w.anchors}
    o = torch.empty_like(layers[0][0])
    ws_a = torch.empty(kas.workspace_size(d, kas.OP_PREFILL_ANCHOR), dtype=torch.uint8, device=dev)
    ws_r = torch.empty(max(256, kas.workspace_size(d, kas.OP_PREFILL_REUSE)), dtype=torch.uint8, device=dev)
    return layers, idx, o, ws_a, ws_r, off


def run_prefill_step(w, st, inputgen, kas, events=None):
    layers, idx, o, ws_a, ws_r, _ = st
    for l, (q, k, v, hm) in enumerate(layers):
        if events is not None:
            events[l][0].record()
        if l in w.anchors:
            kas.prefill_anchor(q, k, v, w.topk_pct, idx_out=idx[l], o=o, ws=ws_a)
        else:
            kas.prefill_reuse(q, k, v, idx[inputgen.anchor_of(w, l)], hm, w.topk_pct, o=o, ws=ws_r)
        if events is not None:
            events[l][1].record()


# ---------------------------------------------------------------- CPU oracle baseline

def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_threads():
    return int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()


def cpu_decode_sample(w, st, budget_s, inputgen):
    """The (untuned) oracle over the first layers of a decode schedule (full
    B, Hkv, N per layer) until the budget is spent: algorithmic GB/s."""
    import oracle
    layers = st[0]
    reuse_b, anchor_b, _ = decode_work(w, oracle.decode_k(w.seq_len, w.topk_pct))
    maps = inputgen.head_maps(w)
    f = lambda t: t.float().cpu().numpy()
    done, spent, n, cur = 0, 0.0, 0, None
    for l, (q, k, v, _) in enumerate(layers):
        if n >= 2 and spent > budget_s:
            break
        qn, kn, vn = f(q), f(k), f(v)
        t0 = time.perf_counter()
        if l in w.anchors:
            cur, _, _ = oracle.decode_anchor(qn, kn, vn, w.topk_pct)
            done += anchor_b
        else:
            oracle.decode_reuse(qn, kn, vn, cur, maps[l])
            done += reuse_b
        spent += time.perf_counter() - t0
        n += 1
    return {"value": round(done / spent / 1e9, 4), "unit": "GB/s", "layers": n, "seconds": round(spent, 2),
            "sample": f"{w.name}: first {n} of {w.n_layers} layers (full B, Hkv, N each)"}


def cpu_prefill_sample(w, st, tiles, inputgen):
    """The oracle on a few tiles of the schedule's first anchor layer and of
    the first reuse layer after it (all KV heads): measured TFLOP/s, and the
    full layer's time extrapolated linearly in flops (labelled as such)."""
    import oracle
    layers, idx = st[0], st[1]
    f = lambda t: t.float().cpu().numpy()
    D, rows = w.head_dim, w.batch * w.n_q_heads * 32
    T = w.seq_len // 32
    off = oracle.prefill_offsets(w.seq_len, 32, w.topk_pct)
    work = prefill_work(w, off)
    res = {}
    a0 = min(w.anchors)
    r0 = next(l for l in range(w.n_layers) if l not in w.anchors)
    maps = inputgen.head_maps(w)
    anc_idx = idx[a0].cpu().numpy()
    for kind, layer in (("anchor_layer", a0), ("reuse_layer", r0)):
        q, k, v, _ = layers[layer]
        kn, vn = f(k), f(v)
        flops, spent = 0.0, 0.0
        for t in tiles:
            qr = f(q[:, :, 32 * t: 32 * t + 32])
            kt = int(off[t + 1] - off[t])
            t0 = time.perf_counter()
            if kind == "anchor_layer":
                oracle.prefill_anchor(qr, kn, vn, w.topk_pct, t0=t, t1=t + 1)
                flops += 2 * D * rows * (32 * t + 16.5) + 2 * D * rows * 32 * t + 4 * D * rows * (kt + 16.5)
            else:
                oracle.prefill_reuse(qr, kn, vn, anc_idx, maps[layer], w.topk_pct, t0=t, t1=t + 1)
                flops += 4 * D * rows * (kt + 16.5)
            spent += time.perf_counter() - t0
        full = (work["prefill_stats"] + work["prefill_pool"] + work["prefill_attn"]) if kind == "anchor_layer" \
            else work["prefill_attn"]
        rate = flops / spent
        res[kind] = {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "tiles": list(tiles), "of_tiles": T,
                     "seconds": round(spent, 2),
                     "extrapolated_full_layer_s": {"value": round(full / rate, 1),
                                                   "note": "linear in flops from the measured tiles, not measured"}}
    return res


def cpu_baseline(wd, dec_state, wp, pre_state, budget_s, inputgen, extra):
    """The oracle (plain fp64 C with OpenMP, never tuned) on bounded samples of
    the same resident workloads, on this host's cores; `value` is the 128K
    decode schedule's algorithmic GB/s (the metric), the rest are per config."""
    dec = cpu_decode_sample(wd, dec_state, budget_s * 0.4, inputgen)
    T = wp.seq_len // 32
    pre = cpu_prefill_sample(wp, pre_state, (T - 1, T // 2), inputgen)
    per = dict(extra)
    per[wd.name] = dec
    per[wp.name] = pre
    return {
        "value": dec["value"], "unit": "GB/s", "cores": _oracle_threads(), "kind": "oracle",
        "precision": "fp64", "cpu_model": _cpu_model(),
        "sample": f"{dec['sample']}; oracle fp64 C with OpenMP; {dec['seconds']} s",
        "prefill": {"value": pre["anchor_layer"]["value"], "unit": "TFLOP/s",
                    "sample": f"{wp.name} anchor layer {min(wp.anchors)}, tiles {pre['anchor_layer']['tiles']} "
                              f"(all KV heads)"},
        "per_config": per,
    }


# ---------------------------------------------------------------- the other workloads

OTHER_CONFIGS = ("tiny_decode_2k", "llama8b_decode_32k", "qwen8b_prefill_32k")


def graph_step_ms(w, st, run, steps, torch, inputgen, kas):
    """Mean device time of one step captured in a HIP graph and replayed (the
    step's calls only enqueue kernels on the current stream, so they capture
    as they are); small decode steps are bound by host launch work otherwise."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(w, st, inputgen, kas)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(w, st, inputgen, kas)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(max(steps, 3))]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    ms = _mean([a.elapsed_time(b) for a, b in ev])
    del g
    return ms


def config_record(name, steps, warmup, dev, torch, inputgen, kas, cpu_budget):
    """One workload's own schedule (every layer resident): `warmup` untimed
    steps, `steps` steps with events around each step, the same steps with an
    event pair around every layer (anchor / reuse layer times), and one pass
    with the library's per-launch timing for the kernels' rooflines. The
    oracle is timed on a sample of the same layers when cpu_budget > 0."""
    w = inputgen.WORKLOADS[name]
    dec = w.phase == "decode"
    log(f"[bench] config {name}: generating {w.n_layers} layers")
    st = (build_decode if dec else build_prefill)(w, dev, torch, inputgen, kas)
    run = run_decode_step if dec else run_prefill_step
    gc.collect()
    for _ in range(warmup):
        run(w, st, inputgen, kas)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e in ev:
        e[0].record()
        run(w, st, inputgen, kas)
        e[1].record()
    torch.cuda.synchronize()
    step_ms = _mean([a.elapsed_time(b) for a, b in ev])
    log(f"[bench] config {name}: eager steps (ms) {[round(a.elapsed_time(b), 3) for a, b in ev]}")
    graph_ms = graph_step_ms(w, st, run, steps, torch, inputgen, kas) if dec else None
    lay = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(w.n_layers)] for _ in range(steps)]
    for s_ in range(steps):
        run(w, st, inputgen, kas, lay[s_])
    torch.cuda.synchronize()
    per_layer = [_mean([lay[s_][l][0].elapsed_time(lay[s_][l][1]) for s_ in range(steps)]) for l in range(w.n_layers)]
    anc = [per_layer[l] for l in range(w.n_layers) if l in w.anchors]
    reu = [per_layer[l] for l in range(w.n_layers) if l not in w.anchors]
    kas.profile_reset()
    kas.profile_enable(True)
    run(w, st, inputgen, kas)
    torch.cuda.synchronize()
    kas.profile_enable(False)
    kern = {}
    for kname in kas.profile_names():
        ms, n = kas.profile_query(kname)
        if n:
            kern[kname] = (ms, n)
    rec = {"workload": name, "batch": w.batch, "seq_len": w.seq_len, "layers": w.n_layers,
           "anchors": list(w.anchors), "topk_pct": w.topk_pct, "dtype": w.dtype, "steps": steps}
    roof = []
    if dec:
        kd = st[5]
        reuse_b, anchor_b, kern_b = decode_work(w, kd)
        step_b = len(anc) * anchor_b + len(reu) * reuse_b
        rec.update({
            "k": kd,
            "us_per_layer": {"anchor": round(1e3 * _mean(anc), 3), "reuse": round(1e3 * _mean(reu), 3),
                             "schedule_mean": round(1e3 * step_ms / w.n_layers, 3)},
            "GB_per_s": {"anchor": _rate(anchor_b, _mean(anc) * 1e-3, 1e9),
                         "reuse": _rate(reuse_b, _mean(reu) * 1e-3, 1e9),
                         "step": _rate(step_b, step_ms * 1e-3, 1e9)},
            "ms_per_step": round(step_ms, 4),
            "tokens_per_s": round(w.batch / (step_ms * 1e-3), 2),
            "graph": {"ms_per_step": round(graph_ms, 4), "tokens_per_s": round(w.batch / (graph_ms * 1e-3), 2),
                      "GB_per_s": _rate(step_b, graph_ms * 1e-3, 1e9),
                      "note": "the whole step captured once in a HIP graph and replayed: no host launch work"}})
        ops = {"decode_attn": len(reu), "decode_attn_anchor": len(anc), "decode_score": len(anc)}
        for kname, b in kern_b.items():
            if kname in kern:
                roof.append(_roof_entry(kname, "hbm", b * ops[kname], kern[kname], HBM_PEAK_GBS, "GB/s", 1e9))
    else:
        off = st[5]
        work = prefill_work(w, off)
        anc_flops = work["prefill_stats"] + work["prefill_pool"] + work["prefill_attn"]
        rec.update({
            "index_entries_per_kv_head": int(off[-1]),
            "ms_per_layer": {"anchor": round(_mean(anc), 4), "reuse": round(_mean(reu), 4),
                             "schedule_mean": round(step_ms / w.n_layers, 4)},
            "TFLOP_per_s": {"anchor_layer": _rate(anc_flops, _mean(anc) * 1e-3, 1e12),
                            "reuse_layer": _rate(work["prefill_attn"], _mean(reu) * 1e-3, 1e12)},
            "ms_per_step": round(step_ms, 3),
            "tokens_per_s": round(w.batch * w.seq_len / (step_ms * 1e-3), 1)})
        ops = {"prefill_stats": len(anc), "prefill_pool": len(anc), "prefill_attn": w.n_layers}
        for kname, fl in work.items():
            if kname in kern:
                roof.append(_roof_entry(kname, "mfma", fl * ops[kname], kern[kname], BF16_PEAK_TFLOPS,
                                        "TFLOP/s", 1e12))
    for r in roof:
        r["frac"] = round(r["achieved"] / r["peak"], 4)
    rec["roofline"] = [{k: r[k] for k in ("kernel", "bound", "achieved", "unit", "frac", "avg_us")} for r in roof]
    if not dec:
        qk = [r for r in roof if r["kernel"] in ("prefill_stats", "prefill_pool")]
        rec["qkt_passes_vs_half_peak"] = {r["kernel"]: {"ms": round(r["avg_us"] / 1e3, 3), "frac": r["frac"],
                                                        "meets_0.5": r["frac"] >= 0.5} for r in qk}
    rec["kernels"] = {n_: {"total_ms": round(ms, 3), "launches": c, "avg_us": round(1e3 * ms / c, 3)}
                      for n_, (ms, c) in sorted(kern.items(), key=lambda x: -x[1][0])}
    cpu = None
    if cpu_budget > 0:
        if dec:
            cpu = cpu_decode_sample(w, st, cpu_budget, inputgen)
        else:
            T = w.seq_len // 32
            cpu = cpu_prefill_sample(w, st, (T - 1, T // 2), inputgen)
    log(f"[bench] config {name}: step {step_ms:.3f} ms")
    del st
    torch.cuda.empty_cache()
    return rec, cpu


# ---------------------------------------------------------------- main

def main():
    gc.disable()   # collected explicitly between measurements
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--phase", choices=["both", "decode", "prefill"], default="both")
    ap.add_argument("--decode-workload", default="llama8b_decode_128k")
    ap.add_argument("--prefill-workload", default="llama8b_prefill_128k")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-attention comparison")
    ap.add_argument("--no-variants", action="store_true", help="skip the selection-variant timings")
    ap.add_argument("--no-fp16", action="store_true", help="skip the fp16 layer timings")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache timings")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config records of the other workloads (tiny 2K decode, 32K decode, "
                         "32K Qwen prefill)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the reference ceilings (a large bf16 GEMM, a device copy)")
    ap.add_argument("--layers", type=int, default=0,
                    help="profiling runs only: keep the first N layers of each schedule")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="profiling runs only: one device copy of this size before timing, as the "
                         "reference for hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import inputgen
    import sparse_attention_long_anchor_amd as kas

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wd = inputgen.WORKLOADS[args.decode_workload]
    wp = inputgen.WORKLOADS[args.prefill_workload]
    if args.layers:
        import dataclasses
        wd = dataclasses.replace(wd, n_layers=min(args.layers, wd.n_layers))
        wp = dataclasses.replace(wp, n_layers=min(args.layers, wp.n_layers))
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 19
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")
        del src, dst
    do_dec = args.phase in ("both", "decode")
    do_pre = args.phase in ("both", "prefill")

    dec_state = pre_state = None
    if do_dec:
        log(f"[bench] generating {wd.name} ({wd.n_layers} layers)")
        dec_state = build_decode(wd, dev, torch, inputgen, kas)
    if do_pre:
        log(f"[bench] generating {wp.name} ({wp.n_layers} layers)")
        pre_state = build_prefill(wp, dev, torch, inputgen, kas)
    torch.cuda.synchronize()
    # the collector runs only between measurements: a collection inside a timed
    # host-bound step would leave the GPU idle for milliseconds
    gc.collect()

    for i in range(args.warmup):
        if do_dec:
            run_decode_step(wd, dec_state, inputgen, kas)
        if do_pre:
            run_prefill_step(wp, pre_state, inputgen, kas)
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")

    # Pass 1 (the timed region): events only around each phase of a step, so
    # that nothing is enqueued between layers. Pass 2: the same steps again
    # with events between layers, for the anchor / reuse layer breakdown (an
    # event record between two layers adds a few microseconds of device
    # time, so step figures come from pass 1). Pass 3: the library's
    # per-launch events on (hipExtLaunchKernel start/stop stamps), for
    # per-kernel device times.
    def ev_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dec_ev = [ev_pair() for _ in range(args.steps)] if do_dec else None
    pre_ev = [ev_pair() for _ in range(args.steps)] if do_pre else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if do_dec:
            dec_ev[s][0].record()
            run_decode_step(wd, dec_state, inputgen, kas)
            dec_ev[s][1].record()
        if do_pre:
            pre_ev[s][0].record()
            run_prefill_step(wp, pre_state, inputgen, kas)
            pre_ev[s][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {wall:.3f} s")

    dec_lay = [[ev_pair() for _ in range(wd.n_layers)] for _ in range(args.steps)] if do_dec else None
    pre_lay = [[ev_pair() for _ in range(wp.n_layers)] for _ in range(args.steps)] if do_pre else None
    for s in range(args.steps):
        if do_dec:
            run_decode_step(wd, dec_state, inputgen, kas, dec_lay[s])
        if do_pre:
            run_prefill_step(wp, pre_state, inputgen, kas, pre_lay[s])
    torch.cuda.synchronize()
    log(f"[bench] per-layer pass: {args.steps} steps")

    kas.profile_reset()
    kas.profile_enable(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(args.steps):
        if do_dec:
            run_decode_step(wd, dec_state, inputgen, kas)
        if do_pre:
            run_prefill_step(wp, pre_state, inputgen, kas)
    torch.cuda.synchronize()
    kas.profile_enable(False)
    wall_k = time.perf_counter() - t1
    log(f"[bench] per-kernel timing pass: {args.steps} steps in {wall_k:.3f} s")

    # The decode step again, captured once in a HIP graph and replayed (how a
    # serving loop would run it: the same kernels on the same inputs, without
    # host launch work). Reported beside the eager figures; the replay's index
    # sets and output are compared bit for bit with the eager step's.
    dec_graph = None
    if do_dec:
        _, d_idx, d_o, _, _, _ = dec_state
        run_decode_step(wd, dec_state, inputgen, kas)
        torch.cuda.synchronize()
        ref_o = d_o.clone()
        ref_idx = {a_: t_.clone() for a_, t_ in d_idx.items()}
        g_ms = graph_step_ms(wd, dec_state, run_decode_step, args.steps, torch, inputgen, kas)
        same = bool(torch.equal(ref_o, d_o)) and all(torch.equal(ref_idx[a_], d_idx[a_]) for a_ in ref_idx)
        dec_graph = (g_ms, same)
        log(f"[bench] decode step from a HIP graph: {g_ms:.4f} ms, outputs bit-identical to eager: {same}")

    kern_ms = {}
    for name in kas.profile_names():
        ms, n = kas.profile_query(name)
        if n:
            kern_ms[name] = (ms, n)

    out = {"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": " + ".join(([wd.name] if do_dec else []) + ([wp.name] if do_pre else [])),
                      "phase": args.phase}}
    out["kernel_timing_pass_ms_per_step"] = round(wall_k * 1e3 / args.steps, 4)
    if args.layers:
        out["config"]["layers_kept"] = args.layers
    roof = []
    if do_dec:
        kd = dec_state[5]
        reuse_b, anchor_b, kern_b = decode_work(wd, kd)
        lay_ms = [[a.elapsed_time(b) for (a, b) in step] for step in dec_lay]
        per_layer = [sum(x[l] for x in lay_ms) / args.steps for l in range(wd.n_layers)]
        anc = [per_layer[l] for l in range(wd.n_layers) if l in wd.anchors]
        reu = [per_layer[l] for l in range(wd.n_layers) if l not in wd.anchors]
        step_ms = _mean([a.elapsed_time(b) for a, b in dec_ev])
        step_bytes = len(anc) * anchor_b + len(reu) * reuse_b
        gbs = step_bytes / (step_ms * 1e-3) / 1e9
        out["value"] = round(gbs, 3)
        out["decode"] = {
            "workload": wd.name, "batch": wd.batch, "seq_len": wd.seq_len, "layers": wd.n_layers,
            "anchors": list(wd.anchors), "topk_pct": wd.topk_pct, "k": kd,
            "us_per_layer": {"anchor": round(1e3 * _mean(anc), 3),
                             "reuse": round(1e3 * _mean(reu), 3),
                             "mean": round(1e3 * step_ms / wd.n_layers, 3),
                             "timing": "anchor, reuse: events between layers; mean: the step's own events"},
            "GB_per_s": {"anchor": _rate(anchor_b, _mean(anc) * 1e-3, 1e9),
                         "reuse": _rate(reuse_b, _mean(reu) * 1e-3, 1e9),
                         "step": round(gbs, 2)},
            "ms_per_step": round(step_ms, 4),
            "tokens_per_s": round(wd.batch / (step_ms * 1e-3), 2),
        }
        if dec_graph is not None:
            g_ms, same = dec_graph
            out["decode"]["graph"] = {
                "ms_per_step": round(g_ms, 4), "tokens_per_s": round(wd.batch / (g_ms * 1e-3), 2),
                "GB_per_s": round(step_bytes / (g_ms * 1e-3) / 1e9, 2),
                "bit_identical_to_eager": same,
                "note": "the whole step captured once in a HIP graph and replayed; value stays the eager figure"}
        n_anc, n_reu = len(anc) * args.steps, len(reu) * args.steps
        ops = {"decode_attn": n_reu, "decode_attn_anchor": n_anc, "decode_score": n_anc}
        for name, b in kern_b.items():
            if name in kern_ms:
                roof.append(_roof_entry(name, "hbm", b * ops[name], kern_ms[name], HBM_PEAK_GBS, "GB/s", 1e9))
    if do_pre:
        off = pre_state[5]
        work = prefill_work(wp, off)
        lay_ms = [[a.elapsed_time(b) for (a, b) in step] for step in pre_lay]
        per_layer = [sum(x[l] for x in lay_ms) / args.steps for l in range(wp.n_layers)]
        anc = [per_layer[l] for l in range(wp.n_layers) if l in wp.anchors]
        reu = [per_layer[l] for l in range(wp.n_layers) if l not in wp.anchors]
        step_ms = _mean([a.elapsed_time(b) for a, b in pre_ev])
        anc_flops = work["prefill_stats"] + work["prefill_pool"] + work["prefill_attn"]
        out["prefill"] = {
            "workload": wp.name, "batch": wp.batch, "seq_len": wp.seq_len, "layers": wp.n_layers,
            "anchors": list(wp.anchors), "topk_pct": wp.topk_pct, "index_entries_per_kv_head": int(off[-1]),
            "ms_per_layer": {"anchor": round(_mean(anc), 4), "reuse": round(_mean(reu), 4)},
            "TFLOP_per_s": {"anchor_layer": _rate(anc_flops, _mean(anc) * 1e-3, 1e12),
                            "reuse_layer": _rate(work["prefill_attn"], _mean(reu) * 1e-3, 1e12)},
            "ms_per_step": round(step_ms, 3),
            "tokens_per_s": round(wp.batch * wp.seq_len / (step_ms * 1e-3), 1),
        }
        n_anc, n_all = len(anc) * args.steps, wp.n_layers * args.steps
        ops = {"prefill_stats": n_anc, "prefill_pool": n_anc, "prefill_attn": n_all}
        for name, f in work.items():
            if name in kern_ms:
                roof.append(_roof_entry(name, "mfma", f * ops[name], kern_ms[name], BF16_PEAK_TFLOPS,
                                        "TFLOP/s", 1e12))
    for r in roof:
        r["frac"] = round(r["achieved"] / r["peak"], 4)
    out["kernels"] = {n: {"total_ms": round(ms, 3), "launches": c, "avg_us": round(1e3 * ms / c, 3)}
                      for n, (ms, c) in sorted(kern_ms.items(), key=lambda x: -x[1][0])}
    if roof:
        dom = max(roof, key=lambda r: r["total_ms"])
        traffic = _traffic(dom["kernel"])
        out["roofline"] = {"kernel": dom["kernel"], "bound": dom["bound"], "achieved": dom["achieved"],
                           "peak": dom["peak"], "unit": dom["unit"], "frac": dom["frac"], "traffic": traffic}
        for r in roof:
            if r["kernel"] == "decode_attn":
                out["roofline_decode_reuse"] = {"kernel": "decode_attn", "bound": "hbm", "achieved": r["achieved"],
                                                "peak": r["peak"], "unit": "GB/s", "frac": r["frac"],
                                                "traffic": _traffic("decode_attn")}
        out["roofline_all"] = [{k: r[k] for k in ("kernel", "bound", "achieved", "unit", "frac", "avg_us")}
                               for r in roof]
    if not args.no_dense:
        out["dense_baseline"], out["roofline_dense"] = dense_baseline(
            args, wd, dec_state, wp, pre_state, out, torch, kas, dev)
    if not args.no_variants:
        out["selection_variants"] = variant_timings(wd, dec_state, wp, pre_state, out, torch, kas, dev, inputgen)
    if not args.no_fp16:
        out["fp16"] = fp16_timings(wd if do_dec else None, wp if do_pre else None, dec_state, pre_state, dev,
                                   torch, inputgen, kas)
    if not args.no_paged and do_dec:
        out["paged_decode"] = paged_timings(wd, dec_state, dev, torch, inputgen, kas)
    if not args.no_paged and do_pre:
        out["paged_prefill"] = paged_prefill_timings(wp, pre_state, dev, torch, inputgen, kas)
    if not args.no_ceilings:
        out["ceilings"] = ceilings(torch, dev)
    cpu_extra = {}
    if not args.no_configs and not args.layers:
        out["configs"] = {}
        for name in OTHER_CONFIGS:
            w = inputgen.WORKLOADS[name]
            if (w.phase == "decode" and not do_dec) or (w.phase == "prefill" and not do_pre):
                continue
            budget = 0.0 if args.no_cpu_baseline else args.cpu_budget * 0.15
            rec, cpu = config_record(name, args.steps, max(1, args.warmup), dev, torch, inputgen, kas, budget)
            out["configs"][name] = rec
            if cpu is not None:
                cpu_extra[name] = cpu
    if not args.no_cpu_baseline and do_dec and do_pre:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wd, dec_state, wp, pre_state, args.cpu_budget, inputgen, cpu_extra)
    print(json.dumps(out), flush=True)


def dense_baseline(args, wd, dec_state, wp, pre_state, out, torch, kas, dev):
    """Every layer of the same resident workloads through the dense calls: one
    pass with per-layer events, one with the library's per-launch timing."""
    dec_b, pre_f = dense_work(wd, wp)
    res, roof = {}, []
    runs = []
    if dec_state is not None:
        layers, _, o, *_ = dec_state
        d = kas.make_desc(wd.batch, wd.n_q_heads, wd.n_kv_heads, wd.head_dim, wd.seq_len, wd.topk_pct,
                          wd.torch_dtype)
        ws = torch.empty(kas.workspace_size(d, kas.OP_DECODE_DENSE), dtype=torch.uint8, device=dev)
        runs.append(("decode", layers, lambda q, k, v, o=o, ws=ws: kas.decode_dense(q, k, v, o=o, ws=ws)))
    if pre_state is not None:
        layers, _, o, *_ = pre_state
        runs.append(("prefill", layers, lambda q, k, v, o=o: kas.prefill_dense(q, k, v, o=o)))
    for phase, layers, call in runs:
        q, k, v, _ = layers[0]
        call(q, k, v)                                  # warm-up
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        torch.cuda.synchronize()
        ev[0].record()                                 # events around the step, as for the sparse step
        for q, k, v, _ in layers:
            call(q, k, v)
        ev[1].record()
        torch.cuda.synchronize()
        per_layer = [ev[0].elapsed_time(ev[1]) / len(layers)] * len(layers)
        kas.profile_reset()
        kas.profile_enable(True)
        for q, k, v, _ in layers:
            call(q, k, v)
        torch.cuda.synchronize()
        kas.profile_enable(False)
        step_ms = sum(per_layer)
        name = phase + "_dense"
        kms = kas.profile_query(name)
        if phase == "decode":
            sparse_ms = out["decode"]["ms_per_step"] if "decode" in out else None
            res[phase] = {"workload": wd.name, "us_per_layer": round(1e3 * _mean(per_layer), 3),
                          "GB_per_s": _rate(dec_b, _mean(per_layer) * 1e-3, 1e9),
                          "ms_per_step": round(step_ms, 4)}
            roof.append(_roof_entry(name, "hbm", dec_b * kms[1], kms, HBM_PEAK_GBS, "GB/s", 1e9))
        else:
            sparse_ms = out["prefill"]["ms_per_step"] if "prefill" in out else None
            res[phase] = {"workload": wp.name, "ms_per_layer": round(_mean(per_layer), 4),
                          "TFLOP_per_s": _rate(pre_f, _mean(per_layer) * 1e-3, 1e12),
                          "ms_per_step": round(step_ms, 3)}
            roof.append(_roof_entry(name, "mfma", pre_f * kms[1], kms, BF16_PEAK_TFLOPS, "TFLOP/s", 1e12))
        if sparse_ms:
            res[phase]["speedup_kascade_step"] = round(step_ms / sparse_ms, 3)
        log(f"[bench] dense {phase}: {step_ms:.3f} ms per {len(layers)}-layer step")
    for r in roof:
        r["frac"] = round(r["achieved"] / r["peak"], 4)
    return res, [dict({k: r[k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac", "avg_us")},
                      traffic=_traffic(r["kernel"])) for r in roof]


VARIANTS = {"group_sum": (0, 0), "group_max": (0, 1), "all_sum": (1, 0), "all_max": (1, 1)}


def variant_timings(wd, dec_state, wp, pre_state, out, torch, kas, dev, inputgen):
    """Anchor-layer time of each selection variant (pooling scope: the KV
    head's group or all heads; operator: sum or max) on layer 0's resident
    inputs, median of repeated calls; plus the schedule in which every layer is
    an anchor, derived from the measured anchor-layer time."""
    res = {}

    def timed(call, reps):
        call()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    if dec_state is not None:
        (q, k, v, _), o, ws = dec_state[0][0], dec_state[2], dec_state[3]
        kd = dec_state[5]
        r = {}
        for name, (sc, op) in VARIANTS.items():
            idx = torch.empty((wd.batch, 1 if sc else wd.n_kv_heads, kd), dtype=torch.int32, device=dev)
            ms = timed(lambda: kas.decode_anchor(q, k, v, wd.topk_pct, idx_out=idx, o=o, ws=ws,
                                                 pool_scope=sc, pool_op=op), 5)
            r[name] = round(1e3 * ms, 3)
        res["decode_anchor_us"] = r
        # reuse layer 1 with a head map per KV head vs one per query head
        (q1, k1, v1, _), ws_r = dec_state[0][1], dec_state[4]
        idx = torch.empty((wd.batch, wd.n_kv_heads, kd), dtype=torch.int32, device=dev)
        anchor = lambda: kas.decode_anchor(q, k, v, wd.topk_pct, idx_out=idx, o=o, ws=ws)
        hm = torch.as_tensor(inputgen.head_maps(wd)[1], device=dev)
        qm = hm.repeat_interleave(wd.group)
        d_q = kas.make_desc(wd.batch, wd.n_q_heads, wd.n_kv_heads, wd.head_dim, wd.seq_len, wd.topk_pct,
                            wd.torch_dtype, query_head_map=1)
        ws_q = torch.empty(kas.workspace_size(d_q, kas.OP_DECODE_REUSE), dtype=torch.uint8, device=dev)
        _, t_kv = _alternate(torch, anchor, lambda: kas.decode_reuse(q1, k1, v1, idx, hm, wd.topk_pct, o=o, ws=ws_r), 7)
        _, t_q = _alternate(torch, anchor, lambda: kas.decode_reuse(q1, k1, v1, idx, qm, wd.topk_pct, o=o, ws=ws_q,
                                                                    query_head_map=True), 7)
        res["decode_reuse_us"] = {"map_per_kv_head": round(1e3 * t_kv, 3), "map_per_query_head": round(1e3 * t_q, 3)}
        # proposal-refined reuse: a proposal anchor at 4x the percentage, the
        # refined layer selecting its own k within that pool
        rho = 4
        pool = torch.empty((wd.batch, wd.n_kv_heads, kas.decode_k(wd.seq_len, rho * wd.topk_pct)), dtype=torch.int32,
                           device=dev)
        d_p = kas.make_desc(wd.batch, wd.n_q_heads, wd.n_kv_heads, wd.head_dim, wd.seq_len, rho * wd.topk_pct,
                            wd.torch_dtype)
        ws_p = torch.empty(kas.workspace_size(d_p, kas.OP_DECODE_ANCHOR), dtype=torch.uint8, device=dev)
        ridx = torch.empty((wd.batch, wd.n_kv_heads, kd), dtype=torch.int32, device=dev)
        t_pa, t_rf = _alternate(torch, lambda: kas.decode_anchor(q, k, v, rho * wd.topk_pct, idx_out=pool, o=o, ws=ws_p),
                                lambda: kas.decode_refine(q1, k1, v1, pool, hm, wd.topk_pct, idx_out=ridx, o=o), 7)
        res["decode_proposal_refined_us"] = {"rho": rho, "proposal_anchor": round(1e3 * t_pa, 3),
                                             "refined_layer": round(1e3 * t_rf, 3)}
        del pool, ws_p, ridx
        if "decode" in out:
            res["decode_every_layer_anchor_ms_per_step"] = {
                "value": round(wd.n_layers * out["decode"]["us_per_layer"]["anchor"] / 1e3, 4),
                "derived": "layers x measured anchor layer"}
    if pre_state is not None:
        (q, k, v, _), o, ws = pre_state[0][0], pre_state[2], pre_state[3]
        total = int(pre_state[5][-1])
        r = {}
        for name, (sc, op) in VARIANTS.items():
            idx = torch.empty((wp.batch, 1 if sc else wp.n_kv_heads, total), dtype=torch.int32, device=dev)
            ms = timed(lambda: kas.prefill_anchor(q, k, v, wp.topk_pct, idx_out=idx, o=o, ws=ws,
                                                  pool_scope=sc, pool_op=op), 2)
            r[name] = round(ms, 3)
        res["prefill_anchor_ms"] = r
        (q1, k1, v1, _), ws_r = pre_state[0][1], pre_state[4]
        idx = torch.empty((wp.batch, wp.n_kv_heads, total), dtype=torch.int32, device=dev)
        anchor = lambda: kas.prefill_anchor(q, k, v, wp.topk_pct, idx_out=idx, o=o, ws=ws)
        hm = torch.as_tensor(inputgen.head_maps(wp)[1], device=dev)
        qm = hm.repeat_interleave(wp.group)
        _, t_kv = _alternate(torch, anchor, lambda: kas.prefill_reuse(q1, k1, v1, idx, hm, wp.topk_pct, o=o, ws=ws_r), 2)
        _, t_q = _alternate(torch, anchor, lambda: kas.prefill_reuse(q1, k1, v1, idx, qm, wp.topk_pct, o=o, ws=ws_r,
                                                                     query_head_map=True), 2)
        res["prefill_reuse_ms"] = {"map_per_kv_head": round(t_kv, 3), "map_per_query_head": round(t_q, 3)}
        if "prefill" in out:
            res["prefill_every_layer_anchor_ms_per_step"] = {
                "value": round(wp.n_layers * out["prefill"]["ms_per_layer"]["anchor"], 3),
                "derived": "layers x measured anchor layer"}
    log(f"[bench] selection variants: {res}")
    return res


def _alternate(torch, anchor, reuse, reps):
    """Median device times of anchor() and reuse() enqueued back to back as
    anchor, reuse, anchor, ... (each reuse finds its rows evicted by the
    anchor's K stream)."""
    anchor()
    reuse()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        anchor()
        e[1].record()
        reuse()
        e[2].record()
    torch.cuda.synchronize()
    ta = sorted(e[0].elapsed_time(e[1]) for e in ev)
    tr = sorted(e[1].elapsed_time(e[2]) for e in ev)
    return ta[reps // 2], tr[reps // 2]


def paged_timings(wd, dec_state, dev, torch, inputgen, kas):
    """Decode anchor and reuse layer times on the contiguous cache and on page
    pools (pages of P keys, [pages, Hkv, P, D], shuffled page ids) holding
    the same layers 0 and 1; same alternating protocol as the dtype timings."""
    (q0, k0, v0, _), (q1, k1, v1, _) = dec_state[0][0], dec_state[0][1]
    o, ws_a, ws_r, kd = dec_state[2], dec_state[3], dec_state[4], dec_state[5]
    B, Hkv, N, D = k0.shape
    hm = torch.as_tensor(inputgen.head_maps(wd)[1], device=dev)
    idx = torch.empty((B, Hkv, kd), dtype=torch.int32, device=dev)
    res = {"workload": wd.name, "unit": "us"}
    ta, tr = _alternate(torch, lambda: kas.decode_anchor(q0, k0, v0, wd.topk_pct, idx_out=idx, o=o, ws=ws_a),
                        lambda: kas.decode_reuse(q1, k1, v1, idx, hm, wd.topk_pct, o=o, ws=ws_r), 7)
    res["contiguous"] = {"anchor": round(1e3 * ta, 3), "reuse": round(1e3 * tr, 3)}
    for P in (16, 64):
        per = N // P
        g = torch.Generator(device="cpu").manual_seed(P)
        ids = torch.randperm(B * per, generator=g).to(torch.int32).view(B, per).to(dev)

        kp0, vp0, kp1, vp1 = (_page_pool(torch, x, ids, P) for x in (k0, v0, k1, v1))
        kw = dict(block_table=ids, seq_len=N)
        wsa = kas.binding._ws_kv(*_kv_desc(kas, q0, kp0, ids, N, wd), kas.OP_DECODE_ANCHOR, None, dev)
        wsr = kas.binding._ws_kv(*_kv_desc(kas, q0, kp0, ids, N, wd), kas.OP_DECODE_REUSE, None, dev)
        ta, tr = _alternate(torch, lambda: kas.decode_anchor(q0, kp0, vp0, wd.topk_pct, idx_out=idx, o=o, ws=wsa, **kw),
                            lambda: kas.decode_reuse(q1, kp1, vp1, idx, hm, wd.topk_pct, o=o, ws=wsr, **kw), 7)
        res[f"paged_P{P}"] = {"anchor": round(1e3 * ta, 3), "reuse": round(1e3 * tr, 3)}
        del kp0, vp0, kp1, vp1, wsa, wsr
        torch.cuda.empty_cache()
    log(f"[bench] paged decode: {res}")
    return res


def _page_pool(torch, x, ids, P):
    """Page pool [pages, Hkv, P, D] holding x [B, Hkv, N, D] at the page ids
    ids [B, N / P] (shuffled, so the pages of a sequence are scattered)."""
    B, Hkv, N, D = x.shape
    per = N // P
    pg = torch.empty((B * per, Hkv, P, D), dtype=x.dtype, device=x.device)
    pg[ids.view(-1).long()] = x.view(B, Hkv, per, P, D).permute(0, 2, 1, 3, 4).reshape(B * per, Hkv, P, D)
    return pg


def ceilings(torch, dev):
    """What this GPU reaches on plain work, beside the published peaks the
    rooflines use: a 16384^3 bf16 GEMM through torch (the vendor BLAS) and a
    2 GiB device-to-device copy (read + written bytes)."""
    res = {}
    n = 16384
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    res["gemm_bf16_16384"] = {"TFLOP_per_s": round(2 * n ** 3 / ms / 1e9, 1),
                              "frac_of_peak": round(2 * n ** 3 / ms / 1e9 / BF16_PEAK_TFLOPS, 4)}
    del a, b, c
    src = torch.empty(1 << 30, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    gbs = 2 * src.numel() * 2 / (ms * 1e-3) / 1e9
    res["copy_2GiB"] = {"GB_per_s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del src, dst
    torch.cuda.empty_cache()
    log(f"[bench] ceilings: {res}")
    return res


def paged_prefill_timings(wp, pre_state, dev, torch, inputgen, kas):
    """Prefill anchor and reuse layer times on the contiguous cache and on page
    pools holding the same layers 0 and 1 (alternating protocol); the paged
    calls include their page copy, also timed on its own."""
    (q0, k0, v0, _), (q1, k1, v1, _) = pre_state[0][0], pre_state[0][1]
    o, ws_a, ws_r = pre_state[2], pre_state[3], pre_state[4]
    total = int(pre_state[5][-1])
    B, Hkv, N, D = k0.shape
    hm = torch.as_tensor(inputgen.head_maps(wp)[1], device=dev)
    idx = torch.empty((B, Hkv, total), dtype=torch.int32, device=dev)
    res = {"workload": wp.name, "unit": "ms"}
    ta, tr = _alternate(torch, lambda: kas.prefill_anchor(q0, k0, v0, wp.topk_pct, idx_out=idx, o=o, ws=ws_a),
                        lambda: kas.prefill_reuse(q1, k1, v1, idx, hm, wp.topk_pct, o=o, ws=ws_r), 3)
    res["contiguous"] = {"anchor": round(ta, 3), "reuse": round(tr, 3)}
    for P in (16, 256):
        g = torch.Generator(device="cpu").manual_seed(P)
        ids = torch.randperm(B * (N // P), generator=g).to(torch.int32).view(B, N // P).to(dev)
        kp0, vp0, kp1, vp1 = (_page_pool(torch, x, ids, P) for x in (k0, v0, k1, v1))
        kw = dict(block_table=ids)
        wsa = kas.binding._ws_kv(*kas.binding._prefill_desc(q0, kp0, wp.topk_pct, 0.0, None, ids, q0),
                                 kas.OP_PREFILL_ANCHOR, None, dev)
        wsr = kas.binding._ws_kv(*kas.binding._prefill_desc(q0, kp0, wp.topk_pct, 0.0, None, ids, q0),
                                 kas.OP_PREFILL_REUSE, None, dev)
        ta, tr = _alternate(torch,
                            lambda: kas.prefill_anchor(q0, kp0, vp0, wp.topk_pct, idx_out=idx, o=o, ws=wsa, **kw),
                            lambda: kas.prefill_reuse(q1, kp1, vp1, idx, hm, wp.topk_pct, o=o, ws=wsr, **kw), 3)
        kas.profile_reset()
        kas.profile_enable(True)
        for _ in range(3):
            kas.prefill_reuse(q1, kp1, vp1, idx, hm, wp.topk_pct, o=o, ws=wsr, **kw)
        torch.cuda.synchronize()
        kas.profile_enable(False)
        ms, n = kas.profile_query("prefill_page_copy")
        res[f"paged_P{P}"] = {"anchor": round(ta, 3), "reuse": round(tr, 3),
                              "page_copy": round(ms / max(n, 1), 4)}
        del kp0, vp0, kp1, vp1, wsa, wsr
        torch.cuda.empty_cache()
    res["page_copy_bytes"] = 2 * 2 * k0.numel() * k0.element_size()   # K and V, read and written
    log(f"[bench] paged prefill: {res}")
    return res


def _kv_desc(kas, q, kp, ids, N, w):
    over, cache = kas.binding._cache(q, kp, None, ids, N)
    return kas.binding._decode_desc(q, kp, w.topk_pct, 0.0, over, q), cache


def fp16_timings(wd, wp, dec_state, pre_state, dev, torch, inputgen, kas):
    """Anchor and reuse layer times with fp16 I/O (the element type of the
    pages' own kernels) beside bf16, same protocol for both: layers 0 (anchor)
    and 1 (reuse) of the workload, calls enqueued back to back as anchor,
    reuse, anchor, ... (each reuse finds its rows evicted by the anchor's full
    K stream), per-call events, medians. bf16 uses the resident layers."""
    import dataclasses
    res = {}
    alternate = lambda anchor, reuse, reps: _alternate(torch, anchor, reuse, reps)

    for phase, w0, st in (("decode", wd, dec_state), ("prefill", wp, pre_state)):
        if w0 is None:
            continue
        dec = phase == "decode"
        reps, scale, unit = (7, 1e3, "us") if dec else (3, 1.0, "ms")
        out = {"workload": w0.name, "unit": unit}
        for dt in ("bf16", "f16"):
            w = dataclasses.replace(w0, dtype=dt)
            hm = torch.as_tensor(inputgen.head_maps(w)[1], device=dev)
            if dt == w0.dtype:
                (qa, ka, va, _), (qr, kr, vr, _) = st[0][0], st[0][1]
            else:
                pos = inputgen.heavy_positions(w)
                qa, ka, va = inputgen.layer_inputs(w, 0, dev, pos)
                qr, kr, vr = inputgen.layer_inputs(w, 1, dev, pos)
            d = kas.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.topk_pct, w.torch_dtype)
            o = torch.empty_like(qa)
            if dec:
                ws_a = torch.empty(kas.workspace_size(d, kas.OP_DECODE_ANCHOR), dtype=torch.uint8, device=dev)
                ws_r = torch.empty(kas.workspace_size(d, kas.OP_DECODE_REUSE), dtype=torch.uint8, device=dev)
                idx = torch.empty((w.batch, w.n_kv_heads, kas.decode_k(w.seq_len, w.topk_pct)),
                                  dtype=torch.int32, device=dev)
                anchor = lambda: kas.decode_anchor(qa, ka, va, w.topk_pct, idx_out=idx, o=o, ws=ws_a)
                reuse = lambda: kas.decode_reuse(qr, kr, vr, idx, hm, w.topk_pct, o=o, ws=ws_r)
            else:
                ws_a = torch.empty(kas.workspace_size(d, kas.OP_PREFILL_ANCHOR), dtype=torch.uint8, device=dev)
                ws_r = torch.empty(max(256, kas.workspace_size(d, kas.OP_PREFILL_REUSE)), dtype=torch.uint8,
                                   device=dev)
                idx = torch.empty((w.batch, w.n_kv_heads, int(kas.prefill_offsets(d)[-1])), dtype=torch.int32,
                                  device=dev)
                anchor = lambda: kas.prefill_anchor(qa, ka, va, w.topk_pct, idx_out=idx, o=o, ws=ws_a)
                reuse = lambda: kas.prefill_reuse(qr, kr, vr, idx, hm, w.topk_pct, o=o, ws=ws_r)
            ta, tr = alternate(anchor, reuse, reps)
            out[dt] = {"anchor": round(scale * ta, 3), "reuse": round(scale * tr, 3)}
            del qa, ka, va, qr, kr, vr, o, ws_a, ws_r, idx
            torch.cuda.empty_cache()
        res[phase] = out
    log(f"[bench] bf16 / fp16 layers: {res}")
    return res


def _mean(xs):
    return sum(xs) / len(xs) if xs else float("nan")


def _rate(work, seconds, scale):
    return round(work / seconds / scale, 3) if seconds == seconds and seconds > 0 else None


def _roof_entry(name, bound, total_work, ms_n, peak, unit, scale):
    """Algorithmic work per launch / average launch duration (equal to total
    work / total device time of the kernel over the per-kernel timing pass)."""
    ms, n = ms_n
    per_launch = total_work / n
    avg_s = ms * 1e-3 / n
    return {"kernel": name, "bound": bound, "achieved": round(per_launch / avg_s / scale, 3), "peak": peak,
            "unit": unit, "total_ms": ms, "avg_us": avg_s * 1e6, "launches": n, "work_per_launch": per_launch}


def _traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else null)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except Exception:
        return None
    ent = data.get(kernel)
    if not ent:
        return None
    import hashlib
    src = os.path.join(ROOT, "sparse_attention_long_anchor_amd", "csrc", ent["source"])
    try:
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except Exception:
        return None
    return ent["bytes_per_launch"] if h == ent.get("source_sha256_16") else None


if __name__ == "__main__":
    main()
