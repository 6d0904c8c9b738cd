#!/usr/bin/env python
"""PBSA benchmark on one MI355X.

Workload (one step = one chunk of a streaming rollout in steady state):
the Wan2.1-T2V-1.3B-shaped chunk - 30 layers, each with 12 heads of 128, a
4680-token chunk (37 blocks of 128, the last 72 tokens), a window of the two
previous chunks (74 slots), a full persistent pool of 32 blocks and top-16
window selection.  Per layer: pbsa_select_attn_fwd (each workgroup routes
its query block, then attends: one launch) on the critical path, then
pbsa_block_mass -> pbsa_memory_update (the 37 blocks of chunk t-2 leave the
window) -> pbsa_window_append (chunk t takes their slots) on a side stream:
the next layer needs only the attention output, the updated cache is needed
by the next chunk.  Every timed step is the seeded Wan-chunk instance
(layer l: seed 1000 + l, pool 0..31, window = chunks 2 and 3, 8 planted
window blocks): the pool and window that the previous step's update and
append changed are restored on the device before each step, outside the
timing.  Inputs are synthetic, generated on the device and resident in HBM.

Prints ONE JSON line: attention TFLOP/s over the whole step (algorithmic
forward FLOPs 4*d*sum_rows|U_r| / step time), per-chunk latency, the
routing + forward kernel's roofline position (HIP events around a rotating
sample of its launches inside the timed region, every layer sampled; the
forward's FLOPs over the whole launch, routing included), a training step
(batch 2, fwd + bwd) and the fp64 CPU oracle timed on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)

# HBM traffic of one routing + forward launch on this workload, from two rocprofv3
# --pmc passes (FETCH_SIZE, WRITE_SIZE in KiB per dispatch), each scaled by
# what the same counter reads for a copy kernel of known size (the window
# append: 28,302 KiB read and 28,302 KiB written per launch; it reads back
# FETCH 14,167 KiB, WRITE 28,304 KiB).  Valid only for the kernel code it
# was measured on (sha1 over FWD_SOURCES below, comments left out); reported
# as null once that code changes.
FWD_TRAFFIC = {"src_sha1": "3ae10adffd1d1288c9f22f6a4b03c09a821cbc7c",
               "fetch_kib": 64153.8, "write_kib": 15156.4,
               "fetch_scale": 28302.0 / 14166.5, "write_scale": 28302.0 / 28304.3}


FWD_SOURCES = ("pbsa_attn_fwd.hip", "pbsa_tiles.h", "pbsa_select_dev.h")


def fwd_source_sha1() -> str:
    """sha1 over the forward kernel's code (the kernel file and the headers
    of tile staging and of the routing it runs first), with comments and
    blank lines left out, so that only a change of code invalidates it."""
    import hashlib
    import re
    h = hashlib.sha1()
    for name in FWD_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_20_amd", "csrc", name)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            line = line.split("//", 1)[0].rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def fwd_traffic_bytes():
    if fwd_source_sha1() != FWD_TRAFFIC["src_sha1"]:
        return None
    t = FWD_TRAFFIC
    return round(1024 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_rollout(n_layers, device, side_group=5):
    import pbsa_synth as syn
    from block_sparse_attention_20_amd.rollout import Rollout
    s = syn.WAN_CHUNK
    ro = Rollout(n_layers, s.B, s.H, s.d, s.T, s.Nq, s.C, s.topk, window_chunks=2, device=device,
                 overlap=True, side_group=side_group)
    for l in range(n_layers):
        st = syn.wan_chunk_state(l, device=device)
        ro.layers[l].load(st)
    # generator ids: pool 0..31, window = chunks 2 and 3 -> the current chunk is 4
    ro.t = 4
    return ro


def time_steps(ro, steps, warmup, torch, sample_every=10):
    """Every step runs the seeded Wan-chunk instance itself: before it, each
    layer's pool and window are restored to their seeded contents (device
    copies on the critical-path stream, outside the timing), so the memory
    update and window append of the previous step leave no trace.  The 30
    layers' PBSA work runs between HIP events on that stream, and the steps
    run back to back (no host synchronisation until the last one).  HIP
    events also bracket a rotating sample of the forward launches: in step
    s, the layers l with (l + s) % sample_every == 0, so every layer is
    sampled over sample_every steps (each event pair delays the launches
    after it by a few microseconds, so bracketing all 30 forwards would add
    ~2.5% to the step it measures).
    Returns ms per step (mean), [(step, layer, fwd ms)], per-layer FLOPs
    (from the selections and pools the forwards saw) and the per-step ms."""
    from block_sparse_attention_20_amd.rollout import attended_tokens
    n_layers = len(ro.layers)
    d = ro.layers[0].d
    seeded = ro.state_dict()
    for _ in range(warmup):
        ro.load_state_dict(seeded)
        ro.run_chunk()
    torch.cuda.synchronize()
    ev = {(s, l): (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for s in range(steps) for l in range(n_layers) if (l + s) % sample_every == 0}
    step_ev, flops = [], [0] * n_layers
    snaps = []
    for s in range(steps):
        ro.load_state_dict(seeded)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for l in range(n_layers):
            ro.run_layer(l, fwd_events=ev.get((s, l)))
        e1.record()
        if s == 0:  # routing of the seeded instance (the same every step)
            snaps = [(L.t["sel"].clone(), L.t["sel_count"].clone()) for L in ro.layers]
        step_ev.append((e0, e1))
        ro.advance()
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in step_ev]
    for l, L in enumerate(ro.layers):
        flops[l] = 4 * d * attended_tokens(L, seeded["layers"][l]["pool_count"],
                                           seeded["layers"][l]["pool_len"], *snaps[l])
    fwd_ms = [(s, l, a.elapsed_time(b)) for (s, l), (a, b) in sorted(ev.items())]
    return sum(step_ms) / steps, fwd_ms, flops, step_ms


def breakdown(ro, torch, reps=3):
    """Average device time of each call, run one after the other on one
    stream (separate, untimed pass)."""
    ro.sync_side()
    names = ("select_fwd", "select", "fwd", "block_mass", "update", "append")
    acc = {n: [] for n in names}
    for _ in range(reps):
        t = ro.t
        for L in ro.layers:
            calls = (L.select_fwd, lambda: L.select(masses=False), L.fwd, L.block_mass,
                     lambda: L.update(ro.leaving[t % ro.window_chunks], ro.n_sink),
                     lambda: L.append_window(ro.first_slot(t), t * ro.QB))
            for n, fn in zip(names, calls):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(); fn(); b.record()
                acc[n].append((a, b))
        ro.advance()
    torch.cuda.synchronize()
    return {n: round(1e3 * sum(a.elapsed_time(b) for a, b in v) / len(v), 2) for n, v in acc.items()}


def train_step(torch, steps=5, warmup=2, device="cuda"):
    """Batch-2 training step of one layer: routing + forward (one launch), then
    the backward; fwd_ms is the routing + forward launch."""
    import pbsa_synth as syn
    from block_sparse_attention_20_amd.layer import PBSALayer
    from block_sparse_attention_20_amd.rollout import attended_tokens
    s = syn.WAN_TRAIN
    L = PBSALayer(s.B, s.H, s.d, s.T, s.Nq, s.W, s.C, s.topk, device=device)
    st = syn.make_state(s, 4000, sigma=1 / math.sqrt(s.d), shift=1.5, n_planted=8,
                        win_len=syn.chunk_window_lens(s.Nq, s.T, 2), device=device)
    L.load(st)
    dout = syn.make_dout(s, 4001, device=device)
    grads = None
    for _ in range(warmup):
        L.select_fwd(); grads = L.bwd(dout, grads)
    torch.cuda.synchronize()
    ef = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    eb = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ef[i][0].record(); L.select_fwd(); ef[i][1].record()
        eb[i][0].record(); grads = L.bwd(dout, grads); eb[i][1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    pairs = attended_tokens(L)
    fwd_ms = sum(a.elapsed_time(b) for a, b in ef) / steps
    bwd_ms = sum(a.elapsed_time(b) for a, b in eb) / steps
    fwd_f, bwd_f = 4 * s.d * pairs, 10 * s.d * pairs
    return {"workload": "wan chunk training step, batch 2 (routing + fwd in one launch, bwd; one layer)",
            "ms_per_step": round(ms, 4), "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "fwd_gflop": round(fwd_f / 1e9, 2), "bwd_gflop": round(bwd_f / 1e9, 2),
            "tflops": round((fwd_f + bwd_f) / (ms * 1e-3) / 1e12, 2),
            "bwd_tflops": round(bwd_f / (bwd_ms * 1e-3) / 1e12, 2),
            "bwd_flop_convention": "10*d per attended (row, token) pair, QK^T recompute included"}


def rollout_bench(n_chunks, config_id, torch, n_layers=30, device="cuda", side_group=5):
    """Streaming rollout in the Wan shape: n_chunks chunks of 4680 tokens,
    30 layers with independent state, window of the two previous chunks,
    pool capped at 64 blocks, Top-C update after every chunk.  Each new chunk
    plants 8 salient blocks along a direction re-drawn every 8 chunks.
    Per-chunk latency = HIP events around the 30 layers' PBSA work on the
    critical-path stream (inputs are generated on the device between
    chunks, outside the events)."""
    import pbsa_synth as syn
    from block_sparse_attention_20_amd.rollout import Rollout, attended_tokens
    s = syn.WAN_CHUNK
    C = syn.ROLLOUT_POOL_CAP
    shape = syn.Shape(B=s.B, H=s.H, d=s.d, T=s.T, Nq=s.Nq, W=0, C=C, topk=s.topk)
    ro = Rollout(n_layers, s.B, s.H, s.d, s.T, s.Nq, C, s.topk, window_chunks=2, device=device,
                 overlap=True, side_group=side_group)
    sigma = 1 / math.sqrt(s.d)
    ms, gflop, pool = [], [], []
    for t in range(n_chunks):
        for l in range(n_layers):
            u = syn.rollout_direction(config_id, l, t, s.d, device=device)
            ch = syn.make_chunk(shape, syn.rollout_seed(config_id, l, t), u, sigma=sigma, shift=1.5,
                                n_planted=8, device=device)
            ro.set_inputs(l, ch["q"], ch["k"], ch["v"])
        # the pools this chunk's forwards attend (each layer's update follows
        # its forward), for the FLOP count after the chunk
        ro.sync_side()
        seen = [(L.t["pool_count"].clone(), L.t["pool_len"].clone()) for L in ro.layers]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for l in range(n_layers):
            ro.run_layer(l)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
        gflop.append(sum(4 * s.d * attended_tokens(L, *pl) for L, pl in zip(ro.layers, seen)) / 1e9)
        pool.append(int(ro.layers[0].t["pool_count"][0, 0].item()))
        ro.advance()
    steady = ms[4:]
    med = sorted(steady)[len(steady) // 2]
    return {"workload": f"streaming rollout, {n_chunks} chunks x {n_layers} layers, pool cap {C}",
            "per_chunk_ms": [round(x, 3) for x in ms],
            "per_chunk_gflop": [round(x, 1) for x in gflop],
            "pool_blocks_after_update": pool,
            "steady_median_ms": round(med, 3),
            "steady_flatness": round((max(steady) - min(steady)) / med, 4),
            "steady_tflops": round(sum(gflop[4:]) / sum(steady), 2)}


def cpu_baseline(ro, budget_s, torch):
    """The fp64 oracle (as it stands) on a bounded sample of the same
    workload: layer 0's select over every head, then the forward of as many
    query blocks as fit in the time budget.  Reported in the metric's unit."""
    import numpy as np
    from oracle import pbsa_oracle as po
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    L = ro.layers[0]
    st = {k: L.t[k].detach().cpu() for k in ("q", "k_cur", "v_cur", "k_win", "v_win", "win_len",
                                                "win_id", "k_pool", "v_pool", "pool_len", "pool_id",
                                                "pool_count")}
    st = po.as_f64_state(st)
    scale = 1 / math.sqrt(L.d)
    t0 = time.perf_counter()
    r = po.select(st, L.topk, scale, L.T)
    t_sel = time.perf_counter() - t0
    blocks, flops = [], 0
    t0 = time.perf_counter()
    QB, H = L.QB, L.H
    order = [(0, h, i) for i in range(QB) for h in range(H)]
    for b, h, i in order:
        po.attn_fwd(st, r["sel"], r["sel_count"], scale, L.T, blocks=[(b, h, i)])
        rows = min(L.T, L.Nq - i * L.T)
        n_u = sum(int(st["pool_len"][b, h, p]) for p in range(int(st["pool_count"][b, h])))
        n_u += sum(int(st["win_len"][w]) for w in r["sel"][b, h, i, :r["sel_count"][b, h, i]])
        n_u += L.Nq
        flops += 4 * L.d * rows * n_u
        blocks.append((h, i))
        if time.perf_counter() - t0 > budget_s:
            break
    t_fwd = time.perf_counter() - t0
    return {"value": round(flops / t_fwd / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"layer 0 of the Wan chunk: coarse routing of all 12 heads ({t_sel:.1f} s), "
                      f"then the fp64 forward of {len(blocks)} of {QB * H} (head, query block) "
                      f"pairs ({t_fwd:.1f} s); value = forward FLOPs / forward time"}


def sweep(torch, device="cuda", reps=3, iters=10):
    """Forward time of the Wan-shaped chunk (12 heads x 128, 4680 tokens,
    blocks of 128) across sparsity and history length, against the same
    kernel at its dense limit (every window block selected, no pool).

    - topk axis: window of 2 chunks (74 slots), pool 32, k in {9, 18, 37, 74}
      (k = 74 is dense over the window);
    - pool axis: window 74, k = 16, pool in {0, 16, 32, 64};
    - history axis: h previous chunks; dense attends all 37 h history blocks
      (W = 37 h, k = W, pool 0); PBSA attends a 2-chunk window (k = 16) and a
      pool holding the blocks that left the window, capped at 64.
    """
    import pbsa_synth as syn
    from block_sparse_attention_20_amd.layer import PBSALayer
    from block_sparse_attention_20_amd.rollout import attended_tokens
    base = syn.WAN_CHUNK
    qb = base.QB

    def fwd_time(W, C, topk, seed):
        shape = syn.Shape(B=1, H=base.H, d=base.d, T=base.T, Nq=base.Nq, W=W, C=C, topk=topk)
        nch = max(1, (W + qb - 1) // qb)
        wl = (syn.chunk_window_lens(base.Nq, base.T, nch) + [base.T] * W)[:W]
        st = syn.make_state(shape, seed, sigma=1 / math.sqrt(base.d), shift=1.5,
                            n_planted=min(8, W), win_len=wl, device=device)
        L = PBSALayer(shape.B, shape.H, shape.d, shape.T, shape.Nq, W, C, topk, device=device).load(st)
        del st
        L.select()
        for _ in range(3):
            L.fwd()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(iters):
                L.fwd()
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b) * 1e3 / iters)
        pairs = attended_tokens(L)
        del L
        torch.cuda.empty_cache()
        return {"W": W, "pool": C, "topk": topk, "fwd_us": round(best, 1),
                "keys_per_query": round(pairs / (base.H * base.Nq), 1),
                "tflops": round(4 * base.d * pairs / (best * 1e-6) / 1e12, 1)}

    out = {"topk": [], "pool": [], "history": []}
    for k in (9, 18, 37, 74):
        log(f"sweep topk {k}")
        out["topk"].append(fwd_time(74, 32, k, 5000 + k))
    for c in (0, 16, 32, 64):
        log(f"sweep pool {c}")
        out["pool"].append(fwd_time(74, c, 16, 5100 + c))
    for h in (1, 2, 4, 8, 16, 27):
        log(f"sweep history {h}")
        dense = fwd_time(qb * h, 0, qb * h, 5200 + h)
        w = qb * min(h, 2)
        sparse = fwd_time(w, min(64, qb * max(0, h - 2)), min(16, w), 5300 + h)
        out["history"].append({"chunks": h, "dense": dense, "pbsa": sparse,
                               "speedup": round(dense["fwd_us"] / sparse["fwd_us"], 2)})
    return out


def small_chunks(torch, device="cuda", iters=20):
    """Forward on short query chunks, where the kernel is bound by memory:
    1-8 query blocks of the Wan head shape (12 heads x 128, blocks of 128)
    against the full-size cache (window 74 slots, pool 32, top-16), and the
    tiny fp32 configuration.  Algorithmic bytes per launch: Q and O, LSE,
    and the valid rows of K and V of every block attended (pool, the union
    of the selected window blocks over the query blocks, the current chunk),
    each moved once.  Cold: L2 and Infinity Cache flushed (a 512 MB write)
    before each timed launch; warm: back-to-back launches."""
    import statistics

    import pbsa_synth as syn
    from block_sparse_attention_20_amd.layer import PBSALayer
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=device)
    base = syn.WAN_CHUNK
    cases = [(f"{qb} query block{'s' if qb > 1 else ''} x 12 heads, Wan cache",
              syn.Shape(B=1, H=base.H, d=base.d, T=base.T, Nq=qb * base.T, W=base.W, C=base.C,
                        topk=base.topk)) for qb in (1, 2, 4, 8)]
    cases.append(("tiny fp32 (1 head x 64, 256 tokens, window 32, pool 4, top-4)", syn.TINY_F32))
    out = []
    for name, shape in cases:
        log(f"small chunks: {name}")
        if shape.dtype == torch.float32:
            st = syn.tiny_f32_state(device=device)
        else:
            st = syn.make_state(shape, 6000 + shape.Nq // shape.T, sigma=1 / math.sqrt(shape.d), shift=1.5,
                                n_planted=8, win_len=syn.chunk_window_lens(base.Nq, base.T, 2),
                                device=device)
        L = PBSALayer(shape.B, shape.H, shape.d, shape.T, shape.Nq, shape.W, shape.C, shape.topk,
                      dtype=shape.dtype, device=device).load(st)
        del st
        L.select()
        L.fwd()
        torch.cuda.synchronize()
        esz = 2 if shape.dtype == torch.bfloat16 else 4
        row_b = shape.d * esz
        t = {k: L.t[k].cpu() for k in ("pool_count", "pool_len", "sel", "sel_count", "win_len")}
        alg = 0
        for b in range(shape.B):
            for h in range(shape.H):
                n_pool = int(t["pool_count"][b, h])
                kv = sum(int(x) for x in t["pool_len"][b, h, :n_pool])
                used = set()
                for i in range(L.QB):
                    used.update(int(w) for w in t["sel"][b, h, i, :int(t["sel_count"][b, h, i])])
                kv += sum(int(t["win_len"][w]) for w in used) + shape.Nq
                alg += 2 * kv * row_b + 2 * shape.Nq * row_b + 4 * shape.Nq
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for r in range(iters):
            flush.fill_(r & 255)
            ev[r][0].record()
            L.fwd()
            ev[r][1].record()
        torch.cuda.synchronize()
        cold = statistics.median(a.elapsed_time(b) * 1e3 for a, b in ev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            L.fwd()
        b.record()
        torch.cuda.synchronize()
        warm = a.elapsed_time(b) * 1e3 / iters
        out.append({"case": name, "query_blocks": L.QB, "items": shape.B * shape.H * L.QB,
                    "dtype": "bf16" if esz == 2 else "f32", "alg_mb": round(alg / 1e6, 2),
                    "cold_us": round(cold, 1), "warm_us": round(warm, 1),
                    "cold_gbs": round(alg / (cold * 1e-6) / 1e9, 1),
                    "warm_gbs": round(alg / (warm * 1e-6) / 1e9, 1),
                    "cold_frac_of_8tbs": round(alg / (cold * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)})
        del L
        torch.cuda.empty_cache()
    del flush
    return {"workload": "forward on short query chunks against the Wan-sized cache, and the tiny "
                        "fp32 configuration (memory-bound sizes)", "rows": out}


def mass_compare(torch, n_chunks=16, n_layers=2, device="cuda"):
    """Coarse vs exact (fine-grained) block mass as the Top-C score, the
    head-shared pool (one pool per layer, coarse masses summed over heads)
    and the sink policy (the first chunk's blocks pinned), on the
    streaming Wan-shaped rollout (pool cap 64, k = 16, 8 planted salient
    blocks per chunk): per chunk, the overlap of the two pools (Jaccard over
    (layer, head)); and for layer 0, with dense attention over the whole
    history (the same kernel with every history block selected) and its
    exact block masses, the share of the dense attention mass on blocks
    older than the window that each pool holds, next to the best 64 blocks
    chosen with hindsight.  Also the time of pbsa_fine_mass."""
    import pbsa_synth as syn
    from block_sparse_attention_20_amd.layer import PBSALayer
    from block_sparse_attention_20_amd.rollout import Rollout
    s = syn.WAN_CHUNK
    C = syn.ROLLOUT_POOL_CAP
    qb = s.QB
    shape = syn.Shape(B=s.B, H=s.H, d=s.d, T=s.T, Nq=s.Nq, W=0, C=C, topk=s.topk)
    ros = {m: Rollout(n_layers, s.B, s.H, s.d, s.T, s.Nq, C, s.topk, window_chunks=2, device=device,
                      overlap=True, mass=m) for m in ("coarse", "fine")}
    # the head-shared pool variant: one pool per layer, coarse masses summed over heads
    ros["shared"] = Rollout(n_layers, s.B, s.H, s.d, s.T, s.Nq, C, s.topk, window_chunks=2,
                            device=device, overlap=True, shared_pool=True)
    # the sink policy: the first chunk's blocks (ids 0 .. QB-1) pinned in the
    # pool once they leave the window, the rest ranked by coarse mass
    ros["sinks"] = Rollout(n_layers, s.B, s.H, s.d, s.T, s.Nq, C, s.topk, n_sink=qb,
                           window_chunks=2, device=device, overlap=True)
    sigma = 1 / math.sqrt(s.d)
    hist = []  # layer 0's chunks: (k, v) padded to whole blocks, [B,H,QB,T,d]
    pad = qb * s.T - s.Nq

    def blocks(x):
        x = torch.nn.functional.pad(x, (0, 0, 0, pad))
        return x.reshape(s.B, s.H, qb, s.T, s.d)

    rows = []
    for t in range(n_chunks):
        for l in range(n_layers):
            u = syn.rollout_direction(4, l, t, s.d, device=device)
            ch = syn.make_chunk(shape, syn.rollout_seed(4, l, t), u, sigma=sigma, shift=1.5,
                                n_planted=8, device=device)
            for ro in ros.values():
                ro.set_inputs(l, ch["q"], ch["k"], ch["v"])
            if l == 0:
                cur = ch
        # layer 0's pool as this chunk attends it (before this chunk's update)
        pools = {m: (ro.layers[0].t["pool_id"].clone(), ro.layers[0].t["pool_count"].clone())
                 for m, ro in ros.items()}
        ms, fwd_ms = {}, {}
        # the rollouts take turns at running first: the first one after an
        # idle gap runs at a higher clock than the ones right behind it
        nr = len(ros)
        order = list(ros)[t % nr:] + list(ros)[:t % nr]
        for m in order:
            ro = ros[m]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(n_layers)]
            e0.record()
            for l in range(n_layers):
                ro.run_layer(l, fwd_events=fe[l])
            e1.record()
            ro.sync_side()
            torch.cuda.synchronize()
            ms[m] = e0.elapsed_time(e1)
            fwd_ms[m] = sum(a.elapsed_time(b) for a, b in fe)
        row = {"chunk": t, "ms_coarse": round(ms["coarse"], 3), "ms_fine": round(ms["fine"], 3),
               "ms_shared": round(ms["shared"], 3), "ms_sinks": round(ms["sinks"], 3),
               "fwd_ms_coarse": round(fwd_ms["coarse"], 3), "fwd_ms_fine": round(fwd_ms["fine"], 3)}
        # pool overlap after this chunk's update
        jac = []
        for l in range(n_layers):
            pa = ros["coarse"].layers[l].t; pb = ros["fine"].layers[l].t
            for h in range(s.H):
                a = set(pa["pool_id"][0, h, :int(pa["pool_count"][0, h])].tolist())
                b = set(pb["pool_id"][0, h, :int(pb["pool_count"][0, h])].tolist())
                jac.append(len(a & b) / len(a | b) if a | b else 1.0)
        row["pool_jaccard"] = round(sum(jac) / len(jac), 4)
        if t >= 3:
            # dense attention over every history chunk, layer 0
            W = qb * t
            D = PBSALayer(s.B, s.H, s.d, s.T, s.Nq, W, 0, W, device=device, ws_fwd=None)
            D.t["q"].copy_(cur["q"]); D.t["k_cur"].copy_(cur["k"]); D.t["v_cur"].copy_(cur["v"])
            D.t["k_win"].copy_(torch.cat([k for k, _ in hist], dim=2))
            D.t["v_win"].copy_(torch.cat([v for _, v in hist], dim=2))
            D.t["win_len"].copy_(torch.tensor(syn.chunk_window_lens(s.Nq, s.T, t), dtype=torch.int32))
            D.t["win_id"].copy_(torch.arange(W, dtype=torch.int64))
            D.refresh_kbar()
            D.select(); D.fwd(); D.fine_mass()
            md = D.t["mass_win"][0].double()            # [H, W]: block id = slot
            old = (t - 2) * qb                           # ids older than the window
            cap = {m: [] for m in ros}
            best = []
            for h in range(s.H):
                tot = float(md[h, :old].sum())
                best.append(float(md[h, :old].topk(min(C, old)).values.sum()) / tot)
                for m in ros:
                    pid, pcnt = pools[m]
                    ids = pid[0, h, :int(pcnt[0, h])].long()
                    cap[m].append(float(md[h, ids[ids < old]].sum()) / tot)
            for m in ros:
                row["pool_share_" + m] = round(sum(cap[m]) / s.H, 4)
            row["pool_share_best"] = round(sum(best) / s.H, 4)
            del D
        hist.append((blocks(cur["k"]).clone(), blocks(cur["v"]).clone()))
        rows.append(row)
        for ro in ros.values():
            ro.advance()
    # on layer 0 of the fine rollout (last chunk's state, pool of 64): the
    # separate exact-mass pass alone, and the forward with and without the
    # fused exact mass (pbsa_attn_fwd_mass vs pbsa_attn_fwd)
    L = ros["fine"].layers[0]

    def per_call_us(fn, n=20):
        fn(); torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record(); torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) * 1e3 / n, 1)

    fine_us = per_call_us(L.fine_mass)
    # alternated, the better of three each, so that both see the same clock
    fwd_us, fwd_mass_us = float("inf"), float("inf")
    for _ in range(3):
        fwd_us = min(fwd_us, per_call_us(L.fwd))
        fwd_mass_us = min(fwd_mass_us, per_call_us(L.fwd_mass))
    return {"workload": f"streaming rollout, {n_chunks} chunks x {n_layers} layers, pool cap {C}, "
                        "coarse vs exact block mass as the Top-C score, a head-shared pool and "
                        "the first chunk's blocks as sinks",
            "per_chunk": rows, "fine_mass_us": fine_us, "fwd_us": fwd_us,
            "fwd_mass_us": fwd_mass_us,
            "fused_mass_extra_frac": round((fwd_mass_us - fwd_us) / fwd_us, 4)}


def train_rollout_bench(torch, n_chunks=8, device="cuda"):
    """Training through a streaming rollout in the Wan shape (one layer,
    12 heads x 128, 4680-token chunks, window of 2 chunks, pool cap 64,
    top-16): the forward over n_chunks records routing and pool decisions;
    the backward runs, per chunk, pbsa_block_gather of the attended pool and
    window slots, pbsa_attn_bwd and pbsa_grad_scatter into fp32 history
    gradients.  HIP events around each chunk's forward and backward, and
    around the gather / scatter calls alone."""
    import pbsa_synth as syn
    from block_sparse_attention_20_amd import pbsa as P
    from block_sparse_attention_20_amd.train import TrainRollout
    s = syn.WAN_CHUNK
    C = syn.ROLLOUT_POOL_CAP
    shape = syn.Shape(B=s.B, H=s.H, d=s.d, T=s.T, Nq=s.Nq, W=0, C=C, topk=s.topk)
    sigma = 1 / math.sqrt(s.d)

    def ev():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(timed):
        tr = TrainRollout(n_chunks, s.B, s.H, s.d, s.T, s.Nq, C, s.topk, device=device)
        fwd = []
        douts = []
        for t in range(n_chunks):
            u = syn.rollout_direction(5, 0, t, s.d, device=device)
            ch = syn.make_chunk(shape, syn.rollout_seed(5, 0, t), u, sigma=sigma, shift=1.5,
                                n_planted=8, device=device)
            douts.append(syn.make_dout(shape, 9000 + t, device=device))
            a, b = ev()
            a.record(); tr.forward(ch["q"], ch["k"], ch["v"]); b.record()
            fwd.append((a, b))
        torch.cuda.synchronize()
        a, b = ev()
        a.record(); tr.backward(douts); b.record()
        torch.cuda.synchronize()
        return tr, [x.elapsed_time(y) for x, y in fwd], a.elapsed_time(b), douts

    run(False)  # warm-up (first launches, allocator)
    tr, fwd_ms, bwd_ms, douts = run(True)
    # gather + scatter alone, on the last chunk's record, repeated
    r, D = tr.rec[-1], tr.D
    g = D.bwd(douts[-1])
    gk = torch.zeros(n_chunks, s.B, s.H, s.Nq, s.d, dtype=torch.float32, device=device)
    gv = torch.zeros_like(gk)
    a, b = ev()
    a.record()
    for _ in range(10):
        P.pbsa_block_gather(D.prob, r["win_id"], 0, None, tr.W, tr.k_hist, tr.v_hist, n_chunks,
                            D.t["k_win"], D.t["v_win"], None)
        P.pbsa_block_gather(D.prob, r["pool_id"], C, r["pool_count"], C, tr.k_hist, tr.v_hist,
                            n_chunks, D.t["k_pool"], D.t["v_pool"], D.t["pool_len"])
        P.pbsa_grad_scatter(D.prob, r["win_id"], 0, None, tr.W, 0, g["dk_win"], g["dv_win"], gk, gv,
                            n_chunks)
        P.pbsa_grad_scatter(D.prob, r["pool_id"], C, r["pool_count"], C, 0, g["dk_pool"], g["dv_pool"],
                            gk, gv, n_chunks)
    b.record()
    torch.cuda.synchronize()
    return {"workload": f"training through a streaming rollout, {n_chunks} chunks of the Wan "
                        f"shape, one layer, pool cap {C}",
            "fwd_ms_per_chunk": [round(x, 3) for x in fwd_ms],
            "bwd_ms_total": round(bwd_ms, 3),
            "bwd_ms_per_chunk": round(bwd_ms / n_chunks, 3),
            "gather_scatter_ms_per_chunk": round(a.elapsed_time(b) / 10, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle forward work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--side-group", type=int, default=5,
                    help="layers whose update + append go to the side stream together")
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--no-rollout", action="store_true", help="skip the 20 s / 1 min rollouts")
    ap.add_argument("--sweep", action="store_true",
                    help="only the sparsity x history sweep of the forward (its own JSON line)")
    ap.add_argument("--train-rollout", action="store_true",
                    help="only the training-through-a-rollout timing (its own JSON line)")
    ap.add_argument("--small-chunks", action="store_true",
                    help="forward on 1-8 query blocks and the tiny fp32 case: HBM GB/s")
    ap.add_argument("--mass-compare", action="store_true",
                    help="only the coarse vs exact block-mass comparison (its own JSON line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (use --gpus 1): PBSA would shard by head with no "
              "exchange between GPUs, so the single-GPU rate is the per-GPU figure.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import block_sparse_attention_20_amd as pkg
    from block_sparse_attention_20_amd.rollout import attended_tokens
    pkg.lib()
    dev = "cuda"
    if args.sweep:
        print(json.dumps({"sweep": sweep(torch, dev)}), flush=True)
        return
    if args.train_rollout:
        print(json.dumps({"train_rollout": train_rollout_bench(torch, device=dev)}), flush=True)
        return
    if args.small_chunks:
        print(json.dumps({"small_chunks": small_chunks(torch, device=dev)}), flush=True)
        return
    if args.mass_compare:
        print(json.dumps({"mass_compare": mass_compare(torch, device=dev)}), flush=True)
        return
    log(f"building 30-layer state ({args.layers} layers)")
    ro = build_rollout(args.layers, dev, args.side_group)
    torch.cuda.synchronize()
    log("timing")
    ms, fwd_samples, flops_layer, step_ms = time_steps(ro, args.steps, args.warmup, torch)
    d = ro.layers[0].d
    step_flops = sum(flops_layer)
    value = step_flops / (ms * 1e-3) / 1e12
    fwd_avg_ms = sum(x for _, _, x in fwd_samples) / len(fwd_samples)
    # the sampled launches' own FLOPs: their layer's mean over the timed steps
    fwd_tflops = (sum(flops_layer[l] for _, l, _ in fwd_samples)
                  / (sum(x for _, _, x in fwd_samples) * 1e-3) / 1e12)
    bd = breakdown(ro, torch)
    out = {
        "metric": "PBSA attention TFLOP/s and per-chunk latency (ms) on one MI355X; % of MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "wan2.1-t2v-1.3b-shaped chunk, seeded instance (state restored "
                               "before every step): "
                               f"{args.layers} layers x (select + fwd in one launch; block "
                               "mass + update + append on a side stream)",
                   "layers": args.layers, "heads": 12, "head_dim": d, "block": 128,
                   "chunk_tokens": 4680, "window_slots": 74, "pool_blocks": 32, "topk": 16,
                   "parallelism": "1 GPU"},
        "per_chunk_latency_ms": round(ms, 4),
        "fwd_gflop_per_layer": round(step_flops / len(ro.layers) / 1e9, 2),
        "pct_of_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"kernel": "attn_fwd_sel_bf16_kernel<128,128> (routing + forward)",
                     "bound": "mfma",
                     "achieved": round(fwd_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": fwd_traffic_bytes(), "traffic_unit": "bytes per launch",
                     "launch_us": round(fwd_avg_ms * 1e3, 2),
                     "launches": len(fwd_samples)},
        "step_ms_min_median_max": [round(min(step_ms), 4), round(sorted(step_ms)[len(step_ms) // 2], 4),
                                   round(max(step_ms), 4)],
        "breakdown_us_per_layer": bd,
    }
    if not args.no_train:
        log("training step")
        out["train"] = train_step(torch)
    if not args.no_rollout:
        log("rollout 27 chunks (20 s)")
        out["rollout_20s"] = rollout_bench(27, 2, torch, side_group=args.side_group)
        log("rollout 80 chunks (1 min)")
        out["rollout_1min"] = rollout_bench(80, 3, torch, side_group=args.side_group)
    if not args.no_cpu_baseline:
        log("cpu baseline")
        out["cpu_baseline"] = cpu_baseline(ro, args.cpu_budget, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
