"""QSA layer forward pass benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload chunked|prefill]
                    [--decode {decode,stack,none}] [--no-cpu-baseline]

One step = one pass of the whole hot path over one batch of synthetic input:
index build of the chunk's new blocks -> block scoring + top-k_B selection ->
sparse attention.  The headline workload is chunked prefill at 128K context
(2 sequences, 131,072 cached tokens, 8,192 new queries each, 16Q/2KV heads,
d=128, K=2048, r=4, bf16); `value` is prefill tokens/s with every input
resident in HBM.  Alongside, the decode loop (8 sequences at 256K context,
one token per sequence per step: index build, selection, split attention)
is timed over 64 steps and reported as microseconds per step.

Timing: torch.cuda events on the stream every kernel is launched on (the
binding launches on torch's current stream), a device synchronisation on
both sides of the timed region.  The dominant kernel's average duration is
taken from events around its launches inside the timed region.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA prefill tok/s + decode µs/step at 128K–1M ctx; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0

# HBM traffic of one sparse_attn_prefill launch on the 128K chunked workload,
# from two rocprofv3 --pmc runs of `bench.py --only prefill` (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for
# a plain 1 GiB device copy (`bench.py --calibrate-copy`: FETCH_SIZE reads
# 524,302 KiB for 1 GiB read -> x2.0; WRITE_SIZE reads 1 GiB -> x1.0).  The
# figures belong to the attention source with this SHA-1; for any other source
# `traffic` is reported as null until the counters are taken again.
ATTN_COUNTERS = {
    "source_sha1": "38e5ddb5601b98a9acf4f1ad2fcc2296dd7e3e68",
    "fetch_kib": 15017750.0, "write_kib": 66673.4,
    "fetch_scale": 2.0, "write_scale": 1.0,
}


def attn_source_digest() -> str:
    """sha1 over the sources the prefill attention kernel is compiled from."""
    import hashlib
    h = hashlib.sha1()
    for f in ("attn.hip", "attn_tile.h"):
        with open(os.path.join(ROOT, "block_sparse_trainable_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def attn_traffic_bytes():
    c = ATTN_COUNTERS
    if attn_source_digest() != c["source_sha1"]:
        return None
    return (c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=["chunked", "prefill", "companion"], default="chunked",
                    help="prefill workload: 2 x 8K over 128K (default), 32K from empty, or "
                         "the last 4K queries of a 1M context")
    ap.add_argument("--decode", choices=["decode", "stack", "none"], default="decode",
                    help="decode workload: 8 x 256K (default) or the 12-layer 1M-context stack")
    ap.add_argument("--only", choices=["prefill", "decode"], default=None,
                    help="profile one leg only (the JSON line then carries that leg)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (3 times), the "
                         "known-size reference for scaling HBM byte counters")
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--block-size", type=int, default=4,
                    help="r of the chunked prefill workload (4 = the pages' configuration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the sparse attention backward on the prefill workload")
    ap.add_argument("--offload", action=argparse.BooleanOptionalAction, default=True,
                    help="also time decode with the KV history in pinned host memory")
    ap.add_argument("--distill", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the stage-1 indexer distillation on the prefill workload")
    ap.add_argument("--cpu-rows", type=int, default=2304,
                    help="query rows in the oracle's timed sample")
    return ap.parse_args()


# ------------------------------------------------------------ workloads ----
def make_prefill_inputs(name, block_size=4):
    from block_sparse_trainable_amd import synth
    if name == "chunked":
        if block_size != 4:
            return synth.chunked(layout=synth.Layout(block_size=block_size)), {
                "workload": f"chunked-prefill-128k-r{block_size}", "batch": 2,
                "cached_tokens": 131072, "chunk_tokens": 8192}
        return synth.chunked(), {"workload": "chunked-prefill-128k", "batch": 2,
                                 "cached_tokens": 131072, "chunk_tokens": 8192}
    if name == "companion":
        return synth.stack_layer(0, companion=4096), {
            "workload": "companion-prefill-1m", "batch": 1, "cached_tokens": 1048576 - 4096,
            "chunk_tokens": 4096}
    return synth.prefill(), {"workload": "prefill-32k", "batch": 1, "cached_tokens": 0,
                             "chunk_tokens": 32768}


def token_visits(x) -> int:
    """sum over queries of |S_i| = r*min(k_B, c_i) + (p_i mod r) + 1."""
    kB, r = x.layout.k_blocks, x.layout.block_size
    tot = 0
    for s in range(x.batch):
        p = x.q_pos0[s] + np.arange(x.n_q, dtype=np.int64)
        c = p // r
        tot += int((r * np.minimum(kB, c) + (p % r) + 1).sum())
    return tot


def score_pairs(x) -> int:
    """sum over queries of c_i (visible candidate blocks)."""
    r = x.layout.block_size
    tot = 0
    for s in range(x.batch):
        p = x.q_pos0[s] + np.arange(x.n_q, dtype=np.int64)
        tot += int((p // r).sum())
    return tot


# ---------------------------------------------------------------- prefill --
def bench_prefill(args, torch):
    from block_sparse_trainable_amd.runtime import DeviceLayer
    t0 = time.time()
    x, cfg = make_prefill_inputs(args.workload, args.block_size)
    log(f"generated {x.name} in {time.time() - t0:.1f}s")
    dl = DeviceLayer(x, "cuda:0")
    dl.build_prefix(x.cache_len)
    torch.cuda.synchronize()
    outs = dl.alloc_prefill_outputs()
    sel, cnt, scs, out, lse = outs
    r = x.layout.block_size
    q_pos0 = dl.i32(x.q_pos0)
    cache_len = dl.i32(x.cache_len)
    end_np = x.q_pos0.astype(np.int64) + x.n_q
    end = dl.i32(end_np)
    max_pos_end = int(end_np.max())
    new_blocks = int((end_np // r - x.cache_len // r).max())
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(rec=None):
        e = [ev() for _ in range(4)] if rec is not None else None
        if e: e[0].record()
        dl.index_build(cache_len, end, new_blocks)
        if e: e[1].record()
        dl.select(dl.q_idx, q_pos0, max_pos_end, sel, cnt, scs)
        if e: e[2].record()
        dl.attend_prefill(dl.q, q_pos0, max_pos_end, sel, cnt, out, lse)
        if e:
            e[3].record()
            rec.append(e)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("prefill warm")
    recs = []
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step(recs)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps
    build_ms = np.mean([e[0].elapsed_time(e[1]) for e in recs])
    select_ms = np.mean([e[1].elapsed_time(e[2]) for e in recs])
    attn_ms = np.mean([e[2].elapsed_time(e[3]) for e in recs])
    toks = x.batch * x.n_q
    visits = token_visits(x)
    pairs = score_pairs(x)
    attn_bytes = visits * x.layout.kv_heads * x.layout.head_dim * 2 * 2
    res = {
        "ms_per_step": ms, "tok_s": toks / (ms / 1e3), "tokens": toks,
        "stages_ms": {"index_build": build_ms, "score_select": select_ms,
                      "sparse_attn_prefill": attn_ms},
        "attn_bytes": attn_bytes, "token_visits": visits, "score_pairs": pairs,
        "score_flops": pairs * 2 * x.layout.idx_heads * x.layout.idx_dim,
    }
    if args.backward:
        res["backward"] = bench_backward(args, torch, x, dl, outs, q_pos0, max_pos_end)
    if args.distill:
        res["distill"] = bench_distill(args, torch, x, dl, q_pos0, max_pos_end)
    cfg.update({"q_heads": x.layout.q_heads, "kv_heads": x.layout.kv_heads,
                "head_dim": x.layout.head_dim, "token_budget": x.layout.token_budget,
                "block_size": r, "idx_heads": x.layout.idx_heads, "idx_dim": x.layout.idx_dim})
    del dl, outs
    torch.cuda.empty_cache()
    return x, cfg, res


# --------------------------------------------------------------- backward --
def group_entries(x, sel, cnt) -> int:
    """(query, 16-token group) pairs of the token sets: the key side's work
    items, each reading the query's transposed q and dO once."""
    r, kB = x.layout.block_size, x.layout.k_blocks
    m = r // 4
    tot = 0
    for s in range(x.batch):
        for j in range(x.n_q):
            p = int(x.q_pos0[s]) + j
            c = p // r
            n = min(max(int(cnt[s, j]), 0), kB, c)
            b = np.clip(sel[s, j, :n].astype(np.int64), 0, max(c - 1, 0))
            units = np.concatenate([(b[:, None] * m + np.arange(m)).ravel(),
                                    c * m + np.arange((p - c * r) // 4 + 1)])
            g = units >> 2
            tot += 1 + int((g[1:] != g[:-1]).sum())
    return tot


def bench_backward(args, torch, x, dl, outs, q_pos0, max_pos_end):
    """Gradients of the chunk's sparse attention (dq, dK, dV) for a seeded
    dL/dout, on the forward's own selections."""
    sel, cnt, scs, out, lse = outs
    g = torch.Generator(device="cuda:0")
    g.manual_seed(5)
    dout = torch.randn(dl.q.shape, generator=g, device="cuda:0", dtype=torch.float32).to(dl.q.dtype)
    dq = torch.empty_like(dl.q)
    dk = torch.zeros(dl.k.shape, dtype=torch.float32, device="cuda:0")
    dv = torch.zeros_like(dk)

    def call():
        dl.attend_backward(dl.q, q_pos0, max_pos_end, sel, cnt, out, lse, dout, dq, dk, dv)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    lay = x.layout
    visits = token_visits(x)
    entries = group_entries(x, sel.cpu().numpy(), cnt.cpu().numpy())
    rows = x.batch * x.n_q
    row_bytes = lay.q_heads * lay.head_dim * 2          # one bf16 row of q, dO, out or dq
    kd = lay.kv_heads * lay.head_dim
    parts = {
        "kv_gather": visits * kd * 2 * 2,               # K and V rows per token visit
        "p_weight_export": visits * lay.q_heads * 8 * 2,  # written by the query side, read back
        "rows": rows * row_bytes * 6 + rows * lay.q_heads * 4 * 2,  # q,dO,out,dq,qT,dOT; lse, D
        "transposed_reads": entries * row_bytes * 2,    # qT and dO^T per group entry
    }
    tot = sum(parts.values())
    log(f"backward {ms:.3f} ms/call, {entries} group entries")
    cpu = None if args.no_cpu_baseline else cpu_baseline_backward(
        x, sel.cpu().numpy(), cnt.cpu().numpy(), dout.float().cpu().numpy(), 96)
    return {"ms_per_call": ms, "tok_s": rows / (ms / 1e3), "token_visits": visits,
            "cpu_baseline": cpu,
            "group_entries": entries, "algorithmic_bytes": parts,
            "achieved_gbs": tot / (ms * 1e-3) / 1e9,
            "hbm_frac": tot / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


# ---------------------------------------------------------------- distill --
def bench_distill(args, torch, x, dl, q_pos0, max_pos_end):
    """Stage-1 indexer distillation on the chunk: the dense teacher over
    tokens 0..p of every query (two passes), the student over its candidate
    blocks, dq_idx and dk_cmp."""
    lay = x.layout
    loss = torch.empty((x.batch, x.n_q), dtype=torch.float32, device="cuda:0")
    dq_idx = torch.empty((x.batch, x.n_q, lay.idx_heads, lay.idx_dim), dtype=torch.float32,
                         device="cuda:0")
    dk_cmp = torch.zeros(dl.k_cmp.shape, dtype=torch.float32, device="cuda:0")

    def call():
        dl.distill(q_pos0, max_pos_end, loss, dq_idx, dk_cmp)

    call()
    torch.cuda.synchronize()
    n = max(1, min(args.steps, 3))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(n):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / n
    r = lay.block_size
    visits = cand = 0
    for s in range(x.batch):
        p = x.q_pos0[s] + np.arange(x.n_q, dtype=np.int64)
        visits += int((p + 1).sum())                    # teacher tokens 0..p
        cand += int((p // r).sum())                     # candidate blocks
    per_tok = 2 * lay.q_heads * lay.head_dim            # one logit for every head
    teacher = visits * per_tok + cand * r * per_tok     # pass 1 over 0..p, pass 2 over candidates
    student = cand * 2 * lay.idx_heads * lay.idx_dim * 4   # dots twice, dq_idx, dk_cmp
    log(f"distill {ms:.3f} ms/call")
    cpu = None if args.no_cpu_baseline else cpu_baseline_distill(x, 8)
    return {"ms_per_call": ms, "rows_per_s": x.batch * x.n_q / (ms / 1e3),
            "cpu_baseline": cpu,
            "teacher_token_visits": visits, "candidate_pairs": cand,
            "flops": {"teacher": teacher, "student": student},
            "mfma_frac": (teacher + student) / (ms * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12),
            "mean_loss": float(loss.mean().item())}


# ----------------------------------------------------------------- decode --
def bench_decode(args, torch):
    """Decode loop: `steps` steps of index_build + select_topk + attention for
    8 sequences at 256K context, as one fused launch per step
    (qsa_decode_step) and as the three separate calls (several scheduling
    variants), each captured in one HIP graph and replayed; the best is
    reported, eager per-step times beside it."""
    from block_sparse_trainable_amd import synth
    from block_sparse_trainable_amd.runtime import DeviceLayer
    steps = args.decode_steps
    t0 = time.time()
    x = synth.decode(steps=steps)
    log(f"generated {x.name} in {time.time() - t0:.1f}s")
    dl = DeviceLayer(x, "cuda:0")
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(steps)
    outs = dl.alloc_decode_outputs()
    torch.cuda.synchronize()
    for t in range(min(8, steps)):          # warm-up (rebuilding a block is idempotent)
        dl.decode_step(plan, t, outs)
    torch.cuda.synchronize()
    # eager, per-step events
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for t in range(steps):
        dl.decode_step(plan, t, outs)
        evs[t + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[t].elapsed_time(evs[t + 1]) for t in range(steps)]) * 1e3
    eager_us = evs[0].elapsed_time(evs[-1]) * 1e3 / steps
    # the same steps through the fused entry point (one launch per step)
    for t in range(min(8, steps)):
        dl.decode_step_fused(plan, t, outs)
    torch.cuda.synchronize()
    evs[0].record()
    for t in range(steps):
        dl.decode_step_fused(plan, t, outs)
        evs[t + 1].record()
    torch.cuda.synchronize()
    per_f = np.array([evs[t].elapsed_time(evs[t + 1]) for t in range(steps)]) * 1e3
    fused_eager_us = evs[0].elapsed_time(evs[-1]) * 1e3 / steps
    dl.check_step()     # raises (the run fails) if a wait for a selection gave up
    # graph replay, for each scheduling variant; the best one is reported
    variants = {}
    for name, kw in (("fused", None), ("inline-build", {}), ("side-build", {"overlap_build": True}),
                     ("2-branch", {"branches": 2}), ("4-branch", {"branches": 4})):
        if kw is None:
            g = dl.capture_decode_fused(plan, steps, outs)
        else:
            g = dl.capture_decode(plan, steps, outs, **kw)
        g.replay()
        torch.cuda.synchronize()
        reps = 5
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(reps):
            g.replay()
        s1.record()
        torch.cuda.synchronize()
        variants[name] = s0.elapsed_time(s1) * 1e3 / (reps * steps)
        if kw is None:
            dl.check_step()
        del g
    log(f"decode graph variants (us/step): {variants}")
    best = min(variants, key=variants.get)
    graph_us = variants[best]
    # cold: the fused graph with step t on replica t % 4 of the caches (equal
    # values, other addresses), so the ~600 MB working set cannot stay in the
    # 256 MB Infinity Cache; every replica holds every block the steps touch
    reps = [dl] + [dl.replica() for _ in range(3)]
    ws = dl.step_workspace(plan[4])
    for r in reps:
        for t in range(min(8, steps)):
            r.decode_step_fused(plan, t, outs, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(steps):
            reps[t % 4].decode_step_fused(plan, t, outs, ws)
    g.replay()
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(5):
        g.replay()
    s1.record()
    torch.cuda.synchronize()
    cold_us = s0.elapsed_time(s1) * 1e3 / (5 * steps)
    dl.check_step(ws)
    del g, reps
    log(f"decode fused, 4 rotating cache replicas: {cold_us:.1f} us/step")
    kB = x.layout.k_blocks
    ctx = x.q_pos0.astype(np.int64)
    scan_bytes = int(sum((ctx[s] + t) // 4 for s in range(x.batch) for t in range(steps))) * 256 // steps
    gather = int(x.batch * (4 * kB + 4) * x.layout.kv_heads * x.layout.head_dim * 4)
    res = {"workload": "decode-256k", "batch": x.batch, "context": int(ctx.min()),
           "steps": steps, "us_per_step": graph_us, "mode": f"hip-graph ({best})",
           "graph_variants_us": variants,
           "eager_us_per_step": eager_us,
           "eager_p50_us": float(np.percentile(per, 50)),
           "eager_p99_us": float(np.percentile(per, 99)),
           "fused_eager_us_per_step": fused_eager_us,
           "fused_eager_p50_us": float(np.percentile(per_f, 50)),
           "fused_eager_p99_us": float(np.percentile(per_f, 99)),
           "algorithmic_bytes_per_step": scan_bytes + gather,
           "hbm_frac": (scan_bytes + gather) / (graph_us * 1e-6) / (HBM_PEAK_GBS * 1e9),
           "step_error_word": dl.step_error_word(ws),
           "cold_4_replicas_us_per_step": cold_us,
           "cold_hbm_frac": (scan_bytes + gather) / (cold_us * 1e-6) / (HBM_PEAK_GBS * 1e9)}
    if args.offload:
        res["offload"] = bench_offload(args, torch, x, dl, plan, steps)
    del dl, outs
    torch.cuda.empty_cache()
    return res


def bench_offload(args, torch, x, dl, plan, steps):
    """The same decode steps with the K/V history in pinned host memory:
    index build + top-k on the GPU-resident index, staging of each step's
    token set (hot cache of 65,536 4-token units per sequence, the rest from
    host), attention over the staging buffer.  Every timed run starts from an
    empty hot cache (its tags reset by a fill kernel)."""
    from block_sparse_trainable_amd.runtime import OffloadedKV
    off = OffloadedKV(dl, 65536)
    outs = dl.alloc_decode_outputs()
    for t in range(min(4, steps)):
        off.decode_step(plan, t, outs)
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # eager, with the per-step hit and miss counts
    off.hot_tag.fill_(-1)
    recs = []
    start, stop = ev(), ev()
    start.record()
    for t in range(steps):
        off.decode_step(plan, t, outs)
        recs.append(off.stats.sum(0))
    stop.record()
    torch.cuda.synchronize()
    eager_us = start.elapsed_time(stop) * 1e3 / steps
    tot = torch.stack(recs).sum(0).cpu().numpy()
    hits, miss = int(tot[0]), int(tot[1])
    # the same run captured in one HIP graph
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        off.hot_tag.fill_(-1)
        for t in range(steps):
            off.decode_step(plan, t, outs)
    g.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(3):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    graph_us = start.elapsed_time(stop) * 1e3 / (3 * steps)
    unit_bytes = 4 * x.layout.kv_heads * x.layout.head_dim * 2 * 2   # K and V of 4 tokens
    host_bytes = miss * unit_bytes / steps
    log(f"decode offloaded: {graph_us:.1f} us/step (graph), {eager_us:.1f} eager, "
        f"hit rate {hits / max(1, hits + miss):.3f}")
    del g, off
    return {"us_per_step": graph_us, "mode": "hip-graph (index build, top-k, staging, attention)",
            "eager_us_per_step": eager_us,
            "hot_units_per_sequence": 65536, "hit_rate": hits / max(1, hits + miss),
            "host_bytes_per_step": host_bytes,
            "host_gbs": host_bytes / (graph_us * 1e-6) / 1e9}


def bench_stack_decode(args, torch):
    """Decode through a stack of 12 independent QSA layers at a 1M-token
    context, batch 1: each step runs the fused decode step of every layer in
    turn (a layer's input depends on the previous layer's output in a model,
    so the layers are not overlapped).  `steps` steps in one HIP graph."""
    from block_sparse_trainable_amd import synth
    from block_sparse_trainable_amd.runtime import DeviceLayer
    steps = args.decode_steps
    n_layers = 12
    layers = []
    t0 = time.time()
    for l in range(n_layers):
        x = synth.stack_layer(l, steps=steps)
        dl = DeviceLayer(x, "cuda:0")
        dl.build_prefix(x.cache_len)
        plan = dl.decode_plan(steps)
        outs = dl.alloc_decode_outputs()
        ws = dl.step_workspace(plan[4])
        scan = int(sum((int(x.q_pos0[0]) + t) // 4 for t in range(steps))) * 256 // steps
        kB = x.layout.k_blocks
        gather = int((4 * kB + 4) * x.layout.kv_heads * x.layout.head_dim * 4)
        dl.x = None  # host copies are no longer needed
        layers.append((dl, plan, outs, ws, scan + gather))
        del x
        torch.cuda.synchronize()
        log(f"stack layer {l} ready ({time.time() - t0:.0f}s)")
    for t in range(min(4, steps)):
        for dl, plan, outs, ws, _ in layers:
            dl.decode_step_fused(plan, t, outs, ws)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for t in range(steps):
        for dl, plan, outs, ws, _ in layers:
            dl.decode_step_fused(plan, t, outs, ws)
        evs[t + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[t].elapsed_time(evs[t + 1]) for t in range(steps)]) * 1e3
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for t in range(steps):
            for dl, plan, outs, ws, _ in layers:
                dl.decode_step_fused(plan, t, outs, ws)
    g.replay()
    torch.cuda.synchronize()
    reps = 3
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(reps):
        g.replay()
    s1.record()
    torch.cuda.synchronize()
    graph_us = s0.elapsed_time(s1) * 1e3 / (reps * steps)
    for dl, plan, outs, ws, _ in layers:
        dl.check_step(ws)
    err_words = sum(dl.step_error_word(ws) for dl, plan, outs, ws, _ in layers)
    bytes_step = sum(b for *_, b in layers)
    res = {"workload": "stack-12x1m-decode", "layers": n_layers, "batch": 1,
           "context": 1048576, "steps": steps, "us_per_step": graph_us,
           "mode": "hip-graph (fused, layers in sequence)", "step_error_word": err_words,
           "eager_us_per_step": float(per.mean()), "eager_p50_us": float(np.percentile(per, 50)),
           "eager_p99_us": float(np.percentile(per, 99)),
           "algorithmic_bytes_per_step": bytes_step,
           "hbm_frac": bytes_step / (graph_us * 1e-6) / (HBM_PEAK_GBS * 1e9)}
    del g, layers
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------ cpu oracle --
def cpu_baseline(x, rows: int):
    """The fp64 oracle on a bounded sample of the same chunk: compression of
    every new block of the chunk, then `rows` query rows (scoring, top-k,
    attention), single-threaded; extrapolated to the full chunk."""
    from threadpoolctl import threadpool_limits
    from oracle import qsa_oracle as O
    from block_sparse_trainable_amd import synth
    lay = x.layout
    f64 = lambda a: synth.as_f32(a, lay.dtype).astype(np.float64)
    rng = np.random.default_rng(7)
    with threadpool_limits(limits=1):
        t_comp = 0.0
        khat = []
        for s in range(x.batch):
            # the cached prefix is setup work on both sides; only the chunk's
            # new blocks are timed
            nb_all = (int(x.q_pos0[s]) + x.n_q) // lay.block_size
            nb_old = int(x.cache_len[s]) // lay.block_size
            k_idx = f64(x.k_idx[s, :nb_all * lay.block_size])
            r = lay.block_size
            kh_old = O.compress_index(k_idx[:nb_old * r], nb_old, r=r,
                                      gain=x.gain.astype(np.float64),
                                      eps=float(np.float32(lay.rms_eps)), storage=lay.dtype)
            t = time.perf_counter()
            kh_all = O.compress_index(k_idx, nb_all, r=r, gain=x.gain.astype(np.float64),
                                      eps=float(np.float32(lay.rms_eps)), storage=lay.dtype)
            t_comp += (time.perf_counter() - t) * (nb_all - nb_old) / max(nb_all, 1)
            khat.append(kh_all)
            del kh_old
        per_seq = max(1, rows // x.batch)
        t_rows = 0.0
        n_rows = 0
        for s in range(x.batch):
            K, V = f64(x.k[s]), f64(x.v[s])
            q_idx, q = f64(x.q_idx[s]), f64(x.q[s])
            for j in rng.choice(x.n_q, size=min(per_seq, x.n_q), replace=False):
                p = int(x.q_pos0[s]) + int(j)
                t = time.perf_counter()
                O.qsa_row(p, q_idx[j], q[j], khat[s], K, V, k_B=lay.k_blocks, r=lay.block_size)
                t_rows += time.perf_counter() - t
                n_rows += 1
    total = x.batch * x.n_q
    est = t_comp + t_rows * total / n_rows
    return {"value": total / est, "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": (f"{n_rows} of {total} query rows (uniform seeded sample) plus the "
                       f"compression of the chunk's new blocks, single thread; extrapolated "
                       f"to the full chunk"),
            "measured_s": t_comp + t_rows}


def _sample_rows(x, rows, seed):
    rng = np.random.default_rng(seed)
    per = max(1, rows // x.batch)
    return [(s, int(j)) for s in range(x.batch)
            for j in rng.choice(x.n_q, size=min(per, x.n_q), replace=False)]


def cpu_baseline_backward(x, sel, cnt, dout, rows: int):
    """The oracle's attention backward on a seeded sample of query rows (the
    GPU's selections), single-threaded; extrapolated to every row."""
    from threadpoolctl import threadpool_limits
    from oracle import qsa_oracle as O
    from block_sparse_trainable_amd import synth
    lay = x.layout
    f64 = lambda a: synth.as_f32(a, lay.dtype).astype(np.float64)
    scale = 1.0 / math.sqrt(lay.head_dim)
    sample = _sample_rows(x, rows, 11)
    t_rows = 0.0
    with threadpool_limits(limits=1):
        for s in range(x.batch):
            K, V, q = f64(x.k[s]), f64(x.v[s]), f64(x.q[s])
            dK = np.zeros_like(K)
            dV = np.zeros_like(V)
            for (ss, j) in sample:
                if ss != s:
                    continue
                p = int(x.q_pos0[s]) + j
                S = O.expand_with_tail(np.sort(sel[s, j, :int(cnt[s, j])]), p, lay.block_size)
                t = time.perf_counter()
                O.sparse_attention_backward(q[j], K, V, S, dout[s, j], scale, dK, dV)
                t_rows += time.perf_counter() - t
    total = x.batch * x.n_q
    return {"value": len(sample) / t_rows, "unit": "query rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(sample)} of {total} query rows (uniform seeded sample), single "
                      f"thread, on the GPU's selections", "measured_s": t_rows}


def cpu_baseline_distill(x, rows: int):
    """The oracle's distillation (dense teacher target, KL, gradients) on a
    seeded sample of query rows, single-threaded; extrapolated."""
    from threadpoolctl import threadpool_limits
    from oracle import qsa_oracle as O
    from block_sparse_trainable_amd import synth
    lay = x.layout
    f64 = lambda a: synth.as_f32(a, lay.dtype).astype(np.float64)
    scale = 1.0 / math.sqrt(lay.head_dim)
    r = lay.block_size
    sample = _sample_rows(x, rows, 12)
    t_rows = 0.0
    with threadpool_limits(limits=1):
        for s in range(x.batch):
            end = int(x.q_pos0[s]) + x.n_q
            kh = O.compress_index(f64(x.k_idx[s, :(end // r) * r]), end // r, r=r,
                                  gain=x.gain.astype(np.float64),
                                  eps=float(np.float32(lay.rms_eps)), storage=lay.dtype)
            K, q, qi = f64(x.k[s]), f64(x.q[s]), f64(x.q_idx[s])
            for (ss, j) in sample:
                if ss != s:
                    continue
                p = int(x.q_pos0[s]) + j
                t = time.perf_counter()
                tb = O.teacher_block_target(q[j], K, p, r, scale)
                I = O.block_importance(qi[j], kh, p // r)
                _, dI = O.distill_row(tb, I)
                O.distill_grads(qi[j], kh, dI)
                t_rows += time.perf_counter() - t
    total = x.batch * x.n_q
    return {"value": len(sample) / t_rows, "unit": "query rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(sample)} of {total} query rows (uniform seeded sample), single "
                      f"thread", "measured_s": t_rows}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the QSA forward path here is single-GPU "
              "(no sharding or collectives are built); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_trainable_amd as qsa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    qsa.load()
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read_per_launch": n,
                          "bytes_written_per_launch": n, "launches": 3}), flush=True)
        return
    run_decode = bench_stack_decode if args.decode == "stack" else bench_decode
    if args.only == "decode":
        dec = run_decode(args, torch)
        print(json.dumps({"metric": METRIC, "value": None, "unit": "tok/s", "n_gpus": 1,
                          "decode": dec, "note": "decode leg only"}), flush=True)
        return
    x, cfg, pre = bench_prefill(args, torch)
    log(f"prefill {pre['tok_s']:.0f} tok/s, {pre['ms_per_step']:.3f} ms/step, "
        f"stages {pre['stages_ms']}")
    dec = run_decode(args, torch) if (args.decode != "none" and args.only is None) else None
    if dec:
        log(f"decode {dec['us_per_step']:.1f} us/step")

    attn_ms = pre["stages_ms"]["sparse_attn_prefill"]
    achieved = pre["attn_bytes"] / (attn_ms * 1e-3) / 1e9
    roofline = {"kernel": "sparse_attn_prefill (attn_mfma_kernel<2,128>)", "bound": "hbm",
                "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": attn_traffic_bytes(),
                "algorithmic_bytes_per_launch": pre["attn_bytes"],
                "avg_launch_ms": attn_ms,
                # the gather kernel's own contraction (QK^T and PV: 8,192 flop
                # per token visit at 16 heads x 128 dims) against the dense
                # bf16 MFMA peak, for reference: it runs at 8 flop per byte
                "mfma_frac": pre["token_visits"] * 4 * x.layout.q_heads * x.layout.head_dim
                             / (attn_ms * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12)}
    score_tflops = pre["score_flops"] / (pre["stages_ms"]["score_select"] * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(x, args.cpu_rows)
        log(f"cpu baseline {cpu['value']:.2f} tok/s over {cpu['measured_s']:.1f}s")

    line = {
        "metric": METRIC, "value": pre["tok_s"], "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": cfg, "roofline": roofline, "cpu_baseline": cpu,
        "stages_ms": pre["stages_ms"],
        "score_select_effective_tflops": score_tflops,
        "decode": dec,
        "backward": pre.get("backward"),
        "distill": pre.get("distill"),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
