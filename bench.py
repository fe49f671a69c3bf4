"""QSA layer forward pass benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--legs LIST] [--block-size R]

One step = one pass of the whole hot path over one batch of synthetic input:
index build of the chunk's new blocks -> block scoring + top-k_B selection ->
sparse attention.  The headline workload is chunked prefill at 128K context
(2 sequences, 131,072 cached tokens, 8,192 new queries each, 16Q/2KV heads,
d=128, K=2048, r=4, bf16); `value` is prefill tokens/s with every input
resident in HBM.  Beside it, one object per other workload:

  prefill_32k   1 x 32,768 queries from an empty cache;
  companion_1m  the last 4,096 queries of a 1,048,576-token context;
  decode        8 sequences at 256K context, 64 decode steps (fused step in a
                HIP graph, a cold variant on 4 rotating cache replicas, the
                three-call variants, the KV history offloaded to host memory);
  stack_1m      12 independent layers at 1M context, batch 1, 64 decode steps,
                the layers strictly in sequence;
  backward, distill   the attention backward and the stage-1 distillation on
                the headline chunk.

Timing: torch.cuda events on the stream every kernel is launched on (the
binding launches on torch's current stream), a device synchronisation on
both sides of the timed region.  The dominant kernel's average duration is
taken from events around its launches inside the timed region.

The oracle (fp64, CPU) is timed last, on the host's cores, one worker process
per usable core (at most 16), on seeded row samples of the same workloads.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import shutil
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA prefill tok/s + decode µs/step at 128K–1M ctx; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
ALL_LEGS = ("chunked", "backward", "distill", "prefill32k", "companion", "decode", "offload",
            "stack", "cpu")

# Bytes that went past the L2 (to the Infinity Cache or HBM) in one
# sparse_attn_prefill launch on the 128K chunked workload, from rocprofv3
# --pmc runs of `bench.py --legs chunked --steps 2 --warmup 1 --cpu-rows 0`:
# 32*TCC_EA0_RDREQ_32B + 64*TCC_EA0_RDREQ_64B + 128*TCC_EA0_RDREQ_128B read,
# 64*TCC_EA0_WRREQ_64B + 32*(TCC_EA0_WRREQ - TCC_EA0_WRREQ_64B) written, each
# scaled by what the same counters give for a plain 1 GiB device copy
# (`bench.py --calibrate-copy`).  They belong to the attention source with
# this SHA-1; for any other source `traffic` is null until they are retaken.
ATTN_COUNTERS = {
    "source_sha1": "4f6c5d6b3b1244ba0162c6782310ca6ccfeb219e",
    "read_bytes": 19240783458.9, "write_bytes": 68166082.9,
    # the 1 GiB copy read back as 1,073,757,227 B and 1,073,741,824 B
    "read_scale": 0.99998566, "write_scale": 1.00000000,
}


def attn_source_digest() -> str:
    """sha1 over the sources the prefill attention kernel is compiled from."""
    import hashlib
    h = hashlib.sha1()
    for f in ("attn.hip", "attn_tile.h", "qsa_common.h", "fast_exp.h"):
        with open(os.path.join(ROOT, "block_sparse_trainable_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def attn_traffic_bytes():
    c = ATTN_COUNTERS
    if c["source_sha1"] is None or attn_source_digest() != c["source_sha1"]:
        return None
    return c["read_bytes"] * c["read_scale"] + c["write_bytes"] * c["write_scale"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default=",".join(ALL_LEGS),
                    help="comma-separated subset of " + ",".join(ALL_LEGS))
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (3 times), the "
                         "known-size reference for scaling HBM byte counters")
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--block-size", type=int, default=4,
                    help="r of the chunked prefill workload (4 = the pages' configuration)")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="query rows in the oracle's timed sample of the chunked workload")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (0: one per usable core, at most 16)")
    a = ap.parse_args(argv)
    a.legs = [l for l in a.legs.split(",") if l]
    bad = [l for l in a.legs if l not in ALL_LEGS]
    if bad:
        ap.error(f"unknown legs {bad}")
    return a


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


def group_entries(x, sel, cnt) -> int:
    """(query, 16-token group) pairs of the token sets: the backward key
    side's work items, each reading the query's transposed q and dO once."""
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


def _ev(torch):
    return torch.cuda.Event(enable_timing=True)


# ---------------------------------------------------------------- prefill --
def bench_prefill(args, torch, name, keep=False):
    """index_build + select_topk + sparse_attn_prefill over one chunk, timed
    per stage.  keep: also return the device layer and outputs (for the
    backward, distillation and cold-attention legs)."""
    from block_sparse_trainable_amd.runtime import DeviceLayer
    t0 = time.time()
    x, cfg = make_prefill_inputs(name, args.block_size if name == "chunked" else 4)
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

    def step(rec=None):
        e = [_ev(torch) for _ in range(4)] if rec is not None else None
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
    recs = []
    start, stop = _ev(torch), _ev(torch)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step(recs)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    build_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in recs]))
    select_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in recs]))
    attn_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in recs]))
    lay = x.layout
    toks = x.batch * x.n_q
    visits = token_visits(x)
    pairs = score_pairs(x)
    gather = visits * lay.kv_heads * lay.head_dim * 2 * 2      # K and V rows, bf16
    attn_flops = visits * 4 * lay.q_heads * lay.head_dim     # q.k and p.v per head
    score_flops = pairs * 2 * lay.idx_heads * lay.idx_dim
    res = {
        "workload": cfg["workload"], "ms_per_step": ms, "tok_s": toks / (ms / 1e3),
        "tokens": toks,
        "stages_ms": {"index_build": build_ms, "score_select": select_ms,
                      "sparse_attn_prefill": attn_ms},
        "score_select": {
            "flops": score_flops,
            "tflops": score_flops / (select_ms * 1e-3) / 1e12,
            "mfma_frac": score_flops / (select_ms * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12),
            "note": "scoring and top-k together (one call, two kernels); scoring's own "
                    "fraction is in the kernel statistics"},
        "attention": {
            "token_visits": visits, "flops": attn_flops, "avg_launch_ms": attn_ms,
            "mfma_frac": attn_flops / (attn_ms * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12),
            "gather_bytes": gather, "gather_gbs": gather / (attn_ms * 1e-3) / 1e9,
            "note": "gather_gbs counts every token visit's K/V rows; rows gathered again "
                    "by other queries are served from L2 or the Infinity Cache, so it can "
                    "exceed the HBM peak"},
    }
    cfg.update({"q_heads": lay.q_heads, "kv_heads": lay.kv_heads, "head_dim": lay.head_dim,
                "token_budget": lay.token_budget, "block_size": r, "idx_heads": lay.idx_heads,
                "idx_dim": lay.idx_dim})
    log(f"{cfg['workload']}: {res['tok_s']:.0f} tok/s, {ms:.3f} ms/step, stages "
        f"{ {k: round(v, 4) for k, v in res['stages_ms'].items()} }")
    if keep:
        return x, cfg, res, (dl, outs, q_pos0, max_pos_end)
    del dl, outs
    torch.cuda.empty_cache()
    return x, cfg, res, None


def bench_attention_cold(args, torch, x, state):
    """sparse_attn_prefill alone with launch i on replica i mod 4 of the KV
    caches (equal values at other addresses): a launch finds nothing of its
    caches left in the Infinity Cache by the previous one."""
    from block_sparse_trainable_amd import _binding as B
    dl, outs, q_pos0, max_pos_end = state
    sel, cnt, scs, out, lse = outs
    reps = [(dl.k, dl.v)] + [(dl.k.clone(), dl.v.clone()) for _ in range(3)]
    ws = dl.workspace(B.QSA_OP_PREFILL, dl.batch, x.n_q, max_pos_end)

    def call(i):
        k, v = reps[i % 4]
        B.qsa_sparse_attn_prefill(dl.cfg, dl.batch, x.n_q, dl.q, k, v, dl.cap, q_pos0,
                                  max_pos_end, sel, cnt, out, lse, ws, ws.numel())

    for i in range(4):
        call(i)
    torch.cuda.synchronize()
    n = 4 * max(1, args.steps // 4)
    start, stop = _ev(torch), _ev(torch)
    start.record()
    for i in range(n):
        call(i)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / n
    del reps
    torch.cuda.empty_cache()
    return ms


# --------------------------------------------------------------- backward --
def bench_backward(args, torch, x, state):
    """Gradients of the chunk's sparse attention (dq, dK, dV) for a seeded
    dL/dout, on the forward's own selections."""
    dl, outs, q_pos0, max_pos_end = state
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
    start, stop = _ev(torch), _ev(torch)
    start.record()
    for _ in range(args.steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    lay = x.layout
    visits = token_visits(x)
    sel_np, cnt_np = sel.cpu().numpy(), cnt.cpu().numpy()
    entries = group_entries(x, sel_np, cnt_np)
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
    flops = visits * lay.q_heads * lay.head_dim * 2 * 4   # S, dP, dq, dK/dV: four contractions
    dout_np = dout.float().cpu().numpy()
    return {"ms_per_call": ms, "rows_per_s": rows / (ms / 1e3), "token_visits": visits,
            "group_entries": entries, "algorithmic_bytes": parts,
            "achieved_gbs": tot / (ms * 1e-3) / 1e9,
            "mfma_frac": flops / (ms * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12),
            "note": "algorithmic bytes count every gather and re-read; most re-reads hit "
                    "L2 or the Infinity Cache, so achieved_gbs is not an HBM rate"}, \
        (sel_np, cnt_np, dout_np)


# ---------------------------------------------------------------- distill --
def bench_distill(args, torch, x, state):
    """Stage-1 indexer distillation on the chunk: the dense teacher over
    tokens 0..p of every query (two passes), the student over its candidate
    blocks, dq_idx and dk_cmp."""
    dl, outs, q_pos0, max_pos_end = state
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
    start, stop = _ev(torch), _ev(torch)
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
    return {"ms_per_call": ms, "rows_per_s": x.batch * x.n_q / (ms / 1e3),
            "teacher_token_visits": visits, "candidate_pairs": cand,
            "flops": {"teacher": teacher, "student": student},
            "mfma_frac": (teacher + student) / (ms * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12),
            "mean_loss": float(loss.mean().item())}


# ----------------------------------------------------------------- decode --
def _graph_us(torch, g, steps, reps=5):
    g.replay()
    torch.cuda.synchronize()
    s0, s1 = _ev(torch), _ev(torch)
    s0.record()
    for _ in range(reps):
        g.replay()
    s1.record()
    torch.cuda.synchronize()
    return s0.elapsed_time(s1) * 1e3 / (reps * steps)


def bench_decode(args, torch, with_offload):
    """Decode loop: `steps` steps of index_build + select_topk + attention for
    8 sequences at 256K context, as one fused launch per step
    (qsa_decode_step) and as the three separate calls (several scheduling
    variants), each captured in one HIP graph and replayed; the fused graph
    is reported, the others and eager per-step times beside it."""
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
    evs = [_ev(torch) for _ in range(steps + 1)]
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
    variants = {}
    for name, kw in (("fused", None), ("inline-build", {}), ("side-build", {"overlap_build": True}),
                     ("2-branch", {"branches": 2}), ("4-branch", {"branches": 4})):
        g = dl.capture_decode_fused(plan, steps, outs) if kw is None else \
            dl.capture_decode(plan, steps, outs, **kw)
        variants[name] = _graph_us(torch, g, steps)
        if kw is None:
            dl.check_step()
        del g
    log(f"decode graph variants (us/step): { {k: round(v, 2) for k, v in variants.items()} }")
    graph_us = variants["fused"]
    # cold: the fused graph with step t on replica t % 4 of the caches (equal
    # values, other addresses), so the ~600 MB working set cannot stay in the
    # 256 MB Infinity Cache; every replica holds every block the steps touch
    reps = [dl] + [dl.replica() for _ in range(3)]
    ws = dl.step_workspace(plan[4])
    for rr in reps:
        for t in range(min(8, steps)):
            rr.decode_step_fused(plan, t, outs, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(steps):
            reps[t % 4].decode_step_fused(plan, t, outs, ws)
    cold_us = _graph_us(torch, g, steps)
    dl.check_step(ws)
    del g, reps
    log(f"decode fused {graph_us:.1f} us/step, cold (4 rotating cache replicas) {cold_us:.1f}")
    kB = x.layout.k_blocks
    ctx = x.q_pos0.astype(np.int64)
    scan_bytes = int(sum((ctx[s] + t) // 4 for s in range(x.batch) for t in range(steps))) * 256 // steps
    gather = int(x.batch * (4 * kB + 4) * x.layout.kv_heads * x.layout.head_dim * 4)
    alg = scan_bytes + gather
    res = {"workload": "decode-256k", "batch": x.batch, "context": int(ctx.min()),
           "steps": steps, "us_per_step": graph_us, "mode": "hip-graph (fused)",
           "graph_variants_us": variants,
           "eager_us_per_step": eager_us,
           "eager_p50_us": float(np.percentile(per, 50)),
           "eager_p99_us": float(np.percentile(per, 99)),
           "fused_eager_us_per_step": fused_eager_us,
           "fused_eager_p50_us": float(np.percentile(per_f, 50)),
           "fused_eager_p99_us": float(np.percentile(per_f, 99)),
           "step_error_word": dl.step_error_word(ws),
           "algorithmic_bytes_per_step": alg,
           "hbm_frac": alg / (graph_us * 1e-6) / (HBM_PEAK_GBS * 1e9),
           "cold_4_replicas_us_per_step": cold_us,
           "cold_hbm_frac": alg / (cold_us * 1e-6) / (HBM_PEAK_GBS * 1e9)}
    if with_offload:
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
    off.hot_tag.fill_(-1)
    recs = []
    start, stop = _ev(torch), _ev(torch)
    start.record()
    for t in range(steps):
        off.decode_step(plan, t, outs)
        recs.append(off.stats.sum(0))
    stop.record()
    torch.cuda.synchronize()
    eager_us = start.elapsed_time(stop) * 1e3 / steps
    tot = torch.stack(recs).sum(0).cpu().numpy()
    hits, miss = int(tot[0]), int(tot[1])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        off.hot_tag.fill_(-1)
        for t in range(steps):
            off.decode_step(plan, t, outs)
    graph_us = _graph_us(torch, g, steps, reps=3)
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
    from concurrent.futures import ThreadPoolExecutor
    from block_sparse_trainable_amd import synth
    from block_sparse_trainable_amd.runtime import DeviceLayer
    steps = args.decode_steps
    n_layers = 12
    t0 = time.time()
    layers = []
    with ThreadPoolExecutor(min(n_layers, max(1, len(os.sched_getaffinity(0))))) as ex:
        futs = [ex.submit(synth.stack_layer, l, steps=steps) for l in range(n_layers)]
        for l in range(n_layers):
            x = futs[l].result()
            futs[l] = None
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
    log(f"stack: 12 layers generated and uploaded in {time.time() - t0:.0f}s")
    for t in range(min(4, steps)):
        for dl, plan, outs, ws, _ in layers:
            dl.decode_step_fused(plan, t, outs, ws)
    torch.cuda.synchronize()
    evs = [_ev(torch) for _ in range(steps + 1)]
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
    graph_us = _graph_us(torch, g, steps, reps=3)
    for dl, plan, outs, ws, _ in layers:
        dl.check_step(ws)
    err_words = sum(dl.step_error_word(ws) for dl, plan, outs, ws, _ in layers)
    bytes_step = sum(b for *_, b in layers)
    log(f"stack 12 x 1M: {graph_us:.1f} us/step")
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
# The oracle runs in worker processes started fresh (spawn: they never touch
# the GPU), one per usable core.  The parent writes each sequence's inputs as
# .npy files that the workers memory-map; a task is one query row.
_OW = None


def _oracle_init(paths, meta):
    global _OW
    _OW = {"meta": meta}
    for k, p in paths.items():
        _OW[k] = np.load(p, mmap_mode="r")


def _oracle_task(task):
    from oracle import qsa_oracle as O
    kind, s, j = task
    W, meta = _OW, _OW["meta"]
    p = int(meta["q_pos0"][s]) + j
    r, kB, scale = meta["r"], meta["k_B"], meta["scale"]
    t = time.perf_counter()
    if kind == "fwd":
        O.qsa_row(p, W[f"qi{s}"][j], W[f"q{s}"][j], W[f"kh{s}"], W[f"K{s}"], W[f"V{s}"],
                  k_B=kB, r=r)
    elif kind == "bwd":
        n = int(W[f"cnt{s}"][j])
        S = O.expand_with_tail(np.sort(np.asarray(W[f"sel{s}"][j, :n])), p, r)
        key = f"dK{s}"
        if key not in W:   # the accumulators of this worker
            W[key] = np.zeros(W[f"K{s}"].shape)
            W[f"dV{s}"] = np.zeros(W[f"V{s}"].shape)
        O.sparse_attention_backward(W[f"q{s}"][j], W[f"K{s}"], W[f"V{s}"], S,
                                    W[f"dout{s}"][j], scale, W[key], W[f"dV{s}"])
    else:  # "distill"
        tb = O.teacher_block_target(W[f"q{s}"][j], W[f"K{s}"], p, r, scale)
        I = O.block_importance(W[f"qi{s}"][j], W[f"kh{s}"], p // r)
        _, dI = O.distill_row(tb, I)
        O.distill_grads(W[f"qi{s}"][j], W[f"kh{s}"], dI)
    return time.perf_counter() - t


def _pool_size(args):
    n = len(os.sched_getaffinity(0))
    return max(1, min(n, 16) if args.cpu_workers <= 0 else args.cpu_workers)


def cpu_baselines(args, x, bwd_data):
    """The fp64 oracle, as it stands, on bounded seeded samples of the
    headline chunk: the forward (compression of the chunk's new blocks in
    this process, then `cpu_rows` query rows: scoring, top-k, attention),
    and, when their legs ran, the backward (on the GPU's selections) and the
    distillation."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import qsa_oracle as O
    from block_sparse_trainable_amd import synth
    lay = x.layout
    r = lay.block_size
    f32 = lambda a: synth.as_f32(a, lay.dtype)
    workers = _pool_size(args)
    host = {"sched_getaffinity": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count()}
    tmp = tempfile.mkdtemp(prefix="qsa_oracle_",
                           dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        paths = {}

        def put(name, arr):
            paths[name] = os.path.join(tmp, name + ".npy")
            np.save(paths[name], np.ascontiguousarray(arr))

        t_comp = 0.0
        with threadpool_limits(limits=1):
            for s in range(x.batch):
                nb_all = (int(x.q_pos0[s]) + x.n_q) // r
                nb_old = int(x.cache_len[s]) // r
                k_idx = f32(x.k_idx[s, :nb_all * r]).astype(np.float64)
                t = time.perf_counter()
                kh = O.compress_index(k_idx, nb_all, r=r, gain=x.gain.astype(np.float64),
                                      eps=float(np.float32(lay.rms_eps)), storage=lay.dtype)
                # the cached prefix is setup work on both sides: only the
                # chunk's new blocks are charged
                t_comp += (time.perf_counter() - t) * (nb_all - nb_old) / max(nb_all, 1)
                put(f"kh{s}", kh)
                put(f"K{s}", f32(x.k[s]))
                put(f"V{s}", f32(x.v[s]))
                put(f"qi{s}", f32(x.q_idx[s]))
                put(f"q{s}", f32(x.q[s]))
                if bwd_data is not None:
                    sel, cnt, dout = bwd_data
                    put(f"sel{s}", sel[s])
                    put(f"cnt{s}", cnt[s])
                    put(f"dout{s}", dout[s])
        meta = {"q_pos0": [int(v) for v in x.q_pos0], "r": r, "k_B": lay.k_blocks,
                "scale": 1.0 / math.sqrt(lay.head_dim)}
        total = x.batch * x.n_q

        def sample(kind, rows, seed):
            g = np.random.default_rng(seed)
            per = max(1, rows // x.batch)
            return [(kind, s, int(j)) for s in range(x.batch)
                    for j in g.choice(x.n_q, size=min(per, x.n_q), replace=False)]

        legs = {"fwd": sample("fwd", args.cpu_rows, 7)}
        if bwd_data is not None:
            legs["bwd"] = sample("bwd", 16 * workers, 11)
        if "distill" in args.legs:
            legs["distill"] = sample("distill", 4 * workers, 12)
        saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                "MKL_NUM_THREADS")}
        for k in saved:
            os.environ[k] = "1"
        out = {}
        try:
            # a worker that dies raises BrokenProcessPool here (no silent respawn)
            with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"),
                                     initializer=_oracle_init,
                                     initargs=(paths, meta)) as pool:
                list(pool.map(_oracle_task, [("fwd", 0, 0)] * (2 * workers)))   # warm
                for kind, tasks in legs.items():
                    t = time.perf_counter()
                    busy = sum(pool.map(_oracle_task, tasks))
                    out[kind] = (len(tasks), time.perf_counter() - t, busy)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    n, wall, busy = out["fwd"]
    est = t_comp + wall * total / n
    res = {"cpu_baseline": {
        "value": total / est, "unit": "tok/s", "cores": workers, "kind": "oracle",
        "sample": (f"{n} of {total} query rows (uniform seeded sample) on {workers} worker "
                   f"processes, plus the compression of the chunk's new blocks in one; "
                   f"extrapolated to the full chunk"),
        "measured_s": t_comp + wall, "cpu_seconds": t_comp + busy, "host_cores": host}}
    if "bwd" in out:
        n, wall, busy = out["bwd"]
        res["backward"] = {"value": n / wall, "unit": "query rows/s", "cores": workers,
                           "kind": "oracle", "sample": f"{n} of {total} query rows, on the "
                           f"GPU's selections", "measured_s": wall, "cpu_seconds": busy}
    if "distill" in out:
        n, wall, busy = out["distill"]
        res["distill"] = {"value": n / wall, "unit": "query rows/s", "cores": workers,
                          "kind": "oracle", "sample": f"{n} of {total} query rows",
                          "measured_s": wall, "cpu_seconds": busy}
    return res


# -------------------------------------------------------------------- main --
def main(argv=None):
    args = parse(argv)
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

    legs = args.legs
    if args.block_size < 4:   # the backward and the distillation work on 4-token units
        legs = [l for l in legs if l not in ("backward", "distill")]
    line = {"metric": METRIC, "value": None, "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": None, "roofline": None, "cpu_baseline": None}
    x = bwd_data = None
    if "chunked" in legs:
        x, cfg, pre, state = bench_prefill(args, torch, "chunked", keep=True)
        cold_ms = bench_attention_cold(args, torch, x, state)
        att = pre["attention"]
        att["cold_4_replicas_avg_launch_ms"] = cold_ms
        att["cold_gather_gbs"] = att["gather_bytes"] / (cold_ms * 1e-3) / 1e9
        achieved = att["flops"] / (att["avg_launch_ms"] * 1e-3) / 1e12
        line.update({
            "value": pre["tok_s"], "ms_per_step": pre["ms_per_step"], "config": cfg,
            # The dominant kernel against its roofline.  Its minimum traffic (each
            # distinct K/V row once, plus q and out) gives an arithmetic intensity
            # far above the MFMA ridge, so the binding roof is the bf16 MFMA peak;
            # the kernel re-gathers rows per query instead of sharing them, which
            # is what keeps it below.  `traffic` is the counter-measured bytes
            # past L2 per launch (null until retaken for the current source).
            "roofline": {"kernel": "sparse_attn_prefill (attn_mfma_kernel<2,128>)",
                         "bound": "mfma", "achieved": achieved,
                         "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                         "traffic": attn_traffic_bytes(),
                         "algorithmic_flops_per_launch": att["flops"],
                         "avg_launch_ms": att["avg_launch_ms"],
                         "gather_gbs": att["gather_gbs"],
                         "cold_gather_gbs": att["cold_gather_gbs"]},
            "stages_ms": pre["stages_ms"], "score_select": pre["score_select"],
            "attention": att,
        })
        if "backward" in legs:
            line["backward"], bwd_data = bench_backward(args, torch, x, state)
        if "distill" in legs:
            line["distill"] = bench_distill(args, torch, x, state)
        del state
        torch.cuda.empty_cache()
    if "prefill32k" in legs:
        _, cfg2, res, _ = bench_prefill(args, torch, "prefill32k")
        res["config"] = cfg2
        line["prefill_32k"] = res
    if "companion" in legs:
        _, cfg5, res, _ = bench_prefill(args, torch, "companion")
        res["config"] = cfg5
        line["companion_1m"] = res
    if "decode" in legs:
        line["decode"] = bench_decode(args, torch, "offload" in legs)
    if "stack" in legs:
        line["stack_1m"] = bench_stack_decode(args, torch)
    if "cpu" in legs and x is not None:
        log(f"cpu baseline (oracle), {_pool_size(args)} worker processes ...")
        cpu = cpu_baselines(args, x, bwd_data if "backward" in legs else None)
        line["cpu_baseline"] = cpu["cpu_baseline"]
        if "backward" in cpu and "backward" in line:
            line["backward"]["cpu_baseline"] = cpu["backward"]
        if "distill" in cpu and "distill" in line:
            line["distill"]["cpu_baseline"] = cpu["distill"]
        log(f"cpu baseline {line['cpu_baseline']['value']:.1f} tok/s on "
            f"{line['cpu_baseline']['cores']} workers")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
