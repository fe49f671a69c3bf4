"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test prints the case it is about to run (flushed) before touching the
GPU.  Inputs come from the seeded generator; the oracle never sees a value
produced by the GPU except the selection it is asked to attend over in the
stage-isolated attention checks.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import qsa_oracle as O
from block_sparse_trainable_amd import _binding as B
from block_sparse_trainable_amd import synth
from block_sparse_trainable_amd.runtime import DeviceLayer, bf16_bits, to_f32
from tests import _compare as C

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _run_prefill(x):
    dl = DeviceLayer(x)
    if (x.cache_len > 0).any():
        dl.build_prefix(x.cache_len)
    outs = dl.prefill_chunk()
    torch.cuda.synchronize()
    return dl, outs


def _host(outs, dtype):
    sel, cnt, scs, out, lse = outs
    return (sel.cpu().numpy(), cnt.cpu().numpy(), scs.cpu().numpy(), to_f32(out),
            lse.cpu().numpy())


def _check_rows(x, dl, outs, rows_by_seq, khat=None, check_attn=True):
    lay = x.layout
    sel, cnt, scs, out, lse = _host(outs, lay.dtype)
    kB = lay.k_blocks
    scale = 1.0 / math.sqrt(lay.head_dim)
    stats = []
    for s, rows in rows_by_seq.items():
        nb_needed = (int(x.q_pos0[s]) + max(rows)) // lay.block_size
        kh = khat[s] if khat is not None else C.oracle_khat(x, s, max(nb_needed, 1))
        q_idx = C.f64(x.q_idx[s], lay.dtype)
        q = C.f64(x.q[s], lay.dtype)
        K = C.f64(x.k[s], lay.dtype)
        V = C.f64(x.v[s], lay.dtype)
        for j in rows:
            p = int(x.q_pos0[s]) + j
            res = O.qsa_row(p, q_idx[j], q[j], kh, K, V, k_B=kB, attend=False)
            rc = C.check_selection(res, sel[s, j], int(cnt[s, j]), scs[s, j], kB)
            stats.append(rc)
            if check_attn:
                count = int(cnt[s, j])
                C.check_attention(p, sel[s, j, :count], q[j], K, V, out[s, j], lse[s, j],
                                  scale, lay.dtype, lay.block_size)
    return stats


# ------------------------------------------------------------ compression --
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_index_build_matches_oracle_with_ragged_ranges(dtype):
    say(f"index_build parity dtype={dtype}")
    lay = synth.Layout(dtype=dtype)
    x = synth.prefill(n=1000, batch=3, layout=lay,
                      gain=np.random.default_rng(5).uniform(0.5, 1.5, 128).astype(np.float32))
    dl = DeviceLayer(x)
    sentinel = -7.0
    dl.k_cmp.fill_(sentinel)
    lb = np.array([0, 13, 401], np.int32)      # ragged: not multiples of 4
    la = np.array([999, 14, 1000], np.int32)
    dl.index_build(dl.i32(lb), dl.i32(la), 250)
    torch.cuda.synchronize()
    got = to_f32(dl.k_cmp)
    for s in range(3):
        kh = C.oracle_khat(x, s, la[s] // 4)
        b0, b1 = lb[s] // 4, la[s] // 4
        built = got[s, b0:b1].astype(np.float64)
        ref = kh[b0:b1]
        # fp64 on both sides then one rounding: equal but for a rare 1-ulp tie case
        ulp = np.abs(ref) * (2.0 ** -7 if dtype == "bf16" else 2.0 ** -23)
        diff = np.abs(built - ref)
        assert (diff <= ulp + 1e-30).all(), f"seq {s}: compression error {diff.max():.3e}"
        if diff.size:
            assert np.mean(diff > 0) < 1e-3
        assert (got[s, :b0] == sentinel).all() and (got[s, b1:] == sentinel).all()


def test_index_build_decode_step_builds_only_completed_block():
    say("index_build single-token steps")
    x = synth.prefill(n=64, batch=4)
    dl = DeviceLayer(x)
    dl.k_cmp.fill_(3.0)
    pos = np.array([3, 4, 6, 11], np.int32)  # (p+1) % 4 == 0 only for 3 and 11
    dl.index_build(dl.i32(pos), dl.i32(pos + 1), 1)
    torch.cuda.synchronize()
    got = to_f32(dl.k_cmp)
    for s, p in enumerate(pos):
        changed = np.nonzero((got[s] != 3.0).any(axis=1))[0].tolist()
        assert changed == ([p // 4] if (p + 1) % 4 == 0 else []), (s, p, changed)


# ------------------------------------------------------------ tiny fp32 ----
@pytest.mark.parametrize("budget", [64, 256])
def test_tiny_fp32_all_rows(budget):
    say(f"tiny fp32 n=256 K={budget}")
    x = synth.tiny(token_budget=budget)
    dl, outs = _run_prefill(x)
    stats = _check_rows(x, dl, outs, {0: list(range(256))})
    assert np.mean([s.exact_eligible for s in stats]) > 0.8


def test_tiny_fp32_full_budget_equals_dense_causal():
    say("tiny fp32 full budget vs dense causal")
    x = synth.tiny(token_budget=256)
    dl, outs = _run_prefill(x)
    out = to_f32(outs[3])[0]
    q = C.f64(x.q[0], "f32")
    K = C.f64(x.k[0, :256], "f32")
    V = C.f64(x.v[0, :256], "f32")
    qt = torch.tensor(q).permute(1, 0, 2)
    kt = torch.tensor(K).permute(1, 0, 2).repeat_interleave(4, 0)
    vt = torch.tensor(V).permute(1, 0, 2).repeat_interleave(4, 0)
    dense = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    dense = dense.permute(1, 0, 2).numpy()
    assert np.abs(out - dense).max() <= C.ATOL["f32"]


# ------------------------------------------------------------- bf16 small --
@pytest.mark.parametrize("n,budget,batch", [(3000, 2048, 1), (2333, 256, 2), (777, 16, 1)])
def test_prefill_bf16_matches_oracle(n, budget, batch):
    say(f"prefill bf16 n={n} K={budget} batch={batch}")
    lay = synth.Layout(token_budget=budget)
    x = synth.prefill(n=n, batch=batch, layout=lay, needle_frac=0.02)
    dl, outs = _run_prefill(x)
    rows = {s: list(range(0, n, 1 if n <= 1000 else 3)) for s in range(batch)}
    stats = _check_rows(x, dl, outs, rows)
    assert len(stats) > 0


def test_prefill_bf16_full_budget_equals_dense_causal():
    say("prefill bf16 full budget vs dense causal")
    lay = synth.Layout(token_budget=2048)
    x = synth.prefill(n=1500, layout=lay)   # every c <= 375 < k_B
    dl, outs = _run_prefill(x)
    sel, cnt, _, out, _ = _host(outs, "bf16")
    assert (cnt[0] == np.arange(1500) // 4).all()
    q = C.f64(x.q[0], "bf16")
    K = C.f64(x.k[0, :1500], "bf16")
    V = C.f64(x.v[0, :1500], "bf16")
    qt = torch.tensor(q).permute(1, 0, 2)
    kt = torch.tensor(K).permute(1, 0, 2).repeat_interleave(8, 0)
    vt = torch.tensor(V).permute(1, 0, 2).repeat_interleave(8, 0)
    dense = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    dense = dense.permute(1, 0, 2).numpy()
    assert np.abs(out[0] - dense).max() <= C.ATOL["bf16"]


def test_chunked_prefill_small_ragged():
    say("chunked prefill bf16 small, ragged cache")
    x = synth.chunked(cache=4098, chunk=701, batch=2, window=256, n_far=4)
    dl, outs = _run_prefill(x)
    _check_rows(x, dl, outs, {s: list(range(0, 701, 2)) for s in range(2)})


def test_prefill_long_rows_match_oracle():
    say("chunked prefill bf16: 64 queries over a 200K-token cache (long-row streaming select)")
    # c ~ 50K blocks per row: past the short-row shape, so the selection
    # streams each row with the rising floor
    x = synth.chunked(cache=200000, chunk=64, batch=1, window=2048, n_far=10)
    dl, outs = _run_prefill(x)
    _check_rows(x, dl, outs, {0: list(range(64))}, check_attn=False)


def test_chunked_equals_monolithic_bitwise():
    say("chunked == monolithic")
    x = synth.prefill(n=2600, needle_frac=0.02)
    dl, outs = _run_prefill(x)
    ref = [t.clone() for t in outs]
    # second layer object: build the prefix of 1001 tokens, then the rest
    split = 1001
    y = synth.LayerInputs(x.layout, x.k_idx, x.q_idx[:, split:], x.q[:, split:], x.k, x.v,
                          q_pos0=np.array([split], np.int32),
                          cache_len=np.array([split], np.int32), gain=x.gain)
    dl2 = DeviceLayer(y)
    dl2.build_prefix(y.cache_len)
    outs2 = dl2.prefill_chunk()
    torch.cuda.synchronize()
    for a, b in zip(ref, outs2):
        assert torch.equal(a[:, split:], b), "chunked result differs from monolithic"
    assert torch.equal(dl.k_cmp, dl2.k_cmp)


@pytest.mark.parametrize("r", [4, 2, 16])
def test_row_order_changes_no_bit(r):
    say(f"prefill attention r={r}: one call over 2 x 3,000 rows (rows run in region order) == "
        "the same rows in calls of 1,000 rows (natural order)")
    x = synth.chunked(cache=20000, chunk=3000, batch=2, window=2048, n_far=6,
                      layout=synth.Layout(block_size=r))
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    outs = dl.alloc_prefill_outputs()
    outs[3].fill_(float("nan"))   # a row the ordered call skipped stays NaN
    outs[4].fill_(float("nan"))
    sel, cnt, _, out, lse = dl.prefill_chunk(outs)
    torch.cuda.synchronize()
    # the call's workspace holds [sort key | walk start | order] per row: the
    # order is a permutation and the workload has clustered rows (key >= 0)
    rows = x.batch * x.n_q
    ws = dl.workspace(B.QSA_OP_PREFILL, x.batch, x.n_q, int(x.q_pos0.max()) + x.n_q)
    w = ws[:12 * rows].view(torch.int32).cpu().numpy()
    assert (np.sort(w[2 * rows:3 * rows]) == np.arange(rows)).all()
    assert (w[:rows] >= 0).sum() > rows // 4, "too few clustered rows to exercise the order"
    end = int(x.q_pos0.max()) + x.n_q
    for j0 in range(0, x.n_q, 500):   # 2 x 500 rows per call: no reordering
        n = min(500, x.n_q - j0)
        o2 = torch.full_like(out[:, j0:j0 + n], float("nan")).contiguous()
        l2 = torch.full_like(lse[:, j0:j0 + n], float("nan")).contiguous()
        dl.attend_prefill(dl.q[:, j0:j0 + n].contiguous(), dl.i32(x.q_pos0 + j0), end,
                          sel[:, j0:j0 + n].contiguous(), cnt[:, j0:j0 + n].contiguous(), o2, l2)
        torch.cuda.synchronize()
        assert torch.equal(out[:, j0:j0 + n], o2), f"rows {j0}..{j0 + n}: output differs"
        assert torch.equal(lse[:, j0:j0 + n], l2), f"rows {j0}..{j0 + n}: lse differs"


def test_prefill_attention_takes_unordered_lists():
    say("prefill attention: each row's selection in a seeded random order (2 x 3,000 rows, "
        "row order on) == the ascending lists, and sampled rows == the oracle")
    x = synth.chunked(cache=20000, chunk=3000, batch=2, window=2048, n_far=6)
    dl, outs = _run_prefill(x)
    sel, cnt, _, out, lse = outs
    rng = np.random.default_rng(7)
    sel_h = sel.cpu().numpy().copy()
    cnt_h = cnt.cpu().numpy()
    for s in range(x.batch):
        for j in range(x.n_q):
            c = int(cnt_h[s, j])
            sel_h[s, j, :c] = rng.permutation(sel_h[s, j, :c])
    shuf = torch.tensor(sel_h, device=sel.device)
    o2 = torch.full_like(out, float("nan"))
    l2 = torch.full_like(lse, float("nan"))
    end = int(x.q_pos0.max()) + x.n_q
    dl.attend_prefill(dl.q, dl.i32(x.q_pos0), end, shuf, cnt, o2, l2)
    torch.cuda.synchronize()
    a, b = to_f32(out), to_f32(o2)
    assert np.isfinite(b).all(), "a row was not written"
    assert np.abs(a - b).max() <= C.ATOL["bf16"]
    assert np.abs(lse.cpu().numpy() - l2.cpu().numpy()).max() <= C.LSE_ATOL["bf16"]
    lay = x.layout
    scale = 1.0 / math.sqrt(lay.head_dim)
    for s in range(x.batch):
        K = C.f64(x.k[s], "bf16")
        V = C.f64(x.v[s], "bf16")
        for j in (0, 1, 777, 2998, 2999):
            p = int(x.q_pos0[s]) + j
            c = int(cnt_h[s, j])
            C.check_attention(p, np.sort(sel_h[s, j, :c]), C.f64(x.q[s, j], "bf16"), K, V,
                              b[s, j], l2.cpu().numpy()[s, j], scale, "bf16")


def test_prefill_deterministic():
    say("determinism")
    x = synth.prefill(n=2100)
    dl, o1 = _run_prefill(x)
    o1 = [t.clone() for t in o1]
    o2 = dl.prefill_chunk()
    torch.cuda.synchronize()
    for a, b in zip(o1, o2):
        assert torch.equal(a, b)


def test_zero_queries_tie_to_lowest_blocks():
    say("all-zero indexer queries -> ties to lowest ids")
    x = synth.prefill(n=2400)
    x.q_idx[:] = 0
    dl, outs = _run_prefill(x)
    sel, cnt, scs, _, _ = _host(outs, "bf16")
    for j in [2052, 2100, 2399]:
        c = j // 4
        assert cnt[0, j] == 512
        assert sel[0, j].tolist() == list(range(512))
        assert (scs[0, j] == 0).all()


def test_exact_ties_prefer_lower_block():
    say("exact score ties -> lower block id")
    lay = synth.Layout(token_budget=64)  # k_B = 16
    x = synth.prefill(n=400, layout=lay, needle_frac=0.0)
    kf = synth.bf16_to_f32(x.k_idx)
    kf[:, :, :64] = 0.0                                      # rotated half zero: no RoPE effect
    rep = kf[0, 0:4].copy()
    for b in range(0, 100, 3):                               # identical blocks 0, 3, 6, ...
        kf[0, 4 * b:4 * b + 4] = rep
    x.k_idx[:] = synth.f32_to_bf16(kf)
    qf = synth.bf16_to_f32(x.q_idx)
    qf[0, :, :, 64:] = rep.mean(0)[None, None, 64:] * 0.5
    x.q_idx[:] = synth.f32_to_bf16(qf)
    dl, outs = _run_prefill(x)
    _check_rows(x, dl, outs, {0: list(range(100, 400, 7))}, check_attn=False)
    sel, cnt, scs, _, _ = _host(outs, "bf16")
    for j in [399, 300]:
        c = j // 4
        tied = list(range(0, min(100, c), 3))
        got = sel[0, j, :16].tolist()
        if len(tied) >= 16:
            assert got == tied[:16], got


def test_many_exact_ties_report_exact_scores():
    """More keys tie at the 16-bit threshold than the row selection resolves
    in LDS (2,500 identical blocks, k_B = 512): the whole-row fallback picks
    the lowest ids and reports their fp32 scores (not the 16-bit keys)."""
    say("2500 identical blocks, nonzero scores: whole-row fallback")
    x = synth.prefill(n=12800, needle_frac=0.0)
    kf = synth.bf16_to_f32(x.k_idx)
    kf[:, :, :64] = 0.0
    rep = kf[0, 0:4].copy()
    for b in range(2500):
        kf[0, 4 * b:4 * b + 4] = rep
    x.k_idx[:] = synth.f32_to_bf16(kf)
    qf = synth.bf16_to_f32(x.q_idx)
    qf[0, :, :, 64:] = rep.mean(0)[None, None, 64:]
    x.q_idx[:] = synth.f32_to_bf16(qf)
    dl, outs = _run_prefill(x)
    _check_rows(x, dl, outs, {0: [10400, 12799]}, check_attn=False)
    sel, cnt, scs, _, _ = _host(outs, "bf16")
    for j in (10400, 12799):
        assert sel[0, j].tolist() == list(range(512))
        assert (scs[0, j] > 100.0).all()


# ----------------------------------------------------------------- decode --
def test_decode_steps_match_oracle_and_prefill_rows():
    say("decode small: 3 seqs x 9 steps")
    x = synth.decode(context=5000, batch=3, steps=9, n_needles=8)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(9)
    outs = dl.alloc_decode_outputs()
    lay = x.layout
    scale = 1.0 / math.sqrt(lay.head_dim)
    per_step = []
    for t in range(9):
        dl.decode_step(plan, t, outs)
        torch.cuda.synchronize()
        per_step.append([o.clone() for o in outs])
    khats = {s: C.oracle_khat(x, s, (int(x.q_pos0[s]) + 9) // 4) for s in range(3)}
    recall = []
    for t, (sel, cnt, scs, out, lse) in enumerate(per_step):
        sel, cnt, scs = sel.cpu().numpy(), cnt.cpu().numpy(), scs.cpu().numpy()
        out, lse = to_f32(out), lse.cpu().numpy()
        for s in range(3):
            p = int(x.q_pos0[s]) + t
            q_idx = C.f64(x.q_idx[s, t], "bf16")
            q = C.f64(x.q[s, t], "bf16")
            K = C.f64(x.k[s], "bf16")
            V = C.f64(x.v[s], "bf16")
            res = O.qsa_row(p, q_idx, q, khats[s], K, V, k_B=lay.k_blocks, attend=False)
            C.check_selection(res, sel[s, 0], int(cnt[s, 0]), scs[s, 0], lay.k_blocks)
            C.check_attention(p, sel[s, 0, :cnt[s, 0]], q, K, V, out[s], lse[s], scale, "bf16")
            recall.append(int(x.target_block[s, t]) in set(sel[s, 0, :cnt[s, 0]].tolist()))
    assert np.mean(recall) == 1.0

    # a decode step equals the prefill row at the same position
    say("decode step == prefill row")
    s_pos = x.q_pos0.copy()
    y = synth.LayerInputs(lay, x.k_idx, x.q_idx, x.q, x.k, x.v, q_pos0=s_pos,
                          cache_len=x.cache_len, gain=x.gain)
    dl2 = DeviceLayer(y)
    dl2.build_prefix(y.cache_len)
    outs2 = dl2.prefill_chunk()
    torch.cuda.synchronize()
    sel2, cnt2, scs2, out2, _ = _host(outs2, "bf16")
    for t in range(9):
        sel, cnt, scs, out, _ = per_step[t]
        assert np.array_equal(sel.cpu().numpy()[:, 0], sel2[:, t])
        assert np.array_equal(scs.cpu().numpy()[:, 0], scs2[:, t])
        assert np.abs(to_f32(out) - out2[:, t]).max() <= 1e-2


def test_decode_graph_replay_matches_eager():
    say("decode graph replay == eager (small)")
    x = synth.decode(context=6000, batch=3, steps=9, n_needles=8)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(9)
    outs = dl.alloc_decode_outputs()
    for t in range(9):
        dl.decode_step(plan, t, outs)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    for kw in ({}, {"overlap_build": True}, {"branches": 2}, {"branches": 3}):
        g = dl.capture_decode(plan, 9, outs, **kw)
        for rep in range(3):
            for o in outs:
                o.zero_()
            g.replay()
            torch.cuda.synchronize()
            for a, b in zip(ref, outs):
                assert torch.equal(a, b), f"replay {rep} ({kw}) differs"
            dl.decode_step(plan, 2, outs)       # eager work between replays
            torch.cuda.synchronize()


def test_long_rows_split_filter_matches_oracle():
    say("select with split filter segments (few long rows)")
    # 3 queries per sequence at ~40K context: rows < 256 and c > 8192, so the
    # row is split over filter workgroups and finished by the last one
    x = synth.decode(context=40000, batch=2, steps=3, n_needles=16)
    y = synth.LayerInputs(x.layout, x.k_idx, x.q_idx, x.q, x.k, x.v, q_pos0=x.q_pos0,
                          cache_len=x.cache_len, gain=x.gain, target_block=x.target_block)
    dl, outs = _run_prefill(y)
    _check_rows(y, dl, outs, {0: [0, 1, 2], 1: [0, 1, 2]})
    sel = outs[0].cpu().numpy()
    for s in range(2):
        for j in range(3):
            assert int(x.target_block[s, j]) in set(sel[s, j].tolist())


def test_decode_single_split_budget_matches_oracle():
    say("decode with k_B = 16 (one attention split, no merge pass)")
    lay = synth.Layout(token_budget=64)
    x = synth.decode(context=3000, batch=2, steps=3, n_needles=4, layout=lay)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(3)
    outs = dl.alloc_decode_outputs()
    scale = 1.0 / math.sqrt(lay.head_dim)
    for t in range(3):
        dl.decode_step(plan, t, outs)
        torch.cuda.synchronize()
        sel, cnt, scs, out, lse = outs
        for s in range(2):
            p = int(x.q_pos0[s]) + t
            kh = C.oracle_khat(x, s, p // 4 + 1)
            K, V = C.f64(x.k[s], "bf16"), C.f64(x.v[s], "bf16")
            q_idx, q = C.f64(x.q_idx[s, t], "bf16"), C.f64(x.q[s, t], "bf16")
            res = O.qsa_row(p, q_idx, q, kh, K, V, k_B=lay.k_blocks, attend=False)
            n = int(cnt[s, 0])
            C.check_selection(res, sel[s, 0].cpu().numpy(), n, scs[s, 0].cpu().numpy(),
                              lay.k_blocks)
            C.check_attention(p, sel[s, 0, :n].cpu().numpy(), q, K, V, to_f32(out[s]),
                              lse[s].cpu().numpy(), scale, "bf16")
