"""GPU parity of the fused decode step (qsa_decode_step: one launch).

The fused step must reproduce, bit for bit, the three-call decode step
(qsa_index_build + qsa_select_topk + qsa_sparse_attn_decode), which is itself
checked against the fp64 oracle; a few steps are also checked against the
oracle directly.  Cases: multi-segment rows, rows with fewer candidates than
k_B and rows crossing k_B, a budget small enough for a single attention
split, the other head layouts, exact score ties at the threshold, many
candidates inside one score segment, the all-equal fallback, batches split
over several launches, graph replay.
After the calls the workspace's control area must hold each row's flags at
its epoch, the next call's counts clear and the error word clear.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import qsa_oracle as O
from block_sparse_trainable_amd import synth
from block_sparse_trainable_amd.runtime import DeviceLayer, to_f32
from tests import _compare as C

pytestmark = pytest.mark.gpu



def say(msg):
    print(f"[gpu-decode-step] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _ctl_clear(dl, max_pos_end):
    C.check_step_control(dl.step_workspace(max_pos_end), dl.batch)


def _fused_vs_unfused(x, steps, check_oracle_steps=()):
    """Runs both paths step by step from the same state; asserts equality."""
    a = DeviceLayer(x)
    b = DeviceLayer(x)
    a.build_prefix(x.cache_len)
    b.build_prefix(x.cache_len)
    pa, pb = a.decode_plan(steps), b.decode_plan(steps)
    oa, ob = a.alloc_decode_outputs(), b.alloc_decode_outputs()
    got = {}
    for t in range(steps):
        a.decode_step(pa, t, oa)
        b.decode_step_fused(pb, t, ob)
        torch.cuda.synchronize()
        for name, u, v in zip(("sel", "cnt", "scores", "out", "lse"), oa, ob):
            assert torch.equal(u, v), f"step {t}: {name} differs from the three-call path"
        if t in check_oracle_steps:
            got[t] = [o.clone() for o in ob]
    assert torch.equal(a.k_cmp, b.k_cmp), "compressed index differs"
    _ctl_clear(b, pb[4])
    if got:
        lay = x.layout
        scale = 1.0 / math.sqrt(lay.head_dim)
        for s in range(x.batch):
            kh = C.oracle_khat(x, s, max((int(x.q_pos0[s]) + steps) // lay.block_size, 1))
            K, V = C.f64(x.k[s], lay.dtype), C.f64(x.v[s], lay.dtype)
            for t, (sel, cnt, scs, out, lse) in got.items():
                p = int(x.q_pos0[s]) + t
                q_idx, q = C.f64(x.q_idx[s, t], lay.dtype), C.f64(x.q[s, t], lay.dtype)
                res = O.qsa_row(p, q_idx, q, kh, K, V, k_B=lay.k_blocks, attend=False)
                n = int(cnt[s, 0])
                C.check_selection(res, sel[s, 0].cpu().numpy(), n, scs[s, 0].cpu().numpy(),
                                  lay.k_blocks)
                C.check_attention(p, sel[s, 0, :n].cpu().numpy(), q, K, V, to_f32(out[s]),
                                  lse[s].cpu().numpy(), scale, lay.dtype, lay.block_size)
    return a, b


def test_fused_step_multi_segment_rows():
    say("fused step: 3 seqs at ~5000 tokens (2 score segments), 9 steps")
    x = synth.decode(context=5000, batch=3, steps=9, n_needles=8)
    _fused_vs_unfused(x, 9, check_oracle_steps=(0, 3, 8))


def test_fused_step_long_rows_over_64_segments():
    say("fused step: ~300K-token rows (73 score segments)")
    x = synth.decode(context=300000, batch=1, steps=3, n_needles=8)
    _fused_vs_unfused(x, 3, check_oracle_steps=(2,))


def test_fused_step_many_rows_and_segments():
    say("fused step: 20 seqs at ~60K tokens (15 segments each, 300 score workgroups)")
    x = synth.decode(context=60000, batch=20, steps=3, n_needles=8)
    _fused_vs_unfused(x, 3, check_oracle_steps=(2,))


def test_fused_step_rows_crossing_the_budget():
    say("fused step: candidate counts crossing k_B = 512 (c <= k_B rows)")
    x = synth.decode(context=2040, batch=2, steps=16, n_needles=4)
    _fused_vs_unfused(x, 16, check_oracle_steps=(0, 9, 15))


def test_fused_step_short_rows():
    say("fused step: 300-token contexts (c << k_B)")
    x = synth.decode(context=300, batch=2, steps=5, n_needles=2)
    _fused_vs_unfused(x, 5, check_oracle_steps=(0, 4))


def test_fused_step_single_split_budget():
    say("fused step: K = 64 (k_B = 16, one attention split)")
    lay = synth.Layout(token_budget=64)
    x = synth.decode(context=3000, batch=2, steps=6, n_needles=4, layout=lay)
    _fused_vs_unfused(x, 6, check_oracle_steps=(0, 5))


@pytest.mark.parametrize("kv_heads,head_dim", [(1, 128), (2, 64)])
def test_fused_step_other_head_layouts(kv_heads, head_dim):
    say(f"fused step: kv_heads={kv_heads} head_dim={head_dim}")
    lay = synth.Layout(kv_heads=kv_heads, head_dim=head_dim)
    x = synth.decode(context=4100, batch=2, steps=5, n_needles=4, layout=lay)
    _fused_vs_unfused(x, 5, check_oracle_steps=(4,))


def test_fused_step_batch_over_several_launches():
    say("fused step: batch 40 (split over several launches)")
    x = synth.decode(context=2600, batch=40, steps=4, n_needles=2)
    _fused_vs_unfused(x, 4, check_oracle_steps=(3,))


def test_fused_step_exact_ties_at_threshold():
    say("fused step: identical blocks tie at the threshold")
    x = synth.decode(context=6000, batch=2, steps=4, n_needles=1)
    kf = synth.bf16_to_f32(x.k_idx)
    kf[:, :, :64] = 0.0                       # rotated half zero: RoPE leaves keys equal
    qf = synth.bf16_to_f32(x.q_idx)
    for s in range(x.batch):
        rep = kf[s, 0:4].copy()
        for bk in range(0, 1400, 2):          # 700 identical blocks > k_B
            kf[s, 4 * bk:4 * bk + 4] = rep
        qf[s, :, :, 64:] = rep.mean(0)[None, None, 64:] * 0.5
    x.q_idx[:] = synth.f32_to_bf16(qf)
    x.k_idx[:] = synth.f32_to_bf16(kf)
    _fused_vs_unfused(x, 4, check_oracle_steps=(0, 3))


def test_fused_step_clustered_candidates():
    say("fused step: 150 high-scoring blocks inside one of 17 score segments")
    x = synth.decode(context=70000, batch=2, steps=3, n_needles=2)
    kf = synth.bf16_to_f32(x.k_idx)
    qf = synth.bf16_to_f32(x.q_idx)
    for s in range(x.batch):
        d = qf[s, :, :, 64:].mean(axis=(0, 1))          # the steps' shared direction
        d = d / np.linalg.norm(d)
        kf[s, 4 * 5200:4 * 5350, 64:] += 4.0 * d         # blocks 5200..5349, one segment
    x.k_idx[:] = synth.f32_to_bf16(kf)
    a, b = _fused_vs_unfused(x, 3, check_oracle_steps=(0, 2))
    plan = b.decode_plan(3)
    outs = b.alloc_decode_outputs()
    b.decode_step_fused(plan, 0, outs)
    torch.cuda.synchronize()
    sel = outs[0][:, 0].cpu().numpy()
    for s in range(x.batch):   # the cluster must really crowd one segment
        assert ((sel[s] >= 5200) & (sel[s] < 5350)).sum() >= 100
    _ctl_clear(b, plan[4])


def test_fused_step_all_equal_scores_fallback():
    say("fused step: all-zero indexer queries (every score 0: exact fallback)")
    x = synth.decode(context=20000, batch=2, steps=3, n_needles=1)
    x.q_idx[:] = 0
    a, b = _fused_vs_unfused(x, 3)
    plan = b.decode_plan(3)
    outs = b.alloc_decode_outputs()
    b.decode_step_fused(plan, 0, outs)
    torch.cuda.synchronize()
    assert outs[0][:, 0].cpu().numpy().tolist() == [list(range(512))] * 2
    _ctl_clear(b, plan[4])


def test_fused_step_graph_replay():
    say("fused step: graph of 9 steps replayed 3 times with eager work between")
    x = synth.decode(context=6000, batch=3, steps=9, n_needles=8)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(9)
    outs = dl.alloc_decode_outputs()
    for t in range(9):
        dl.decode_step_fused(plan, t, outs)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = dl.capture_decode_fused(plan, 9, outs)
    for rep in range(3):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for u, v in zip(ref, outs):
            assert torch.equal(u, v), f"replay {rep} differs"
        dl.decode_step_fused(plan, 2, outs)
        torch.cuda.synchronize()
        _ctl_clear(dl, plan[4])
