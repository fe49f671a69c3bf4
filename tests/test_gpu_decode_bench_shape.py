"""The decode configuration the benchmark times, tested as it is timed.

8 sequences at 256K context, 64 decode steps of the fused step
(qsa_decode_step) captured in one HIP graph, and the benchmark's cold
variant: the same graph with step t on replica t mod 4 of the caches.  Every
step's outputs (selection, count, scores, output, log-sum-exp) must equal the
three-call path's (qsa_index_build + qsa_select_topk + qsa_sparse_attn_decode)
bit for bit; sampled steps are checked against the fp64 oracle (selection
protocol, attention within 2e-2); the control area must afterwards hold
every row's flags at its epoch, with the error word clear.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import qsa_oracle as O
from block_sparse_trainable_amd import _binding as B
from block_sparse_trainable_amd import synth
from block_sparse_trainable_amd.runtime import DeviceLayer, to_f32
from tests import _compare as C

pytestmark = pytest.mark.gpu

STEPS = 64
NAMES = ("sel", "cnt", "scores", "out", "lse")


def say(msg):
    print(f"[gpu-decode-bench-shape] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def _control_clear(ws, rows=8):
    C.check_step_control(ws, rows)


def _capture(layers, plan, per_step, ws):
    """One graph of STEPS fused steps, step t on layers[t % len(layers)],
    writing its outputs into per_step[t]."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for t in range(STEPS):
            layers[t % len(layers)].decode_step_fused(plan, t, per_step[t], ws)
    return g


def test_fused_decode_graph_at_bench_shape():
    x = synth.decode(steps=STEPS)
    say(f"{x.name}: three-call path, eager")
    ref_layer = DeviceLayer(x)
    ref_layer.build_prefix(x.cache_len)
    plan = ref_layer.decode_plan(STEPS)
    outs = ref_layer.alloc_decode_outputs()
    ref = []
    for t in range(STEPS):
        ref_layer.decode_step(plan, t, outs)
        ref.append([o.clone() for o in outs])
    torch.cuda.synchronize()
    ref_kcmp = ref_layer.k_cmp.clone()
    del ref_layer, outs
    torch.cuda.empty_cache()

    say("fused step: one graph of 64 steps")
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    fplan = dl.decode_plan(STEPS)
    ws = dl.step_workspace(fplan[4])
    per_step = [dl.alloc_decode_outputs() for _ in range(STEPS)]
    g = _capture([dl], fplan, per_step, ws)
    for rep in range(2):
        for o in per_step:
            for u in o:
                u.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert dl.step_error_word(ws) == 0
        for t in range(STEPS):
            for name, u, v in zip(NAMES, ref[t], per_step[t]):
                assert torch.equal(u, v), f"replay {rep}, step {t}: {name} differs"
    assert torch.equal(dl.k_cmp, ref_kcmp), "compressed index differs"
    _control_clear(ws)
    del g

    say("fused step, cold: step t on replica t % 4 of the caches")
    reps = [dl] + [dl.replica() for _ in range(3)]
    for o in per_step:
        for u in o:
            u.fill_(-7)
    g = _capture(reps, fplan, per_step, ws)
    g.replay()
    torch.cuda.synchronize()
    assert dl.step_error_word(ws) == 0
    for t in range(STEPS):
        for name, u, v in zip(NAMES, ref[t], per_step[t]):
            assert torch.equal(u, v), f"cold graph, step {t}: {name} differs"
    _control_clear(ws)
    del g, reps, dl
    torch.cuda.empty_cache()

    say("oracle on sampled steps")
    lay = x.layout
    scale = 1.0 / math.sqrt(lay.head_dim)
    check_steps = (0, 1, 2, 3, 31, 63)
    recall = []
    for s in range(x.batch):
        kh = C.oracle_khat(x, s, (int(x.q_pos0[s]) + STEPS) // 4)
        K, V = C.f64(x.k[s], "bf16"), C.f64(x.v[s], "bf16")
        for t in check_steps:
            sel, cnt, scs, out, lse = ref[t]
            p = int(x.q_pos0[s]) + t
            q_idx, q = C.f64(x.q_idx[s, t], "bf16"), C.f64(x.q[s, t], "bf16")
            res = O.qsa_row(p, q_idx, q, kh, K, V, k_B=lay.k_blocks, attend=False)
            c_sel = sel[s, 0].cpu().numpy()
            n = int(cnt[s, 0])
            C.check_selection(res, c_sel, n, scs[s, 0].cpu().numpy(), lay.k_blocks)
            C.check_attention(p, c_sel[:n], q, K, V, to_f32(out[s]), lse[s].cpu().numpy(),
                              scale, "bf16")
            recall.append(int(x.target_block[s, t]) in set(c_sel[:n].tolist()))
        say(f"seq {s} checked against the oracle")
    assert np.mean(recall) == 1.0
