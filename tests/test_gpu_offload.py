"""GPU parity of decode with the KV history in pinned host memory
(qsa_offload_stage + qsa_sparse_attn_decode on the staging buffer).

Every step is run twice: the resident path (K/V in GPU memory) and the
offloaded one.  Selections are the same call on the same index; the
offloaded attention visits the same token set in another order, so its
output is compared with the resident one and with the fp64 oracle at the
attention tolerance.  The hot cache must hold exactly the host rows of the
units it names, the first step must read everything from host, a unit
selected again must be found, and staging a step a second time must hit
every unit that kept its slot (the synthetic queries are independent draws,
so consecutive steps share few blocks; correlated queries would share more).
"""
import math
import sys

import numpy as np
import pytest
import torch

from block_sparse_trainable_amd import synth
from block_sparse_trainable_amd.runtime import DeviceLayer, OffloadedKV, to_f32
from tests import _compare as C

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-offload] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("r,hot_units,steps", [(4, 4096, 6), (4, 64, 5), (16, 1024, 5)])
def test_offloaded_decode_matches_resident(r, hot_units, steps):
    say(f"offloaded decode r={r} hot_units={hot_units} steps={steps}")
    lay = synth.Layout(block_size=r)
    x = synth.decode(context=30000, batch=2, steps=steps, n_needles=8, layout=lay)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(steps)
    off = OffloadedKV(dl, hot_units)
    res = dl.alloc_decode_outputs()
    ofs = dl.alloc_decode_outputs()
    scale = 1.0 / math.sqrt(lay.head_dim)
    K = [C.f64(x.k[s], "bf16") for s in range(2)]
    V = [C.f64(x.v[s], "bf16") for s in range(2)]
    for t in range(steps):
        dl.decode_step(plan, t, res)
        off.decode_step(plan, t, ofs)
        torch.cuda.synchronize()
        sel_r, cnt_r = res[0].cpu().numpy(), res[1].cpu().numpy()
        sel_o, cnt_o = ofs[0].cpu().numpy(), ofs[1].cpu().numpy()
        assert (sel_r == sel_o).all() and (cnt_r == cnt_o).all()
        out_r, out_o = to_f32(res[3]), to_f32(ofs[3])
        assert np.abs(out_r - out_o).max() <= C.ATOL["bf16"]
        assert np.abs(res[4].cpu().numpy() - ofs[4].cpu().numpy()).max() <= 1e-3
        stats = off.stats.cpu().numpy()
        for s in range(2):
            p = int(x.q_pos0[s]) + t
            c = p // r
            n = int(cnt_o[s, 0])
            units = n * (r // 4) + (p - c * r) // 4 + 1
            assert stats[s].sum() == units
            if t == 0:
                assert stats[s, 0] == 0                  # a cold cache: everything from host
            elif hot_units >= 1024:
                assert stats[s, 0] > 0                   # blocks selected again are found
            if t in (0, steps - 1):
                q = C.f64(x.q[s, t], "bf16")
                C.check_attention(p, sel_o[s, 0, :n], q, K[s], V[s], out_o[s], ofs[4][s].cpu().numpy(),
                                  scale, "bf16", r)
        say(f"step {t}: hits/misses {stats.tolist()}")
    # staging the last step again: every unit that kept its slot is a hit
    # (units of one set that share a slot evict each other)
    last = steps - 1
    tags = off.hot_tag.cpu().numpy()                    # before the repeat
    off.stage(plan[2][last], ofs[0][:, 0], ofs[1][:, 0])
    torch.cuda.synchronize()
    again = off.stats.cpu().numpy()
    cnt_o = ofs[1].cpu().numpy()
    for s in range(2):
        p = int(x.q_pos0[s]) + last
        c = p // r
        n = int(cnt_o[s, 0])
        m = r // 4
        sel = ofs[0].cpu().numpy()[s, 0, :n].astype(np.int64)
        units = np.concatenate([(sel[:, None] * m + np.arange(m)).ravel(),
                                c * m + np.arange((p - c * r) // 4 + 1)])
        held = int((tags[s, units % hot_units] == units).sum())
        assert again[s, 0] == held and again[s].sum() == len(units)
        if hot_units >= 4096:
            assert held >= 0.9 * len(units)
    # the hot cache holds exactly the host rows of the units it names
    tags = off.hot_tag.cpu().numpy()
    hk = off.hot_k.cpu()
    for s in range(2):
        for slot in np.nonzero(tags[s] >= 0)[0][:200]:
            u = int(tags[s, slot])
            assert u % hot_units == slot
            assert torch.equal(hk[s, slot], off.k_host[s, 4 * u:4 * u + 4])


def test_offloaded_decode_graph_replays():
    """The offloaded steps captured in one HIP graph (the hot cache emptied by
    a fill kernel at its start) replay bit for bit as the eager run, with
    eager work between the replays."""
    say("offloaded decode: 4 steps in a graph, 3 replays vs eager")
    x = synth.decode(context=30000, batch=2, steps=4, n_needles=8)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(4)
    off = OffloadedKV(dl, 2048)
    outs = dl.alloc_decode_outputs()
    off.hot_tag.fill_(-1)
    eager = []
    for t in range(4):
        off.decode_step(plan, t, outs)
        eager.append((outs[3].clone(), outs[4].clone(), off.stats.clone()))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        off.hot_tag.fill_(-1)
        for t in range(4):
            off.decode_step(plan, t, outs)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs[3], eager[-1][0]) and torch.equal(outs[4], eager[-1][1])
        assert torch.equal(off.stats, eager[-1][2])
        dl.decode_step(plan, rep, dl.alloc_decode_outputs())   # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("r", [4, 16])
def test_offloaded_decode_rows_written_step_by_step(r):
    """Real decode writes row p into host memory only just before step p.
    The unit holding p also spans rows p+1.. that are not written yet, so
    it must never be served from the hot cache: with garbage in every host
    row past the current position, each step must still match the
    resident path."""
    say(f"offloaded decode, host rows written step by step, r={r}")
    steps = 9
    lay = synth.Layout(block_size=r)
    x = synth.decode(context=20000, batch=2, steps=steps, n_needles=4, layout=lay)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(steps)
    off = OffloadedKV(dl, 4096)
    garbage = torch.full(off.k_host.shape[2:], 7.5, dtype=off.k_host.dtype)
    for s in range(2):
        p0 = int(x.q_pos0[s])
        off.k_host[s, p0:] = garbage
        off.v_host[s, p0:] = -garbage
    k_cpu, v_cpu = dl.k.cpu(), dl.v.cpu()
    res = dl.alloc_decode_outputs()
    ofs = dl.alloc_decode_outputs()
    for t in range(steps):
        torch.cuda.synchronize()
        for s in range(2):                  # the new token's row arrives now
            p = int(x.q_pos0[s]) + t
            off.k_host[s, p] = k_cpu[s, p]
            off.v_host[s, p] = v_cpu[s, p]
        dl.decode_step(plan, t, res)
        off.decode_step(plan, t, ofs)
        torch.cuda.synchronize()
        assert torch.equal(res[0], ofs[0]) and torch.equal(res[1], ofs[1])
        err = np.abs(to_f32(res[3]) - to_f32(ofs[3])).max()
        assert err <= C.ATOL["bf16"], f"step {t}: offloaded output off by {err:.3e}"
        assert np.abs(res[4].cpu().numpy() - ofs[4].cpu().numpy()).max() <= 1e-3
    # no cached unit reaches past the last position
    tags = off.hot_tag.cpu().numpy()
    for s in range(2):
        p = int(x.q_pos0[s]) + steps - 1
        u = tags[s][tags[s] >= 0].astype(np.int64)
        assert (4 * u + 3 <= p).all()
