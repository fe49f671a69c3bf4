"""qsa_decode_step_noalloc, the fused decode step with the library's own
per-device step workspace (for callers that cannot allocate), against
qsa_decode_step with a caller workspace: bitwise equal outputs over two
calls in a row, the second with a smaller input; replays of a captured
graph; and the size limit rejected on the host before any launch."""
import sys

import pytest
import torch

from block_sparse_trainable_amd import _binding as B
from block_sparse_trainable_amd import synth
from block_sparse_trainable_amd.runtime import DeviceLayer

pytestmark = pytest.mark.gpu

NAMES = ("sel", "cnt", "scores", "out", "lse")


def say(msg):
    print(f"[gpu-no-alloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _pair(context, batch, steps):
    x = synth.decode(context=context, batch=batch, steps=steps, n_needles=8)
    a, b = DeviceLayer(x), DeviceLayer(x)
    a.build_prefix(x.cache_len)
    b.build_prefix(x.cache_len)
    return x, a, b


def test_noalloc_matches_workspace_call_large_then_small():
    for context, batch, steps in ((70000, 4, 6), (5000, 2, 4)):
        say(f"noalloc vs workspace call: batch {batch}, context {context}, {steps} steps")
        x, a, b = _pair(context, batch, steps)
        pa, pb = a.decode_plan(steps), b.decode_plan(steps)
        oa, ob = a.alloc_decode_outputs(), b.alloc_decode_outputs()
        for t in range(steps):
            a.decode_step_fused(pa, t, oa)
            b.decode_step_noalloc(pb, t, ob)
            torch.cuda.synchronize()
            for name, u, v in zip(NAMES, oa, ob):
                assert torch.equal(u, v), f"step {t}: {name} differs from qsa_decode_step"
        assert torch.equal(a.k_cmp, b.k_cmp)
        a.check_step()


def test_noalloc_graph_replays():
    say("noalloc: 5 steps captured in a graph, replayed 3 times with eager work between")
    x, a, b = _pair(9000, 3, 5)
    pa, pb = a.decode_plan(5), b.decode_plan(5)
    oa, ob = a.alloc_decode_outputs(), b.alloc_decode_outputs()
    for t in range(5):
        a.decode_step_fused(pa, t, oa)
    torch.cuda.synchronize()
    b.decode_step_noalloc(pb, 0, ob)          # an eager call before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(5):
            b.decode_step_noalloc(pb, t, ob)
    for rep in range(3):
        for o in ob:
            o.fill_(-3)
        g.replay()
        torch.cuda.synchronize()
        for name, u, v in zip(NAMES, oa, ob):
            assert torch.equal(u, v), f"replay {rep}: {name} differs"
        b.decode_step_noalloc(pb, 2, b.alloc_decode_outputs())   # eager work between
        torch.cuda.synchronize()


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lay = synth.Layout()
    cfg = B.QsaConfig.from_layout(lay)
    t = torch.zeros(4096, dtype=torch.uint8, device="cuda:0")
    cap = (1 << 20) + 64
    with pytest.raises(B.QsaError) as e:
        B.qsa_decode_step_noalloc(cfg, 64, t, t, t, t, None, t, t, cap, t, 1 << 20, t, t, t, t,
                                  t)
    assert e.value.status == B.QSA_ERR_UNSUPPORTED
    assert "scratch" in str(e.value)
