"""GPU parity of the sparse attention backward (qsa_sparse_attn_backward)
against the fp64 oracle's exact derivative, on the GPU's own selections.

Tolerance (the pages fix none for a backward): every element within
1e-2 * max(|ref|, RMS of the checked tensor) in bf16 layers (dq is rounded
to bf16; the forward's log-sum-exp is fp32), 1e-4 in fp32 layers.  Cases: bf16 prefill (r = 4 and r = 16; the three head shapes of the MFMA
path), a chunk over a cache
(gradients reach cached rows), an fp32 layer on the generic path, and the
accumulating contract of dk/dv.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import qsa_oracle as O
from block_sparse_trainable_amd import synth
from block_sparse_trainable_amd.runtime import DeviceLayer, to_device, to_f32
from tests import _compare as C

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-backward] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _run(x, seed=21):
    """Forward (index build + select + attention), then the backward with a
    seeded dL/dout.  Returns the host copies and dout."""
    lay = x.layout
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    outs = dl.prefill_chunk()
    sel, cnt, scs, out, lse = outs
    rng = np.random.default_rng(seed)
    dout_np = synth._store(rng.standard_normal(x.q.shape).astype(np.float32), lay.dtype)
    dout = to_device(dout_np, lay.dtype, dl.device)
    dq = torch.empty_like(dl.q)
    dk = torch.zeros(dl.k.shape, dtype=torch.float32, device=dl.device)
    dv = torch.zeros_like(dk)
    q_pos0 = dl.i32(x.q_pos0)
    mpe = int((x.q_pos0.astype(np.int64) + x.n_q).max())
    dl.attend_backward(dl.q, q_pos0, mpe, sel, cnt, out, lse, dout, dq, dk, dv)
    torch.cuda.synchronize()
    return dl, (sel, cnt, out, lse, dout, dq, dk, dv), C.f64(dout_np, lay.dtype)


def _oracle(x, sel, cnt, dO, rows_by_seq):
    """Oracle dq for the given rows and dK/dV summed over ALL rows (every row
    adds to them), on the GPU's selections."""
    lay = x.layout
    r = lay.block_size
    scale = 1.0 / math.sqrt(lay.head_dim)
    dq = {}
    dK = np.zeros((x.batch,) + x.k.shape[1:])
    dV = np.zeros_like(dK)
    for s in range(x.batch):
        q = C.f64(x.q[s], lay.dtype)
        K = C.f64(x.k[s], lay.dtype)
        V = C.f64(x.v[s], lay.dtype)
        for j in range(x.n_q):
            p = int(x.q_pos0[s]) + j
            n = int(cnt[s, j])
            S = O.expand_with_tail(np.sort(sel[s, j, :n]), p, r)
            g = O.sparse_attention_backward(q[j], K, V, S, dO[s, j], scale, dK[s], dV[s])
            if j in rows_by_seq.get(s, ()):
                dq[(s, j)] = g
    return dq, dK, dV


def _close(got, ref, rel, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    floor = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    err = np.abs(got - ref)
    bound = rel * np.maximum(np.abs(ref), floor)
    worst = float((err / np.maximum(bound, 1e-30)).max()) if ref.size else 0.0
    assert (err <= bound).all(), f"{what}: worst error {worst:.3g} x the bound"
    return worst


def _check(x, res, dO, rel, rows):
    sel, cnt, out, lse, dout, dq, dk, dv = res
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    ref_dq, ref_dK, ref_dV = _oracle(x, sel_h, cnt_h, dO, rows)
    dq_h = to_f32(dq)
    keys = sorted(ref_dq)
    w0 = _close(np.stack([dq_h[s, j] for s, j in keys]), np.stack([ref_dq[k] for k in keys]),
                rel, "dq")
    w1 = _close(dk.cpu().numpy(), ref_dK, rel, "dk")
    w2 = _close(dv.cpu().numpy(), ref_dV, rel, "dv")
    say(f"worst error / bound: dq {w0:.3f}, dk {w1:.3f}, dv {w2:.3f}")


@pytest.mark.parametrize("r", [4, 16])
def test_backward_bf16_prefill(r):
    say(f"backward bf16 prefill n=1100 r={r}")
    lay = synth.Layout(block_size=r, token_budget=512)
    x = synth.prefill(n=1100, layout=lay, needle_frac=0.05)
    dl, res, dO = _run(x)
    _check(x, res, dO, 1e-2, {0: set(range(0, 1100, 5)) | {1099}})


@pytest.mark.parametrize("kv_heads,head_dim", [(1, 128), (2, 64)])
def test_backward_bf16_head_shapes(kv_heads, head_dim):
    say(f"backward bf16 prefill n=900, {kv_heads} KV heads, d={head_dim}")
    lay = synth.Layout(token_budget=256, kv_heads=kv_heads, head_dim=head_dim)
    x = synth.prefill(n=900, layout=lay, needle_frac=0.05)
    dl, res, dO = _run(x)
    _check(x, res, dO, 1e-2, {0: set(range(0, 900, 4)) | {899}})


def test_backward_chunk_over_cache():
    say("backward bf16: 300 queries over a 3001-token cache, batch 2")
    lay = synth.Layout(token_budget=256)
    x = synth.chunked(cache=3001, chunk=300, batch=2, window=256, n_far=4, layout=lay)
    dl, res, dO = _run(x)
    _check(x, res, dO, 1e-2, {s: set(range(0, 300, 3)) for s in range(2)})


def test_backward_fp32_generic():
    say("backward fp32, 4 heads / 1 KV head, d=64, r=8")
    lay = synth.Layout(block_size=8, token_budget=128, dtype="f32", q_heads=4, kv_heads=1,
                       head_dim=64)
    x = synth.prefill(n=600, layout=lay, needle_frac=0.05)
    dl, res, dO = _run(x)
    _check(x, res, dO, 1e-4, {0: set(range(600))})


def test_backward_adds_into_dk_dv():
    say("backward: dk/dv are added into")
    lay = synth.Layout(token_budget=256)
    x = synth.prefill(n=500, layout=lay)
    dl, res, dO = _run(x)
    sel, cnt, out, lse, dout, dq, dk, dv = res
    k1, v1 = dk.clone(), dv.clone()
    q_pos0 = dl.i32(x.q_pos0)
    dl.attend_backward(dl.q, q_pos0, 500, sel, cnt, out, lse, dout, dq, dk, dv)
    torch.cuda.synchronize()
    # equal up to the order of each block's fp32 sum over its queries
    for got, one in ((dk, k1), (dv, v1)):
        err = (got - 2 * one).abs().max().item()
        assert err <= 1e-5 * one.abs().max().item(), err
    assert not dk[0, 500:].any()                      # rows no query attends stay untouched
