"""GPU parity at block sizes other than 4 (r = 8 .. 128) against the fp64 oracle.

The pages fix r = 4 for their configuration and show the selection unit as
a parameter of the method ("Qwen Sparse Attention" gallery page, selection
unit/budget table; "QSA (Qwen Sparse Attention)", Key math (A): blocks of r
tokens, k_B = ceil(K/r)).  The kernels take any power of two from 4 to 128
with k_B * r <= 2048; the oracle is the same code as for r = 4 with r passed
through.  Covered: compression over ragged ranges, bf16 prefill on the MFMA
path (selection + attention), fp32 on the VALU scoring path and the generic
attention, a ragged chunk, the three-call decode (split attention + merge),
and the full budget equal to dense causal attention.
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
    print(f"[gpu-block-sizes] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _host(outs, dtype):
    sel, cnt, scs, out, lse = outs
    return (sel.cpu().numpy(), cnt.cpu().numpy(), scs.cpu().numpy(), to_f32(out),
            lse.cpu().numpy())


def _check_rows(x, outs, rows_by_seq, check_attn=True):
    lay = x.layout
    r = lay.block_size
    sel, cnt, scs, out, lse = _host(outs, lay.dtype)
    kB = lay.k_blocks
    scale = 1.0 / math.sqrt(lay.head_dim)
    n = 0
    for s, rows in rows_by_seq.items():
        nb = max((int(x.q_pos0[s]) + max(rows)) // r, 1)
        kh = C.oracle_khat(x, s, nb)
        q_idx = C.f64(x.q_idx[s], lay.dtype)
        q = C.f64(x.q[s], lay.dtype)
        K = C.f64(x.k[s], lay.dtype)
        V = C.f64(x.v[s], lay.dtype)
        for j in rows:
            p = int(x.q_pos0[s]) + j
            res = O.qsa_row(p, q_idx[j], q[j], kh, K, V, k_B=kB, r=r, attend=False)
            C.check_selection(res, sel[s, j], int(cnt[s, j]), scs[s, j], kB)
            if check_attn:
                count = int(cnt[s, j])
                C.check_attention(p, sel[s, j, :count], q[j], K, V, out[s, j], lse[s, j],
                                  scale, lay.dtype, r)
            n += 1
    return n


@pytest.mark.parametrize("r", [8, 16, 64])
def test_index_build_block_sizes(r):
    say(f"index_build r={r}, ragged ranges")
    lay = synth.Layout(block_size=r)
    x = synth.prefill(n=1500, batch=3, layout=lay,
                      gain=np.random.default_rng(7).uniform(0.5, 1.5, 128).astype(np.float32))
    dl = DeviceLayer(x)
    dl.k_cmp.fill_(-7.0)
    lb = np.array([0, 13, 3 * r + 1], np.int32)        # not multiples of r
    la = np.array([1499, 13 + 2 * r, 1500], np.int32)
    dl.index_build(dl.i32(lb), dl.i32(la), 1500 // r + 1)
    torch.cuda.synchronize()
    got = to_f32(dl.k_cmp)
    for s in range(3):
        nb_all = la[s] // r
        ref = C.oracle_khat(x, s, nb_all)
        b0, b1 = lb[s] // r, la[s] // r
        np.testing.assert_allclose(got[s, b0:b1], ref[b0:b1].astype(np.float32), rtol=2 ** -7,
                                   atol=1e-6)
        assert (got[s, :b0] == -7.0).all() and (got[s, b1:] == -7.0).all()


@pytest.mark.parametrize("r,n,budget,batch", [(8, 2500, 2048, 1), (16, 3000, 2048, 2),
                                              (64, 3000, 2048, 1), (32, 1500, 512, 1),
                                              (128, 4000, 2048, 1)])
def test_prefill_bf16_block_sizes(r, n, budget, batch):
    say(f"prefill bf16 r={r} n={n} K={budget} batch={batch}")
    lay = synth.Layout(block_size=r, token_budget=budget)
    x = synth.prefill(n=n, batch=batch, layout=lay, needle_frac=0.05)
    dl = DeviceLayer(x)
    outs = dl.prefill_chunk()
    torch.cuda.synchronize()
    assert _check_rows(x, outs, {s: list(range(0, n, 7)) + [n - 1] for s in range(batch)}) > 0


@pytest.mark.parametrize("r", [8, 32])
def test_prefill_fp32_block_sizes(r):
    say(f"prefill fp32 r={r} (VALU scoring, generic attention)")
    lay = synth.Layout(block_size=r, token_budget=128, dtype="f32", q_heads=4, kv_heads=1,
                       head_dim=64)
    x = synth.prefill(n=700, layout=lay, needle_frac=0.05)
    dl = DeviceLayer(x)
    outs = dl.prefill_chunk()
    torch.cuda.synchronize()
    _check_rows(x, outs, {0: list(range(700))})


def test_chunked_ragged_block_size():
    say("chunked prefill r=16, ragged cache")
    lay = synth.Layout(block_size=16)
    x = synth.chunked(cache=4101, chunk=777, batch=2, window=512, n_far=4, layout=lay)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    outs = dl.prefill_chunk()
    torch.cuda.synchronize()
    _check_rows(x, outs, {s: list(range(0, 777, 3)) for s in range(2)})


def test_full_budget_equals_dense_causal_block_size():
    say("prefill bf16 r=16 full budget vs dense causal")
    lay = synth.Layout(block_size=16, token_budget=2048)
    x = synth.prefill(n=1900, layout=lay)               # every c <= 118 < k_B = 128
    dl = DeviceLayer(x)
    outs = dl.prefill_chunk()
    torch.cuda.synchronize()
    sel, cnt, _, out, _ = _host(outs, "bf16")
    assert (cnt[0] == np.arange(1900) // 16).all()
    q = C.f64(x.q[0], "bf16")
    K = C.f64(x.k[0, :1900], "bf16")
    V = C.f64(x.v[0, :1900], "bf16")
    qt = torch.tensor(q).permute(1, 0, 2)
    kt = torch.tensor(K).permute(1, 0, 2).repeat_interleave(8, 0)
    vt = torch.tensor(V).permute(1, 0, 2).repeat_interleave(8, 0)
    dense = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    dense = dense.permute(1, 0, 2).numpy()
    assert np.abs(out[0] - dense).max() <= C.ATOL["bf16"]


@pytest.mark.parametrize("r", [16, 128])
def test_decode_three_calls_block_size(r):
    say(f"decode r={r}: 2 seqs x 2r+1 steps through the three calls")
    steps = 2 * r + 1                                   # crosses two block completions
    lay = synth.Layout(block_size=r)
    x = synth.decode(context=40000, batch=2, steps=steps, n_needles=8, layout=lay)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(steps)
    outs = dl.alloc_decode_outputs()
    scale = 1.0 / math.sqrt(lay.head_dim)
    khats = {s: C.oracle_khat(x, s, (int(x.q_pos0[s]) + steps) // r) for s in range(2)}
    checked = (0, r - 1, r, steps - 1)
    for t in range(steps):
        dl.decode_step(plan, t, outs)
        torch.cuda.synchronize()
        if t not in checked:
            continue
        sel, cnt, scs, out, lse = _host(outs, "bf16")
        for s in range(2):
            p = int(x.q_pos0[s]) + t
            q_idx = C.f64(x.q_idx[s, t], "bf16")
            q = C.f64(x.q[s, t], "bf16")
            K = C.f64(x.k[s], "bf16")
            V = C.f64(x.v[s], "bf16")
            res = O.qsa_row(p, q_idx, q, khats[s], K, V, k_B=lay.k_blocks, r=r, attend=False)
            C.check_selection(res, sel[s, 0], int(cnt[s, 0]), scs[s, 0], lay.k_blocks)
            C.check_attention(p, sel[s, 0, :cnt[s, 0]], q, K, V, out[s], lse[s], scale, "bf16", r)
            assert int(x.target_block[s, t]) in set(sel[s, 0, :cnt[s, 0]].tolist())
