"""GPU parity at the token-level end of the block size: r = 1 (single tokens,
k_B = K up to 2048) and r = 2, against the fp64 oracle.

"Qwen Sparse Attention" gallery page, QSA-vs-DSA table: a selection unit of
single token positions with a 2,048-token budget is the DeepSeek-style
extreme of the same design; "QSA (Qwen Sparse Attention)", Definition: the
indexer's cost falls with the compression ratio r, r = 1 meaning no
compression.  The kernels take r = 1 and 2 with k_B * r <= 2048: the
compression pools r rows (the identity at r = 1), the scoring and selection
use c = floor(p/r) candidates, and the attention reads the token set from an
explicit list.  Covered: compression over ragged ranges, bf16 prefill on the
MFMA path with rows longer than the budget (2048 of up to ~60K candidates,
including the long-row pruning selection), fp32 on the VALU path, a ragged
chunk, exact ties, the full budget equal to dense causal attention, and the
three-call decode (split attention + merge).
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
    print(f"[gpu-token-level] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _host(outs):
    sel, cnt, scs, out, lse = outs
    return (sel.cpu().numpy(), cnt.cpu().numpy(), scs.cpu().numpy(), to_f32(out),
            lse.cpu().numpy())


def _check_rows(x, outs, rows_by_seq):
    lay = x.layout
    r = lay.block_size
    sel, cnt, scs, out, lse = _host(outs)
    kB = lay.k_blocks
    scale = 1.0 / math.sqrt(lay.head_dim)
    stats = []
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
            stats.append(C.check_selection(res, sel[s, j], int(cnt[s, j]), scs[s, j], kB))
            count = int(cnt[s, j])
            C.check_attention(p, sel[s, j, :count], q[j], K, V, out[s, j], lse[s, j], scale,
                              lay.dtype, r)
    say(f"{len(stats)} rows: {np.mean([t.exact_eligible for t in stats]):.2f} margin-eligible, "
        f"{np.mean([t.exact for t in stats]):.2f} identical to the oracle")
    return stats


@pytest.mark.parametrize("r", [1, 2])
def test_index_build_token_level(r):
    say(f"index_build r={r}, ragged ranges")
    lay = synth.Layout(block_size=r)
    x = synth.prefill(n=900, batch=3, layout=lay,
                      gain=np.random.default_rng(7).uniform(0.5, 1.5, 128).astype(np.float32))
    dl = DeviceLayer(x)
    dl.k_cmp.fill_(-7.0)
    lb = np.array([0, 13, 3 * r + 1], np.int32)
    la = np.array([899, 13 + 5 * r, 900], np.int32)
    dl.index_build(dl.i32(lb), dl.i32(la), 900 // r + 1)
    torch.cuda.synchronize()
    got = to_f32(dl.k_cmp)
    for s in range(3):
        b0, b1 = lb[s] // r, la[s] // r
        ref = C.oracle_khat(x, s, b1)
        np.testing.assert_allclose(got[s, b0:b1], ref[b0:b1].astype(np.float32), rtol=2 ** -7,
                                   atol=1e-6)
        assert (got[s, :b0] == -7.0).all() and (got[s, b1:] == -7.0).all()


@pytest.mark.parametrize("r,n,budget,batch", [(1, 3000, 2048, 1), (1, 1500, 256, 2),
                                              (2, 2600, 2048, 1)])
def test_prefill_bf16_token_level(r, n, budget, batch):
    say(f"prefill bf16 r={r} n={n} K={budget} batch={batch}")
    lay = synth.Layout(block_size=r, token_budget=budget)
    x = synth.prefill(n=n, batch=batch, layout=lay, needle_frac=0.05)
    dl = DeviceLayer(x)
    outs = dl.prefill_chunk()
    torch.cuda.synchronize()
    rows = list(range(0, n, 9)) + [n - 1]
    stats = _check_rows(x, outs, {s: rows for s in range(batch)})
    assert stats


def test_prefill_fp32_token_level():
    say("prefill fp32 r=1 (VALU scoring, generic attention)")
    lay = synth.Layout(block_size=1, token_budget=128, dtype="f32", q_heads=4, kv_heads=1,
                       head_dim=64)
    x = synth.prefill(n=500, layout=lay, needle_frac=0.05)
    dl = DeviceLayer(x)
    outs = dl.prefill_chunk()
    torch.cuda.synchronize()
    _check_rows(x, outs, {0: list(range(500))})


def test_chunked_ragged_token_level():
    say("chunked prefill r=1, ragged cache, K=2048")
    lay = synth.Layout(block_size=1)
    x = synth.chunked(cache=5001, chunk=300, batch=2, window=512, n_far=4, layout=lay)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    outs = dl.prefill_chunk()
    torch.cuda.synchronize()
    _check_rows(x, outs, {s: list(range(0, 300, 3)) for s in range(2)})


def test_long_rows_token_level():
    say("chunked prefill r=1: 48 queries over a 60K-token cache (long-row selection)")
    lay = synth.Layout(block_size=1)
    x = synth.chunked(cache=60000, chunk=48, batch=1, window=2048, n_far=6, layout=lay)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    outs = dl.prefill_chunk()
    torch.cuda.synchronize()
    _check_rows(x, outs, {0: list(range(48))})


def test_exact_ties_token_level():
    say("prefill r=1: 2500 identical tokens tie at the threshold")
    lay = synth.Layout(block_size=1, token_budget=2048)
    x = synth.prefill(n=3200, layout=lay, needle_frac=0.0)
    kf = synth.bf16_to_f32(x.k_idx)
    kf[:, :, :64] = 0.0                       # rotated half zero: RoPE leaves keys equal
    rep = kf[0, 0].copy()
    kf[0, 0:2500] = rep                       # tokens 0..2499 identical
    x.k_idx[:] = synth.f32_to_bf16(kf)
    qf = synth.bf16_to_f32(x.q_idx)
    qf[0, :, :, 64:] = rep[None, None, 64:]   # every identical token scores far above the rest
    x.q_idx[:] = synth.f32_to_bf16(qf)
    dl = DeviceLayer(x)
    outs = dl.prefill_chunk()
    torch.cuda.synchronize()
    _check_rows(x, outs, {0: [2100, 2500, 2600, 3199]})
    sel = outs[0].cpu().numpy()
    for p in (2100, 2500, 2600, 3199):      # equal scores go to the lower positions
        assert sel[0, p].tolist() == list(range(2048))


def test_full_budget_equals_dense_causal_token_level():
    say("prefill bf16 r=1 full budget vs dense causal")
    lay = synth.Layout(block_size=1, token_budget=2048)
    x = synth.prefill(n=1900, layout=lay)               # every c = p < k_B = 2048
    dl = DeviceLayer(x)
    outs = dl.prefill_chunk()
    torch.cuda.synchronize()
    sel, cnt, _, out, _ = _host(outs)
    assert (cnt[0] == np.arange(1900)).all()
    q = C.f64(x.q[0], "bf16")
    K = C.f64(x.k[0, :1900], "bf16")
    V = C.f64(x.v[0, :1900], "bf16")
    qt = torch.tensor(q).permute(1, 0, 2)
    kt = torch.tensor(K).permute(1, 0, 2).repeat_interleave(8, 0)
    vt = torch.tensor(V).permute(1, 0, 2).repeat_interleave(8, 0)
    dense = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    dense = dense.permute(1, 0, 2).numpy()
    assert np.abs(out[0] - dense).max() <= C.ATOL["bf16"]


@pytest.mark.parametrize("r", [1, 2])
def test_decode_three_calls_token_level(r):
    say(f"decode r={r}: 2 seqs x 5 steps through the three calls")
    steps = 5
    lay = synth.Layout(block_size=r)
    x = synth.decode(context=30000, batch=2, steps=steps, n_needles=8, layout=lay)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(steps)
    outs = dl.alloc_decode_outputs()
    scale = 1.0 / math.sqrt(lay.head_dim)
    khats = {s: C.oracle_khat(x, s, (int(x.q_pos0[s]) + steps) // r) for s in range(2)}
    for t in range(steps):
        dl.decode_step(plan, t, outs)
        torch.cuda.synchronize()
        sel, cnt, scs, out, lse = _host(outs)
        for s in range(2):
            p = int(x.q_pos0[s]) + t
            q_idx = C.f64(x.q_idx[s, t], "bf16")
            q = C.f64(x.q[s, t], "bf16")
            K = C.f64(x.k[s], "bf16")
            V = C.f64(x.v[s], "bf16")
            res = O.qsa_row(p, q_idx, q, khats[s], K, V, k_B=lay.k_blocks, r=r, attend=False)
            C.check_selection(res, sel[s, 0], int(cnt[s, 0]), scs[s, 0], lay.k_blocks)
            C.check_attention(p, sel[s, 0, :cnt[s, 0]], q, K, V, out[s], lse[s], scale, "bf16", r)
