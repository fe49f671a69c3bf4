"""GPU parity of the stage-1 indexer distillation (qsa_indexer_distill) and of
the gradient back through the block compression (qsa_index_build_backward)
against the fp64 oracle.

Tolerance (the pages fix none): every element within 1e-3 * max(|ref|, RMS of
the checked tensor) -- the kernels take the same rounded inputs as the oracle
and compute in fp32 (the compression backward in fp64).  A ReLU mask decided by
a dot product within 1e-5 |q| |k| of zero (the fp32 rounding bound of a
128-term dot) can differ between fp32 and fp64: each such (query, block, head)
term widens the bound of the elements it feeds by its own magnitude.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import qsa_oracle as O
from block_sparse_trainable_amd import synth
from block_sparse_trainable_amd.runtime import DeviceLayer
from tests import _compare as C

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-distill] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _close(got, ref, rel, what, extra=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    floor = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    err = np.abs(got - ref)
    bound = rel * np.maximum(np.abs(ref), floor)
    if extra is not None:
        bound = bound + extra
    worst = float((err / np.maximum(bound, 1e-30)).max()) if ref.size else 0.0
    assert (err <= bound).all(), f"{what}: worst error {worst:.3g} x the bound"
    return worst


def _run(x):
    lay = x.layout
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    dl.prefill_chunk()                                  # builds the chunk's blocks
    q_pos0 = dl.i32(x.q_pos0)
    mpe = int((x.q_pos0.astype(np.int64) + x.n_q).max())
    loss = torch.full((x.batch, x.n_q), -1.0, dtype=torch.float32, device=dl.device)
    dq_idx = torch.full((x.batch, x.n_q, lay.idx_heads, lay.idx_dim), 7.0, dtype=torch.float32,
                        device=dl.device)
    dk_cmp = torch.zeros(dl.k_cmp.shape, dtype=torch.float32, device=dl.device)
    dl.distill(q_pos0, mpe, loss, dq_idx, dk_cmp)
    torch.cuda.synchronize()
    return dl, loss.cpu().numpy(), dq_idx.cpu().numpy(), dk_cmp.cpu().numpy()


def _oracle(x, rows_by_seq):
    """Per-row loss and dq_idx for the given rows, dk_cmp summed over every
    row, and the widening of each element's bound by the ambiguous terms."""
    lay = x.layout
    r = lay.block_size
    scale = 1.0 / math.sqrt(lay.head_dim)
    loss, dq, dq_extra = {}, {}, {}
    cap_blocks = x.k.shape[1] // r
    dk = np.zeros((x.batch, cap_blocks, lay.idx_dim))
    dk_extra = np.zeros_like(dk)
    n_amb = 0
    for s in range(x.batch):
        end = int(x.q_pos0[s]) + x.n_q
        kh = C.oracle_khat(x, s, max(end // r, 1))
        q = C.f64(x.q[s], lay.dtype)
        K = C.f64(x.k[s], lay.dtype)
        qi = C.f64(x.q_idx[s], lay.dtype)
        for j in range(x.n_q):
            p = int(x.q_pos0[s]) + j
            c = p // r
            t = O.teacher_block_target(q[j], K, p, r, scale)
            I = O.block_importance(qi[j], kh, c)
            lo, dI = O.distill_row(t, I)
            g_q, g_k = O.distill_grads(qi[j], kh, dI)
            dk[s, :c] += g_k
            ex_q = np.zeros_like(g_q)
            if c:
                dots = kh[:c] @ qi[j].T
                tau = 1e-5 * np.outer(np.linalg.norm(kh[:c], axis=1), np.linalg.norm(qi[j], axis=1))
                near = (np.abs(dots) < tau) * np.abs(dI)[:, None]        # [c, H]
                if near.any():
                    n_amb += int((near > 0).sum())
                    ex_q = near.T @ np.abs(kh[:c])
                    dk_extra[s, :c] += near @ np.abs(qi[j])
            if j in rows_by_seq.get(s, ()):
                loss[(s, j)] = lo
                dq[(s, j)] = g_q
                dq_extra[(s, j)] = ex_q
    return loss, dq, dq_extra, dk, dk_extra, n_amb


def _check(x, res, rows_by_seq, rel=1e-3):
    dl, loss, dq_idx, dk_cmp = res
    ref_loss, ref_dq, ex_dq, ref_dk, ex_dk, n_amb = _oracle(x, rows_by_seq)
    keys = sorted(ref_loss)
    w0 = _close([loss[k] for k in keys], [ref_loss[k] for k in keys], rel, "loss")
    w1 = _close(np.stack([dq_idx[k] for k in keys]), np.stack([ref_dq[k] for k in keys]), rel,
                "dq_idx", np.stack([ex_dq[k] for k in keys]))
    w2 = _close(dk_cmp[:, : ref_dk.shape[1]], ref_dk, rel, "dk_cmp", ex_dk)
    say(f"worst error / bound: loss {w0:.3f}, dq_idx {w1:.3f}, dk_cmp {w2:.3f}; "
        f"{n_amb} (query, block, head) dots within the fp32 bound of zero")
    # rows with no candidate: zero loss and gradient
    for s in range(x.batch):
        for j in range(x.n_q):
            if (int(x.q_pos0[s]) + j) // x.layout.block_size == 0:
                assert loss[s, j] == 0.0 and not dq_idx[s, j].any()


def test_distill_bf16_prefill():
    say("distill bf16 prefill n=700 r=4")
    x = synth.prefill(n=700, layout=synth.Layout(token_budget=512), needle_frac=0.05)
    _check(x, _run(x), {0: set(range(0, 700, 3)) | {699}})


def test_distill_bf16_block_size_16():
    say("distill bf16 prefill n=900 r=16")
    x = synth.prefill(n=900, layout=synth.Layout(block_size=16, token_budget=512),
                      needle_frac=0.05)
    _check(x, _run(x), {0: set(range(0, 900, 4))})


def test_distill_chunk_over_cache():
    say("distill bf16: 160 queries over a 1500-token cache, batch 2")
    lay = synth.Layout(token_budget=256)
    x = synth.chunked(cache=1500, chunk=160, batch=2, window=256, n_far=3, layout=lay)
    _check(x, _run(x), {s: set(range(0, 160, 2)) for s in range(2)})


@pytest.mark.parametrize("kv_heads,head_dim", [(1, 128), (2, 64)])
def test_distill_bf16_other_head_shapes(kv_heads, head_dim):
    """The MFMA teacher's other two shapes (16 query heads over one KV head of
    128 dims, or two of 64), with a query count that is not a multiple of
    the 16 rows a teacher workgroup takes."""
    say(f"distill bf16 kv_heads={kv_heads} head_dim={head_dim}, n=613")
    lay = synth.Layout(token_budget=512, kv_heads=kv_heads, head_dim=head_dim)
    x = synth.prefill(n=613, layout=lay, needle_frac=0.05)
    _check(x, _run(x), {0: set(range(0, 613, 3)) | {612}})


@pytest.mark.parametrize("kv_heads,head_dim", [(1, 128), (2, 64)])
def test_distill_other_head_shapes_chunk_over_cache(kv_heads, head_dim):
    say(f"distill bf16 kv_heads={kv_heads} head_dim={head_dim}: 75 queries over 1300 cached")
    lay = synth.Layout(token_budget=256, kv_heads=kv_heads, head_dim=head_dim)
    x = synth.chunked(cache=1300, chunk=75, batch=2, window=256, n_far=3, layout=lay)
    _check(x, _run(x), {s: set(range(75)) for s in range(2)})


def test_distill_fp32_small_heads():
    say("distill fp32, 4 heads / 1 KV head, d=64, r=8")
    lay = synth.Layout(block_size=8, token_budget=128, dtype="f32", q_heads=4, kv_heads=1,
                       head_dim=64)
    x = synth.prefill(n=500, layout=lay, needle_frac=0.05)
    _check(x, _run(x), {0: set(range(500))})


@pytest.mark.parametrize("r", [4, 16])
def test_index_build_backward(r):
    say(f"index_build_backward r={r}, ragged ranges, added into")
    lay = synth.Layout(block_size=r)
    x = synth.prefill(n=1500, batch=3, layout=lay,
                      gain=np.random.default_rng(8).uniform(0.5, 1.5, 128).astype(np.float32))
    dl = DeviceLayer(x)
    rng = np.random.default_rng(9)
    cap_blocks = dl.k_cmp.shape[1]
    g_np = rng.standard_normal((3, cap_blocks, 128)).astype(np.float32)
    dk_cmp = torch.from_numpy(g_np).to(dl.device)
    base = rng.standard_normal((3,) + tuple(dl.k_idx.shape[1:])).astype(np.float32)
    dk_idx = torch.from_numpy(base).to(dl.device)
    lb = np.array([0, 13, 3 * r + 1], np.int32)
    la = np.array([1499, 13 + 5 * r, 1500], np.int32)
    dl.index_build_backward(dl.i32(lb), dl.i32(la), 1500 // r + 1, dk_cmp, dk_idx)
    torch.cuda.synchronize()
    got = dk_idx.cpu().numpy() - base
    for s in range(3):
        b0, b1 = lb[s] // r, la[s] // r
        k_all = C.f64(x.k_idx[s, : b1 * r], "bf16")
        ref = O.compress_index_backward(k_all, b1, g_np[s, :b1].astype(np.float64), r=r,
                                        gain=x.gain.astype(np.float64), eps=float(np.float32(lay.rms_eps)),
                                        rope_dims=lay.rope_dims, base=lay.rope_base)
        rows = slice(b0 * r, b1 * r)
        np.testing.assert_allclose(got[s, rows], ref[rows], rtol=1e-5,
                                   atol=1e-6 * np.abs(ref).max())
        assert not got[s, : b0 * r].any() and not got[s, b1 * r:].any()
