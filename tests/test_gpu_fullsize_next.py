"""GPU parity of the backward, the distillation and the offloaded decode at
the full workload sizes the benchmark times, on sampled rows, plus
properties that hold at any size:
  * every softmax row sums to 1, so sum_j dV_j = sum over the rows of their
    heads' dO (per KV head), and sum_j dS_j = 0, so sum_j dK_j = 0;
  * the offloaded decode equals the resident one up to the attention tolerance.
"""
import math
import sys
import time

import numpy as np
import pytest
import torch

from oracle import qsa_oracle as O
from block_sparse_trainable_amd import synth
from block_sparse_trainable_amd.runtime import DeviceLayer, OffloadedKV, to_f32
from tests import _compare as C

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-fullsize-next] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def _rows(n_q, k, seed):
    rng = np.random.default_rng(seed)
    return sorted({0, 1, n_q - 1} | set(rng.choice(n_q, size=k, replace=False).tolist()))


def test_backward_chunked_128k_sampled():
    x = synth.chunked()
    lay = x.layout
    say("chunked 2 x 8192 over 131072: forward + backward")
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    sel, cnt, scs, out, lse = dl.prefill_chunk()
    g = torch.Generator(device="cuda:0")
    g.manual_seed(5)
    dout = torch.randn(dl.q.shape, generator=g, device="cuda:0").to(dl.q.dtype)
    dq = torch.empty_like(dl.q)
    dk = torch.zeros(dl.k.shape, dtype=torch.float32, device=dl.device)
    dv = torch.zeros_like(dk)
    q_pos0 = dl.i32(x.q_pos0)
    mpe = int((x.q_pos0.astype(np.int64) + x.n_q).max())
    dl.attend_backward(dl.q, q_pos0, mpe, sel, cnt, out, lse, dout, dq, dk, dv)
    torch.cuda.synchronize()
    # the sums over tokens (float64 on the device)
    do64 = dout.double()
    for gk in range(lay.kv_heads):
        hs = slice(gk * lay.q_heads // lay.kv_heads, (gk + 1) * lay.q_heads // lay.kv_heads)
        want = do64[:, :, hs].sum(dim=(0, 1, 2))                     # [d]
        got = dv[:, :, gk].double().sum(dim=(0, 1))
        assert (got - want).abs().max().item() <= 1e-3 * want.abs().max().item() + 1e-2
        sk = dk[:, :, gk].double().sum(dim=(0, 1))
        assert sk.abs().max().item() <= 1e-4 * dk[:, :, gk].double().abs().sum().item() / 128
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    dq_h, do_h = to_f32(dq), to_f32(dout)
    scale = 1.0 / math.sqrt(lay.head_dim)
    got, ref = [], []
    for s in range(x.batch):
        K, V, q = C.f64(x.k[s], "bf16"), C.f64(x.v[s], "bf16"), C.f64(x.q[s], "bf16")
        sK, sV = np.zeros_like(K), np.zeros_like(V)
        t0 = time.time()
        for j in _rows(x.n_q, 6, 20 + s):
            p = int(x.q_pos0[s]) + j
            S = O.expand_with_tail(np.sort(sel_h[s, j, :int(cnt_h[s, j])]), p, lay.block_size)
            ref.append(O.sparse_attention_backward(q[j], K, V, S, do_h[s, j].astype(np.float64),
                                                   scale, sK, sV))
            got.append(dq_h[s, j])
        say(f"seq {s}: sampled rows checked in {time.time() - t0:.1f}s")
    got, ref = np.stack(got).astype(np.float64), np.stack(ref)
    floor = np.sqrt(np.mean(ref ** 2))
    assert (np.abs(got - ref) <= 1e-2 * np.maximum(np.abs(ref), floor)).all()


def test_distill_chunked_128k_sampled():
    x = synth.chunked()
    lay = x.layout
    r = lay.block_size
    say("chunked 2 x 8192 over 131072: distillation")
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    dl.prefill_chunk()
    q_pos0 = dl.i32(x.q_pos0)
    mpe = int((x.q_pos0.astype(np.int64) + x.n_q).max())
    loss = torch.empty((x.batch, x.n_q), dtype=torch.float32, device=dl.device)
    dq = torch.empty((x.batch, x.n_q, 4, 128), dtype=torch.float32, device=dl.device)
    dkc = torch.zeros(dl.k_cmp.shape, dtype=torch.float32, device=dl.device)
    dl.distill(q_pos0, mpe, loss, dq, dkc)
    torch.cuda.synchronize()
    loss_h, dq_h = loss.cpu().numpy(), dq.cpu().numpy()
    scale = 1.0 / math.sqrt(lay.head_dim)
    for s in range(x.batch):
        end = int(x.q_pos0[s]) + x.n_q
        kh = C.oracle_khat(x, s, end // r)
        K, q, qi = C.f64(x.k[s], "bf16"), C.f64(x.q[s], "bf16"), C.f64(x.q_idx[s], "bf16")
        t0 = time.time()
        for j in _rows(x.n_q, 3, 30 + s):
            p = int(x.q_pos0[s]) + j
            t = O.teacher_block_target(q[j], K, p, r, scale)
            I = O.block_importance(qi[j], kh, p // r)
            lo, dI = O.distill_row(t, I)
            g_q, _ = O.distill_grads(qi[j], kh, dI)
            assert abs(loss_h[s, j] - lo) <= 1e-3 * max(abs(lo), 1e-2)
            dots = kh[: p // r] @ qi[j].T
            tau = 1e-5 * np.outer(np.linalg.norm(kh[: p // r], axis=1), np.linalg.norm(qi[j], axis=1))
            extra = ((np.abs(dots) < tau) * np.abs(dI)[:, None]).T @ np.abs(kh[: p // r])
            floor = np.sqrt(np.mean(g_q ** 2))
            assert (np.abs(dq_h[s, j] - g_q) <= 1e-3 * np.maximum(np.abs(g_q), floor) + extra).all()
        say(f"seq {s}: sampled rows checked in {time.time() - t0:.1f}s")


def test_offload_decode_256k():
    x = synth.decode()
    say("decode 8 x 256K: resident vs offloaded, 3 steps")
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(3)
    off = OffloadedKV(dl, 65536)
    res, ofs = dl.alloc_decode_outputs(), dl.alloc_decode_outputs()
    for t in range(3):
        dl.decode_step(plan, t, res)
        off.decode_step(plan, t, ofs)
        torch.cuda.synchronize()
        assert torch.equal(res[0], ofs[0]) and torch.equal(res[1], ofs[1])
        assert np.abs(to_f32(res[3]) - to_f32(ofs[3])).max() <= C.ATOL["bf16"]
        st = off.stats.cpu().numpy()
        units = ofs[1][:, 0].cpu().numpy().astype(np.int64) + 1   # r = 4: a unit per block + the tail
        assert (st.sum(1) == units).all()
        say(f"step {t}: hits {st[:, 0].sum()} of {st.sum()}")
