"""The library never allocates device memory: after one warm-up call of each
entry point (code objects load on first use), 1,000 further calls of every
entry point leave the device's free memory (hipMemGetInfo, through
torch.cuda.mem_get_info) exactly unchanged.  Every tensor and workspace is
allocated before the measured loop."""
import sys

import numpy as np
import pytest
import torch

from block_sparse_trainable_amd import _binding as B
from block_sparse_trainable_amd import synth
from block_sparse_trainable_amd.runtime import DeviceLayer, OffloadedKV

pytestmark = pytest.mark.gpu

CALLS = 1000


def say(msg):
    print(f"[gpu-no-allocation] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def test_entry_points_allocate_nothing():
    x = synth.decode(context=3000, batch=2, steps=4, n_needles=4)
    dl = DeviceLayer(x)
    dl.build_prefix(x.cache_len)
    plan = dl.decode_plan(4)
    q_idx_s, q_s, pos_t, pos1_t, mpe = plan
    outs = dl.alloc_decode_outputs()
    sel, cnt, scs, out, lse = outs
    lay = x.layout
    # prefill-shaped inputs over the same caches: 4 queries per sequence
    nq = 4
    q_idx_p = q_idx_s[:nq].transpose(0, 1).contiguous()
    q_p = q_s[:nq].transpose(0, 1).contiguous()
    pre = dl.alloc_select(dl.batch, nq)
    out_p = torch.empty_like(q_p)
    lse_p = torch.empty((dl.batch, nq, lay.q_heads), dtype=torch.float32, device=dl.device)
    dout = torch.randn(q_p.shape, device=dl.device).to(q_p.dtype)
    dq = torch.empty_like(q_p)
    dk = torch.zeros(dl.k.shape, dtype=torch.float32, device=dl.device)
    dv = torch.zeros_like(dk)
    loss = torch.empty((dl.batch, nq), dtype=torch.float32, device=dl.device)
    dq_idx = torch.empty((dl.batch, nq, lay.idx_heads, lay.idx_dim), dtype=torch.float32,
                         device=dl.device)
    dk_cmp = torch.zeros(dl.k_cmp.shape, dtype=torch.float32, device=dl.device)
    dk_idx = torch.zeros(dl.k_idx.shape, dtype=torch.float32, device=dl.device)
    off = OffloadedKV(dl, 256)
    ws = {op: dl.workspace(op, dl.batch, nq, mpe)
          for op in (B.QSA_OP_SELECT, B.QSA_OP_PREFILL, B.QSA_OP_BACKWARD, B.QSA_OP_DISTILL)}
    ws_dec = dl.workspace(B.QSA_OP_DECODE, dl.batch, 1, mpe)
    ws_step = dl.step_workspace(mpe)
    ws_stage = dl.workspace(B.QSA_OP_DECODE, dl.batch, 1, off.stage_tokens)
    cfg, cap = dl.cfg, dl.cap
    t = 3

    calls = {
        "qsa_index_build": lambda: B.qsa_index_build(
            cfg, dl.batch, dl.k_idx, cap, pos_t[t], pos1_t[t], 1, dl.gain, dl.k_cmp),
        "qsa_select_topk": lambda: B.qsa_select_topk(
            cfg, dl.batch, nq, q_idx_p, pos_t[0], mpe, dl.k_cmp, cap, pre[0], pre[1], pre[2],
            ws[B.QSA_OP_SELECT], ws[B.QSA_OP_SELECT].numel()),
        "qsa_sparse_attn_prefill": lambda: B.qsa_sparse_attn_prefill(
            cfg, dl.batch, nq, q_p, dl.k, dl.v, cap, pos_t[0], mpe, pre[0], pre[1], out_p, lse_p,
            ws[B.QSA_OP_PREFILL], ws[B.QSA_OP_PREFILL].numel()),
        "qsa_sparse_attn_decode": lambda: B.qsa_sparse_attn_decode(
            cfg, dl.batch, q_s[t], dl.k, dl.v, cap, pos_t[t], mpe, sel, cnt, out, lse, ws_dec,
            ws_dec.numel()),
        "qsa_decode_step": lambda: B.qsa_decode_step(
            cfg, dl.batch, q_idx_s[t], q_s[t], dl.k_idx, dl.k_cmp, dl.gain, dl.k, dl.v, cap,
            pos_t[t], mpe, sel[:, 0], cnt[:, 0], scs[:, 0], out, lse, ws_step, ws_step.numel()),
        "qsa_decode_step_noalloc": lambda: B.qsa_decode_step_noalloc(
            cfg, dl.batch, q_idx_s[t], q_s[t], dl.k_idx, dl.k_cmp, dl.gain, dl.k, dl.v, cap,
            pos_t[t], mpe, sel[:, 0], cnt[:, 0], scs[:, 0], out, lse),
        "qsa_sparse_attn_backward": lambda: B.qsa_sparse_attn_backward(
            cfg, dl.batch, nq, q_p, dl.k, dl.v, cap, pos_t[0], mpe, pre[0], pre[1], out_p, lse_p,
            dout, dq, dk, dv, ws[B.QSA_OP_BACKWARD], ws[B.QSA_OP_BACKWARD].numel()),
        "qsa_indexer_distill": lambda: B.qsa_indexer_distill(
            cfg, dl.batch, nq, q_p, dl.k, cap, pos_t[0], mpe, q_idx_p, dl.k_cmp, loss, dq_idx,
            dk_cmp, ws[B.QSA_OP_DISTILL], ws[B.QSA_OP_DISTILL].numel()),
        "qsa_index_build_backward": lambda: B.qsa_index_build_backward(
            cfg, dl.batch, dl.k_idx, cap, pos_t[0], pos1_t[t], 2, dl.gain, dk_cmp, dk_idx),
        "qsa_offload_stage": lambda: B.qsa_offload_stage(
            cfg, dl.batch, pos_t[t], sel[:, 0], cnt[:, 0], off.k_host.data_ptr(),
            off.v_host.data_ptr(), cap, off.hot_k, off.hot_v, off.hot_tag, off.hot_units,
            off.stage_k, off.stage_v, off.stage_tokens, off.stage_sel, off.stage_cnt,
            off.stage_pos, off.stats),
    }
    # every declared compute entry point is exercised
    assert set(calls) | {"qsa_workspace_size", "qsa_status_string", "qsa_last_error",
                         "qsa_abi_version"} == set(B.EXPORTED)
    for name, f in calls.items():
        f()
    torch.cuda.synchronize()
    for name, f in calls.items():
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info()
        for _ in range(CALLS):
            f()
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        say(f"{name}: {CALLS} calls, free device memory {free0} -> {free1}")
        assert free1 == free0, f"{name}: free device memory changed by {free0 - free1} bytes"
    dl.check_step(ws_step)
