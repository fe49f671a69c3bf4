"""Device buffers of one QSA layer and the call sequences that drive it.

Marshalling only: tensors are uploaded once, outputs and workspaces are
allocated once, and each method enqueues the C-ABI entry points on the
current stream.  A prefill chunk is index_build (blocks completed by the
chunk) -> select_topk -> sparse_attn_prefill; a decode step is
index_build (the block the new token may complete) -> select_topk (one
query per sequence) -> sparse_attn_decode.
"""
from __future__ import annotations

import copy
import numpy as np
import torch

from . import _binding as B
from .synth import LayerInputs


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """numpy storage tensor (uint16 bf16 bits or fp32) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 numpy bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


class DeviceLayer:
    """One layer's caches and query tensors on the GPU."""

    def __init__(self, x: LayerInputs, device="cuda:0"):
        self.x = x
        self.layout = x.layout
        self.cfg = B.QsaConfig.from_layout(x.layout)
        self.device = torch.device(device)
        dt = x.layout.dtype
        self.tdtype = torch.bfloat16 if dt == "bf16" else torch.float32
        self.batch = x.batch
        self.cap = x.cap_tokens
        self.n_q = x.n_q
        self.k_idx = to_device(x.k_idx, dt, self.device)
        self.k = to_device(x.k, dt, self.device)
        self.v = to_device(x.v, dt, self.device)
        self.q_idx = to_device(x.q_idx, dt, self.device)
        self.q = to_device(x.q, dt, self.device)
        self.gain = torch.from_numpy(np.ascontiguousarray(x.gain, np.float32)).to(self.device)
        self.k_cmp = torch.zeros((self.batch, self.cap // self.layout.block_size,
                                  self.layout.idx_dim), dtype=self.tdtype, device=self.device)
        self.kB = self.cfg.k_blocks
        self._ws = {}

    def replica(self) -> "DeviceLayer":
        """The same layer with its caches (raw and compressed index, K, V)
        copied to new device memory: equal values at other addresses, for
        runs whose working set must not stay in the on-chip caches.  Queries
        and workspaces are shared."""
        r = copy.copy(self)
        r.k_idx, r.k, r.v = self.k_idx.clone(), self.k.clone(), self.v.clone()
        r.k_cmp = self.k_cmp.clone()
        return r

    # ------------------------------------------------------------ helpers --
    def i32(self, values) -> torch.Tensor:
        return torch.tensor(np.asarray(values, dtype=np.int32), device=self.device)

    def workspace(self, op: int, batch: int, n_q: int, max_pos_end: int) -> torch.Tensor:
        """One workspace per op, grown on demand (no state is kept in it
        between calls)."""
        n = B.qsa_workspace_size(self.cfg, op, batch, n_q, max_pos_end)
        key = (op,)
        ws = self._ws.get(key)
        if ws is None or ws.numel() < max(n, 16):
            ws = torch.zeros(max(n, 16), dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws

    # -------------------------------------------------------- entry points --
    def index_build(self, len_before, len_after, max_new_blocks: int) -> None:
        B.qsa_index_build(self.cfg, self.batch, self.k_idx, self.cap, len_before, len_after,
                          int(max_new_blocks), self.gain, self.k_cmp)

    def build_prefix(self, lengths) -> None:
        """Build every complete block of the first lengths[s] tokens (setup)."""
        lengths = np.asarray(lengths, np.int64)
        self.index_build(self.i32(np.zeros(self.batch)), self.i32(lengths),
                         int(lengths.max()) // self.layout.block_size + 1)

    def alloc_select(self, batch: int, n_q: int):
        sel = torch.empty((batch, n_q, self.kB), dtype=torch.int32, device=self.device)
        cnt = torch.empty((batch, n_q), dtype=torch.int32, device=self.device)
        scs = torch.empty((batch, n_q, self.kB), dtype=torch.float32, device=self.device)
        return sel, cnt, scs

    def select(self, q_idx, q_pos0, max_pos_end: int, sel, cnt, scs, batch=None, n_q=None):
        batch = self.batch if batch is None else batch
        n_q = q_idx.shape[1] if n_q is None else n_q
        ws = self.workspace(B.QSA_OP_SELECT, batch, n_q, max_pos_end)
        B.qsa_select_topk(self.cfg, batch, n_q, q_idx, q_pos0, int(max_pos_end), self.k_cmp,
                          self.cap, sel, cnt, scs, ws, ws.numel())

    def attend_prefill(self, q, q_pos0, max_pos_end: int, sel, cnt, out, lse):
        n_q = q.shape[1]
        ws = self.workspace(B.QSA_OP_PREFILL, self.batch, n_q, max_pos_end)
        B.qsa_sparse_attn_prefill(self.cfg, self.batch, n_q, q, self.k, self.v, self.cap, q_pos0,
                                  int(max_pos_end), sel, cnt, out, lse, ws, ws.numel())

    def attend_backward(self, q, q_pos0, max_pos_end: int, sel, cnt, out, lse, dout, dq, dk,
                        dv):
        """Gradients of attend_prefill: dq written, dk/dv (fp32, [B][cap][Hkv][d]) added."""
        n_q = q.shape[1]
        ws = self.workspace(B.QSA_OP_BACKWARD, self.batch, n_q, max_pos_end)
        B.qsa_sparse_attn_backward(self.cfg, self.batch, n_q, q, self.k, self.v, self.cap, q_pos0,
                                   int(max_pos_end), sel, cnt, out, lse, dout, dq, dk, dv, ws,
                                   ws.numel())

    def distill(self, q_pos0, max_pos_end: int, loss, dq_idx, dk_cmp):
        """Stage-1 distillation loss of the chunk's queries (per row) with
        dq_idx written and dk_cmp (fp32, [B][cap/r][128]) added."""
        n_q = self.q.shape[1]
        ws = self.workspace(B.QSA_OP_DISTILL, self.batch, n_q, max_pos_end)
        B.qsa_indexer_distill(self.cfg, self.batch, n_q, self.q, self.k, self.cap, q_pos0,
                              int(max_pos_end), self.q_idx, self.k_cmp, loss, dq_idx, dk_cmp,
                              ws, ws.numel())

    def index_build_backward(self, len_before, len_after, max_new_blocks: int, dk_cmp,
                             dk_idx) -> None:
        B.qsa_index_build_backward(self.cfg, self.batch, self.k_idx, self.cap, len_before,
                                   len_after, int(max_new_blocks), self.gain, dk_cmp, dk_idx)

    def attend_decode(self, q, q_pos, max_pos_end: int, sel, cnt, out, lse):
        ws = self.workspace(B.QSA_OP_DECODE, self.batch, 1, max_pos_end)
        B.qsa_sparse_attn_decode(self.cfg, self.batch, q, self.k, self.v, self.cap, q_pos,
                                 int(max_pos_end), sel, cnt, out, lse, ws, ws.numel())

    # -------------------------------------------------------- call chains --
    def prefill_chunk(self, outputs=None):
        """index_build + select_topk + sparse_attn_prefill for the chunk of
        n_q queries at q_pos0 (blocks before cache_len already built)."""
        x = self.x
        r = self.layout.block_size
        q_pos0 = self.i32(x.q_pos0)
        end = x.q_pos0.astype(np.int64) + self.n_q
        max_pos_end = int(end.max())
        new_blocks = int((end // r - x.cache_len // r).max())
        if outputs is None:
            outputs = self.alloc_prefill_outputs()
        sel, cnt, scs, out, lse = outputs
        self.index_build(self.i32(x.cache_len), self.i32(end), new_blocks)
        self.select(self.q_idx, q_pos0, max_pos_end, sel, cnt, scs)
        self.attend_prefill(self.q, q_pos0, max_pos_end, sel, cnt, out, lse)
        return outputs

    def alloc_prefill_outputs(self):
        sel, cnt, scs = self.alloc_select(self.batch, self.n_q)
        out = torch.empty_like(self.q)
        lse = torch.empty((self.batch, self.n_q, self.layout.q_heads), dtype=torch.float32,
                          device=self.device)
        return sel, cnt, scs, out, lse

    def decode_plan(self, steps: int):
        """Per-step device inputs of a decode run: step-major copies of the
        indexer/main queries and the position arrays."""
        x = self.x
        q_idx_s = self.q_idx.transpose(0, 1).contiguous()    # [steps][B][H][d]
        q_s = self.q.transpose(0, 1).contiguous()
        pos = np.stack([x.q_pos0 + t for t in range(steps)]).astype(np.int32)
        pos_t = torch.tensor(pos, device=self.device)          # [steps][B]
        pos1_t = torch.tensor(pos + 1, device=self.device)
        max_pos_end = int(pos.max()) + 1
        return q_idx_s, q_s, pos_t, pos1_t, max_pos_end

    def alloc_decode_outputs(self):
        sel, cnt, scs = self.alloc_select(self.batch, 1)
        out = torch.empty((self.batch, self.layout.q_heads, self.layout.head_dim),
                          dtype=self.tdtype, device=self.device)
        lse = torch.empty((self.batch, self.layout.q_heads), dtype=torch.float32,
                          device=self.device)
        return sel, cnt, scs, out, lse

    def decode_step(self, plan, t: int, outputs):
        q_idx_s, q_s, pos_t, pos1_t, max_pos_end = plan
        sel, cnt, scs, out, lse = outputs
        self.index_build(pos_t[t], pos1_t[t], 1)
        self.select(q_idx_s[t].unsqueeze(1), pos_t[t], max_pos_end, sel, cnt, scs, n_q=1)
        self.attend_decode(q_s[t], pos_t[t], max_pos_end, sel, cnt, out, lse)
        return outputs

    def step_workspace(self, max_pos_end: int) -> torch.Tensor:
        """Zero-filled workspace of the fused decode step (its control area
        must be zero before the first call; the calls keep their state there)."""
        n = B.qsa_workspace_size(self.cfg, B.QSA_OP_DECODE_STEP, self.batch, 1, max_pos_end)
        ws = self._ws.get("step")
        if ws is None or ws.numel() < n:
            ws = torch.zeros(n, dtype=torch.uint8, device=self.device)
            self._ws["step"] = ws
        return ws

    def step_error_word(self, ws=None) -> int:
        """The fused step's error word (reads device memory: synchronises).
        Non-zero means a wait gave up in some call since the control area was
        last cleared, and those calls' outputs are invalid."""
        ws = self._ws.get("step") if ws is None else ws
        if ws is None:
            return 0
        e = B.QSA_STEP_ERROR_BYTE
        return int(ws[e:e + 4].view(torch.int32).item())

    def check_step(self, ws=None) -> None:
        """Raises if the fused step's error word is set, after zero-filling
        the control area again (a call that gave up can leave flags and
        counts behind that the next call would misread)."""
        ws = self._ws.get("step") if ws is None else ws
        err = self.step_error_word(ws)
        if err:
            ws[:B.QSA_STEP_CONTROL_BYTES].zero_()
            torch.cuda.synchronize(self.device)
            raise B.QsaError(B.QSA_ERR_DEVICE,
                             f"qsa_decode_step: a wait gave up (error word {err})")

    def decode_step_fused(self, plan, t: int, outputs, ws=None):
        """The same decode step as decode_step, in one launch (qsa_decode_step)."""
        q_idx_s, q_s, pos_t, pos1_t, max_pos_end = plan
        sel, cnt, scs, out, lse = outputs
        ws = self.step_workspace(max_pos_end) if ws is None else ws
        B.qsa_decode_step(self.cfg, self.batch, q_idx_s[t], q_s[t], self.k_idx, self.k_cmp,
                          self.gain, self.k, self.v, self.cap, pos_t[t], int(max_pos_end),
                          sel[:, 0], cnt[:, 0], scs[:, 0], out, lse, ws, ws.numel())
        return outputs

    def decode_step_noalloc(self, plan, t: int, outputs):
        """decode_step_fused through qsa_decode_step_noalloc (the library's
        own per-device step workspace: nothing is allocated)."""
        q_idx_s, q_s, pos_t, pos1_t, max_pos_end = plan
        sel, cnt, scs, out, lse = outputs
        B.qsa_decode_step_noalloc(self.cfg, self.batch, q_idx_s[t], q_s[t], self.k_idx,
                                  self.k_cmp, self.gain, self.k, self.v, self.cap, pos_t[t],
                                  int(max_pos_end), sel[:, 0], cnt[:, 0], scs[:, 0], out, lse)
        return outputs

    def capture_decode_fused(self, plan, steps: int, outputs):
        """Capture `steps` fused decode steps into one HIP graph."""
        ws = self.step_workspace(plan[4])
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize(self.device)
        with torch.cuda.graph(g):
            for t in range(steps):
                self.decode_step_fused(plan, t, outputs, ws)
        return g

    def capture_decode(self, plan, steps: int, outputs, overlap_build: bool = False,
                       branches: int = 1):
        """Capture `steps` decode steps into one HIP graph (torch.cuda.CUDAGraph).

        overlap_build: step t's index_build runs on a side stream (the block it
        may complete is first a candidate at step t+1), joined before step
        t+1's selection.
        branches: the batch is split into this many contiguous sequence groups,
        each driven on its own stream (its own workspaces), so one group's
        latency-bound selection/attention overlaps another's HBM-bound scan.
        """
        q_idx_s, q_s, pos_t, pos1_t, max_pos_end = plan
        sel, cnt, scs, out, lse = outputs
        B_ = self.batch
        bounds = [round(i * B_ / branches) for i in range(branches + 1)]
        groups = [(a, b) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
        # per-group workspaces allocated outside the capture
        ws = []
        for a, b in groups:
            nsel = B.qsa_workspace_size(self.cfg, B.QSA_OP_SELECT, b - a, 1, max_pos_end)
            ndec = B.qsa_workspace_size(self.cfg, B.QSA_OP_DECODE, b - a, 1, max_pos_end)
            ws.append((torch.zeros(max(nsel, 16), dtype=torch.uint8, device=self.device),
                       torch.zeros(max(ndec, 16), dtype=torch.uint8, device=self.device)))
        g = torch.cuda.CUDAGraph()
        streams = [torch.cuda.Stream(device=self.device) for _ in range(len(groups) + 1)]
        torch.cuda.synchronize(self.device)
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream(self.device)
            for t in range(steps):
                if overlap_build and t > 0:
                    cap.wait_event(built)
                if overlap_build:
                    streams[-1].wait_stream(cap)
                    with torch.cuda.stream(streams[-1]):
                        self.index_build(pos_t[t], pos1_t[t], 1)
                    built = torch.cuda.Event()
                    built.record(streams[-1])
                else:
                    self.index_build(pos_t[t], pos1_t[t], 1)
                for gi, (a, b) in enumerate(groups):
                    st = streams[gi] if len(groups) > 1 else cap
                    if st is not cap:
                        st.wait_stream(cap)
                    with torch.cuda.stream(st):
                        self._decode_group(plan, t, outputs, a, b, ws[gi])
                for gi in range(len(groups)):
                    if len(groups) > 1:
                        cap.wait_stream(streams[gi])
            if overlap_build:
                cap.wait_event(built)
        return g

    def _decode_group(self, plan, t, outputs, a, b, ws):
        """select_topk + sparse_attn_decode for sequences [a, b) of step t."""
        q_idx_s, q_s, pos_t, pos1_t, max_pos_end = plan
        sel, cnt, scs, out, lse = outputs
        nb = b - a
        wsel, wdec = ws
        k_cmp = self.k_cmp[a:b]
        B.qsa_select_topk(self.cfg, nb, 1, q_idx_s[t, a:b].unsqueeze(1), pos_t[t, a:b],
                          int(max_pos_end), k_cmp, self.cap, sel[a:b], cnt[a:b], scs[a:b],
                          wsel, wsel.numel())
        B.qsa_sparse_attn_decode(self.cfg, nb, q_s[t, a:b], self.k[a:b], self.v[a:b], self.cap,
                                 pos_t[t, a:b], int(max_pos_end), sel[a:b], cnt[a:b], out[a:b],
                                 lse[a:b], wdec, wdec.numel())


class OffloadedKV:
    """Decode with a layer's KV history in pinned host memory: a hot cache of
    `hot_units` 4-token units per sequence and a staging buffer in GPU
    memory, filled per step by qsa_offload_stage (plumbing only)."""

    def __init__(self, dl: "DeviceLayer", hot_units: int):
        lay = dl.layout
        self.dl = dl
        self.hot_units = int(hot_units)
        # pinned host copies of the caches (the history the GPU no longer holds)
        self.k_host = torch.empty(dl.k.shape, dtype=dl.k.dtype, pin_memory=True)
        self.v_host = torch.empty(dl.v.shape, dtype=dl.v.dtype, pin_memory=True)
        self.k_host.copy_(dl.k.cpu())
        self.v_host.copy_(dl.v.cpu())
        kd = (lay.kv_heads, lay.head_dim)
        self.hot_k = torch.zeros((dl.batch, self.hot_units, 4) + kd, dtype=dl.k.dtype,
                                 device=dl.device)
        self.hot_v = torch.zeros_like(self.hot_k)
        self.hot_tag = torch.full((dl.batch, self.hot_units), -1, dtype=torch.int32,
                                  device=dl.device)
        self.stage_tokens = (dl.kB + 1) * lay.block_size
        self.stage_k = torch.zeros((dl.batch, self.stage_tokens) + kd, dtype=dl.k.dtype,
                                   device=dl.device)
        self.stage_v = torch.zeros_like(self.stage_k)
        self.stage_sel = torch.empty((dl.batch, dl.kB), dtype=torch.int32, device=dl.device)
        self.stage_cnt = torch.empty((dl.batch,), dtype=torch.int32, device=dl.device)
        self.stage_pos = torch.empty((dl.batch,), dtype=torch.int32, device=dl.device)
        self.stats = torch.zeros((dl.batch, 2), dtype=torch.int32, device=dl.device)

    def stage(self, q_pos, sel, cnt) -> None:
        dl = self.dl
        B.qsa_offload_stage(dl.cfg, dl.batch, q_pos, sel, cnt, self.k_host.data_ptr(),
                            self.v_host.data_ptr(), dl.cap, self.hot_k, self.hot_v, self.hot_tag,
                            self.hot_units, self.stage_k, self.stage_v, self.stage_tokens,
                            self.stage_sel, self.stage_cnt, self.stage_pos, self.stats)

    def decode_step(self, plan, t: int, outputs):
        """index build + select on the GPU-resident index, staging, attention
        over the staging buffer."""
        dl = self.dl
        q_idx_s, q_s, pos_t, pos1_t, max_pos_end = plan
        sel, cnt, scs, out, lse = outputs
        dl.index_build(pos_t[t], pos1_t[t], 1)
        dl.select(q_idx_s[t].unsqueeze(1), pos_t[t], max_pos_end, sel, cnt, scs, n_q=1)
        self.stage(pos_t[t], sel[:, 0], cnt[:, 0])
        ws = dl.workspace(B.QSA_OP_DECODE, dl.batch, 1, self.stage_tokens)
        B.qsa_sparse_attn_decode(dl.cfg, dl.batch, q_s[t], self.stage_k, self.stage_v,
                                 self.stage_tokens, self.stage_pos, self.stage_tokens,
                                 self.stage_sel, self.stage_cnt, out, lse, ws, ws.numel())
        return outputs
