"""ctypes binding of libqsa (include/qsa.h).

Argument marshalling only: every function takes device tensors (torch) or
raw device pointers (int), passes their addresses and the stream to the C
ABI, and raises :class:`QsaError` on a non-OK status.  Nothing here computes
any part of the method; there is no fallback when the library is missing.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

# QSA_LIBRARY names another build of the same library (the host-sanitized
# one the sanitizer test loads); by default the in-tree libqsa.so.
_LIB_PATH = os.environ.get("QSA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libqsa.so")
_lib = None

QSA_OK, QSA_ERR_INVALID_ARGUMENT, QSA_ERR_UNSUPPORTED, QSA_ERR_WORKSPACE, QSA_ERR_DEVICE = range(5)
QSA_F32, QSA_BF16 = 0, 1
(QSA_OP_INDEX_BUILD, QSA_OP_SELECT, QSA_OP_PREFILL, QSA_OP_DECODE, QSA_OP_DECODE_STEP,
 QSA_OP_BACKWARD, QSA_OP_DISTILL) = range(7)
# qsa_decode_step's workspace (qsa.h): a control area of this many bytes at
# its start (zero-filled before the first call, the calls' state after),
# whose int32 at this byte offset is the error word (non-zero once a wait
# gave up).
QSA_STEP_CONTROL_BYTES = 3325952
QSA_STEP_ERROR_BYTE = 8192

EXPORTED = (
    "qsa_index_build", "qsa_select_topk", "qsa_sparse_attn_prefill", "qsa_sparse_attn_decode",
    "qsa_decode_step", "qsa_sparse_attn_backward", "qsa_index_build_backward",
    "qsa_indexer_distill", "qsa_offload_stage", "qsa_workspace_size", "qsa_status_string",
    "qsa_last_error", "qsa_abi_version", "qsa_decode_step_noalloc",
)


class QsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class QsaConfig(ctypes.Structure):
    """Mirror of qsa_config (field order and types must match qsa.h)."""

    _fields_ = [
        ("block_size", ctypes.c_int32),
        ("token_budget", ctypes.c_int32),
        ("idx_heads", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("rope_dims", ctypes.c_int32),
        ("q_heads", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("rope_base", ctypes.c_double),
    ]

    @classmethod
    def from_layout(cls, layout) -> "QsaConfig":
        """Build from any object with the attributes of synth.Layout."""
        return cls(block_size=layout.block_size, token_budget=layout.token_budget,
                   idx_heads=layout.idx_heads, idx_dim=layout.idx_dim,
                   rope_dims=layout.rope_dims, q_heads=layout.q_heads,
                   kv_heads=layout.kv_heads, head_dim=layout.head_dim,
                   dtype=QSA_BF16 if layout.dtype == "bf16" else QSA_F32,
                   rms_eps=layout.rms_eps, softmax_scale=0.0, rope_base=layout.rope_base)

    @property
    def k_blocks(self) -> int:
        return -(-self.token_budget // self.block_size)


def library_path() -> str:
    return _LIB_PATH


def load(path: str | None = None):
    """Load libqsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libqsa.so not found at {p}; build it with "
                           "`python -m block_sparse_trainable_amd.build`")
    lib = ctypes.CDLL(p)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    CFG = ctypes.POINTER(QsaConfig)
    sig = {
        "qsa_index_build": [CFG, I32, P, I64, P, P, I32, P, P, P],
        "qsa_select_topk": [CFG, I32, I32, P, P, I32, P, I64, P, P, P, P, SZ, P],
        "qsa_sparse_attn_prefill": [CFG, I32, I32, P, P, P, I64, P, I32, P, P, P, P, P, SZ, P],
        "qsa_sparse_attn_decode": [CFG, I32, P, P, P, I64, P, I32, P, P, P, P, P, SZ, P],
        "qsa_decode_step": [CFG, I32, P, P, P, P, P, P, P, I64, P, I32, P, P, P, P, P, P, SZ, P],
        "qsa_decode_step_noalloc": [CFG, I32, P, P, P, P, P, P, P, I64, P, I32, P, P, P, P, P, P],
        "qsa_sparse_attn_backward": [CFG, I32, I32, P, P, P, I64, P, I32, P, P, P, P, P, P, P,
                                     P, P, SZ, P],
        "qsa_index_build_backward": [CFG, I32, P, I64, P, P, I32, P, P, P, P],
        "qsa_indexer_distill": [CFG, I32, I32, P, P, I64, P, I32, P, P, P, P, P, P, SZ, P],
        "qsa_offload_stage": [CFG, I32, P, P, P, P, P, I64, P, P, P, I32, P, P, I64, P, P, P, P,
                              P],
        "qsa_workspace_size": [CFG, I32, I32, I32, I32, ctypes.POINTER(SZ)],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.qsa_status_string.argtypes = [ctypes.c_int]
    lib.qsa_status_string.restype = ctypes.c_char_p
    lib.qsa_last_error.argtypes = []
    lib.qsa_last_error.restype = ctypes.c_char_p
    lib.qsa_abi_version.argtypes = []
    lib.qsa_abi_version.restype = ctypes.c_int32
    if path is None:
        _lib = lib
    return lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(lib, st: int) -> None:
    if st != QSA_OK:
        raise QsaError(st, lib.qsa_last_error().decode())


def qsa_workspace_size(cfg: QsaConfig, op: int, batch: int, n_q: int, max_pos_end: int) -> int:
    lib = load()
    out = ctypes.c_size_t(0)
    _check(lib, lib.qsa_workspace_size(ctypes.byref(cfg), op, batch, n_q, max_pos_end,
                                       ctypes.byref(out)))
    return out.value


def qsa_index_build(cfg, batch, k_idx, cap_tokens, len_before, len_after, max_new_blocks,
                    rms_gain, k_cmp, stream=None) -> None:
    lib = load()
    _check(lib, lib.qsa_index_build(ctypes.byref(cfg), batch, _ptr(k_idx), cap_tokens,
                                    _ptr(len_before), _ptr(len_after), max_new_blocks,
                                    _ptr(rms_gain), _ptr(k_cmp), _stream(stream)))


def qsa_select_topk(cfg, batch, n_q, q_idx, q_pos0, max_pos_end, k_cmp, cap_tokens,
                    sel_blocks, sel_count, sel_scores, workspace, workspace_bytes,
                    stream=None) -> None:
    lib = load()
    _check(lib, lib.qsa_select_topk(ctypes.byref(cfg), batch, n_q, _ptr(q_idx), _ptr(q_pos0),
                                    max_pos_end, _ptr(k_cmp), cap_tokens, _ptr(sel_blocks),
                                    _ptr(sel_count), _ptr(sel_scores), _ptr(workspace),
                                    workspace_bytes, _stream(stream)))


def qsa_sparse_attn_prefill(cfg, batch, n_q, q, k_cache, v_cache, cap_tokens, q_pos0,
                            max_pos_end, sel_blocks, sel_count, out, lse, workspace,
                            workspace_bytes, stream=None) -> None:
    lib = load()
    _check(lib, lib.qsa_sparse_attn_prefill(ctypes.byref(cfg), batch, n_q, _ptr(q),
                                            _ptr(k_cache), _ptr(v_cache), cap_tokens,
                                            _ptr(q_pos0), max_pos_end, _ptr(sel_blocks),
                                            _ptr(sel_count), _ptr(out), _ptr(lse),
                                            _ptr(workspace), workspace_bytes, _stream(stream)))


def qsa_sparse_attn_decode(cfg, batch, q, k_cache, v_cache, cap_tokens, q_pos, max_pos_end,
                           sel_blocks, sel_count, out, lse, workspace, workspace_bytes,
                           stream=None) -> None:
    lib = load()
    _check(lib, lib.qsa_sparse_attn_decode(ctypes.byref(cfg), batch, _ptr(q), _ptr(k_cache),
                                           _ptr(v_cache), cap_tokens, _ptr(q_pos), max_pos_end,
                                           _ptr(sel_blocks), _ptr(sel_count), _ptr(out),
                                           _ptr(lse), _ptr(workspace), workspace_bytes,
                                           _stream(stream)))


def qsa_decode_step(cfg, batch, q_idx, q, k_idx, k_cmp, rms_gain, k_cache, v_cache, cap_tokens,
                    q_pos, max_pos_end, sel_blocks, sel_count, sel_scores, out, lse, workspace,
                    workspace_bytes, stream=None) -> None:
    lib = load()
    _check(lib, lib.qsa_decode_step(ctypes.byref(cfg), batch, _ptr(q_idx), _ptr(q), _ptr(k_idx),
                                    _ptr(k_cmp), _ptr(rms_gain), _ptr(k_cache), _ptr(v_cache),
                                    cap_tokens, _ptr(q_pos), max_pos_end, _ptr(sel_blocks),
                                    _ptr(sel_count), _ptr(sel_scores), _ptr(out), _ptr(lse),
                                    _ptr(workspace), workspace_bytes, _stream(stream)))


def qsa_decode_step_noalloc(cfg, batch, q_idx, q, k_idx, k_cmp, rms_gain, k_cache, v_cache,
                            cap_tokens, q_pos, max_pos_end, sel_blocks, sel_count, sel_scores,
                            out, lse, stream=None) -> None:
    lib = load()
    _check(lib, lib.qsa_decode_step_noalloc(ctypes.byref(cfg), batch, _ptr(q_idx), _ptr(q),
                                            _ptr(k_idx), _ptr(k_cmp), _ptr(rms_gain),
                                            _ptr(k_cache), _ptr(v_cache), cap_tokens, _ptr(q_pos),
                                            max_pos_end, _ptr(sel_blocks), _ptr(sel_count),
                                            _ptr(sel_scores), _ptr(out), _ptr(lse),
                                            _stream(stream)))


def qsa_sparse_attn_backward(cfg, batch, n_q, q, k_cache, v_cache, cap_tokens, q_pos0,
                             max_pos_end, sel_blocks, sel_count, out, lse, dout, dq, dk, dv,
                             workspace, workspace_bytes, stream=None) -> None:
    lib = load()
    _check(lib, lib.qsa_sparse_attn_backward(ctypes.byref(cfg), batch, n_q, _ptr(q),
                                             _ptr(k_cache), _ptr(v_cache), cap_tokens,
                                             _ptr(q_pos0), max_pos_end, _ptr(sel_blocks),
                                             _ptr(sel_count), _ptr(out), _ptr(lse), _ptr(dout),
                                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                             workspace_bytes, _stream(stream)))


def qsa_index_build_backward(cfg, batch, k_idx, cap_tokens, len_before, len_after,
                             max_new_blocks, rms_gain, dk_cmp, dk_idx, stream=None) -> None:
    lib = load()
    _check(lib, lib.qsa_index_build_backward(ctypes.byref(cfg), batch, _ptr(k_idx), cap_tokens,
                                             _ptr(len_before), _ptr(len_after), max_new_blocks,
                                             _ptr(rms_gain), _ptr(dk_cmp), _ptr(dk_idx),
                                             _stream(stream)))


def qsa_indexer_distill(cfg, batch, n_q, q, k_cache, cap_tokens, q_pos0, max_pos_end, q_idx,
                        k_cmp, loss, dq_idx, dk_cmp, workspace, workspace_bytes,
                        stream=None) -> None:
    lib = load()
    _check(lib, lib.qsa_indexer_distill(ctypes.byref(cfg), batch, n_q, _ptr(q), _ptr(k_cache),
                                        cap_tokens, _ptr(q_pos0), max_pos_end, _ptr(q_idx),
                                        _ptr(k_cmp), _ptr(loss), _ptr(dq_idx), _ptr(dk_cmp),
                                        _ptr(workspace), workspace_bytes, _stream(stream)))


def qsa_offload_stage(cfg, batch, q_pos, sel_blocks, sel_count, k_host, v_host, cap_tokens,
                      hot_k, hot_v, hot_tag, hot_units, stage_k, stage_v, stage_tokens, stage_sel,
                      stage_cnt, stage_pos, stats, stream=None) -> None:
    lib = load()
    _check(lib, lib.qsa_offload_stage(ctypes.byref(cfg), batch, _ptr(q_pos), _ptr(sel_blocks),
                                      _ptr(sel_count), _ptr(k_host), _ptr(v_host), cap_tokens,
                                      _ptr(hot_k), _ptr(hot_v), _ptr(hot_tag), hot_units,
                                      _ptr(stage_k), _ptr(stage_v), stage_tokens, _ptr(stage_sel),
                                      _ptr(stage_cnt), _ptr(stage_pos), _ptr(stats),
                                      _stream(stream)))
