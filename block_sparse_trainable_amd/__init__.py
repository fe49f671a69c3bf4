"""QSA (Qwen Sparse Attention) layer forward pass for MI355X (gfx950), the
backward of its sparse attention, and the stage-1 indexer distillation.

The compute lives in libqsa.so (HIP kernels behind the C ABI of
include/qsa.h); this package is its ctypes binding plus plumbing:

* :mod:`._binding` -- the four entry points, the fused decode step, the
  attention backward, the distillation loss and the compression backward,
  and helpers, same names as the C ABI.
* :mod:`.runtime`  -- device buffers for one layer and the call sequences of a
  prefill chunk and of a decode step (marshalling only).
* :mod:`.synth`    -- seeded synthetic inputs (no method arithmetic).
* :mod:`.build`    -- in-tree hipcc build of libqsa.so.
"""
from ._binding import (  # noqa: F401
    EXPORTED, QSA_BF16, QSA_F32, QSA_OP_BACKWARD, QSA_OP_DECODE, QSA_OP_DECODE_STEP,
    QSA_OP_DISTILL, QSA_OP_INDEX_BUILD, QSA_OP_PREFILL, QSA_OP_SELECT, QsaConfig, QsaError,
    library_path, load, qsa_decode_step, qsa_index_build, qsa_index_build_backward,
    qsa_indexer_distill, qsa_offload_stage, qsa_select_topk, qsa_sparse_attn_backward,
    qsa_sparse_attn_decode, qsa_sparse_attn_prefill, qsa_workspace_size,
)
