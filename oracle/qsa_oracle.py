"""fp64 CPU oracle of the QSA layer forward pass (and of the sparse attention's
backward, the next step the pages point to).

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and it
imports nothing from the product.

It follows the method step by step, in the pages' order and notation, in
plain NumPy fp64, one query row at a time.  Sources:

[concept] "QSA (Qwen Sparse Attention)" research-hub concept page,
    section "Key math / How it works": (A) compressed lightweight indexer --
    MQA layout (4 query heads, one shared key head, dim 128); block
    compression k_hat_b = RMSNorm(AvgPool(keys of a block of r tokens));
    partial RoPE on 64 of 128 dims, applied after compression; block
    importance I_ib = sum_h ReLU(<q_i^h, k_bar_b>) with block-causal masking;
    top-k_B selection, k_B = ceil(K/r), expanded to tokens plus the tail of
    the current block.  (B) sparse core attention: softmax attention with
    the 1/sqrt(d) logit scale over the selected tokens only.  "Config":
    K=2048, r=4.
[gallery] "Qwen Sparse Attention" architecture-gallery page: the selection
    unit/budget table (complete four-token blocks, up to 512 blocks plus the
    current tail); "How block selection works" (blocks of keys preceding the
    query, mean per complete block, normalisation, RoPE at each block's first
    position, relu-sum scoring over indexer heads, top-k, expansion to token
    positions plus the current incomplete block); the QSA-vs-DSA table (the
    current incomplete block is included directly).

Readings where the pages are silent:
  * k_hat_b and k_bar_b are one vector: AvgPool -> RMSNorm -> partial RoPE.
  * RMSNorm(x) = x / sqrt(mean(x^2) + eps) * g, over all idx_dim dims.
  * RoPE rotates dims [0, rope_dims) in rotate-half pairs (j, j + rope_dims/2)
    with theta_j = base^(-2j/rope_dims), at absolute position r*b.
    PARITY UNPINNED: the pages fix neither the pairing nor the frequency
    schedule; the tests pin only properties every RoPE has.
  * Candidate blocks of a query at position p: b < floor(p/r) (complete
    blocks strictly before the query's own block).  Tail: positions
    r*floor(p/r) .. p inclusive (always contains p).
  * Ties in I are broken toward the lower block index; the selection is
    reported in ascending block order.
  * Attention scale 1/sqrt(head_dim); main head h reads KV head
    floor(h * Hkv / Hq); one selection per query is shared by every main head.
  * Index rows are stored in the layer's storage dtype (bf16 or fp32),
    rounded to nearest-even, before scoring ("storage" argument).
  * Backward (the pages give none): the exact derivative of the sparse
    attention with each query's token set held fixed; no gradient reaches
    the indexer through the top-k_B choice.
  * Stage-1 indexer distillation ([concept] "Native trainability": an
    indexer-only warm-up fits the indexer scores to a block-maxpooled dense
    teacher attention distribution with a KL loss while the model runs dense
    attention).  Unstated, read as: the teacher is the dense causal
    attention of the query at p over tokens 0..p, averaged over the main
    heads; its max over each candidate block's r tokens (b < floor(p/r)),
    renormalised over the candidates, is the target t; the indexer
    distribution is softmax over the candidates of I_b (no temperature); the
    loss of a query is KL(t || softmax(I)), 0 when it has no candidate.  The
    teacher sends no gradient.  ReLU'(0) = 0.  Gradients reach the stored
    index rows k_hat (its storage rounding passed straight through) and,
    through RMSNorm, RoPE and the block mean, the raw indexer keys.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "round_to_bf16", "round_to_f32", "avg_pool_blocks", "rms_norm", "rope_angles",
    "partial_rope", "compress_index", "block_importance", "top_k_blocks",
    "expand_with_tail", "sparse_attention", "sparse_attention_backward", "RowResult",
    "qsa_row", "teacher_block_target", "distill_row", "distill_grads",
    "compress_index_backward",
]


# ---------------------------------------------------------------------------
# storage rounding (the index rows are kept in the layer's dtype)
# ---------------------------------------------------------------------------
def round_to_bf16(x) -> np.ndarray:
    """Nearest bf16 value (8 significant bits), ties to even, as fp64.

    Written from the definition: x = m * 2^e with m in [0.5, 1); keep 8 bits
    of m with round-half-even (np.rint).  Values are O(1) here, so the bf16
    exponent range (that of fp32) is never exceeded.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_to_f32(x) -> np.ndarray:
    """Nearest fp32 value, ties to even, as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


_STORAGE = {"bf16": round_to_bf16, "f32": round_to_f32, "f64": lambda x: np.asarray(x, np.float64)}


# ---------------------------------------------------------------------------
# (A) compressed lightweight indexer -- block compression
# ---------------------------------------------------------------------------
def avg_pool_blocks(k_idx: np.ndarray, r: int, n_blocks: int) -> np.ndarray:
    """AvgPool of the raw indexer keys over each complete block of r tokens.

    [concept] (A) block compression; [gallery] "How block selection works":
    the keys of each complete block are averaged.  Block b covers positions
    r*b .. r*b + r - 1.
    """
    k = np.asarray(k_idx, dtype=np.float64)[: n_blocks * r]
    return k.reshape(n_blocks, r, k.shape[-1]).mean(axis=1)


def rms_norm(x: np.ndarray, gain, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.

    [concept] (A): k_hat_b = RMSNorm(AvgPool(...)); [gallery]: a normalisation
    step follows the mean.  eps and g are not given by the pages.
    """
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gain, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_angles(positions, rope_dims: int, base: float) -> np.ndarray:
    """Rotation angle of pair j at each position: pos * base^(-2j/rope_dims)."""
    j = np.arange(rope_dims // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * j / rope_dims)
    return np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]


def partial_rope(x: np.ndarray, positions, rope_dims: int, base: float) -> np.ndarray:
    """Rotate dims [0, rope_dims) of each row at its position; keep the rest.

    [concept] (A): RoPE on 64 of 128 dims, applied after compression.
    Pair j = (j, j + rope_dims/2) is rotated by angle pos*theta_j:
      x'_j = x_j cos a - x_{j+h} sin a ;  x'_{j+h} = x_{j+h} cos a + x_j sin a.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    h = rope_dims // 2
    a = rope_angles(positions, rope_dims, base)
    c, s = np.cos(a), np.sin(a)
    lo = x[:, :h].copy()
    hi = x[:, h:rope_dims].copy()
    x[:, :h] = lo * c - hi * s
    x[:, h:rope_dims] = hi * c + lo * s
    return x


def compress_index(k_idx: np.ndarray, n_blocks: int, *, r: int = 4, gain=None,
                   eps: float = 1e-6, rope_dims: int = 64, base: float = 10000.0,
                   storage: str = "bf16") -> np.ndarray:
    """k_hat for blocks 0..n_blocks-1 of one sequence: AvgPool -> RMSNorm ->
    partial RoPE at the block's first position r*b -> storage rounding.

    [gallery] "How block selection works": mean per complete block, then a
    normalisation step, then RoPE using the first position in each block.
    """
    d = np.asarray(k_idx).shape[-1]
    g = np.ones(d) if gain is None else gain
    pooled = avg_pool_blocks(k_idx, r, n_blocks)
    normed = rms_norm(pooled, g, eps)
    rotated = partial_rope(normed, r * np.arange(n_blocks), rope_dims, base)
    return _STORAGE[storage](rotated)


# ---------------------------------------------------------------------------
# (A) block importance and top-k_B selection
# ---------------------------------------------------------------------------
def block_importance(q_idx_row: np.ndarray, k_hat: np.ndarray, c: int) -> np.ndarray:
    """I_b = sum over indexer heads h of ReLU(<q^h, k_hat_b>) for b < c.

    [concept] (A), block-importance equation; [gallery] pseudocode "scores"
    line.  Block-causal masking: only the c complete blocks before the
    query's own block are candidates.  ReLU returns +0.0 for x <= 0.
    """
    q = np.asarray(q_idx_row, dtype=np.float64)           # [H, d]
    if c == 0:
        return np.zeros(0)
    dots = q @ np.asarray(k_hat[:c], dtype=np.float64).T  # [H, c]
    return np.where(dots > 0.0, dots, 0.0).sum(axis=0)


@dataclass
class Selection:
    blocks: np.ndarray   # ascending block ids, length count
    count: int
    order: np.ndarray    # all candidates by (I desc, b asc)
    margin: float        # (I_(k) - I_(k+1)) / |I_(k)|, inf when c <= k_B


def top_k_blocks(I: np.ndarray, k_B: int) -> Selection:
    """The min(k_B, c) highest-scoring blocks, ties to the lower index.

    [concept] (A): keep the k_B = ceil(K/r) highest-scoring blocks; the
    selection is returned in ascending block order.
    """
    c = I.shape[0]
    order = np.argsort(-I, kind="stable")  # stable: equal I keep index order
    count = min(k_B, c)
    blocks = np.sort(order[:count])
    if c > k_B:
        ik, ik1 = I[order[k_B - 1]], I[order[k_B]]
        margin = (ik - ik1) / abs(ik) if ik != 0.0 else 0.0
    else:
        margin = math.inf
    return Selection(blocks=blocks.astype(np.int64), count=count, order=order, margin=margin)


def expand_with_tail(blocks: np.ndarray, p: int, r: int = 4) -> np.ndarray:
    """Token positions attended by the query at position p.

    [gallery] pseudocode "attention_input" line and the QSA-vs-DSA table:
    every token of each selected block, plus the visible tokens of the
    current incomplete block, positions r*floor(p/r) .. p.
    """
    toks = (r * np.asarray(blocks, dtype=np.int64)[:, None] + np.arange(r)[None, :]).reshape(-1)
    tail = np.arange(r * (p // r), p + 1, dtype=np.int64)
    return np.concatenate([toks, tail])


# ---------------------------------------------------------------------------
# (B) sparse core attention
# ---------------------------------------------------------------------------
def sparse_attention(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, S: np.ndarray,
                     scale: float):
    """Scaled-dot-product attention of one query over the token set S.

    [concept] (B).  q_row [Hq, d]; K, V [T, Hkv, d] of the query's sequence.
    Head h reads KV head floor(h*Hkv/Hq).  Returns (o [Hq, d], lse [Hq]) with
    lse the natural-log sum of exp of the scaled logits.
    """
    q = np.asarray(q_row, dtype=np.float64)
    Hq, d = q.shape
    Hkv = K.shape[1]
    Ks = np.asarray(K[S], dtype=np.float64)   # [|S|, Hkv, d]
    Vs = np.asarray(V[S], dtype=np.float64)
    o = np.empty((Hq, d))
    lse = np.empty(Hq)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        logits = scale * (Ks[:, g, :] @ q[h])
        m = logits.max()
        w = np.exp(logits - m)
        z = w.sum()
        o[h] = (w @ Vs[:, g, :]) / z
        lse[h] = m + math.log(z)
    return o, lse


def sparse_attention_backward(q_row: np.ndarray, K: np.ndarray, V: np.ndarray,
                              S: np.ndarray, dout_row: np.ndarray, scale: float,
                              dK: np.ndarray, dV: np.ndarray) -> np.ndarray:
    """Gradient of sparse_attention for one query, given dL/do = dout_row.

    The pages define the forward only ([concept] (B)); this is its exact
    derivative with the token set S held fixed (the top-k_B choice is
    piecewise constant in its inputs, so the attention loss sends no gradient
    through it).  Per head h with KV head g:
        P_j  = softmax_j(scale * <q_h, K_j>)          over j in S
        dP_j = <dO_h, V_j>
        dS_j = P_j * (dP_j - sum_k P_k dP_k)
        dq_h = scale * sum_j dS_j K_j
        dK_j += scale * dS_j q_h,   dV_j += P_j dO_h.
    Returns dq [Hq, d]; adds into dK, dV [T, Hkv, d] (fp64) at the rows of S.
    """
    q = np.asarray(q_row, dtype=np.float64)
    do = np.asarray(dout_row, dtype=np.float64)
    Hq, d = q.shape
    Hkv = K.shape[1]
    S = np.asarray(S, dtype=np.int64)
    Ks = np.asarray(K[S], dtype=np.float64)
    Vs = np.asarray(V[S], dtype=np.float64)
    dq = np.empty((Hq, d))
    for h in range(Hq):
        g = (h * Hkv) // Hq
        logits = scale * (Ks[:, g, :] @ q[h])
        w = np.exp(logits - logits.max())
        P = w / w.sum()
        dP = Vs[:, g, :] @ do[h]
        dS = P * (dP - P @ dP)
        dq[h] = scale * (dS @ Ks[:, g, :])
        np.add.at(dK[:, g, :], S, scale * dS[:, None] * q[h][None, :])
        np.add.at(dV[:, g, :], S, P[:, None] * do[h][None, :])
    return dq


# ---------------------------------------------------------------------------
# stage-1 indexer distillation (loss and its gradients)
# ---------------------------------------------------------------------------
def teacher_block_target(q_row: np.ndarray, K: np.ndarray, p: int, r: int,
                         scale: float) -> np.ndarray:
    """Target distribution over the candidate blocks b < floor(p/r) of the
    query at p: the dense causal attention of every main head over tokens
    0..p, averaged over the heads, max-pooled over each block's r tokens,
    renormalised over the candidates.

    [concept] "Native trainability", stage 1 (the dense attention, maxed
    over each block, as the indexer's target).  Head h reads KV head
    floor(h*Hkv/Hq), scale as in (B).  Empty when there is no candidate.
    """
    c = p // r
    if c == 0:
        return np.zeros(0)
    q = np.asarray(q_row, dtype=np.float64)
    Hq, d = q.shape
    Hkv = K.shape[1]
    Kp = np.asarray(K[: p + 1], dtype=np.float64)
    mean = np.zeros(p + 1)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        logits = scale * (Kp[:, g, :] @ q[h])
        w = np.exp(logits - logits.max())
        mean += w / w.sum()
    mean /= Hq
    t = mean[: c * r].reshape(c, r).max(axis=1)
    return t / t.sum()


def distill_row(t: np.ndarray, I: np.ndarray):
    """KL(t || softmax(I)) over one query's candidates and its gradient with
    respect to I: dL/dI_b = softmax(I)_b - t_b.

    Terms with t_b = 0 contribute 0 to the loss.  Returns (loss, dI).
    """
    t = np.asarray(t, dtype=np.float64)
    I = np.asarray(I, dtype=np.float64)
    if t.size == 0:
        return 0.0, np.zeros(0)
    m = I.max()
    lse = m + math.log(np.exp(I - m).sum())
    logQ = I - lse
    nz = t > 0
    loss = float(np.sum(t[nz] * (np.log(t[nz]) - logQ[nz])))
    return loss, np.exp(logQ) - t


def distill_grads(q_idx_row: np.ndarray, k_hat: np.ndarray, dI: np.ndarray):
    """Back through I_b = sum_h ReLU(<q^h, k_hat_b>) for b < c = len(dI):
        dq^h     = sum_b dI_b [<q^h, k_hat_b> > 0] k_hat_b
        dk_hat_b = dI_b sum_h [<q^h, k_hat_b> > 0] q^h
    Returns (dq_idx [H, D], dk_hat [c, D]); ReLU'(0) = 0.
    """
    q = np.asarray(q_idx_row, dtype=np.float64)
    c = len(dI)
    kh = np.asarray(k_hat, dtype=np.float64)[:c]
    on = (kh @ q.T) > 0                      # [c, H]
    w = on * np.asarray(dI, dtype=np.float64)[:, None]
    return w.T @ kh, w @ q


def compress_index_backward(k_idx: np.ndarray, n_blocks: int, dk_hat: np.ndarray, *,
                            r: int = 4, gain=None, eps: float = 1e-6, rope_dims: int = 64,
                            base: float = 10000.0) -> np.ndarray:
    """dL/dk_idx for rows 0 .. n_blocks*r - 1 given dL/dk_hat of blocks
    0 .. n_blocks-1, back through compress_index (the storage rounding passed
    straight through): RoPE's rotation transposed (the same rotation at minus
    the angle), then RMSNorm's Jacobian
        dx = (g*dy)/rms - x * sum(g*dy*x) / (D rms^3),  rms = sqrt(mean(x^2)+eps),
    then 1/r to each of the block's r rows.
    """
    d = np.asarray(k_idx).shape[-1]
    g = np.ones(d) if gain is None else np.asarray(gain, dtype=np.float64)
    x = avg_pool_blocks(k_idx, r, n_blocks)
    dy = partial_rope(np.asarray(dk_hat, dtype=np.float64)[:n_blocks],
                      -r * np.arange(n_blocks), rope_dims, base)
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    gdy = g * dy
    dx = gdy / rms - x * np.sum(gdy * x, axis=-1, keepdims=True) / (d * rms ** 3)
    return np.repeat(dx / r, r, axis=0)


# ---------------------------------------------------------------------------
# one query row, end to end
# ---------------------------------------------------------------------------
@dataclass
class RowResult:
    p: int
    c: int
    scores: np.ndarray      # full I row, length c
    sel: Selection
    S: np.ndarray
    o: np.ndarray
    lse: np.ndarray


def qsa_row(p: int, q_idx_row, q_row, k_hat, K, V, *, k_B: int, r: int = 4,
            scale: float | None = None, attend: bool = True) -> RowResult:
    """Every step for the query at absolute position p of one sequence.

    k_hat must hold at least floor(p/r) compressed blocks.
    """
    c = p // r
    I = block_importance(q_idx_row, k_hat, c)
    sel = top_k_blocks(I, k_B)
    S = expand_with_tail(sel.blocks, p, r)
    if attend:
        d = np.asarray(q_row).shape[-1]
        s = 1.0 / math.sqrt(d) if scale is None else scale
        o, lse = sparse_attention(q_row, K, V, S, s)
    else:
        o = lse = None
    return RowResult(p=p, c=c, scores=I, sel=sel, S=S, o=o, lse=lse)
