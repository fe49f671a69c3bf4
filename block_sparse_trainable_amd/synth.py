"""Seeded synthetic inputs for the QSA layer forward pass.

This module is the only code shared by the GPU path's tests/benchmark and the
CPU oracle's callers.  It holds none of the method's arithmetic: it draws
random numbers, rounds those draws to the storage dtype, and plants the
structure (needle blocks, positional locality) that the workloads describe.
Both sides receive the exact same arrays.

Workloads (the sizes of the five layer configurations measured here; the
planted structure is a reading of the pages' workloads):

* ``tiny``      -- fp32, 1 x 256 tokens, 4Q/1KV heads, d=64, K=64 (k_B=16).
* ``prefill``   -- bf16, 1 x 32,768 tokens, 16Q/2KV, d=128, K=2048.
* ``chunked``   -- bf16, 2 x (131,072 cached + 8,192 new) tokens.
* ``decode``    -- bf16, 8 x ~262,144 cached tokens, 64 decode steps.
* ``stack``     -- bf16, 12 layers x 1,048,576 tokens (generated per layer).

Every function takes explicit sizes so the same recipe can be produced at
parity-test scale.  Random streams: ``numpy.random.SeedSequence(seed)``
spawns one child per tensor in a fixed order, so a tensor never depends on
the sizes of the others.

bf16 tensors are carried as ``uint16`` bit patterns (round-to-nearest-even
from the fp32 draw); :func:`bf16_to_f32` decodes them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEEDS = {"tiny": 1001, "prefill": 1002, "chunked": 1003, "decode": 1004, "stack": 1005}

# Order of the spawned child streams.  Never reorder: it would change every
# workload's bytes.
_STREAMS = ("k_idx", "q_idx", "q", "k", "v", "structure", "steps")


# --------------------------------------------------------------------------
# storage dtype helpers (input preparation only)
# --------------------------------------------------------------------------
def f32_to_bf16(x: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    uint32 arithmetic cannot overflow for finite inputs (the largest finite
    pattern plus the rounding bias stays below 2^32); chunked to bound memory.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    out = np.empty(u.size, dtype=np.uint16)
    for s in range(0, u.size, chunk):
        v = u[s:s + chunk]
        out[s:s + chunk] = ((v + np.uint32(0x7FFF) + ((v >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    return out.reshape(x.shape)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exactly equal fp32 values."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Decode a stored tensor of the given storage dtype to fp32 values."""
    return bf16_to_f32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _normal(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """fp32 N(0,1) draws; chunked so huge tensors do not need an fp64 copy."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    for s in range(0, flat.size, chunk):
        e = min(flat.size, s + chunk)
        flat[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out


def _draws(st, shapes: dict) -> list:
    """fp32 N(0,1) tensors, one per named stream, drawn concurrently: each
    tensor has a stream of its own, so the values do not depend on the
    order (numpy releases the GIL while it fills)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(shapes)) as ex:
        futs = [ex.submit(_normal, st[name], shape) for name, shape in shapes.items()]
        return [f.result() for f in futs]


def _stores(arrays, dtype: str) -> list:
    """_store of each array, concurrently."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(arrays)) as ex:
        return list(ex.map(lambda a: _store(a, dtype), arrays))


# --------------------------------------------------------------------------
# layer description
# --------------------------------------------------------------------------
@dataclass
class Layout:
    """Head layout and method constants of one QSA layer."""

    idx_heads: int = 4        # indexer query heads (one shared key head)
    idx_dim: int = 128        # indexer head dim
    rope_dims: int = 64       # rotated dims [0, rope_dims)
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    block_size: int = 4       # r
    token_budget: int = 2048  # K; k_B = ceil(K / r)
    q_heads: int = 16
    kv_heads: int = 2
    head_dim: int = 128
    dtype: str = "bf16"       # storage dtype of every tensor: "bf16" or "f32"

    @property
    def k_blocks(self) -> int:
        return -(-self.token_budget // self.block_size)


@dataclass
class LayerInputs:
    """One layer's tensors for one forward call (prefill chunk or decode run).

    Shapes (B = batch, T = cap_tokens, n = queries per sequence):
      k_idx [B][T][idx_dim]                raw indexer keys, row = absolute position
      q_idx [B][n][idx_heads][idx_dim]     indexer queries
      q     [B][n][q_heads][head_dim]
      k, v  [B][T][kv_heads][head_dim]
      q_pos0 [B] int32                     position of query 0 of sequence s
      cache_len [B] int32                  tokens whose blocks exist before the call
      gain [idx_dim] float32               RMSNorm gain
    For decode runs ``n`` is the number of steps: query j of sequence s is the
    token generated at step j, at position q_pos0[s] + j.
    """

    layout: Layout
    k_idx: np.ndarray
    q_idx: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_pos0: np.ndarray
    cache_len: np.ndarray
    gain: np.ndarray
    # planted structure, for recall checks: target block per query, -1 = none
    target_block: np.ndarray = field(default=None)
    needles: list = field(default_factory=list)
    name: str = ""

    @property
    def batch(self) -> int:
        return self.k_idx.shape[0]

    @property
    def cap_tokens(self) -> int:
        return self.k_idx.shape[1]

    @property
    def n_q(self) -> int:
        return self.q_idx.shape[1]


def _streams(seed: int, layer: int = 0):
    ss = np.random.SeedSequence([seed, layer])
    kids = ss.spawn(len(_STREAMS))
    return {name: np.random.default_rng(k) for name, k in zip(_STREAMS, kids)}


def _needle_vector(rng: np.random.Generator, layout: Layout) -> np.ndarray:
    """A direction confined to the unrotated dims, norm^2 about idx_dim."""
    u = np.zeros(layout.idx_dim, dtype=np.float32)
    u[layout.rope_dims:] = rng.standard_normal(layout.idx_dim - layout.rope_dims,
                                               dtype=np.float32) * np.float32(np.sqrt(2.0))
    return u


def _plant_needle(k_idx_f: np.ndarray, block: int, u: np.ndarray, rng, r: int) -> None:
    rows = slice(block * r, block * r + r)
    k_idx_f[rows] = u[None, :] + np.float32(0.1) * rng.standard_normal(
        (r, u.size), dtype=np.float32)


def _cap(n: int, align: int = 64) -> int:
    return -(-n // align) * align


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
def tiny(n: int = 256, seed: int = SEEDS["tiny"], token_budget: int = 64) -> LayerInputs:
    """fp32 single layer, one sequence, causal prefill of all ``n`` queries.

    Needles: m = mean of all indexer query vectors; the 4 raw indexer keys of
    3 distinct random blocks are shifted by +2m.
    """
    lay = Layout(q_heads=4, kv_heads=1, head_dim=64, token_budget=token_budget, dtype="f32")
    st = _streams(seed)
    T = _cap(n, 4)
    k_idx, q_idx, q, k, v = _draws(st, {
        "k_idx": (1, T, lay.idx_dim), "q_idx": (1, n, lay.idx_heads, lay.idx_dim),
        "q": (1, n, lay.q_heads, lay.head_dim), "k": (1, T, lay.kv_heads, lay.head_dim),
        "v": (1, T, lay.kv_heads, lay.head_dim)})
    m = q_idx.reshape(-1, lay.idx_dim).mean(axis=0, dtype=np.float64).astype(np.float32)
    nb = n // lay.block_size
    needles = sorted(st["structure"].choice(nb, size=min(3, nb), replace=False).tolist())
    for b in needles:
        k_idx[0, b * 4:(b + 1) * 4] += 2.0 * m
    return LayerInputs(lay, k_idx, q_idx, q, k, v,
                       q_pos0=np.zeros(1, np.int32), cache_len=np.zeros(1, np.int32),
                       gain=np.ones(lay.idx_dim, np.float32),
                       target_block=np.full((1, n), -1, np.int32), needles=[needles],
                       name=f"tiny-n{n}")


def prefill(n: int = 32768, seed: int = SEEDS["prefill"], batch: int = 1,
            needle_frac: float = 0.01, layout: Optional[Layout] = None,
            gain: Optional[np.ndarray] = None) -> LayerInputs:
    """bf16 prefill from an empty cache, queries at positions 0..n-1.

    Needles: round(needle_frac * n/4) blocks per sequence, uniform without
    replacement; their raw indexer keys become u_j + 0.1*noise.  A query with
    at least one visible needle targets one of them, chosen uniformly, with
    probability 1/2: its indexer query gets +0.5*u_j on every head.
    """
    lay = layout or Layout()
    st = _streams(seed)
    T = _cap(n)
    r = lay.block_size
    k_idx, q_idx, q, k, v = _draws(st, {
        "k_idx": (batch, T, lay.idx_dim), "q_idx": (batch, n, lay.idx_heads, lay.idx_dim),
        "q": (batch, n, lay.q_heads, lay.head_dim), "k": (batch, T, lay.kv_heads, lay.head_dim),
        "v": (batch, T, lay.kv_heads, lay.head_dim)})
    rs = st["structure"]
    nb = n // r
    n_needles = int(round(needle_frac * nb))
    target = np.full((batch, n), -1, np.int32)
    all_needles = []
    for s in range(batch):
        blocks = np.sort(rs.choice(nb, size=n_needles, replace=False)) if n_needles else np.zeros(0, int)
        us = [_needle_vector(rs, lay) for _ in blocks]
        for b, u in zip(blocks, us):
            _plant_needle(k_idx[s], int(b), u, rs, r)
        coin = rs.random(n)
        pick = rs.random(n)
        for i in range(n):
            c = i // r
            vis = int(np.searchsorted(blocks, c))  # needles with block < c
            if vis and coin[i] < 0.5:
                j = int(pick[i] * vis)
                target[s, i] = int(blocks[j])
                q_idx[s, i] += np.float32(0.5) * us[j][None, :]
        all_needles.append(blocks.tolist())
    g = np.ones(lay.idx_dim, np.float32) if gain is None else np.asarray(gain, np.float32)
    return LayerInputs(lay, *_stores([k_idx, q_idx, q, k, v], lay.dtype),
                       q_pos0=np.zeros(batch, np.int32), cache_len=np.zeros(batch, np.int32),
                       gain=g, target_block=target, needles=all_needles,
                       name=f"prefill-n{n}-b{batch}")


def chunked(cache: int = 131072, chunk: int = 8192, batch: int = 2,
            seed: int = SEEDS["chunked"], window: int = 2048, local_frac: float = 0.3,
            n_far: int = 10, layout: Optional[Layout] = None) -> LayerInputs:
    """bf16 chunked prefill: ``chunk`` new queries after ``cache`` cached tokens.

    Locality: window directions r_w (zero on rotated dims) are added to every
    raw indexer key at t as r_{t//W} + r_{t//W+1}; a seeded ``local_frac`` of
    the chunk's queries get +0.5*r_{p//W}, which favours keys W..2W-1 tokens
    back.  Far needles: ``n_far`` blocks per sequence in the first half of the
    cache (recipe of :func:`prefill`); every local query also targets one.
    """
    lay = layout or Layout()
    st = _streams(seed)
    r = lay.block_size
    total = cache + chunk
    T = _cap(total)
    k_idx, q_idx, q, k, v = _draws(st, {
        "k_idx": (batch, T, lay.idx_dim), "q_idx": (batch, chunk, lay.idx_heads, lay.idx_dim),
        "q": (batch, chunk, lay.q_heads, lay.head_dim), "k": (batch, T, lay.kv_heads, lay.head_dim),
        "v": (batch, T, lay.kv_heads, lay.head_dim)})
    rs = st["structure"]
    n_win = T // window + 2
    target = np.full((batch, chunk), -1, np.int32)
    all_needles = []
    for s in range(batch):
        dirs = np.zeros((n_win, lay.idx_dim), np.float32)
        dirs[:, lay.rope_dims:] = rs.standard_normal((n_win, lay.idx_dim - lay.rope_dims),
                                                     dtype=np.float32)
        w = np.arange(T) // window
        k_idx[s] += dirs[w] + dirs[w + 1]
        far_hi = max(1, (cache // 2) // r)
        blocks = np.sort(rs.choice(far_hi, size=min(n_far, far_hi), replace=False))
        us = [_needle_vector(rs, lay) for _ in blocks]
        for b, u in zip(blocks, us):
            _plant_needle(k_idx[s], int(b), u, rs, r)
        local = rs.random(chunk) < local_frac
        pick = rs.integers(0, len(blocks), size=chunk)
        for j in np.nonzero(local)[0]:
            p = cache + int(j)
            q_idx[s, j] += np.float32(0.5) * dirs[p // window][None, :]
            q_idx[s, j] += np.float32(0.5) * us[pick[j]][None, :]
            target[s, j] = int(blocks[pick[j]])
        all_needles.append(blocks.tolist())
    return LayerInputs(lay, *_stores([k_idx, q_idx, q, k, v], lay.dtype),
                       q_pos0=np.full(batch, cache, np.int32),
                       cache_len=np.full(batch, cache, np.int32),
                       gain=np.ones(lay.idx_dim, np.float32), target_block=target,
                       needles=all_needles, name=f"chunked-c{cache}-n{chunk}-b{batch}")


def decode(context: int = 262144, batch: int = 8, steps: int = 64,
           seed: int = SEEDS["decode"], n_needles: int = 64,
           layout: Optional[Layout] = None) -> LayerInputs:
    """bf16 decode run: sequence s holds L_s = context + t_s cached tokens,
    t_s in {0..3}; step j generates the token at position L_s + j.

    The rows of all ``steps`` future tokens are part of the tensors (the
    upstream projections would write them one step at a time; a step only
    reads rows at or before its own position).  Needles: ``n_needles`` blocks
    per sequence in [0, context/4); every step's indexer query targets one.
    """
    lay = layout or Layout()
    st = _streams(seed)
    r = lay.block_size
    rs = st["structure"]
    tails = rs.integers(0, r, size=batch).astype(np.int32)
    lens = (context + tails).astype(np.int32)
    T = _cap(int(lens.max()) + steps)
    k_idx, q_idx, q, k, v = _draws(st, {
        "k_idx": (batch, T, lay.idx_dim), "q_idx": (batch, steps, lay.idx_heads, lay.idx_dim),
        "q": (batch, steps, lay.q_heads, lay.head_dim), "k": (batch, T, lay.kv_heads, lay.head_dim),
        "v": (batch, T, lay.kv_heads, lay.head_dim)})
    nb = context // r
    target = np.full((batch, steps), -1, np.int32)
    all_needles = []
    for s in range(batch):
        blocks = np.sort(rs.choice(nb, size=min(n_needles, nb), replace=False))
        us = [_needle_vector(rs, lay) for _ in blocks]
        for b, u in zip(blocks, us):
            _plant_needle(k_idx[s], int(b), u, rs, r)
        pick = rs.integers(0, len(blocks), size=steps)
        for j in range(steps):
            q_idx[s, j] += np.float32(0.5) * us[pick[j]][None, :]
            target[s, j] = int(blocks[pick[j]])
        all_needles.append(blocks.tolist())
    return LayerInputs(lay, *_stores([k_idx, q_idx, q, k, v], lay.dtype),
                       q_pos0=lens.copy(), cache_len=lens.copy(),
                       gain=np.ones(lay.idx_dim, np.float32), target_block=target,
                       needles=all_needles, name=f"decode-c{context}-b{batch}-s{steps}")


def stack_layer(layer: int, context: int = 1048576, steps: int = 64,
                seed: int = SEEDS["stack"], n_needles: int = 16, n_layers: int = 12,
                companion: int = 0, layout: Optional[Layout] = None) -> LayerInputs:
    """One layer of the 12-layer long-context stack, batch 1.

    ``companion == 0``: a decode run of ``steps`` tokens after ``context``
    cached tokens; at step j the query targets needle (j + layer) mod 16.
    ``companion > 0``: a prefill chunk of the last ``companion`` queries of
    the context (cache = context - companion); each query targets a random
    visible needle with probability 1/2.  Needles sit at blocks
    floor((m + 1/2) * (context/4) / n_needles).
    """
    lay = layout or Layout()
    st = _streams(seed, layer)
    r = lay.block_size
    rs = st["structure"]
    nb = context // r
    blocks = [int((m + 0.5) * nb / n_needles) for m in range(n_needles)]
    us = [_needle_vector(rs, lay) for _ in blocks]
    if companion:
        n = companion
        start = context - companion
        T = _cap(context)
    else:
        n = steps
        start = context
        T = _cap(context + steps)
    k_idx, q_idx, q, k, v = _draws(st, {
        "k_idx": (1, T, lay.idx_dim), "q_idx": (1, n, lay.idx_heads, lay.idx_dim),
        "q": (1, n, lay.q_heads, lay.head_dim), "k": (1, T, lay.kv_heads, lay.head_dim),
        "v": (1, T, lay.kv_heads, lay.head_dim)})
    for b, u in zip(blocks, us):
        _plant_needle(k_idx[0], b, u, rs, r)
    target = np.full((1, n), -1, np.int32)
    if companion:
        coin = rs.random(n)
        pick = rs.random(n)
        for j in range(n):
            c = (start + j) // r
            vis = int(np.searchsorted(blocks, c))
            if vis and coin[j] < 0.5:
                m = int(pick[j] * vis)
                q_idx[0, j] += np.float32(0.5) * us[m][None, :]
                target[0, j] = blocks[m]
    else:
        for j in range(n):
            m = (j + layer) % n_needles
            q_idx[0, j] += np.float32(0.5) * us[m][None, :]
            target[0, j] = blocks[m]
    return LayerInputs(lay, *_stores([k_idx, q_idx, q, k, v], lay.dtype),
                       q_pos0=np.array([start], np.int32), cache_len=np.array([start], np.int32),
                       gain=np.ones(lay.idx_dim, np.float32), target_block=target,
                       needles=[blocks],
                       name=f"stack-l{layer}-c{context}" + (f"-comp{companion}" if companion else ""))
