"""Comparison protocol between the HIP path and the fp64 oracle.

Tolerances (written in the tests that call these):
  * indexer scores: |I_gpu - I_ref| <= 1e-2 * max(|I_ref|, rms of the row)
    (relative 1e-2 is undefined at I = 0, common under ReLU; the row RMS
    is the floor);
  * selection: rows with c <= k_B keep every block; rows whose oracle margin
    (I_(k) - I_(k+1)) / |I_(k)| exceeds 1e-3 must match bit-exactly; other
    rows must be rank-consistent: every selected block scores at least
    I_(k) - 1e-3|I_(k)| - 1e-6 rms, and every block above
    I_(k) + 1e-3|I_(k)| + 1e-6 rms is selected;
  * attention: max-abs 2e-2 with bf16 I/O, 1e-4 with fp32 I/O, measured
    against the oracle applied to the GPU's own selection.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from oracle import qsa_oracle as O
from block_sparse_trainable_amd import synth

SCORE_RTOL = 1e-2
MARGIN = 1e-3
ATOL = {"bf16": 2e-2, "f32": 1e-4}
LSE_ATOL = {"bf16": 2e-2, "f32": 1e-4}


@dataclass
class RowCheck:
    exact_eligible: bool
    exact: bool
    overlap: float


def f64(a, dtype):
    return synth.as_f32(a, dtype).astype(np.float64)


def oracle_khat(x: synth.LayerInputs, s: int, n_blocks: int) -> np.ndarray:
    lay = x.layout
    k_idx = f64(x.k_idx[s, : n_blocks * lay.block_size], lay.dtype)
    return O.compress_index(k_idx, n_blocks, r=lay.block_size, gain=x.gain.astype(np.float64),
                            eps=float(np.float32(lay.rms_eps)), rope_dims=lay.rope_dims,
                            base=lay.rope_base, storage=lay.dtype)


def check_selection(res, sel_row, cnt, scores_row, kB) -> RowCheck:
    c = res.c
    count = min(kB, c)
    assert cnt == count, f"p={res.p}: count {cnt} != {count}"
    g = np.asarray(sel_row[:count], dtype=np.int64)
    assert (np.asarray(sel_row[count:]) == -1).all(), f"p={res.p}: padding not -1"
    if count:
        assert (np.diff(g) > 0).all(), f"p={res.p}: selection not ascending/distinct"
        assert g.min() >= 0 and g.max() < c, f"p={res.p}: selected block outside [0, c)"
    I = res.scores
    rms = float(np.sqrt(np.mean(I * I))) if c else 0.0
    if count and scores_row is not None:
        ref = I[g]
        err = np.abs(np.asarray(scores_row[:count], np.float64) - ref)
        bound = SCORE_RTOL * np.maximum(np.abs(ref), rms)
        bad = err > bound
        assert not bad.any(), (f"p={res.p}: score error {err[bad][:4]} > {bound[bad][:4]} "
                               f"at blocks {g[bad][:4]}")
    if c <= kB:
        assert g.tolist() == list(range(c)), f"p={res.p}: c <= k_B must keep every block"
        return RowCheck(True, True, 1.0)
    ref_sel = res.sel.blocks
    overlap = len(set(g.tolist()) & set(ref_sel.tolist())) / kB
    if res.sel.margin > MARGIN:
        assert g.tolist() == ref_sel.tolist(), (
            f"p={res.p}: margin {res.sel.margin:.2e} > 1e-3 but selection differs "
            f"(overlap {overlap:.4f})")
        return RowCheck(True, True, overlap)
    Ik = I[res.sel.order[kB - 1]]
    delta = 1e-6 * rms
    lo = Ik - MARGIN * abs(Ik) - delta
    hi = Ik + MARGIN * abs(Ik) + delta
    assert (I[g] >= lo).all(), f"p={res.p}: a selected block scores below the k-th band"
    must = np.nonzero(I > hi)[0]
    missing = set(must.tolist()) - set(g.tolist())
    assert not missing, f"p={res.p}: blocks {sorted(missing)[:4]} above the band not selected"
    return RowCheck(False, g.tolist() == ref_sel.tolist(), overlap)


def check_attention(p, sel_blocks, q_row, K, V, out_row, lse_row, scale, dtype, r=4):
    """Oracle attention over the GPU's own selection vs the GPU output."""
    S = O.expand_with_tail(np.asarray(sel_blocks, np.int64), p, r)
    o, lse = O.sparse_attention(q_row, K, V, S, scale)
    err = np.abs(np.asarray(out_row, np.float64) - o).max()
    assert err <= ATOL[dtype], f"p={p}: attention max-abs error {err:.3e} > {ATOL[dtype]}"
    if lse_row is not None:
        le = np.abs(np.asarray(lse_row, np.float64) - lse).max()
        assert le <= LSE_ATOL[dtype], f"p={p}: lse error {le:.3e}"
    return err


def stratified_rows(n: int, q_pos0: int, extra=(), k=96, seed=0) -> list:
    """A seeded sample of query rows: first/last rows, every p mod 4 residue,
    rows around the c = k_B boundary, plus ``extra`` rows."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(n, 8))) | set(range(max(0, n - 8), n))
    for target in (2048, 2052, 2056, 2180):
        j = target - q_pos0
        for d in range(-3, 4):
            if 0 <= j + d < n:
                rows.add(j + d)
    rows |= set(int(v) for v in rng.choice(n, size=min(n, k), replace=False))
    rows |= set(int(e) for e in extra if 0 <= e < n)
    return sorted(rows)


# Fused decode step control area (int32 words; include/qsa.h): per-row
# generation words at 0, the error word at 2048, per-row split flags at
# 4096 + 32 s + k, per-row score-bin counts (two buffers of 256, used by
# epoch parity) at 307200 + 512 s.
STEP_GEN, STEP_ERR, STEP_FC, STEP_ACC = 0, 2048, 4096, 307200
STEP_SPLITS = 17


def check_step_control(ws, rows):
    """After fused steps on workspace ws (rows 0 .. rows-1 stepped at least
    once since it was zero-filled): no wait gave up; each row's last call
    raised all its split flags with its own epoch (the row's generation
    word); the count buffer its next call adds into is clear; rows never
    stepped are untouched."""
    import torch
    from block_sparse_trainable_amd import _binding as B
    ctl = ws[:B.QSA_STEP_CONTROL_BYTES].view(torch.int32).cpu().numpy().astype(np.int64)
    assert ctl[STEP_ERR] == 0, "a wait gave up (error word set)"
    gen = ctl[STEP_GEN:STEP_GEN + 1024]
    assert (gen[:rows] >= 1).all(), "a row's generation word did not advance"
    assert (gen[rows:] == 0).all(), "a row that was not stepped has a generation"
    for s in range(rows):
        fc = ctl[STEP_FC + 32 * s:STEP_FC + 32 * s + STEP_SPLITS]
        assert (fc == gen[s]).all(), f"row {s}: split flags {fc} vs epoch {gen[s]}"
        nxt = STEP_ACC + 512 * s + 256 * ((gen[s] + 1) & 1)
        assert not ctl[nxt:nxt + 256].any(), f"row {s}: next call's counts not clear"
