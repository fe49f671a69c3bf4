"""Host-side counting in bench.py (no GPU): the token-visit and group-entry
counts that the backward's throughput and traffic figures are built on,
against brute force over explicit token sets."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from block_sparse_trainable_amd import synth  # noqa: E402


def _sets(x, sel, cnt):
    r, kB = x.layout.block_size, x.layout.k_blocks
    for s in range(x.batch):
        for j in range(x.n_q):
            p = int(x.q_pos0[s]) + j
            c = p // r
            n = min(int(cnt[s, j]), kB, c)
            toks = [b * r + t for b in sel[s, j, :n] for t in range(r)]
            toks += list(range(c * r, p + 1))
            yield toks


def test_counts_match_brute_force():
    rng = np.random.default_rng(3)
    for r in (4, 8, 32):
        lay = synth.Layout(block_size=r, token_budget=8 * r)      # k_B = 8
        x = synth.chunked(cache=300, chunk=40, batch=2, window=64, n_far=2, layout=lay)
        kB = lay.k_blocks
        sel = np.full((x.batch, x.n_q, kB), -1, np.int32)
        cnt = np.zeros((x.batch, x.n_q), np.int32)
        for s in range(x.batch):
            for j in range(x.n_q):
                c = (int(x.q_pos0[s]) + j) // r
                n = min(kB, c)
                sel[s, j, :n] = np.sort(rng.choice(c, n, replace=False))
                cnt[s, j] = n
        sets = list(_sets(x, sel, cnt))
        assert bench.token_visits(x) == sum(len(t) for t in sets)
        want = sum(len({t // 16 for t in toks}) for toks in sets)
        assert bench.group_entries(x, sel, cnt) == want
