"""Algorithmic work of merged branch + causal attention (host arithmetic on
the index structure; no kernels).

Visible (query, key) pairs per q-head, from the closed forms of the mask:
  * a main row at position p sees p + 1 main keys;
  * a branch token sees its anchor's position + 1 main keys, plus t + 1 branch
    keys (causal kinds) or the whole branch (bidirectional kind).
FLOPs per pair and q-head: 4d forward (QK^T and PV), 10d backward (the
recomputed QK^T plus dP, dV, dQ, dK).  Masked-out tile work and recomputation
beyond these five products are not counted.
"""

from __future__ import annotations

import numpy as np


def pair_counts_rows(main_pos, branch_pos, branch_t, local_branch_cu, kind, branch_kinds=None):
    """(main, branch->main, branch-local) pairs for a set of rows.  ``kind`` is
    'causal' or 'bidir' for every branch; with ``branch_kinds`` (one entry per
    branch, 1 = bidirectional) each branch takes its own."""
    main = int(np.sum(np.asarray(main_pos, dtype=np.int64) + 1))
    br_main = int(np.sum(np.asarray(branch_pos, dtype=np.int64) + 1))
    lens = np.diff(np.asarray(local_branch_cu, dtype=np.int64))
    if branch_kinds is not None:
        bid = np.asarray(branch_kinds) == 1
        local = int(np.sum(np.where(bid, lens * lens, lens * (lens + 1) // 2)))
    elif kind == "bidir":
        local = int(np.sum(lens * lens))
    else:
        local = int(np.sum(np.asarray(branch_t, dtype=np.int64) + 1))
    return main, br_main, local


def pair_counts(cu_seqlens, branch_cu, branch_anchor, kind, branch_kinds=None):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lens = np.diff(cu)
    seq_of = np.repeat(np.arange(lens.size), lens)
    pos = np.arange(int(cu[-1]), dtype=np.int64) - cu[seq_of]
    bcu = np.asarray(branch_cu, dtype=np.int64)
    blen = np.diff(bcu)
    anc = np.asarray(branch_anchor, dtype=np.int64)
    apos = pos[anc] if anc.size else np.zeros(0, np.int64)
    branch_pos = np.repeat(apos, blen)
    branch_t = np.arange(int(bcu[-1]), dtype=np.int64) - np.repeat(bcu[:-1], blen)
    return pair_counts_rows(pos, branch_pos, branch_t, bcu, kind, branch_kinds)


def flops(pairs: int, hq: int, d: int, phase: str = "fwd+bwd") -> float:
    per = {"fwd": 4 * d, "bwd": 10 * d, "fwd+bwd": 14 * d}[phase]
    return float(pairs) * hq * per
