"""Padding and balance accounting: packed zigzag sharding against a padded
layout of the same batch ([G] 核心创新: packing avoids the padding of the
USP-style layout, which the pages put at about 2.25x; [R] 长上下文才是系统设计的
主场: the variable-length CP operator test at CP 2/4/8).

Host arithmetic only; nothing here launches a kernel.

Packed layout: the sequences are packed back to back and every sequence is
cut into 2C zigzag chunks by the library's own plan (zigzag_shard_plan).

Padded layout: every sequence, with its branch structure, is padded to one
common length Lp -- the longest sequence rounded up to a multiple of 2C, so
that each padded sequence splits into 2C equal chunks -- and then sharded the
same way.  A kernel over the padded tensors cannot tell padding from tokens,
so it computes every row and every (row, key) pair of the padded structure;
only the pairs between real positions are useful.

Per rank and layout the module counts rows (main + branch tokens), computed
(row, key) pairs per q-head and useful ones; imbalance is the largest rank's
computed pairs over the mean.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence

import numpy as np

from . import api
from .flops import pair_counts_rows


@dataclass
class BranchRule:
    """Branches of `length` tokens anchored every `stride` positions of each
    sequence (EAGLE-3 TTT: stride 1, length = depth)."""
    length: int
    stride: int
    kind: str = "causal"


@dataclass
class RankCount:
    rows: int
    pairs: int          # computed (row, key) pairs per q-head
    useful: int         # pairs whose row and key are both real positions


@dataclass
class Layout:
    name: str
    tokens: int         # main tokens held over all ranks
    ranks: List[RankCount]

    @property
    def rows(self) -> int:
        return sum(r.rows for r in self.ranks)

    @property
    def pairs(self) -> int:
        return sum(r.pairs for r in self.ranks)

    @property
    def useful(self) -> int:
        return sum(r.useful for r in self.ranks)

    @property
    def imbalance(self) -> float:
        p = [r.pairs for r in self.ranks]
        return max(p) / (sum(p) / len(p)) if sum(p) else 1.0


def _structure(seqlens: Sequence[int], rule: BranchRule | None):
    lens = np.asarray(seqlens, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    if rule is None:
        return cu, np.zeros(1, np.int64), np.zeros(0, np.int64)
    anchors = np.concatenate([cu[s] + np.arange(0, L, rule.stride, dtype=np.int64)
                              for s, L in enumerate(lens)] or [np.zeros(0, np.int64)])
    bcu = np.arange(anchors.size + 1, dtype=np.int64) * rule.length
    return cu, bcu, anchors


def _count(cu, bcu, anchors, real_len, C: int, kind: str) -> List[RankCount]:
    """Per-rank counts from the library plan; `real_len[s]` is the number of
    real positions of sequence s (positions past it are padding)."""
    out = []
    for r in range(C):
        p = api.zigzag_shard_plan(cu, bcu, anchors, C, r)
        mseq, mpos = p["main_seq"].astype(np.int64), p["main_pos"].astype(np.int64)
        bseq, bpos = p["branch_seq"].astype(np.int64), p["branch_pos"].astype(np.int64)
        bt, lcu = p["branch_t"].astype(np.int64), p["local_branch_cu"].astype(np.int64)
        pm, pbm, pl = pair_counts_rows(mpos, bpos, bt, lcu, kind)
        # useful: a real row (position below the sequence's real length) and
        # real keys only -- main keys at positions below the real length, and
        # its branch's keys when the anchor is real
        rl_m = np.asarray(real_len, np.int64)[mseq]
        rl_b = np.asarray(real_len, np.int64)[bseq]
        real_m = mpos < rl_m
        real_b = bpos < rl_b
        um = int(np.sum(np.minimum(mpos + 1, rl_m)[real_m]))
        ubm = int(np.sum(np.minimum(bpos + 1, rl_b)[real_b]))
        # a branch is real when its anchor is (all its tokens share the anchor)
        if kind == "bidir":
            lens = np.diff(lcu)
            first = np.minimum(lcu[:-1], max(bpos.size - 1, 0))
            ul = int(np.sum((lens * lens)[(lens > 0) & real_b[first]])) if bpos.size else 0
        else:
            ul = int(np.sum((bt + 1)[real_b]))
        out.append(RankCount(rows=mpos.size + bpos.size, pairs=pm + pbm + pl, useful=um + ubm + ul))
    return out


def packed(seqlens: Sequence[int], C: int, rule: BranchRule | None = None) -> Layout:
    cu, bcu, anc = _structure(seqlens, rule)
    kind = rule.kind if rule else "causal"
    return Layout("packed zigzag", int(cu[-1]), _count(cu, bcu, anc, list(seqlens), C, kind))


def padded(seqlens: Sequence[int], C: int, rule: BranchRule | None = None) -> Layout:
    lp = -(-max(seqlens) // (2 * C)) * (2 * C)
    cu, bcu, anc = _structure([lp] * len(seqlens), rule)
    kind = rule.kind if rule else "causal"
    return Layout(f"padded to {lp}", int(cu[-1]), _count(cu, bcu, anc, list(seqlens), C, kind))


def table(seqlens: Sequence[int], cps=(2, 4, 8), rule: BranchRule | None = None) -> str:
    """Markdown table of both layouts at each ring size."""
    n = sum(seqlens)
    lines = ["| C | layout | main tokens | rows | computed pairs/head | useful pairs/head | "
             "tokens vs packed | pairs vs packed | rank imbalance |",
             "|---|---|---|---|---|---|---|---|---|"]
    for C in cps:
        a, b = packed(seqlens, C, rule), padded(seqlens, C, rule)
        for lay in (a, b):
            lines.append(f"| {C} | {lay.name} | {lay.tokens:,} | {lay.rows:,} | {lay.pairs:,} | "
                         f"{lay.useful:,} | {lay.tokens / n:.3f} | {lay.pairs / a.pairs:.3f} | "
                         f"{lay.imbalance:.4f} |")
    return "\n".join(lines)


if __name__ == "__main__":
    import sys
    import os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from workloads import WORKLOADS
    w = WORKLOADS["eagle3_varlen_20k"]
    print(f"sequence lengths {w.seqlens}, EAGLE-3 TTT depth {w.branch_len}")
    print(table(w.seqlens, rule=BranchRule(w.branch_len, 1, "causal")))
    print()
    print("main sequence only (no branches)")
    print(table(w.seqlens))
