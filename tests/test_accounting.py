"""Padding / balance accounting (host arithmetic over the library's plan)
against hand counts and closed forms."""

import numpy as np
import pytest

from branch_aware_causal_amd import accounting as acc
from workloads import WORKLOADS


def test_hand_counted_two_sequences_no_branches():
    # lengths 9 and 3, C = 2.  Packed: L=9 bounds 0 2 4 6 9, L=3 bounds 0 0 1 2 3;
    # rank 0 holds positions {0,1,6,7,8} and {2}: pairs 1+2+7+8+9 + 3 = 30;
    # rank 1 holds {2,3,4,5} and {0,1}: 3+4+5+6 + 1+2 = 21.
    p = acc.packed([9, 3], 2)
    assert [(r.rows, r.pairs, r.useful) for r in p.ranks] == [(6, 30, 30), (6, 21, 21)]
    assert p.tokens == 12 and p.pairs == 9 * 10 // 2 + 3 * 4 // 2
    # Padded to 12 (9 rounded up to a multiple of 4): chunks of 3; each rank
    # computes 2 x ((1+2+3) + (10+11+12)) = 78 pairs; useful: rank 0 keeps
    # positions 0..2 of both sequences (6 + 6), rank 1 positions 3..8 of the first (39).
    q = acc.padded([9, 3], 2)
    assert [(r.rows, r.pairs, r.useful) for r in q.ranks] == [(12, 78, 12), (12, 78, 39)]
    assert q.tokens == 24 and q.useful == p.pairs


def test_hand_counted_with_eagle3_depth_2():
    # same lengths, a depth-2 chain at every position: a branch row anchored at
    # p sees p+1 main keys and t+1 keys of its chain (3 pairs per chain).
    rule = acc.BranchRule(2, 1, "causal")
    p = acc.packed([9, 3], 2, rule)
    assert [(r.rows, r.pairs) for r in p.ranks] == [(18, 30 + 2 * 30 + 6 * 3), (18, 21 + 2 * 21 + 6 * 3)]
    q = acc.padded([9, 3], 2, rule)
    assert [(r.rows, r.pairs) for r in q.ranks] == [(36, 78 * 3 + 12 * 3), (36, 78 * 3 + 12 * 3)]
    assert [r.useful for r in q.ranks] == [12 + 24 + 18, 39 + 78 + 18]
    assert q.useful == p.pairs


@pytest.mark.parametrize("C", [2, 4, 8])
def test_closed_forms_on_the_20k_length_mix(C):
    w = WORKLOADS["eagle3_varlen_20k"]
    L = np.asarray(w.seqlens, np.int64)
    p, q = acc.packed(w.seqlens, C), acc.padded(w.seqlens, C)
    lp = -(-int(L.max()) // (2 * C)) * (2 * C)
    assert p.tokens == 20480 and q.tokens == L.size * lp
    assert p.pairs == int(np.sum(L * (L + 1) // 2))
    assert q.pairs == L.size * lp * (lp + 1) // 2
    assert q.useful == p.pairs
    # the padded layout splits each padded sequence exactly, so it is balanced
    assert q.imbalance == 1.0
    # packed zigzag with the floor split stays within 0.2% of balance here
    assert p.imbalance < 1.002
    assert 2.3 < q.tokens / p.tokens < 2.33


def test_bidirectional_blocks():
    # one sequence of 10, DFlash-style blocks of 4 every 4 positions (anchors
    # 0, 4, 8), C = 1: main 55, branch->main 4*(1+5+9) = 60, local 3*16 = 48
    rule = acc.BranchRule(4, 4, "bidir")
    p = acc.packed([10], 1, rule)
    assert p.pairs == 55 + 60 + 48
    # padded to 10 (already a multiple of 2): nothing changes
    assert acc.padded([10], 1, rule).pairs == p.pairs
