"""FLOP accounting of the package (host arithmetic) against the oracle's
visibility rule and the closed-form counts."""

import numpy as np
import pytest

from branch_aware_causal_amd import flops
from oracle import zigzag as ozz
from oracle.problem import Problem
from workloads import WORKLOADS, make_structure
from workloads.gen import make_structure_custom


def _prob(st, hq=2, hkv=1, d=2):
    z = lambda n, h: np.zeros((n, h, d))
    return Problem(st.cu_seqlens, st.branch_cu, st.branch_anchor, st.kind_names, hq, hkv, d,
                   z(st.n_main, hq), z(st.n_main, hkv), z(st.n_main, hkv),
                   z(st.n_branch_tok, hq), z(st.n_branch_tok, hkv), z(st.n_branch_tok, hkv))


@pytest.mark.parametrize("st", [
    make_structure_custom((9, 16, 3), [list(range(9)), list(range(16)), list(range(3))], [3] * 28, "causal"),
    make_structure_custom((32, 20), [list(range(0, 32, 8)), list(range(0, 20, 8))], [8] * 7, "bidir"),
    make_structure_custom((5, 7), [[0, 4], [1, 2, 6]], [2, 1, 4, 3, 2], "causal"),
])
def test_pair_counts_match_visibility(st):
    assert sum(flops.pair_counts(st.cu_seqlens, st.branch_cu, st.branch_anchor, st.kind)) == \
        _prob(st).count_visible()


def test_mixed_pack_pair_counts_match_visibility():
    from workloads import specs
    w = specs.small("mix", (40, 48, 24), branch="mixed",
                    mix=(("eagle3", 3, 1), ("dflash", 16, 16), ("dspark", 8, 8)))
    st = make_structure(w)
    assert st.kind == "mixed" and set(st.branch_kinds.tolist()) == {0, 1}
    got = flops.pair_counts(st.cu_seqlens, st.branch_cu, st.branch_anchor, st.kind, st.branch_kinds)
    assert sum(got) == _prob(st).count_visible()


@pytest.mark.parametrize("C", [2, 4])
def test_rank_pair_counts_match_visibility(C):
    st = make_structure_custom((17, 40), [list(range(17)), list(range(40))], [2] * 57, "causal")
    prob = _prob(st)
    allk = np.arange(prob.N + prob.Nb)
    for r in range(C):
        p = ozz.plan(st.cu_seqlens, st.branch_cu, st.branch_anchor, C, r)
        rows = np.concatenate([p["main_index"], prob.N + p["branch_index"]])
        got = sum(flops.pair_counts_rows(p["main_pos"], p["branch_pos"], p["branch_t"],
                                         p["local_branch_cu"], st.kind))
        assert got == int(prob.visibility(rows, allk).sum())


def test_named_workload_counts():
    w = WORKLOADS["eagle3_256k"]
    st = make_structure(w)
    m, bm, lo = flops.pair_counts(st.cu_seqlens, st.branch_cu, st.branch_anchor, st.kind)
    assert (m, bm, lo) == (34359869440, 103079608320, 1572864)
    total = flops.flops(m + bm + lo, 32, 128)
    assert abs(total / 1e12 - 7881.42) < 0.01
