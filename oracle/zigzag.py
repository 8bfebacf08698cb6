"""Zigzag mode: the oracle's own shard plan and a ring emulation of all ranks.

Test infrastructure only.  Written independently of the C++ plan of the HIP
library; tests compare the two arrays element by element.

Plan ([G] 新颖性 and 核心创新: packed, load-balanced zigzag ring; [R] section
"两条路，绕开并行训练的堵点": packing and interleaved assignment avoid padding
and imbalance).  Readings where the pages are silent: a sequence of length L
is cut into 2C chunks at floor(k*L/(2C)) with no padding; chunk k belongs to
rank k for k < C and to rank 2C-1-k otherwise; a branch belongs to the rank
that owns its anchor position ([G] 核心创新: branch K/V stays on the anchor's
rank); ring step s on rank r uses the main K/V shard of rank (r - s) mod C
([G] 方法详解 · CP计算: the main K/V makes C ring steps while branch queries
stay on their rank).
"""

from __future__ import annotations

import numpy as np

from .attention import partial, grads, lse_merge, delta
from .problem import Problem


def chunk_bounds(L: int, C: int):
    return [(k * L) // (2 * C) for k in range(2 * C + 1)]


def chunk_owner(k: int, C: int) -> int:
    return k if k < C else 2 * C - 1 - k


def plan(cu_seqlens, branch_cu, branch_anchor, C: int, r: int):
    """Rank r's share.  Returns a dict of int64 arrays:

    main_index/main_seq/main_pos [n_main]: owned main tokens in (seq, pos) order;
    branch_ids [n_branches]: owned branches in global order;
    branch_index/branch_seq/branch_pos/branch_t [n_branch_tok]: their tokens,
        with pos = the anchor's position and t = index inside the branch;
    local_branch_cu [n_branches+1];
    kv_src [C]: rank whose main K/V shard is used at ring step s.
    """
    cu = [int(x) for x in cu_seqlens]
    bcu = [int(x) for x in branch_cu]
    anchor = [int(x) for x in branch_anchor]
    S = len(cu) - 1
    main_index, main_seq, main_pos = [], [], []
    bounds = []
    for s in range(S):
        L = cu[s + 1] - cu[s]
        b = chunk_bounds(L, C)
        bounds.append(b)
        for k in sorted({r, 2 * C - 1 - r}):
            for p in range(b[k], b[k + 1]):
                main_index.append(cu[s] + p)
                main_seq.append(s)
                main_pos.append(p)
    branch_ids, bi, bs, bp, bt, lcu = [], [], [], [], [], [0]
    for a, ag in enumerate(anchor):
        s = max(i for i in range(S) if cu[i] <= ag)
        p = ag - cu[s]
        b = bounds[s]
        k = next(i for i in range(2 * C) if b[i] <= p < b[i + 1])
        if chunk_owner(k, C) != r:
            continue
        branch_ids.append(a)
        for t, tok in enumerate(range(bcu[a], bcu[a + 1])):
            bi.append(tok)
            bs.append(s)
            bp.append(p)
            bt.append(t)
        lcu.append(len(bi))
    i64 = lambda x: np.asarray(x, dtype=np.int64)
    return dict(main_index=i64(main_index), main_seq=i64(main_seq), main_pos=i64(main_pos),
                branch_ids=i64(branch_ids), branch_index=i64(bi), branch_seq=i64(bs),
                branch_pos=i64(bp), branch_t=i64(bt), local_branch_cu=i64(lcu),
                kv_src=i64([(r - s) % C for s in range(C)]))


def _rank_rows(prob: Problem, pl):
    return np.concatenate([pl["main_index"], prob.N + pl["branch_index"]])


def ring_forward(prob: Problem, C: int):
    """Every rank's rows, main shards merged in ring order, then the local
    branch part; outputs scattered to global row order."""
    n = prob.N + prob.Nb
    O = np.zeros((n, prob.hq, prob.d))
    lse = np.full((n, prob.hq), -np.inf)
    plans = [plan(prob.cu, prob.bcu, prob.anchor, C, r) for r in range(C)]
    for r in range(C):
        rows = _rank_rows(prob, plans[r])
        acc_o = np.zeros((rows.shape[0], prob.hq, prob.d))
        acc_l = np.full((rows.shape[0], prob.hq), -np.inf)
        for s in range(C):
            src = int(plans[r]["kv_src"][s])
            o, l = partial(prob, rows, plans[src]["main_index"])
            acc_o, acc_l = lse_merge(acc_o, acc_l, o, l)
        o, l = partial(prob, rows, prob.N + plans[r]["branch_index"])
        acc_o, acc_l = lse_merge(acc_o, acc_l, o, l)
        O[rows], lse[rows] = acc_o, acc_l
    return O, lse


def ring_backward(prob: Problem, C: int, dO, fwd=None):
    """Per-rank, per-step gradient partials; dK/dV partials of each shard are
    summed into the owner's rows (the return trip of a real ring)."""
    if fwd is None:
        fwd = ring_forward(prob, C)
    O, lse = fwd
    dO = np.asarray(dO, dtype=np.float64)
    dlt = delta(O, dO)
    n = prob.N + prob.Nb
    dQ = np.zeros((n, prob.hq, prob.d))
    dK = np.zeros((n, prob.hkv, prob.d))
    dV = np.zeros((n, prob.hkv, prob.d))
    plans = [plan(prob.cu, prob.bcu, prob.anchor, C, r) for r in range(C)]
    for r in range(C):
        rows = _rank_rows(prob, plans[r])
        steps = [plans[int(plans[r]["kv_src"][s])]["main_index"] for s in range(C)]
        steps.append(prob.N + plans[r]["branch_index"])
        for keys in steps:
            dq, dk, dv = grads(prob, rows, keys, lse[rows], dO[rows], dlt[rows])
            dQ[rows] += dq
            dK[keys] += dk
            dV[keys] += dv
    return dQ, dK, dV


def ring_bytes_received(cu_seqlens, branch_cu, branch_anchor, C: int, r: int,
                        hkv: int, d: int, elem_bytes: int) -> int:
    """Bytes of main K and V rank r receives over one forward: the shards of
    ring steps 1..C-1 (step 0 is its own shard)."""
    pl = plan(cu_seqlens, branch_cu, branch_anchor, C, r)
    total = 0
    for s in range(1, C):
        src = int(pl["kv_src"][s])
        n_src = plan(cu_seqlens, branch_cu, branch_anchor, C, src)["main_index"].shape[0]
        total += 2 * n_src * hkv * d * elem_bytes
    return total
