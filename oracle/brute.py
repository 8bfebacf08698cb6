"""Brute-force mode: pure-Python loops with math.exp and math.fsum.

Test infrastructure only.  Tiny inputs only (a few hundred rows).  The
visibility rule is written out here again, directly from the branch patterns
([G] 深度分析 · 研究背景: EAGLE-3 TTT chains, DFlash blocks, DSpark Markov
blocks; [G] 方法详解 · CP计算: each branch query sees the causal main prefix up
to its anchor and its own local branch), without calling
``oracle.problem.Problem.visibility``, so that the two implementations check
each other.
"""

from __future__ import annotations

import math


def _kind_of(kind, a):
    """Kind of branch a: one kind for every branch, or one per branch."""
    return kind if isinstance(kind, str) else kind[a]


def _row_keys(cu, bcu, anchor, kind, row):
    """Visible keys of a row as ('m', global_idx) / ('b', branch_token_idx)."""
    S = len(cu) - 1
    keys = []
    if row[0] == "m":
        gi = row[1]
        s = max(i for i in range(S) if cu[i] <= gi)
        p = gi - cu[s]
        for kpos in range(0, p + 1):
            keys.append(("m", cu[s] + kpos))
    else:
        bt = row[1]
        a = max(i for i in range(len(bcu) - 1) if bcu[i] <= bt and bcu[i + 1] > bt)
        t = bt - bcu[a]
        ag = anchor[a]
        s = max(i for i in range(S) if cu[i] <= ag)
        j = ag - cu[s]
        for kpos in range(0, j + 1):
            keys.append(("m", cu[s] + kpos))
        blen = bcu[a + 1] - bcu[a]
        for u in range(blen):
            if _kind_of(kind, a) == "bidir" or u <= t:
                keys.append(("b", bcu[a] + u))
    return keys


def forward(cu, bcu, anchor, kind, hq, hkv, d, q, k, v, qb, kb, vb, scale=None):
    """Returns dict row -> (O [hq][d] lists, lse [hq]) for every row.

    Rows are ('m', i) for main tokens and ('b', i) for branch tokens.  Tensors
    are nested sequences (numpy arrays work) indexed [token][head][dim].
    """
    cu = [int(x) for x in cu]
    bcu = [int(x) for x in bcu]
    anchor = [int(x) for x in anchor]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = [("m", i) for i in range(cu[-1])] + [("b", i) for i in range(bcu[-1] if bcu else 0)]
    out = {}
    for row in rows:
        keys = _row_keys(cu, bcu, anchor, kind, row)
        qsrc = q if row[0] == "m" else qb
        Os, lses = [], []
        for h in range(hq):
            g = (h * hkv) // hq
            qv = [float(x) for x in qsrc[row[1]][h]]
            scores = []
            for kk in keys:
                ksrc = k if kk[0] == "m" else kb
                kv = ksrc[kk[1]][g]
                scores.append(scale * math.fsum(qv[c] * float(kv[c]) for c in range(d)))
            m = max(scores)
            ex = [math.exp(s - m) for s in scores]
            l = math.fsum(ex)
            lse = m + math.log(l)
            o = []
            for c in range(d):
                terms = []
                for e, kk in zip(ex, keys):
                    vsrc = v if kk[0] == "m" else vb
                    terms.append(e * float(vsrc[kk[1]][g][c]))
                o.append(math.fsum(terms) / l)
            Os.append(o)
            lses.append(lse)
        out[row] = (Os, lses)
    return out


def count_pairs(cu, bcu, anchor, kind):
    """Visible (query, key) pairs per q-head by explicit enumeration."""
    cu = [int(x) for x in cu]
    bcu = [int(x) for x in bcu]
    anchor = [int(x) for x in anchor]
    rows = [("m", i) for i in range(cu[-1])] + [("b", i) for i in range(bcu[-1] if bcu else 0)]
    return sum(len(_row_keys(cu, bcu, anchor, kind, r)) for r in rows)
