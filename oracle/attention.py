"""Forward and backward of merged branch + causal attention in fp64.

Test infrastructure only (see oracle/__init__.py).

Definition ([G] 技术贡献, 方法详解 · CP计算): for query row q and q-head h with
kv-head g = floor(h*Hkv/Hq) and s_{q,k} = scale * <Q_{q,h}, K_{k,g}>, over the
visible key set V(q) of oracle.problem:

    lse_{q,h} = ln sum_{k in V(q)} exp(s_{q,k})
    O_{q,h}   = sum_{k in V(q)} exp(s_{q,k} - lse_{q,h}) V_{k,g}

The merged output is one softmax over the main and branch keys together; the
merge of a main part and a branch part ([G] 技术贡献) reaches it exactly.

Backward (the pages say nothing about it; this is the vector-Jacobian product
of the definition for an upstream dO, with no gradient flowing into lse):

    P = exp(s - lse),  Delta_{q,h} = <dO_{q,h}, O_{q,h}>,
    dS = P * (<dO_{q,h}, V_{k,g}> - Delta),
    dQ_{q,h} = scale * sum_k dS K_{k,g},
    dK_{k,g} = scale * sum_{h in g} sum_q dS Q_{q,h},
    dV_{k,g} = sum_{h in g} sum_q P dO_{q,h}.
"""

from __future__ import annotations

import numpy as np

from .problem import Problem

_NEG_INF = -np.inf


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Online-softmax merge of two partial results ([G] 技术贡献 and
    方法详解 · CP计算): lse = ln(e^lse_a + e^lse_b),
    O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b.

    An empty part has lse = -inf and O = 0 and is the identity; two empty
    parts give (0, -inf).  Shapes: o [..., d], lse [...].
    """
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(under="ignore"):
        wa = np.exp(lse_a - m_safe)      # exp(-inf) = 0
        wb = np.exp(lse_b - m_safe)
    tot = wa + wb
    nonempty = tot > 0
    safe_tot = np.where(nonempty, tot, 1.0)
    lse = np.where(nonempty, m_safe + np.log(safe_tot), _NEG_INF)
    # e^(lse_a - lse) = wa / tot
    ca = (wa / safe_tot)[..., None]
    cb = (wb / safe_tot)[..., None]
    o = ca * np.asarray(o_a, dtype=np.float64) + cb * np.asarray(o_b, dtype=np.float64)
    return o, lse


def partial(prob: Problem, rows, keys, heads=None):
    """Softmax attention of ``rows`` over the subset ``keys`` under the mask.

    Returns O [R, Hq, d] and lse [R, Hq]; a row that sees none of the keys gets
    O = 0 and lse = -inf.  ``heads`` restricts the evaluation to those q-heads
    (the others are left at O = 0, lse = -inf).
    """
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    R = rows.shape[0]
    O = np.zeros((R, prob.hq, prob.d))
    lse = np.full((R, prob.hq), _NEG_INF)
    if R == 0 or keys.shape[0] == 0:
        return O, lse
    mask = prob.visibility(rows, keys)
    Q, K, V = prob.qrows(rows), prob.krows(keys), prob.vrows(keys)
    for h in (range(prob.hq) if heads is None else heads):
        g = prob.group[h]
        S = prob.scale * (Q[:, h, :] @ K[:, g, :].T)
        S = np.where(mask, S, _NEG_INF)
        m = S.max(axis=1)
        m_safe = np.where(np.isfinite(m), m, 0.0)
        with np.errstate(under="ignore"):
            P = np.exp(S - m_safe[:, None])
        l = P.sum(axis=1)
        has = l > 0
        l_safe = np.where(has, l, 1.0)
        lse[:, h] = np.where(has, m_safe + np.log(l_safe), _NEG_INF)
        O[:, h, :] = (P @ V[:, g, :]) / l_safe[:, None]
    return O, lse


def delta(O, dO):
    """Delta_{q,h} = <dO_{q,h}, O_{q,h}> (fp64)."""
    return np.einsum("rhd,rhd->rh", np.asarray(dO, np.float64), np.asarray(O, np.float64))


def grads(prob: Problem, rows, keys, lse, dO, dlt, heads=None):
    """Gradient contributions of the (rows x keys) block, recomputed from the
    merged lse of the rows.

    Returns dQ [R, Hq, d] (this block's share) and dK, dV [len(keys), Hkv, d].
    ``heads`` restricts the sums to those q-heads.
    """
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    R, Kn = rows.shape[0], keys.shape[0]
    dQ = np.zeros((R, prob.hq, prob.d))
    dK = np.zeros((Kn, prob.hkv, prob.d))
    dV = np.zeros((Kn, prob.hkv, prob.d))
    if R == 0 or Kn == 0:
        return dQ, dK, dV
    mask = prob.visibility(rows, keys)
    Q, K, V = prob.qrows(rows), prob.krows(keys), prob.vrows(keys)
    dO = np.asarray(dO, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    for h in (range(prob.hq) if heads is None else heads):
        g = prob.group[h]
        S = prob.scale * (Q[:, h, :] @ K[:, g, :].T)
        ref = np.where(np.isfinite(lse[:, h]), lse[:, h], 0.0)
        with np.errstate(under="ignore", over="ignore"):
            P = np.where(mask, np.exp(np.where(mask, S, 0.0) - ref[:, None]), 0.0)
        dP = dO[:, h, :] @ V[:, g, :].T
        dS = P * (dP - dlt[:, h][:, None])
        dQ[:, h, :] = prob.scale * (dS @ K[:, g, :])
        dK[:, g, :] += prob.scale * (dS.T @ Q[:, h, :])
        dV[:, g, :] += P.T @ dO[:, h, :]
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# Definition mode over the whole problem, in blocks of query positions.
# ---------------------------------------------------------------------------

def _blocks(prob: Problem, block_pos: int):
    """Yield (rows, keys): for each sequence and each block of positions
    [p0, p1), the main rows of the block plus the branch rows anchored in it;
    keys are the main prefix [0, p1) of the sequence plus those branches'
    tokens.  Every row's visible keys lie inside its block's keys."""
    for s in range(prob.S):
        L = int(prob.cu[s + 1] - prob.cu[s])
        for p0 in range(0, L, block_pos):
            p1 = min(L, p0 + block_pos)
            main_rows = prob.cu[s] + np.arange(p0, p1, dtype=np.int64)
            sel = np.nonzero((prob.anchor_seq == s) & (prob.anchor_pos >= p0) &
                             (prob.anchor_pos < p1))[0]
            br_tok = [np.arange(prob.bcu[a], prob.bcu[a + 1], dtype=np.int64) for a in sel]
            br_ids = prob.N + (np.concatenate(br_tok) if br_tok else np.zeros(0, np.int64))
            rows = np.concatenate([main_rows, br_ids])
            keys = np.concatenate([prob.cu[s] + np.arange(0, p1, dtype=np.int64), br_ids])
            yield rows, keys


def forward(prob: Problem, block_pos: int = 128):
    """O [N+Nb, Hq, d] and lse [N+Nb, Hq] for every row (definition mode)."""
    n = prob.N + prob.Nb
    O = np.zeros((n, prob.hq, prob.d))
    lse = np.full((n, prob.hq), _NEG_INF)
    for rows, keys in _blocks(prob, block_pos):
        o, l = partial(prob, rows, keys)
        O[rows], lse[rows] = o, l
    return O, lse


def backward(prob: Problem, dO, fwd=None, block_pos: int = 128):
    """dQ [N+Nb, Hq, d], dK, dV [N+Nb, Hkv, d] for upstream dO [N+Nb, Hq, d]."""
    if fwd is None:
        fwd = forward(prob, block_pos)
    O, lse = fwd
    dO = np.asarray(dO, dtype=np.float64)
    dlt = delta(O, dO)
    n = prob.N + prob.Nb
    dQ = np.zeros((n, prob.hq, prob.d))
    dK = np.zeros((n, prob.hkv, prob.d))
    dV = np.zeros((n, prob.hkv, prob.d))
    for rows, keys in _blocks(prob, block_pos):
        dq, dk, dv = grads(prob, rows, keys, lse[rows], dO[rows], dlt[rows])
        dQ[rows] += dq
        dK[keys] += dk
        dV[keys] += dv
    return dQ, dK, dV


def forward_decomposed(prob: Problem):
    """Decomposed mode: (Om, lse_m) over main keys only, (Ob, lse_b) over
    branch keys only, combined with lse_merge ([G] 技术贡献)."""
    n = prob.N + prob.Nb
    rows = np.arange(n, dtype=np.int64)
    om, lm = partial(prob, rows, prob.main_ids())
    ob, lb = partial(prob, rows, prob.branch_ids())
    return lse_merge(om, lm, ob, lb)


# ---------------------------------------------------------------------------
# Sampled evaluation for workloads too large for the full oracle.
# ---------------------------------------------------------------------------

def forward_rows(prob: Problem, rows, heads=None):
    """O, lse of the given rows only, each over its full visible key set."""
    rows = np.asarray(rows, dtype=np.int64)
    return partial(prob, rows, prob.visible_keys(rows), heads)


def backward_rows(prob: Problem, rows, dO_rows, heads=None):
    """dQ of the given rows (their O, lse and Delta computed here)."""
    rows = np.asarray(rows, dtype=np.int64)
    keys = prob.visible_keys(rows)
    O, lse = partial(prob, rows, keys, heads)
    dlt = delta(O, dO_rows)
    dq, _, _ = grads(prob, rows, keys, lse, dO_rows, dlt, heads)
    return dq, O, lse


def rows_seeing(prob: Problem, keys):
    """Every query row that sees at least one of ``keys``.

    Candidates: for each sequence holding a main key, its main rows and its
    branch rows positioned at or after the earliest such key; the rows of
    every branch holding a branch key.  The visibility rule then keeps the
    candidates that see one of the keys."""
    kb, ks, kp, kbr, kt = prob.describe(keys)
    cand = []
    for s in set(ks[~kb].tolist()):
        p0 = int(kp[~kb][ks[~kb] == s].min())
        cand.append(prob.cu[s] + np.arange(p0, prob.cu[s + 1] - prob.cu[s], dtype=np.int64))
        if prob.Nb:
            sel = (prob.anchor_seq == s) & (prob.anchor_pos >= p0)          # per branch
            cand.append(prob.N + np.nonzero(sel[prob.branch_of_tok])[0])
    if kb.any() and prob.Nb:
        cand.append(prob.N + np.nonzero(np.isin(prob.branch_of_tok, kbr[kb]))[0])
    if not cand:
        return np.zeros(0, np.int64)
    rows = np.unique(np.concatenate(cand))
    vis = prob.visibility(rows, keys).any(axis=1)
    return rows[vis]


def key_grads(prob: Problem, keys, dO_source, heads=None, row_chunk=64, rows=None):
    """dK, dV [len(keys), Hkv, d] for selected keys, summed over every row that
    sees them.  ``dO_source[ids]`` returns dO rows [.., Hq, d] for row ids.
    ``heads`` optionally restricts the sum to those q-heads (all by default);
    ``rows`` optionally restricts it to those query rows -- the share of the
    key gradients that one rank's rows produce in a ring, whose sum over the
    ranks is the whole.  Each row's lse and Delta are still over its full
    visible key set."""
    keys = np.asarray(keys, dtype=np.int64)
    rows_all = rows_seeing(prob, keys)
    rows = rows_all if rows is None else np.intersect1d(rows_all, np.asarray(rows, np.int64))
    dK = np.zeros((keys.shape[0], prob.hkv, prob.d))
    dV = np.zeros((keys.shape[0], prob.hkv, prob.d))
    for i in range(0, rows.shape[0], row_chunk):
        r = rows[i:i + row_chunk]
        full = prob.visible_keys(r)
        O, lse = partial(prob, r, full, heads)
        dO = np.asarray(dO_source[r], dtype=np.float64)
        if heads is not None:
            keep = np.zeros(prob.hq, bool)
            keep[list(heads)] = True
            dO = np.where(keep[None, :, None], dO, 0.0)
        dlt = delta(O, dO)
        _, dk, dv = grads(prob, r, keys, lse, dO, dlt, heads)
        dK += dk
        dV += dv
    return dK, dV
