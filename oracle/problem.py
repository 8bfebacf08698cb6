"""The attention problem and its visibility rule (test infrastructure only).

Token ids: main tokens are 0..N-1 in packed order; branch tokens are
N..N+Nb-1 (branch token i has id N+i).  Both query rows and keys use these ids.

Visibility, from [G] 技术贡献 and 方法详解 · CP计算 (a branch query sees the
causal main part and its own local branch part) and the branch patterns of
[G] 深度分析 · 研究背景 (EAGLE-3 TTT chains, DFlash blocks, DSpark Markov
blocks):

* main row (s, p) sees main keys (s, k) with k <= p, and no branch key;
* branch row (a, t), anchored at main position (s_a, j_a), sees main keys
  (s_a, k) with k <= j_a, plus keys (a, u) of its own branch with u <= t for
  causal kinds (EAGLE-3 TTT, DSpark) or every u for the bidirectional kind
  (DFlash).  It never sees another branch's keys.  Each branch carries its
  own kind, so one packed batch may mix the three draft families ([G] 技术贡献:
  one design serves EAGLE-3, DFlash and DSpark).

Readings where the pages are silent: the anchor itself is part of the visible
prefix; a branch token sees itself; sequences packed together never see each
other; the softmax scale is 1/sqrt(d); q-head h reads kv-head
floor(h*Hkv/Hq).
"""

from __future__ import annotations

import math

import numpy as np


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


class Problem:
    """Packed main sequences plus branches.

    Tensor arguments may be numpy arrays or any object whose ``[index_array]``
    returns rows as an array (values are upcast to fp64 on access).
    ``kind`` is "causal" or "bidir" for every branch, or a sequence with one
    of them per branch.
    """

    def __init__(self, cu_seqlens, branch_cu, branch_anchor, kind, hq, hkv, d,
                 q, k, v, qb, kb, vb, scale=None):
        self.cu = np.asarray(cu_seqlens, dtype=np.int64)
        self.bcu = np.asarray(branch_cu, dtype=np.int64)
        self.anchor = np.asarray(branch_anchor, dtype=np.int64)
        self.kind = kind
        self.hq, self.hkv, self.d = int(hq), int(hkv), int(d)
        assert self.hq % self.hkv == 0
        self.scale = 1.0 / math.sqrt(self.d) if scale is None else float(scale)
        self.q, self.k, self.v = q, k, v
        self.qb, self.kb, self.vb = qb, kb, vb
        self.N = int(self.cu[-1])
        self.Nb = int(self.bcu[-1]) if self.bcu.size else 0
        self.S = self.cu.shape[0] - 1
        self.A = self.anchor.shape[0]
        # per main token: sequence and position
        self.seq_of_main = np.repeat(np.arange(self.S, dtype=np.int64), np.diff(self.cu))
        self.pos_of_main = np.arange(self.N, dtype=np.int64) - self.cu[self.seq_of_main]
        # per branch token: branch id and index t inside the branch
        self.branch_of_tok = np.repeat(np.arange(self.A, dtype=np.int64), np.diff(self.bcu))
        self.t_of_tok = np.arange(self.Nb, dtype=np.int64) - self.bcu[self.branch_of_tok]
        if isinstance(kind, str):
            assert kind in ("causal", "bidir")
            kinds = [kind] * self.A
        else:
            kinds = list(kind)
            assert len(kinds) == self.A and all(k in ("causal", "bidir") for k in kinds)
        self.bidir_of_branch = np.asarray([k == "bidir" for k in kinds], dtype=bool)
        self.anchor_seq = self.seq_of_main[self.anchor] if self.A else np.zeros(0, np.int64)
        self.anchor_pos = self.pos_of_main[self.anchor] if self.A else np.zeros(0, np.int64)
        self.group = np.arange(self.hq) * self.hkv // self.hq   # kv-head of each q-head

    # ---- token descriptors -------------------------------------------------
    def describe(self, ids):
        """(is_branch, seq, pos, branch, t) for token ids; pos of a branch token
        is its anchor's position, branch/t are -1 for main tokens."""
        ids = np.asarray(ids, dtype=np.int64)
        is_br = ids >= self.N
        mi = np.where(is_br, 0, ids)
        bi = np.where(is_br, ids - self.N, 0)
        br = self.branch_of_tok[bi] if self.Nb else np.zeros_like(ids)
        seq = np.where(is_br, self.anchor_seq[br] if self.A else 0, self.seq_of_main[mi] if self.N else 0)
        pos = np.where(is_br, self.anchor_pos[br] if self.A else 0, self.pos_of_main[mi] if self.N else 0)
        t = np.where(is_br, self.t_of_tok[bi] if self.Nb else 0, -1)
        br = np.where(is_br, br, -1)
        return is_br, seq, pos, br, t

    def visibility(self, rows, keys):
        """bool [len(rows), len(keys)]: does query row see key."""
        rb, rs, rp, rbr, rt = self.describe(rows)
        kb, ks, kp, kbr, kt = self.describe(keys)
        main_vis = (~kb)[None, :] & (ks[None, :] == rs[:, None]) & (kp[None, :] <= rp[:, None])
        same = kb[None, :] & rb[:, None] & (kbr[None, :] == rbr[:, None])
        bidir = self.bidir_of_branch[np.maximum(rbr, 0)] if self.A else np.zeros(rbr.shape, bool)
        same &= (kt[None, :] <= rt[:, None]) | (rb & bidir)[:, None]
        return main_vis | same

    def visible_keys(self, rows):
        """Sorted union of the keys visible to any of ``rows``."""
        rb, rs, rp, rbr, _ = self.describe(rows)
        parts = []
        for s, p in set(zip(rs.tolist(), rp.tolist())):
            parts.append(np.arange(self.cu[s], self.cu[s] + p + 1, dtype=np.int64))
        for a in set(rbr[rb].tolist()):
            parts.append(self.N + np.arange(self.bcu[a], self.bcu[a + 1], dtype=np.int64))
        if not parts:
            return np.zeros(0, np.int64)
        return np.unique(np.concatenate(parts))

    # ---- row access (fp64) --------------------------------------------------
    def _rows(self, main_src, br_src, ids, heads):
        ids = np.asarray(ids, dtype=np.int64)
        out = np.zeros((ids.shape[0], heads, self.d), dtype=np.float64)
        m = ids < self.N
        if m.any():
            out[m] = _as_f64(main_src[ids[m]])
        if (~m).any():
            out[~m] = _as_f64(br_src[ids[~m] - self.N])
        return out

    def qrows(self, ids):
        return self._rows(self.q, self.qb, ids, self.hq)

    def krows(self, ids):
        return self._rows(self.k, self.kb, ids, self.hkv)

    def vrows(self, ids):
        return self._rows(self.v, self.vb, ids, self.hkv)

    def main_ids(self):
        return np.arange(self.N, dtype=np.int64)

    def branch_ids(self):
        return self.N + np.arange(self.Nb, dtype=np.int64)

    def count_visible(self):
        """Visible (query, key) pairs per q-head, by brute enumeration of the
        visibility rule (small problems only)."""
        rows = np.arange(self.N + self.Nb)
        return int(self.visibility(rows, rows).sum())
