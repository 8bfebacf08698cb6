"""Seeded generation of the packed token structure and of the tensors.

Structure: sequences are packed back to back (``cu_seqlens``); branches are
listed in (sequence, anchor) order, each with ``branch_len`` tokens stored
contiguously (``branch_cu``); ``branch_anchor`` holds the anchor's global
main-token index.

Values: Q, K, V (main and branch) ~ N(0,1) * value_scale and dO ~ N(0,1),
drawn in fp32 with ``torch.randn`` from ``torch.Generator(device)`` seeded
with seed_base + {1..8} for (Q, K, V, Qb, Kb, Vb, dO, dOb), then rounded to
bf16 (round-to-nearest-even) for bf16 workloads.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .specs import Workload


@dataclass
class Structure:
    cu_seqlens: np.ndarray      # int32 [S+1]
    branch_cu: np.ndarray       # int32 [A+1]
    branch_anchor: np.ndarray   # int32 [A] global main index of each anchor
    kind: str                   # 'causal' | 'bidir' | 'mixed'
    max_branch_len: int
    branch_kinds: np.ndarray = None   # int32 [A]: 0 causal, 1 bidirectional

    def __post_init__(self):
        if self.branch_kinds is None:
            fill = 1 if self.kind == "bidir" else 0
            self.branch_kinds = np.full(self.branch_anchor.shape[0], fill, dtype=np.int32)

    @property
    def kind_names(self):
        """Per-branch kind names (the oracle's form)."""
        if self.kind in ("causal", "bidir"):
            return self.kind
        return ["bidir" if k == 1 else "causal" for k in self.branch_kinds.tolist()]

    @property
    def n_main(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_branch_tok(self) -> int:
        return int(self.branch_cu[-1])

    @property
    def n_branches(self) -> int:
        return int(self.branch_anchor.shape[0])


def make_structure(w: Workload) -> Structure:
    lens = np.asarray(w.seqlens, dtype=np.int64)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    rules = w.mix if w.branch == "mixed" else ((w.branch, w.branch_len, w.anchor_stride),) * len(lens)
    assert len(rules) == len(lens)
    anchors, blens, kinds = [], [], []
    for s, L in enumerate(lens):
        fam, blen_s, stride = rules[s]
        a = cu[s] + np.arange(0, L, stride, dtype=np.int64)
        anchors.append(a)
        blens.append(np.full(a.shape[0], blen_s, dtype=np.int64))
        kinds.append(np.full(a.shape[0], 1 if fam == "dflash" else 0, dtype=np.int32))
    anchor = np.concatenate(anchors) if anchors else np.zeros(0, np.int64)
    blen = np.concatenate(blens) if blens else np.zeros(0, np.int64)
    bcu = np.zeros(anchor.shape[0] + 1, dtype=np.int64)
    bcu[1:] = np.cumsum(blen)
    assert cu[-1] < 2**31 and bcu[-1] < 2**31
    return Structure(cu.astype(np.int32), bcu.astype(np.int32), anchor.astype(np.int32),
                     w.kind, int(blen.max()) if blen.size else 1,
                     np.concatenate(kinds) if kinds else np.zeros(0, np.int32))


def make_structure_custom(seqlens, anchors_per_seq, branch_lens, kind) -> Structure:
    """Arbitrary structure for edge-case tests.

    anchors_per_seq: list (one per sequence) of anchor positions (ascending);
    branch_lens: flat list of branch lengths, one per anchor in order.
    """
    lens = np.asarray(seqlens, dtype=np.int64)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    anchor = [cu[s] + int(p) for s, ps in enumerate(anchors_per_seq) for p in ps]
    anchor = np.asarray(anchor, dtype=np.int64)
    blen = np.asarray(branch_lens, dtype=np.int64)
    assert blen.shape[0] == anchor.shape[0]
    bcu = np.zeros(anchor.shape[0] + 1, dtype=np.int64)
    bcu[1:] = np.cumsum(blen)
    if isinstance(kind, str):
        return Structure(cu.astype(np.int32), bcu.astype(np.int32), anchor.astype(np.int32),
                         kind, int(blen.max()) if blen.size else 0)
    kinds = np.asarray([1 if k == "bidir" else 0 for k in kind], dtype=np.int32)
    return Structure(cu.astype(np.int32), bcu.astype(np.int32), anchor.astype(np.int32),
                     "mixed", int(blen.max()) if blen.size else 0, kinds)


def _torch_dtype(w_dtype: str):
    import torch
    return torch.float32 if w_dtype == "f32" else torch.bfloat16


def make_tensors(w: Workload, st: Structure, device="cpu", which=None,
                 dtype: str | None = None, value_scale: float | None = None,
                 seed_base: int | None = None):
    """Return a dict of seeded tensors on ``device``.

    Keys: q [N,Hq,d], k [N,Hkv,d], v [N,Hkv,d], qb [Nb,Hq,d], kb, vb [Nb,Hkv,d],
    do [N,Hq,d], dob [Nb,Hq,d].
    """
    import torch
    dt = _torch_dtype(dtype or w.dtype)
    scale = w.value_scale if value_scale is None else value_scale
    base = w.seed_base if seed_base is None else seed_base
    N, Nb = st.n_main, st.n_branch_tok
    shapes = {
        "q": (N, w.hq, w.d), "k": (N, w.hkv, w.d), "v": (N, w.hkv, w.d),
        "qb": (Nb, w.hq, w.d), "kb": (Nb, w.hkv, w.d), "vb": (Nb, w.hkv, w.d),
        "do": (N, w.hq, w.d), "dob": (Nb, w.hq, w.d),
    }
    order = ["q", "k", "v", "qb", "kb", "vb", "do", "dob"]
    out = {}
    for i, name in enumerate(order):
        if which is not None and name not in which:
            continue
        g = torch.Generator(device=device)
        g.manual_seed(base + i + 1)
        x = torch.randn(shapes[name], generator=g, device=device, dtype=torch.float32)
        if name not in ("do", "dob") and scale != 1.0:
            x.mul_(scale)
        out[name] = x.to(dt)
        del x
    return out


class numpy_rows:
    """Row source that copies requested rows of a torch tensor to host fp64.

    The oracle indexes arrays by token; for very large workloads this avoids
    materialising whole tensors on the host.
    """

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        import torch
        if isinstance(idx, slice):
            sub = self.t[idx]
        else:
            ii = torch.as_tensor(np.asarray(idx, dtype=np.int64), device=self.t.device)
            sub = self.t.index_select(0, ii)
        return sub.to(torch.float64).cpu().numpy()
