"""One rank's share of branch-aware zigzag ring attention, driven over the C ABI.

[G] 方法详解 · CP计算: branch queries stay on their rank while the main K/V
makes C ring steps; after each step the partial result is merged into the
running (O, lse) with the online-softmax merge, and the rank-local branch
part is merged last.  On one GPU the shards that a real ring would receive
are resident buffers; this module only sequences the library calls.

Backward (pages silent; plain ring reading): Delta once per row, then per
ring step the main-part gradients -- dQ accumulates locally, the shard's
dK/dV partial goes into that shard's accumulator (the return trip of a real
ring) -- and finally the local branch gradients.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from . import api


@dataclass
class Shard:
    """Main K/V of one ring step, with the (seq, pos) of each key."""
    k: object
    v: object
    seq: object
    pos: object
    src: int = 0


@dataclass
class RankInputs:
    q_main: object
    seq_main: object
    pos_main: object
    q_br: object
    seq_br: object            # anchor's sequence
    pos_br: object            # anchor's position
    kb: object
    vb: object
    branch_cu: object         # device int32 [n_local_branches + 1]
    max_branch_len: int
    kind: str                 # "causal", "bidir", or "mixed" (per-branch kinds below)
    branch_kinds: object = None   # device int32 [n_local_branches] when mixed
    shards: List[Shard] = field(default_factory=list)
    do_main: object = None
    do_br: object = None


def _empty_like_rows(torch, n, hq, d, device):
    return (torch.empty((n, hq, d), dtype=torch.float32, device=device),
            torch.empty((hq, n), dtype=torch.float32, device=device))


def forward(ri: RankInputs, scale=None, stream=None, out=None):
    """Merged forward of the rank's main and branch rows.

    Returns dict: o_main_acc, lse_main, o_br_acc, lse_br (fp32) and o_main,
    o_br (input dtype, rounded from the merged accumulators)."""
    import torch
    hq, d = ri.q_main.shape[1], ri.q_main.shape[2]
    dev = ri.q_main.device
    nm, nb = ri.q_main.shape[0], ri.q_br.shape[0]
    if out is None:
        o_m, l_m = _empty_like_rows(torch, nm, hq, d, dev)
        o_b, l_b = _empty_like_rows(torch, nb, hq, d, dev)
        out = dict(o_main_acc=o_m, lse_main=l_m, o_br_acc=o_b, lse_br=l_b,
                   o_main=torch.empty_like(ri.q_main), o_br=torch.empty_like(ri.q_br))
    C = len(ri.shards)
    for s, sh in enumerate(ri.shards):
        mode = api.WRITE if s == 0 else api.MERGE
        last = s == C - 1
        api.attn_main_fwd(ri.q_main, ri.seq_main, ri.pos_main, sh.k, sh.v, sh.seq, sh.pos,
                          out["o_main_acc"], out["lse_main"], mode,
                          o_out=out["o_main"] if last else None, scale=scale, stream=stream)
        api.attn_main_fwd(ri.q_br, ri.seq_br, ri.pos_br, sh.k, sh.v, sh.seq, sh.pos,
                          out["o_br_acc"], out["lse_br"], mode, scale=scale, stream=stream)
    api.attn_branch_fwd(ri.q_br, ri.kb, ri.vb, ri.branch_cu, ri.max_branch_len, ri.kind,
                        out["o_br_acc"], out["lse_br"], api.MERGE if C > 0 else api.WRITE,
                        o_out=out["o_br"], scale=scale, stream=stream,
                        branch_kinds=ri.branch_kinds)
    return out


def backward(ri: RankInputs, fwd, scale=None, stream=None, grads=None, delta_from="acc"):
    """Gradients of the rank's rows.  Returns dict: dq_main, dq_br (fp32),
    dk/dv (lists, one fp32 accumulator per ring step's shard) and dkb, dvb."""
    import torch
    hq, d = ri.q_main.shape[1], ri.q_main.shape[2]
    hkv = ri.kb.shape[1]
    dev = ri.q_main.device
    nm, nb = ri.q_main.shape[0], ri.q_br.shape[0]
    if grads is None:
        z = lambda *s: torch.zeros(s, dtype=torch.float32, device=dev)
        grads = dict(dq_main=z(nm, hq, d), dq_br=z(nb, hq, d),
                     dk=[z(sh.k.shape[0], hkv, d) for sh in ri.shards],
                     dv=[z(sh.k.shape[0], hkv, d) for sh in ri.shards],
                     dkb=z(nb, hkv, d), dvb=z(nb, hkv, d),
                     delta_main=torch.empty((hq, nm), dtype=torch.float32, device=dev),
                     delta_br=torch.empty((hq, nb), dtype=torch.float32, device=dev))
    om = fwd["o_main_acc"] if delta_from == "acc" else fwd["o_main"]
    ob = fwd["o_br_acc"] if delta_from == "acc" else fwd["o_br"]
    api.attn_bwd_delta(om, ri.do_main, grads["delta_main"], stream=stream)
    api.attn_bwd_delta(ob, ri.do_br, grads["delta_br"], stream=stream)
    for s, sh in enumerate(ri.shards):
        api.attn_main_bwd(ri.q_main, ri.seq_main, ri.pos_main, sh.k, sh.v, sh.seq, sh.pos,
                          ri.do_main, fwd["lse_main"], grads["delta_main"], grads["dq_main"],
                          grads["dk"][s], grads["dv"][s], scale=scale, stream=stream)
        api.attn_main_bwd(ri.q_br, ri.seq_br, ri.pos_br, sh.k, sh.v, sh.seq, sh.pos,
                          ri.do_br, fwd["lse_br"], grads["delta_br"], grads["dq_br"],
                          grads["dk"][s], grads["dv"][s], scale=scale, stream=stream)
    api.attn_branch_bwd(ri.q_br, ri.kb, ri.vb, ri.branch_cu, ri.max_branch_len, ri.kind,
                        ri.do_br, fwd["lse_br"], grads["delta_br"], grads["dq_br"], grads["dkb"],
                        grads["dvb"], scale=scale, stream=stream, branch_kinds=ri.branch_kinds)
    return grads


def plan_all(cu_seqlens, branch_cu, branch_anchor, cp_size):
    return [api.zigzag_shard_plan(cu_seqlens, branch_cu, branch_anchor, cp_size, r)
            for r in range(cp_size)]


def rank_inputs(struct, tensors, cp_size: int, rank: int, plans=None, device=None):
    """Gather rank `rank`'s rows and its ring-ordered K/V shards from packed
    global tensors (set-up, outside any timed region).  With cp_size == 1 the
    global tensors are used as they are."""
    import torch
    dev = device or tensors["q"].device
    if plans is None:
        plans = plan_all(struct.cu_seqlens, struct.branch_cu, struct.branch_anchor, cp_size)
    pl = plans[rank]
    i32 = lambda a: torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=dev)
    full = cp_size == 1

    def rows(t, idx):
        if full:
            return t
        return t.index_select(0, torch.as_tensor(idx, dtype=torch.int64, device=t.device)).contiguous()

    shards = []
    for s in range(cp_size):
        src = int(pl["kv_src"][s])
        ps = plans[src]
        shards.append(Shard(k=rows(tensors["k"], ps["main_index"]),
                            v=rows(tensors["v"], ps["main_index"]),
                            seq=i32(ps["main_seq"]), pos=i32(ps["main_pos"]), src=src))
    ri = RankInputs(
        q_main=rows(tensors["q"], pl["main_index"]), seq_main=i32(pl["main_seq"]),
        pos_main=i32(pl["main_pos"]),
        q_br=rows(tensors["qb"], pl["branch_index"]), seq_br=i32(pl["branch_seq"]),
        pos_br=i32(pl["branch_pos"]),
        kb=rows(tensors["kb"], pl["branch_index"]), vb=rows(tensors["vb"], pl["branch_index"]),
        branch_cu=i32(pl["local_branch_cu"]), max_branch_len=int(struct.max_branch_len),
        kind=struct.kind, shards=shards,
        branch_kinds=(i32(np.asarray(struct.branch_kinds)[pl["branch_ids"]])
                      if struct.kind == "mixed" else None),
        do_main=rows(tensors["do"], pl["main_index"]) if "do" in tensors else None,
        do_br=rows(tensors["dob"], pl["branch_index"]) if "dob" in tensors else None)
    return ri, pl
