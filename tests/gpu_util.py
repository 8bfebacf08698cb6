"""Helpers shared by the GPU parity tests: run the HIP path through the
Python binding of the C ABI, run the oracle on the same seeded inputs, and
compare.  Not collected by pytest (no test_ prefix)."""

from __future__ import annotations

import math
import sys

import numpy as np

import oracle
from oracle.problem import Problem
from workloads import make_structure, make_tensors, numpy_rows

TOL = {"bf16": dict(o=2e-2, grad=2e-2, lse=1e-3), "f32": dict(o=1e-5, grad=1e-5, lse=1e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(w, device="cuda", st=None):
    st = st or make_structure(w)
    t = make_tensors(w, st, device=device)
    return st, t


def run_path(st, t, cp=1, ranks=None, delta_from="acc"):
    """Run forward + backward of every rank in `ranks` (all by default) and
    scatter the results to global row order (torch tensors on the device)."""
    import torch
    from branch_aware_causal_amd import ring
    N, Nb = st.n_main, st.n_branch_tok
    hq, d = t["q"].shape[1], t["q"].shape[2]
    hkv = t["k"].shape[1]
    dev = t["q"].device
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(o_main_acc=torch.zeros(N, hq, d, **f32), lse_main=torch.zeros(hq, N, **f32),
               o_br_acc=torch.zeros(Nb, hq, d, **f32), lse_br=torch.zeros(hq, Nb, **f32),
               o_main=torch.zeros_like(t["q"]), o_br=torch.zeros_like(t["qb"]),
               dq_main=torch.zeros(N, hq, d, **f32), dq_br=torch.zeros(Nb, hq, d, **f32),
               dk=torch.zeros(N, hkv, d, **f32), dv=torch.zeros(N, hkv, d, **f32),
               dkb=torch.zeros(Nb, hkv, d, **f32), dvb=torch.zeros(Nb, hkv, d, **f32))
    plans = ring.plan_all(st.cu_seqlens, st.branch_cu, st.branch_anchor, cp)
    for r in (range(cp) if ranks is None else ranks):
        ri, pl = ring.rank_inputs(st, t, cp, r, plans)
        f = ring.forward(ri)
        g = ring.backward(ri, f, delta_from=delta_from)
        mi = torch.as_tensor(pl["main_index"], dtype=torch.int64, device=dev)
        bi = torch.as_tensor(pl["branch_index"], dtype=torch.int64, device=dev)
        for key, idx in (("o_main_acc", mi), ("o_main", mi), ("dq_main", mi)):
            out[key][idx] = f[key] if key in f else g[key]
        for key, idx in (("o_br_acc", bi), ("o_br", bi), ("dq_br", bi), ("dkb", bi), ("dvb", bi)):
            out[key][idx] = f[key] if key in f else g[key]
        out["lse_main"][:, mi] = f["lse_main"]
        out["lse_br"][:, bi] = f["lse_br"]
        for s, sh in enumerate(ri.shards):
            si = torch.as_tensor(plans[sh.src]["main_index"], dtype=torch.int64, device=dev)
            out["dk"].index_add_(0, si, g["dk"][s])
            out["dv"].index_add_(0, si, g["dv"][s])
    torch.cuda.synchronize()
    return out


def host64(x):
    import torch
    return x.detach().to(torch.float64).cpu().numpy()


def problem(st, t, lazy=False):
    """Oracle problem on the exact (bf16-rounded) input values."""
    hq, hkv, d = t["q"].shape[1], t["k"].shape[1], t["q"].shape[2]
    src = (lambda x: numpy_rows(x)) if lazy else host64
    return Problem(st.cu_seqlens, st.branch_cu, st.branch_anchor, st.kind_names, hq, hkv, d,
                   src(t["q"]), src(t["k"]), src(t["v"]), src(t["qb"]), src(t["kb"]), src(t["vb"]))


def maxdiff(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    fin = np.isfinite(b)
    if not np.array_equal(np.isfinite(a), fin):
        return math.inf
    if not np.array_equal(a[~fin], b[~fin]):
        return math.inf
    return float(np.max(np.abs(a[fin] - b[fin]))) if fin.any() else 0.0


def compare_full(st, t, gpu, tol, label=""):
    """Full oracle (definition mode) vs the GPU results; returns the errors."""
    prob = problem(st, t)
    N = st.n_main
    O, lse = oracle.forward(prob)
    dO = np.concatenate([host64(t["do"]), host64(t["dob"])])
    dQ, dK, dV = oracle.backward(prob, dO, fwd=(O, lse))
    err = dict(
        o_main=maxdiff(host64(gpu["o_main_acc"]), O[:N]),
        o_br=maxdiff(host64(gpu["o_br_acc"]), O[N:]),
        lse_main=maxdiff(host64(gpu["lse_main"]).T, lse[:N]),
        lse_br=maxdiff(host64(gpu["lse_br"]).T, lse[N:]),
        dq_main=maxdiff(host64(gpu["dq_main"]), dQ[:N]),
        dq_br=maxdiff(host64(gpu["dq_br"]), dQ[N:]),
        dk=maxdiff(host64(gpu["dk"]), dK[:N]),
        dv=maxdiff(host64(gpu["dv"]), dV[:N]),
        dkb=maxdiff(host64(gpu["dkb"]), dK[N:]),
        dvb=maxdiff(host64(gpu["dvb"]), dV[N:]),
    )
    say(f"[{label}] max abs err vs oracle: " + ", ".join(f"{k}={v:.2e}" for k, v in err.items()))
    for k, v in err.items():
        kind = "lse" if k.startswith("lse") else ("o" if k.startswith("o") else "grad")
        assert v <= tol[kind], (label, k, v, tol[kind])
    return err


def check_rne(gpu):
    """bf16 outputs equal round-to-nearest-even of the fp32 accumulators."""
    import torch
    for acc, out in (("o_main_acc", "o_main"), ("o_br_acc", "o_br")):
        if gpu[out].dtype == torch.bfloat16:
            assert torch.equal(gpu[acc].to(torch.bfloat16), gpu[out]), out
        else:
            assert torch.equal(gpu[acc], gpu[out]), out


def workers():
    """Host threads for the oracle: the machine's CPU share is 16 cores."""
    import os
    return max(1, min(16, os.cpu_count() or 1))


def _parallel(fn, parts):
    """fn over parts on a thread pool, one BLAS thread per worker (NumPy
    releases the GIL inside BLAS and large elementwise loops)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers()) as ex:
        return list(ex.map(fn, parts))


def par_backward_rows(prob, rows, dO_rows, heads=None, chunk=32):
    """oracle.backward_rows over row chunks in parallel: (dq, O, lse) in the
    order of ``rows``.  Rows are grouped by (sequence, position) -- a branch
    row sits at its anchor -- so a chunk's rows share most of their keys."""
    rows = np.asarray(rows, np.int64)
    _, seq, pos, _, _ = prob.describe(rows)
    order = np.lexsort((pos, seq))
    idx = [order[i:i + chunk] for i in range(0, rows.size, chunk)]
    res = _parallel(lambda ii: oracle.backward_rows(prob, rows[ii], dO_rows[ii], heads=heads), idx)
    out = []
    for j in range(3):
        cat = np.concatenate([r[j] for r in res])
        back = np.empty_like(cat)
        back[order] = cat
        out.append(back)
    return tuple(out)


def full_group_reference(prob, dO_rows_fn, group=0, block_pos=128):
    """Definition mode over the whole problem for one kv-head group: O, lse
    and dQ of every row on the group's q-heads, dK and dV of every key of
    kv-head `group`.  Blocks of positions run in parallel; dO_rows_fn(rows)
    returns dO [len(rows), Hq, d] (fp64)."""
    from oracle.attention import _blocks, delta, grads, partial
    G = prob.hq // prob.hkv
    heads = list(range(group * G, (group + 1) * G))
    n = prob.N + prob.Nb
    blocks = list(_blocks(prob, block_pos))

    import threading
    lock = threading.Lock()
    O = np.zeros((n, G, prob.d))
    lse = np.full((n, G), -np.inf)
    dQ = np.zeros((n, G, prob.d))
    dK = np.zeros((n, prob.d))
    dV = np.zeros((n, prob.d))

    def run(rk):
        rows, keys = rk
        o, l = partial(prob, rows, keys, heads)
        dO = np.zeros((rows.size, prob.hq, prob.d))
        dO[:, heads] = dO_rows_fn(rows)[:, heads]
        dq, dk, dv = grads(prob, rows, keys, l, dO, delta(o, dO), heads)
        with lock:      # a block's rows are its own; its keys recur in later blocks
            O[rows], lse[rows] = o[:, heads], l[:, heads]
            dQ[rows] += dq[:, heads]
            dK[keys] += dk[:, group]
            dV[keys] += dv[:, group]

    _parallel(run, blocks)
    return O, lse, dQ, dK, dV


def par_key_grads(prob, keys, dO_source, heads=None, rows=None, row_chunk=64):
    """oracle.key_grads with its rows split over the workers, summed."""
    from oracle.attention import rows_seeing
    keys = np.asarray(keys, np.int64)
    cand = rows_seeing(prob, keys)
    if rows is not None:
        cand = np.intersect1d(cand, np.asarray(rows, np.int64))
    n = max(1, min(workers() * 4, cand.size // row_chunk + 1))
    # interleave so every part gets early and late (short and long) rows
    parts = [cand[i::n] for i in range(n)]
    res = _parallel(lambda part: oracle.key_grads(prob, keys, dO_source, heads=heads,
                                                  row_chunk=row_chunk, rows=part), parts)
    return sum(r[0] for r in res), sum(r[1] for r in res)
