#!/usr/bin/env python3
"""Benchmark of merged branch + causal attention, forward + backward, on one
MI355X (gfx950).

One step is one pass of the whole hot path over one batch of synthetic
input: the zigzag shard plan (host), upload of its index arrays, the main
attention of the main rows and of the branch rows (positioned at their
anchors) over every K/V shard with the online-softmax merge fused, the
rank-local branch attention with the final merge and bf16 rounding, Delta,
the main backward (dQ and dK/dV kernels) and the branch backward.  Inputs
are resident in HBM before the timed region.

Default workload: one 262,144-token sequence, EAGLE-3 TTT depth 3 at every
position, Hq=32, Hkv=8, d=128, bf16, CP=1 (the 256K-token test of [R]
"长上下文才是系统设计的主场").  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 bf16 FLOP/clk x 2.4 GHz, dense (AMD: 2.5 PF)
PEAK_HBM_GBS = 8000.0
METRIC = "merged branch+causal attention fwd+bwd TFLOP/s and % bf16 MFMA peak at 256K"
KERNEL_SOURCES = {
    "main_fwd": "branch_aware_causal_amd/csrc/mfma_fwd.hip",
    "main_bwd_dq": "branch_aware_causal_amd/csrc/mfma_bwd.hip",
    "main_bwd_dkdv": "branch_aware_causal_amd/csrc/mfma_bwd.hip",
}
KERNEL_NAMES = {
    "main_fwd": "main_fwd_mfma_kernel",
    "main_bwd_dq": "main_bwd_dq_kernel",
    "main_bwd_dkdv": "main_bwd_dkdv_kernel",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# headers the MFMA kernel sources include (a change in any of them changes the kernels)
KERNEL_HEADERS = ["branch_aware_causal_amd/csrc/mfma_common.hpp",
                  "branch_aware_causal_amd/csrc/device_common.hpp",
                  "branch_aware_causal_amd/csrc/launch.hpp"]


def source_sha(rel):
    h = hashlib.sha256()
    for p in [rel] + KERNEL_HEADERS:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Timer:
    """HIP events around each library call on the working stream."""

    def __init__(self, torch, stream, enabled=True):
        self.torch, self.stream, self.enabled = torch, stream, enabled
        self.pending = []
        self.total = {}
        self.count = {}
        self.work = {}
        self.bytes = {}

    def __call__(self, name, work, fn, *args, nbytes=0, **kw):
        if not self.enabled:
            return fn(*args, **kw)
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        fn(*args, **kw)
        b.record(self.stream)
        self.pending.append((name, work, nbytes, a, b))

    def collect(self):
        for name, work, nbytes, a, b in self.pending:
            self.total[name] = self.total.get(name, 0.0) + a.elapsed_time(b) / 1e3
            self.count[name] = self.count.get(name, 0) + 1
            self.work[name] = self.work.get(name, 0.0) + work
            self.bytes[name] = self.bytes.get(name, 0.0) + nbytes
        self.pending = []


def pairs_rows_keys(row_seq, row_pos, key_seq, key_pos):
    """Visible (row, key) pairs per head: keys of the row's sequence with
    pos <= the row's pos (keys sorted by (seq, pos))."""
    rk = np.asarray(row_seq, np.int64) * (1 << 32) + np.asarray(row_pos, np.int64)
    kk = np.asarray(key_seq, np.int64) * (1 << 32) + np.asarray(key_pos, np.int64)
    hi = np.searchsorted(kk, rk, side="right")
    lo = np.searchsorted(kk, np.asarray(row_seq, np.int64) * (1 << 32), side="left")
    return int(np.sum(hi - lo))


def build_step(torch, api, ring, w, st, t, dev, timer):
    """Return (step_fn, work) for the workload; work holds algorithmic FLOPs
    per launch class and totals."""
    from branch_aware_causal_amd import flops as flops_mod
    hq, hkv, d = w.hq, w.hkv, w.d
    C, r = w.cp, w.rank
    plans = ring.plan_all(st.cu_seqlens, st.branch_cu, st.branch_anchor, C)
    pl = plans[r]
    # resident inputs of this rank: its rows and the K/V shards of every ring step
    ri, _ = ring.rank_inputs(st, t, C, r, plans)
    nm, nb = ri.q_main.shape[0], ri.q_br.shape[0]
    f32 = dict(dtype=torch.float32, device=dev)
    bufs = dict(o_main_acc=torch.empty(nm, hq, d, **f32), lse_main=torch.empty(hq, nm, **f32),
                o_br_acc=torch.empty(nb, hq, d, **f32), lse_br=torch.empty(hq, nb, **f32),
                o_main=torch.empty_like(ri.q_main), o_br=torch.empty_like(ri.q_br),
                dq_main=torch.empty(nm, hq, d, **f32), dq_br=torch.empty(nb, hq, d, **f32),
                dk=[torch.empty(sh.k.shape[0], hkv, d, **f32) for sh in ri.shards],
                dv=[torch.empty(sh.k.shape[0], hkv, d, **f32) for sh in ri.shards],
                dkb=torch.empty(nb, hkv, d, **f32), dvb=torch.empty(nb, hkv, d, **f32),
                delta_main=torch.empty(hq, nm, **f32), delta_br=torch.empty(hq, nb, **f32))
    # algorithmic work per launch
    per_shard = []
    for s, sh in enumerate(ri.shards):
        ps = plans[sh.src]
        pm = pairs_rows_keys(pl["main_seq"], pl["main_pos"], ps["main_seq"], ps["main_pos"])
        pb = pairs_rows_keys(pl["branch_seq"], pl["branch_pos"], ps["main_seq"], ps["main_pos"])
        per_shard.append((pm, pb))
    local = flops_mod.pair_counts_rows([], [], pl["branch_t"], pl["local_branch_cu"], st.kind,
                                       st.branch_kinds[pl["branch_ids"]])[2]
    main_pairs = sum(a + b for a, b in per_shard)
    total_pairs = main_pairs + local
    kb_branch = 2 * 2 * nb * hkv * d * 2   # branch fwd bytes are reported, not priced
    work = dict(pairs=total_pairs, local_pairs=local, flops=total_pairs * hq * 14 * d,
                fwd_flops=total_pairs * hq * 4 * d, bwd_flops=total_pairs * hq * 10 * d)
    # algorithmic HBM bytes of the bandwidth-bound launches (each tensor element
    # read or written once; the merge into the accumulators and the bf16 output
    # are fused into the branch forward)
    qrow, krow = hq * d, hkv * d
    bytes_branch_fwd = nb * (2 * qrow + 2 * 2 * krow + 2 * 4 * qrow + 2 * 4 * hq + 2 * qrow)
    bytes_branch_bwd = nb * (2 * 2 * qrow + 2 * 2 * krow + 2 * 4 * hq + 2 * 4 * qrow + 2 * 2 * 4 * krow)
    bytes_delta = lambda n: n * (4 * qrow + 2 * qrow + 4 * hq)
    work["bytes"] = dict(branch_fwd=bytes_branch_fwd, branch_bwd=bytes_branch_bwd,
                         delta=bytes_delta(nm) + bytes_delta(nb))
    i32 = lambda a: torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32))
    cu, bcu, anc = st.cu_seqlens, st.branch_cu, st.branch_anchor

    def step():
        # (a1, a2) plan and index arrays: host integer work, uploaded each step
        p = api.zigzag_shard_plan(cu, bcu, anc, C, r)
        seq_m = i32(p["main_seq"]).to(dev, non_blocking=True)
        pos_m = i32(p["main_pos"]).to(dev, non_blocking=True)
        seq_b = i32(p["branch_seq"]).to(dev, non_blocking=True)
        pos_b = i32(p["branch_pos"]).to(dev, non_blocking=True)
        lbcu = i32(p["local_branch_cu"]).to(dev, non_blocking=True)
        kinds = (i32(st.branch_kinds[p["branch_ids"]]).to(dev, non_blocking=True)
                 if st.kind == "mixed" else None)
        kidx = []
        for sh in ri.shards:
            if C == 1:
                kidx.append((seq_m, pos_m))
            else:
                ps = api.zigzag_shard_plan(cu, bcu, anc, C, sh.src)
                kidx.append((i32(ps["main_seq"]).to(dev, non_blocking=True),
                             i32(ps["main_pos"]).to(dev, non_blocking=True)))
        # (a3, a4) main part, merged after every ring step
        for s, sh in enumerate(ri.shards):
            ks, kp = kidx[s]
            mode = api.WRITE if s == 0 else api.MERGE
            pm, pb = per_shard[s]
            timer("main_fwd", pm * hq * 4 * d, api.attn_main_fwd, ri.q_main, seq_m, pos_m, sh.k,
                  sh.v, ks, kp, bufs["o_main_acc"], bufs["lse_main"], mode,
                  o_out=bufs["o_main"] if s == C - 1 else None)
            timer("main_fwd", pb * hq * 4 * d, api.attn_main_fwd, ri.q_br, seq_b, pos_b, sh.k,
                  sh.v, ks, kp, bufs["o_br_acc"], bufs["lse_br"], mode)
        # (a5, a6) rank-local branch part, final merge and bf16 rounding
        timer("branch_fwd", local * hq * 4 * d, api.attn_branch_fwd, ri.q_br, ri.kb, ri.vb, lbcu,
              ri.max_branch_len, ri.kind, bufs["o_br_acc"], bufs["lse_br"], api.MERGE,
              o_out=bufs["o_br"], nbytes=bytes_branch_fwd, branch_kinds=kinds)
        # (a7) Delta
        timer("delta", 0, api.attn_bwd_delta, bufs["o_main_acc"], ri.do_main, bufs["delta_main"],
              nbytes=bytes_delta(nm))
        timer("delta", 0, api.attn_bwd_delta, bufs["o_br_acc"], ri.do_br, bufs["delta_br"],
              nbytes=bytes_delta(nb))
        for key in ("dq_main", "dq_br", "dkb", "dvb"):
            bufs[key].zero_()
        for s in range(C):
            bufs["dk"][s].zero_()
            bufs["dv"][s].zero_()
        # (a8, a10) main backward per ring step; dK/dV partials per shard
        for s, sh in enumerate(ri.shards):
            ks, kp = kidx[s]
            pm, pb = per_shard[s]
            for q, qs, qp, do, lse, dl, dq, pr in (
                    (ri.q_main, seq_m, pos_m, ri.do_main, bufs["lse_main"], bufs["delta_main"],
                     bufs["dq_main"], pm),
                    (ri.q_br, seq_b, pos_b, ri.do_br, bufs["lse_br"], bufs["delta_br"],
                     bufs["dq_br"], pb)):
                timer("main_bwd_dq", pr * hq * 2 * d, api.attn_main_bwd_dq, q, qs, qp, sh.k, sh.v,
                      ks, kp, do, lse, dl, dq)
                timer("main_bwd_dkdv", pr * hq * 8 * d, api.attn_main_bwd_dkdv, q, qs, qp, sh.k,
                      sh.v, ks, kp, do, lse, dl, bufs["dk"][s], bufs["dv"][s])
        # (a9) branch backward
        timer("branch_bwd", local * hq * 10 * d, api.attn_branch_bwd, ri.q_br, ri.kb, ri.vb, lbcu,
              ri.max_branch_len, ri.kind, ri.do_br, bufs["lse_br"], bufs["delta_br"],
              bufs["dq_br"], bufs["dkb"], bufs["dvb"], nbytes=bytes_branch_bwd,
              branch_kinds=kinds)

    return step, work, ri, pl, bufs


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/<kernel>_<workload>.md: FETCH_SIZE and WRITE_SIZE passes scaled by
    a plain-copy calibration), only while the kernel source is the profiled one."""
    path = os.path.join(ROOT, "profiles", f"{KERNEL_NAMES[kernel]}_{workload}.md")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, st, t, n_anchor, log_fn, full_flops):
    """The oracle, timed on the host on the rows of the last n_anchor anchors
    (their main rows and every token of their branches), each row over its full
    visible key set, all heads: O, lse and the gradients of the block."""
    import torch
    import oracle
    from oracle.problem import Problem
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:  # threadpoolctl missing
        cores = os.cpu_count()
    N = st.n_main
    a_hi = st.n_branches
    anchors = np.arange(a_hi - n_anchor, a_hi)
    main_rows = st.branch_anchor[anchors].astype(np.int64)
    br_tok = np.concatenate([np.arange(st.branch_cu[a], st.branch_cu[a + 1]) for a in anchors])
    rows = np.concatenate([main_rows, N + br_tok])

    class Sparse:
        """Row source holding only the sampled rows (host fp32, exact bf16 values)."""

        def __init__(self, src, ids):
            ids = np.asarray(ids, np.int64)
            self.map = {int(i): j for j, i in enumerate(ids)}
            ii = torch.as_tensor(ids, device=src.device)
            self.data = src.index_select(0, ii).float().cpu().numpy()

        def __getitem__(self, idx):
            return self.data[[self.map[int(i)] for i in np.asarray(idx).ravel()]]

    k = t["k"].float().cpu().numpy()
    v = t["v"].float().cpu().numpy()
    prob = Problem(st.cu_seqlens, st.branch_cu, st.branch_anchor, st.kind_names, w.hq, w.hkv, w.d,
                   Sparse(t["q"], main_rows), k, v, Sparse(t["qb"], br_tok), Sparse(t["kb"], br_tok),
                   Sparse(t["vb"], br_tok))
    dO = np.concatenate([t["do"].index_select(0, torch.as_tensor(main_rows, device=t["do"].device))
                         .double().cpu().numpy(),
                         t["dob"].index_select(0, torch.as_tensor(br_tok, device=t["dob"].device))
                         .double().cpu().numpy()])
    vis = prob.visibility(rows, prob.visible_keys(rows))
    pairs = int(vis.sum()) * w.hq
    del vis
    t0 = time.perf_counter()
    oracle.backward_rows(prob, rows, dO)
    dt = time.perf_counter() - t0
    flop = pairs * 14 * w.d
    rate = flop / dt
    log_fn(f"cpu_baseline: {rows.size} rows, {pairs:,} (row, key, head) triples, {dt:.1f} s; "
           f"whole step extrapolated at this rate: {full_flops / rate / 3600:.1f} h")
    return dict(value=rate / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                extrapolated_full_step_s=round(full_flops / rate, 1),
                extrapolated_note=("EXTRAPOLATED, not measured: the whole step's algorithmic "
                                   "FLOP divided by the sampled oracle rate"),
                sample=(f"fp64 NumPy oracle, fwd+bwd (O, lse, dQ and the block's dK/dV) of the "
                        f"rows of the last {n_anchor} anchors of the {w.name} workload "
                        f"({main_rows.size} main + {br_tok.size} branch rows over ~{N:,} keys, "
                        f"all {w.hq} heads), {dt:.1f} s; 14d FLOP per visible (row, key, head)"))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="eagle3_256k")
    ap.add_argument("--cpu-anchors", type=int, default=16,
                    help="anchors whose rows the CPU oracle processes for cpu_baseline (0: skip)")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run a plain device copy of this many GiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the ring is emulated on one device); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from branch_aware_causal_amd import api, ring
    from workloads import WORKLOADS, make_structure, make_tensors

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    st = make_structure(w)
    log(f"workload {w.name}: seqs={len(w.seqlens)} N={st.n_main} branches={st.n_branches} "
        f"branch tokens={st.n_branch_tok} hq={w.hq} hkv={w.hkv} d={w.d} cp={w.cp} rank={w.rank}")
    t = make_tensors(w, st, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream, enabled=False)
    step, work, ri, pl, bufs = build_step(torch, api, ring, w, st, t, dev, timer)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i} done")

    timer.enabled = True
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timer.collect()
    ms = elapsed / max(args.steps, 1) * 1e3
    value = work["flops"] * args.steps / elapsed / 1e12
    log(f"{args.steps} steps in {elapsed:.3f} s: {ms:.1f} ms/step, {value:.1f} TFLOP/s")

    kernels = {}
    for name, tot in sorted(timer.total.items(), key=lambda kv: -kv[1]):
        n = timer.count[name]
        entry = dict(ms_total=round(tot / args.steps * 1e3, 3), launches=n // max(args.steps, 1),
                     avg_ms=round(tot / n * 1e3, 4))
        if timer.work[name] > 0:
            entry["tflops"] = round(timer.work[name] / tot / 1e12, 1)
        if timer.bytes.get(name, 0) > 0:
            gbs = timer.bytes[name] / tot / 1e9
            entry.update(hbm_gbs=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4),
                         bytes_per_launch=int(timer.bytes[name] / n))
        kernels[name] = entry
        log(f"  {name:14s} {entry}")
    mfma = {k: v for k, v in timer.total.items() if k in KERNEL_SOURCES}
    dom = max(mfma, key=mfma.get)
    n_launch = timer.count[dom]
    flops_per_launch = timer.work[dom] / n_launch
    avg_s = timer.total[dom] / n_launch
    achieved = flops_per_launch / avg_s / 1e12
    traffic = traffic_for(dom, w.name)
    roofline = dict(bound="mfma", kernel=KERNEL_NAMES[dom], achieved=round(achieved, 1),
                    peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4),
                    traffic=traffic, avg_launch_ms=round(avg_s * 1e3, 3),
                    algorithmic_tflop_per_launch=round(flops_per_launch / 1e12, 4))

    if args.calib_copy_gib > 0:
        nbytes = int(args.calib_copy_gib * (1 << 30))
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"calibration copy of {nbytes} bytes done")
        del a, b

    # the standalone online-softmax merge (fused into every forward epilogue of
    # the step above), timed on the branch rows' fp32 accumulators: two fp32
    # O and two lse read, one O and one lse written per (row, head)
    nb = bufs["o_br_acc"].shape[0]
    o_part = torch.zeros_like(bufs["o_br_acc"])
    lse_part = torch.zeros_like(bufs["lse_br"])
    merge_ms = []
    for rep in range(4):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        api.lse_merge(bufs["o_br_acc"], bufs["lse_br"], o_part, lse_part)
        ev1.record(stream)
        torch.cuda.synchronize()
        if rep > 0:
            merge_ms.append(ev0.elapsed_time(ev1))
    del o_part, lse_part
    merge_bytes = nb * w.hq * (3 * 4 * w.d + 3 * 4)
    merge_s = float(np.median(merge_ms)) / 1e3
    kernels["lse_merge_standalone"] = dict(
        avg_ms=round(merge_s * 1e3, 4), rows=nb, heads=w.hq, bytes_per_launch=merge_bytes,
        hbm_gbs=round(merge_bytes / merge_s / 1e9, 1),
        hbm_frac=round(merge_bytes / merge_s / 1e9 / PEAK_HBM_GBS, 4))
    log(f"  lse_merge (standalone, {nb} rows x {w.hq} heads) {kernels['lse_merge_standalone']}")

    cpu = None
    if args.cpu_anchors > 0:
        try:
            cpu = cpu_baseline(w, st, t, args.cpu_anchors, log, work["flops"])
        except Exception as e:  # report, keep the GPU result
            log(f"cpu_baseline failed: {e!r}")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 2),
        "higher_is_better": True, "scaling": "strong", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "seq_lens": list(w.seqlens)[:8], "tokens": st.n_main,
                   "branch": f"{w.branch} length {w.branch_len} every {w.anchor_stride}",
                   "branch_tokens": st.n_branch_tok, "hq": w.hq, "hkv": w.hkv, "d": w.d,
                   "cp": w.cp, "rank": w.rank, "visible_pairs_per_head": work["pairs"],
                   "algorithmic_tflop_per_step": round(work["flops"] / 1e12, 2)},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
