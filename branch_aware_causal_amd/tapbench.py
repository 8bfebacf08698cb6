"""Microbenchmark of the stamped-slot feature hand-off on one GPU against
staging through pinned host memory ([G] 结果分析: TapChannel against host
staging for pipeline-parallel feature fan-in).

For each payload size: the mailbox path sends from a producer stream
(tap_send: copy into a preallocated slot, then the stamp) while a consumer
stream waits for the stamp and copies the slot out (tap_recv), with no host
synchronisation between them; the staging path copies the payload to pinned
host memory and back on one stream.  Each figure is the median over the
repetitions of the time from the producer's first enqueue to the consumer's
last write (HIP events), reported as payload GB/s.

Run: python -m branch_aware_causal_amd.tapbench [--reps N] [--sizes-mib ...]
Prints one JSON line per size and a summary line.
"""

from __future__ import annotations

import argparse
import json
import statistics
import sys


def run(sizes_mib, reps):
    import torch
    from . import api
    dev = torch.device("cuda:0")
    prod, cons = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    rows = []
    for mib in sizes_mib:
        n = int(mib * (1 << 20))
        slots = torch.zeros(2, n, dtype=torch.uint8, device=dev)
        stamps = torch.zeros(2, dtype=torch.int64, device=dev)
        payload = torch.randint(0, 256, (n,), dtype=torch.int32, device=dev).to(torch.uint8)
        out = torch.empty_like(payload)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        pinned = torch.empty(n, dtype=torch.uint8, pin_memory=True)
        torch.cuda.synchronize()
        t_mail, t_host = [], []
        for rep in range(reps + 1):
            seq = rep + 1
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(prod)
            api.tap_send(slots, stamps, seq % 2, payload, seq, stream=prod)
            api.tap_recv(slots, stamps, seq % 2, seq, out, status, spin_limit=1 << 26, stream=cons)
            e1.record(cons)
            torch.cuda.synchronize()
            if int(status.item()) != 0 or not torch.equal(out, payload):
                raise RuntimeError(f"mailbox hand-off of {mib} MiB failed (status {int(status.item())})")
            if rep:
                t_mail.append(e0.elapsed_time(e1) / 1e3)
            out.zero_()
            h0 = torch.cuda.Event(enable_timing=True)
            h1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(prod):
                h0.record(prod)
                pinned.copy_(payload, non_blocking=True)
                out.copy_(pinned, non_blocking=True)
                h1.record(prod)
            torch.cuda.synchronize()
            if not torch.equal(out, payload):
                raise RuntimeError(f"host staging of {mib} MiB failed")
            if rep:
                t_host.append(h0.elapsed_time(h1) / 1e3)
            out.zero_()
        tm, th = statistics.median(t_mail), statistics.median(t_host)
        row = dict(metric="stamped-slot hand-off vs host staging", payload_mib=mib,
                   mailbox_gbs=round(n / tm / 1e9, 1), host_staging_gbs=round(n / th / 1e9, 1),
                   mailbox_ms=round(tm * 1e3, 4), host_staging_ms=round(th * 1e3, 4),
                   speedup=round(th / tm, 2), reps=reps)
        rows.append(row)
        print(json.dumps(row), flush=True)
        del slots, payload, out, pinned
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--sizes-mib", type=float, nargs="+", default=[1, 4, 16, 64, 256])
    args = ap.parse_args()
    rows = run(args.sizes_mib, args.reps)
    print(json.dumps(dict(summary="speedup of the mailbox over host staging",
                          by_size={str(r["payload_mib"]): r["speedup"] for r in rows})),
          flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
