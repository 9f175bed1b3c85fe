"""Text summaries of rocprofv3 output (the files kept under profiles/).

Kernel durations from a kernel trace:

    python -m mixture_experts_ffn_02_amd.profiling stats DIR --cmd "<profiled command>"

HBM traffic of one kernel from two counter runs (FETCH_SIZE, then WRITE_SIZE,
both in KiB per dispatch), scaled by what the same counters read for a plain
device-to-device copy of known size that ran in the same process:

    python -m mixture_experts_ffn_02_amd.profiling traffic --fetch DIR1 --write DIR2 \\
        --kernel "k_gemm<unsigned short, true, true" --copy-bytes 268435456 --cmd "..."

Both print a summary to stdout; the traffic summary carries the hash of the
kernel source it was measured on, so that stale numbers can be recognised.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_SOURCES = ["mixture_experts_ffn_02_amd/csrc/gemm.hip", "mixture_experts_ffn_02_amd/csrc/moe_api.cpp"]


def source_hash(paths=GEMM_SOURCES) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _find(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def stats(args) -> None:
    path = _find(args.dir, "kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    print(f"# rocprofv3 kernel statistics")
    print(f"# command: {args.cmd}")
    print(f"# source: {os.path.basename(path)}")
    print(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel")
    for r in rows:
        name = r["Name"].replace("moe::(anonymous namespace)::", "")
        print(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
              f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}  {name}")


def _counter(d: str, counter: str):
    path = _find(d, "counter_collection.csv")
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def traffic(args) -> None:
    fetch = _counter(args.fetch, "FETCH_SIZE")
    write = _counter(args.write, "WRITE_SIZE")

    def pick(table, key):
        vals = [v for k, vs in table.items() if key in k for v in vs]
        if not vals:
            raise SystemExit(f"kernel matching {key!r} not found")
        return statistics.mean(vals), len(vals)

    copy_kib = args.copy_bytes / 1024.0
    cf, _ = pick(fetch, args.copy_kernel)
    cw, _ = pick(write, args.copy_kernel)
    kf, n = pick(fetch, args.kernel)
    kw, _ = pick(write, args.kernel)
    sf, sw = copy_kib / cf, copy_kib / cw
    total = (kf * sf + kw * sw) * 1024.0
    print("# HBM traffic of one kernel from rocprofv3 counters")
    print(f"# command (FETCH_SIZE run): {args.cmd.replace('COUNTER', 'FETCH_SIZE')}")
    print(f"# command (WRITE_SIZE run): {args.cmd.replace('COUNTER', 'WRITE_SIZE')}")
    print(f"kernel: {args.kernel}")
    print(f"dispatches: {n}")
    print(f"fetch_kib_per_dispatch: {kf:.1f}")
    print(f"write_kib_per_dispatch: {kw:.1f}")
    print(f"copy_bytes: {args.copy_bytes}")
    print(f"copy_fetch_kib: {cf:.1f}")
    print(f"copy_write_kib: {cw:.1f}")
    print(f"fetch_scale: {sf:.4f}")
    print(f"write_scale: {sw:.4f}")
    print(f"hbm_bytes_per_launch: {total:.0f}")
    if args.rdreq:
        rq = _counter(args.rdreq, "TCC_EA0_RDREQ_128B_sum")
        r6 = _counter(args.rdreq, "TCC_EA0_RDREQ_64B_sum")
        k128, _ = pick(rq, args.kernel)
        k64, _ = pick(r6, args.kernel)
        c128, _ = pick(rq, args.copy_kernel)
        c64, _ = pick(r6, args.copy_kernel)
        print(f"# cross-check: EA read requests by size (128 B and 64 B); command: "
              f"{args.cmd.replace('COUNTER', 'TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum')}")
        print(f"rdreq_bytes_per_dispatch: {128 * k128 + 64 * k64:.0f}")
        print(f"copy_rdreq_bytes: {128 * c128 + 64 * c64:.0f}")
    print(f"source_sha256: {source_hash()}")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("--cmd", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", required=True)
    b.add_argument("--copy-kernel", default="vectorized_elementwise_kernel")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--rdreq", default=None, help="optional run with TCC_EA0_RDREQ_{128B,64B}_sum")
    b.add_argument("--cmd", required=True)
    args = ap.parse_args(argv)
    {"stats": stats, "traffic": traffic}[args.what](args)


if __name__ == "__main__":
    main(sys.argv[1:])
