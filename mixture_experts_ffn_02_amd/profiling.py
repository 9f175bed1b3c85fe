"""Text summaries of rocprofv3 output (the files kept under profiles/).

Kernel durations from a kernel trace:

    python -m mixture_experts_ffn_02_amd.profiling stats DIR --cmd "<profiled command>"

HBM traffic of one kernel from two counter runs (FETCH_SIZE, then WRITE_SIZE,
both in KiB per dispatch), scaled by what the same counters read for a plain
device-to-device copy of known size that ran in the same process:

    python -m mixture_experts_ffn_02_amd.profiling traffic --fetch DIR1 --write DIR2 \\
        --kernel "k_gemm8<true, true" --copy-bytes 268435456 --cmd "..."

Matrix-core use of the GEMM launches from one counter run (SQ_VALU_MFMA_BUSY_CYCLES,
SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE):

    python -m mixture_experts_ffn_02_amd.profiling mfma DIR --cmd "..."

Each prints a summary to stdout; the traffic summary carries the hash of the
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
# the GEMM kernels and the host code that picks their tiles (gemm_bm and the
# launchers live in these files)
GEMM_SOURCES = ["mixture_experts_ffn_02_amd/csrc/gemm.hip", "mixture_experts_ffn_02_amd/csrc/gemm8.hip"]


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

    def pick(table, key, large=False):
        vals = [v for k, vs in table.items() if key in k for v in vs]
        if not vals:
            raise SystemExit(f"kernel matching {key!r} not found")
        if large:  # the dispatches of the kind that moves data (see --large)
            vals = [v for v in vals if v >= 0.5 * max(vals)]
        return statistics.mean(vals), len(vals)

    copy_kib = args.copy_bytes / 1024.0
    cf, _ = pick(fetch, args.copy_kernel)
    cw, _ = pick(write, args.copy_kernel)
    kf, n = pick(fetch, args.kernel, args.large)
    kw, _ = pick(write, args.kernel, args.large)
    sf, sw = copy_kib / cf, copy_kib / cw
    total = (kf * sf + kw * sw) * 1024.0
    print("# HBM traffic of one kernel from rocprofv3 counters (bytes that leave L2 for memory)")
    print(f"# command (FETCH_SIZE run): {args.cmd.replace('COUNTER', 'FETCH_SIZE')}")
    print(f"# command (WRITE_SIZE run): {args.cmd.replace('COUNTER', 'WRITE_SIZE')}")
    print("# scale: the counters of a plain elementwise copy (torch.mul by 1.0, 16 bytes per lane) of copy_bytes")
    print("# run in the same process")
    if args.note:
        print(f"# {args.note}")
    print(f"kernel: {args.kernel}")
    print(f"dispatches: {n}")
    print(f"fetch_kib_per_dispatch: {kf:.1f}")
    print(f"write_kib_per_dispatch: {kw:.1f}")
    print(f"copy_bytes: {args.copy_bytes}")
    print(f"copy_fetch_kib: {cf:.1f}")
    print(f"copy_write_kib: {cw:.1f}")
    print(f"fetch_scale: {sf:.4f}")
    print(f"write_scale: {sw:.4f}")
    print(f"read_bytes_per_launch: {kf * sf * 1024.0:.0f}")
    print(f"write_bytes_per_launch: {kw * sw * 1024.0:.0f}")
    print(f"hbm_bytes_per_launch: {total:.0f}")
    if args.algorithmic:
        print(f"algorithmic_bytes_per_launch: {args.algorithmic:.0f}")
        print(f"traffic_over_algorithmic: {total / args.algorithmic:.3f}")
    if args.rdreq:
        rq = _counter(args.rdreq, "TCC_EA0_RDREQ_128B_sum")
        r6 = _counter(args.rdreq, "TCC_EA0_RDREQ_64B_sum")
        r3 = _counter(args.rdreq, "TCC_EA0_RDREQ_32B_sum")
        k128, _ = pick(rq, args.kernel, args.large)
        k64, _ = pick(r6, args.kernel, args.large)
        k32, _ = pick(r3, args.kernel, args.large)
        c128, _ = pick(rq, args.copy_kernel)
        c64, _ = pick(r6, args.copy_kernel)
        c32, _ = pick(r3, args.copy_kernel)
        rq_cmd = args.cmd.replace("--pmc COUNTER", "--pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum "
                                  "TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum").replace("COUNTER", "TCC_EA0_RDREQ")
        kb = 128 * k128 + 64 * k64 + 32 * k32
        cb = 128 * c128 + 64 * c64 + 32 * c32
        print(f"# cross-check: read requests to memory by size (32, 64 and 128 bytes); command: "
              f"{rq_cmd}")
        print(f"rdreq_bytes_per_dispatch: {kb:.0f}")
        print(f"copy_rdreq_bytes: {cb:.0f}")
        print(f"rdreq_over_scaled_fetch: {kb / (kf * sf * 1024.0):.4f}")
    srcs = [os.path.join("mixture_experts_ffn_02_amd/csrc", f) for f in args.sources] if args.sources else GEMM_SOURCES
    print(f"sources: {' '.join(os.path.basename(f) for f in srcs)}")
    print(f"source_sha256: {source_hash(srcs)}")


def _durations(d: str):
    """Kernel durations (ns) per dispatch from a counter run's timestamps."""
    path = _find(d, "counter_collection.csv")
    out, seen = {}, set()
    for r in csv.DictReader(open(path)):
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        if key in seen:
            continue
        seen.add(key)
        out.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def mfma(args) -> None:
    """Matrix-core use of every launch of the kernels matching --kernel:
    SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs) over the cycles of the
    launch (GRBM_GUI_ACTIVE, summed over the XCDs, so divided by their count)
    times the SIMD count; the clock those cycles imply over the dispatch's
    duration; and the bf16 MFMA work (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts
    units of 512 flops)."""
    busy = _counter(args.dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    mops = _counter(args.dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    gui = _counter(args.dir, "GRBM_GUI_ACTIVE")
    dur = _durations(args.dir)
    print("# matrix-core use from rocprofv3 counters")
    print(f"# command: {args.cmd}")
    print(f"# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {args.xcds} * {args.simds}); "
          f"clock = GRBM_GUI_ACTIVE / {args.xcds} / duration; flops = 512 * SQ_INSTS_VALU_MFMA_MOPS_BF16; "
          f"pf_at_clock = the bf16 MFMA rate the clock allows (2.5 PFLOP/s at 2.4 GHz)")
    print(f"{'launches':>8} {'mfma_busy':>9} {'clock_ghz':>9} {'pf_at_clock':>11} {'gflop':>10} {'avg_us':>10}  kernel")
    for name in busy:
        if not any(k in name for k in args.kernel):
            continue
        b = statistics.mean(busy[name])
        m = statistics.mean(mops.get(name, [0.0]))
        g = statistics.mean(gui.get(name, [0.0])) / args.xcds
        us = statistics.mean(dur.get(name, [0])) / 1e3
        util = b / (g * args.simds) if g else 0.0
        ghz = g / (us * 1e3) if us else 0.0
        short = name.replace("moe::(anonymous namespace)::", "")[:80]
        print(f"{len(busy[name]):8d} {util:9.3f} {ghz:9.2f} {2.5 * ghz / 2.4:11.2f} {m * 512 / 1e9:10.1f} {us:10.1f}  {short}")


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
    b.add_argument("--copy-kernel", default="MulFunctor<float>")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--rdreq", default=None, help="optional run with TCC_EA0_RDREQ_{128B,64B}_sum")
    b.add_argument("--large", action="store_true",
                   help="average only the dispatches reading at least half the largest value (a kernel launched "
                        "both with and without a data-moving option)")
    b.add_argument("--algorithmic", type=float, default=0.0, help="algorithmic bytes per launch, for the ratio")
    b.add_argument("--note", default="")
    b.add_argument("--sources", nargs="*", default=None,
                   help="kernel sources (file names under csrc/) whose hash the summary records (default: the GEMM's)")
    b.add_argument("--cmd", required=True)
    c = sub.add_parser("mfma")
    c.add_argument("dir")
    c.add_argument("--kernel", nargs="+", default=["k_gemm"])
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--simds", type=int, default=1024)
    c.add_argument("--cmd", required=True)
    args = ap.parse_args(argv)
    {"stats": stats, "traffic": traffic, "mfma": mfma}[args.what](args)


if __name__ == "__main__":
    main(sys.argv[1:])
