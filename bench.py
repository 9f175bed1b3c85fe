"""Throughput of the MoE FFN layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload deepseek_fine]

One step is one moe_forward call (route, dispatch, routed and shared SwiGLU
experts, combine) over one batch of seeded synthetic tokens that are already
resident in HBM. The default workload is the largest layer that fits one GPU
(DeepSeek-style: 65,536 tokens, d_model 7168, 256 routed experts + 1 shared,
top-8, d_ff 2048). Prints one JSON line with the whole-job throughput, the
roofline of the dominant kernel (the routed gate/up grouped GEMM, timed with
hipEvents on the layer's stream around each of its launches in the timed
region), per-phase times from a second pass of the same steps with every
phase boundary timed, the same phases with cold caches (a 1 GiB copy between
steps, outside the timed events, evicts L2 and the 256 MB last-level cache),
the backward pass where it fits, and the CPU oracle timed on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec @1 MI355X; grouped-GEMM % MFMA peak; route/permute % HBM"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA peaks
PEAK_VALU_F32_TFLOPS = 78.6                       # fp32 FMA on the VALU without packed instructions
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 256 << 20  # plain device-to-device copy used to calibrate HBM counters


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="deepseek_fine")
    ap.add_argument("--tokens", type=int, default=0, help="override the workload's token count (small-T sweeps)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU-oracle sample time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (reference for HBM counters)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--cold-steps", type=int, default=10, help="steps timed with cold caches (0: none)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time torch.matmul (the vendor GEMM library) on dense products of the routed GEMMs' "
                         "sizes, as a reference")
    return ap.parse_args()


FLUSH_BYTES = 1 << 30  # copied between cold steps: 4x the last-level cache


def host_cpu():
    """CPU model and logical CPU count from lscpu (None when unavailable)."""
    import subprocess

    info = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return None, None
    for line in out.splitlines():
        if ":" in line:
            k, v = line.split(":", 1)
            info[k.strip()] = v.strip()
    n = info.get("CPU(s)")
    return info.get("Model name"), (int(n) if n and n.isdigit() else None)


def oracle_threads() -> int:
    """Every CPU of the affinity mask, within the CPU share the environment
    grants (OMP_NUM_THREADS, when it is set)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch from the committed PMC summary, or None when the
    summary is missing or the kernel source changed since it was taken."""
    from mixture_experts_ffn_02_amd.profiling import source_hash

    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    try:
        if vals.get("source_sha256") != source_hash():
            return None
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def shared_as_group(cfg) -> bool:
    """The library runs the shared expert as one more group of the routed
    grouped GEMMs when it has the routed width and T * d_ff <= 2^25."""
    return cfg.d_ff_s > 0 and cfg.d_ff_s == cfg.d_ff and cfg.T * cfg.d_ff_s <= 1 << 25


def phase_bytes_and_flops(cfg, used=None):
    """Algorithmic work per phase (activated experts only): `used` experts
    received tokens (all of them when None), and only their weights count as
    read."""
    T, d, E, k, f, fs = cfg.T, cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_ff, cfg.d_ff_s
    Eu = E if used is None else used
    b = 2 if cfg.dtype == "bf16" else 4
    rows = T * k
    work = {
        # x, W_r in; ids, weights, ranks out
        "route": {"bytes": T * d * b + E * d * 4 + rows * 12, "flops": 2.0 * T * d * E},
        "gateup": {"flops": 4.0 * rows * d * f, "bytes": rows * d * b + Eu * 2 * f * d * b + rows * f * b},
        "down": {"flops": 2.0 * rows * f * d, "bytes": rows * f * b + Eu * d * f * b + rows * d * 4},
        "shared_gateup": {"flops": 4.0 * T * d * fs, "bytes": (T * d * b + 2 * fs * d * b + T * fs * b) if fs else 0},
        "shared_down": {"flops": 2.0 * T * fs * d, "bytes": (T * fs * b + d * fs * b + T * d * 4) if fs else 0},
        # Y rows, weights and ids, shared rows in; y out
        "combine": {"bytes": rows * d * 4 + rows * 8 + (T * d * 4 if fs else 0) + T * d * 4},
    }
    if shared_as_group(cfg):
        # one gate/up and one down launch cover the routed and the shared expert
        for a, s in (("gateup", "shared_gateup"), ("down", "shared_down")):
            for key in ("flops", "bytes"):
                work[a][key] += work[s][key]
            del work[s]
    return work


def gemm_row_tile(rows: int, groups: int, n: int, d_in: int, cu: int = 256) -> int:
    """The library's row tile for the forward products of a bf16 grouped
    launch (host rules gemm_bm and gemm_bm_fwd of gemm.hip: 64 for few rows
    per group, 256 for many rows or a long K, or where the eight-wave kernel
    runs both products and the groups average more than 64 rows)."""
    avg = rows // max(groups, 1)
    busy = min(groups, rows)
    long_k = d_in >= 4096
    if avg <= 128 and busy * (n // 128 if n % 128 == 0 else n // 64) >= 2 * cu:
        bm = 64
    elif rows <= 32 * busy:  # a handful of rows per busy group
        bm = 64
    else:
        bm = 256 if (avg >= 768 or long_k) and (rows // 256) * (n // 128) >= 4 * cu else 128
    if bm == 256 or rows <= 32 * busy:
        return bm
    fits8 = n % 128 == 0 and d_in % 256 == 0 and n >= 192 and d_in >= 192
    if fits8 and avg > 64 and max(rows // 256, busy) * (n // 128) >= 2 * cu:
        return 256
    if bm == 64 and avg > 48 and d_in >= 2048 and groups >= 64:
        return 128
    return bm


def gateup_kernel(cfg) -> str:
    merged = shared_as_group(cfg)
    rows = cfg.T * cfg.top_k + (cfg.T if merged else 0)
    groups = cfg.n_experts + (1 if merged else 0)
    if cfg.dtype == "bf16" and gemm_row_tile(rows, groups, cfg.d_ff, cfg.d_model) == 256 and cfg.d_ff % 128 == 0:
        return "k_gemm8<gate/up, grouped> (256 x 256 tiles, eight waves)"
    return f"k_gemm<{cfg.dtype}, gate/up, grouped>"


def gateup_roofline(cfg, work, gateup_ms: float, traffic):
    """Roofline of the routed gate/up launch: against the matrix cores when
    its algorithmic flops per byte reach the ridge of the two peaks, else
    (a few rows per expert) against HBM, the weights it must read."""
    peak = PEAK_TFLOPS[cfg.dtype]
    what = "routed experts + the shared expert as one more group" if shared_as_group(cfg) else "routed experts"
    gw = work["gateup"]
    if gw["flops"] / gw["bytes"] >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        gu = gw["flops"] / (gateup_ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": f"{gateup_kernel(cfg)} ({what})", "achieved": round(gu, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(gu / peak, 4), "traffic": traffic}
    gbs = gw["bytes"] / (gateup_ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": f"{gateup_kernel(cfg)} ({what})", "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}


def measure_permute(cfg, layer, x, reps: int):
    """moe_permute with the permuted copy of x (x_perm), which moe_forward
    itself never writes (its gate/up GEMM gathers the rows): ms per call and
    algorithmic bytes: x read once, T*k rows written, ids read and row ids
    written (int32 each)."""
    import torch

    idx = layer.route(x)["idx"]
    layer.permute(x, idx)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        layer.permute(x, idx)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    eb = 2 if cfg.dtype == "bf16" else 4
    by = cfg.T * cfg.d_model * eb * (1 + cfg.top_k) + cfg.T * cfg.top_k * 8
    gbs = by / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "bytes": by, "gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
            "note": "moe_permute writing x_perm (not part of moe_forward, whose GEMM gathers the rows)"}


def measure_library_gemm(cfg, reps: int):
    """Reference, not part of the layer: torch.matmul (the vendor GEMM library
    behind it) on dense products with the routed expert GEMMs' sizes,
    [T*k, d] x [d, 2 d_ff] (gate and up as one product) and [T*k, d_ff] x
    [d_ff, d] (down), both operands contiguous, output in the operand dtype.
    One weight for all rows: no gather, no groups, no SwiGLU, no fp32 output,
    so it bounds what a plain product of that size reaches on this chip."""
    import torch

    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    rows = cfg.T * cfg.top_k
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    peak = PEAK_TFLOPS[cfg.dtype]
    out = {"note": "torch.matmul on dense operands of the routed GEMMs' sizes (reference only)"}
    for name, (m, kk, n) in {"gateup_equiv": (rows, cfg.d_model, 2 * cfg.d_ff),
                             "down_equiv": (rows, cfg.d_ff, cfg.d_model)}.items():
        a = torch.randn((m, kk), generator=gen, device="cuda", dtype=torch.float32).to(dt)
        b = torch.randn((kk, n), generator=gen, device="cuda", dtype=torch.float32).to(dt)
        c = torch.matmul(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 2.0 * m * kk * n / (ms * 1e-3) / 1e12
        out[name] = {"m": m, "k": kk, "n": n, "ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / peak, 4)}
        del a, b, c
        torch.cuda.empty_cache()
    return out


def measure_backward(cfg, layer, x, steps: int, warmup: int):
    """moe_backward for the forward's routing and a seeded dy: ms per call
    (HIP events on the layer's stream) and its algorithmic expert-GEMM work:
    dgrad and wgrad of gate/up and down, 12 rows*d*d_ff flops (the gate/up
    recompute inside the call, 4 rows*d*d_ff more, is not counted)."""
    import numpy as np
    import torch

    fw = layer.forward(x)
    dy = torch.from_numpy(np.random.default_rng(1).standard_normal((cfg.T, cfg.d_model)).astype(np.float32)).cuda()
    for _ in range(warmup):
        layer.backward(x, fw["idx"], fw["w"], dy)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        layer.backward(x, fw["idx"], fw["w"], dy)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    rows = cfg.T * cfg.top_k + (cfg.T if cfg.d_ff_s else 0)
    flops = 12.0 * rows * cfg.d_model * cfg.d_ff
    peak = PEAK_TFLOPS[cfg.dtype]
    return {"ms": round(ms, 4), "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
            "expert_gemm_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / peak, 4),
            "note": "one moe_backward call (gate/up recompute included in the time, not in the flops)"}


def cpu_baseline(cfg, inputs, target_s: float):
    threads = oracle_threads()
    os.environ["OMP_NUM_THREADS"] = str(threads)
    import oracle
    import numpy as np

    def run(n):
        sub = dict(inputs)
        sub["x"] = inputs["x"][:n]
        t0 = time.perf_counter()
        oracle.forward(sub, cfg.top_k, cfg.score, cfg.renorm)
        return time.perf_counter() - t0

    n0 = min(cfg.T, 256)
    t_small = run(n0)
    n = int(min(cfg.T, max(n0, n0 * target_s / max(t_small, 1e-6))))
    t = run(n) if n > n0 else t_small
    reps = 1
    while t < target_s and reps < 64:  # the whole layer takes less than the target: repeat it
        t += run(n)
        reps += 1
    model, ncpu = host_cpu()
    return {"value": round(n * reps / t, 2), "unit": "tokens/s", "cores": oracle.lib().oracle_num_threads(),
            "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens of the same layer, {reps} run(s): fp32 router + fp64 experts "
                      f"and combine, {t:.2f} s in all",
            "cpu_model": model, "host_cpus": ncpu, "affinity_cpus": len(os.sched_getaffinity(0))}


def cold_phases(layer, x, y, steps: int):
    """Per-phase times (ms) of `steps` forward calls, each after a 1 GiB
    device copy that evicts L2 and the last-level cache; the copy runs
    before the step's first event, so no phase includes it."""
    import numpy as np
    import torch

    from mixture_experts_ffn_02_amd.layer import Timing

    src = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=x.device).fill_(1.0)
    dst = torch.empty_like(src)
    timings = [Timing() for _ in range(steps)]
    for t in timings:
        dst.copy_(src)
        layer.forward(x, y, want_routing=False, timing=t)
    torch.cuda.synchronize()
    ph = [t.read() for t in timings]
    for t in timings:
        t.close()
    del src, dst
    return {k: float(np.mean([p[k] for p in ph])) for k in ph[0]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer's data-parallel "
              f"shards run independently, one per GPU, and exchange nothing in the forward pass)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from mixture_experts_ffn_02_amd.inputs import CONFIGS, make_layer
    from mixture_experts_ffn_02_amd.layer import MoELayer, Timing, to_device

    cfg = CONFIGS[args.workload]
    if args.tokens > 0:
        cfg = cfg.with_tokens(args.tokens)
    inputs = make_layer(cfg)
    layer = MoELayer.from_host(cfg, inputs)
    x = to_device(inputs["x"])
    y = torch.empty((cfg.T, cfg.d_model), dtype=torch.float32, device="cuda")
    layer.workspace(cfg.T)
    for _ in range(args.warmup):
        layer.forward(x, y, want_routing=False)
    # Timed region: the gate/up launch of every step is bracketed by two
    # hipEvents on the layer's stream (each event between kernels costs a
    # few microseconds of stream time, so no other phase is timed here).
    timings = [Timing(phases=["gateup"]) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        layer.forward(x, y, want_routing=False, timing=timings[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    gateup_ms = float(np.mean([t.read()["gateup"] for t in timings]))
    for t in timings:
        t.close()
    # Phase breakdown: the same steps again with every boundary timed
    timings = [Timing() for _ in range(min(args.steps, 10))]
    for t in timings:
        layer.forward(x, y, want_routing=False, timing=t)
    torch.cuda.synchronize()
    if args.copy_calibration:
        # a plain elementwise copy (16 bytes per lane, whole grid) of known size
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    phases = [t.read() for t in timings]
    phase_ms = {k: float(np.mean([p[k] for p in phases])) for k in phases[0]}
    for t in timings:
        t.close()

    # experts that received tokens: only their weights are read
    counts = layer.route(x)["counts"].cpu().numpy()
    used = int((counts > 0).sum())
    work = phase_bytes_and_flops(cfg, used)
    peak = PEAK_TFLOPS[cfg.dtype]
    # the committed counter summaries were taken at the workload's own size
    traffic = traffic_from_profile("gateup", args.workload) if args.tokens in (0, CONFIGS[args.workload].T) else None
    roofline = gateup_roofline(cfg, work, gateup_ms, traffic)
    def phase_detail(pms):
        detail = {}
        for name, w in work.items():
            t_s = pms[name] * 1e-3
            if t_s <= 0 or not (w.get("flops") or w.get("bytes")):
                continue  # a phase that launched nothing (no shared expert)
            e = {"ms": round(pms[name], 4)}
            if "flops" in w and w["flops"]:
                tf = w["flops"] / t_s / 1e12
                pk = PEAK_VALU_F32_TFLOPS if name == "route" else peak
                e.update(tflops=round(tf, 2), frac_compute_peak=round(tf / pk, 4))
            if w.get("bytes"):
                gbs = w["bytes"] / t_s / 1e9
                e.update(gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
            detail[name] = e
        for name in ("scan", "scatter"):
            detail[name] = {"ms": round(pms[name], 4)}
        return detail

    detail = phase_detail(phase_ms)
    # expert GEMM phases that ran (the shared expert's own launches only when it has them)
    gemm_phases = [n for n in ("gateup", "down", "shared_gateup", "shared_down") if n in work and work[n]["flops"]]

    out = {
        "metric": METRIC,
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d_model, "n_experts": cfg.n_experts,
                   "top_k": cfg.top_k, "d_ff": cfg.d_ff, "shared_d_ff": cfg.d_ff_s, "score": cfg.score,
                   "selection_bias": cfg.bias_range > 0},
        "roofline": roofline,
        "phases": detail,
        "grouped_gemm_frac_mfma": round(
            sum(work[n]["flops"] for n in gemm_phases) / (sum(phase_ms[n] for n in gemm_phases) * 1e-3)
            / 1e12 / peak, 4),
    }
    if args.cold_steps > 0:
        cold = cold_phases(layer, x, y, args.cold_steps)
        out["phases_cold"] = phase_detail(cold)
        out["phases_cold"]["ms_per_step"] = round(sum(cold.values()), 4)
        out["phases_cold"]["note"] = (f"{args.cold_steps} steps, each after a {FLUSH_BYTES >> 20} MiB device copy "
                                      "outside the timed events (L2 and the last-level cache evicted)")
    out["permute"] = measure_permute(cfg, layer, x, max(3, min(args.steps, 20)))
    # expert weights the step had to read: experts that received tokens (+ the shared one)
    wbytes = (2 if cfg.dtype == "bf16" else 4) * 3 * cfg.d_model * (used * cfg.d_ff + cfg.d_ff_s)
    gemm_ms = sum(phase_ms[n] for n in gemm_phases)
    out["expert_weights"] = {"experts_used": used, "bytes": wbytes,
                             "gbs_over_expert_gemms": round(wbytes / (gemm_ms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(wbytes / (gemm_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if not args.no_backward:
        # weights, fp32 gradients and the backward workspace must fit comfortably
        bw_bytes = layer.backward_workspace_bytes(cfg.T) + 4 * 3 * cfg.n_experts * cfg.d_model * cfg.d_ff
        if bw_bytes < 120e9:
            out["backward"] = measure_backward(cfg, layer, x, max(1, min(args.steps // 4, 50)), 2)
    if args.library_gemm:
        out["library_gemm"] = measure_library_gemm(cfg, max(3, min(args.steps, 20)))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inputs, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
