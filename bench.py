"""Benchmark of the fused GEMM + tile-reduce path on one MI355X.

One step = one mk_gemm_reduce_local launch over the whole workload: the
local partial C_r = A.B on MFMA plus the tile-granular reduction of every
output tile with the R-1 peer partials, inputs resident in HBM.  Prints one
JSON line.

Legs (all on the same seeded inputs, same stream):
  fused (adaptive partition)  -> value, roofline
  unfused: GEMM kernel then reduce kernel -> fused_vs_unfused
  static partitions 2..64 reduce workgroups -> adaptive_vs_best_static
  CPU oracle on a bounded sample of the same workload -> cpu_baseline
Before each timed launch a 512 MiB scratch buffer is rewritten (outside the
timed events) so the 256 MB Infinity Cache and the L2s start cold.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 4096 flop/clk x 2.4 GHz, dense
STATIC_SWEEP = (2, 4, 8, 16, 32, 64)          # the pages' sweep range
STATIC_SWEEP_EXT = (96, 128, 160, 192, 224)   # beyond it, for MI355X's reduce role


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="tp_share")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-sweep", action="store_true", help="skip the static partition sweep")
    ap.add_argument("--fused-only", action="store_true",
                    help="only the fused leg (for profiler runs)")
    ap.add_argument("--gemm-only", action="store_true",
                    help="only the GEMM kernel of the unfused baseline, no peers (for counter "
                         "runs on the MFMA core); prints its own JSON line")
    ap.add_argument("--reduce-scatter", action="store_true",
                    help="one rank's share of GEMM+ReduceScatter instead (fused and unfused legs); "
                         "prints its own JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def time_leg(fn, steps, warmup, flush, stream, torch):
    """Per-launch durations (ms) from HIP events on the launch stream."""
    for _ in range(warmup):
        if flush is not None:
            flush()
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in evs:
        if flush is not None:
            flush()
        s.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [s.elapsed_time(e) for s, e in evs]
    return ms, wall


def summary(ms):
    return {"mean": statistics.fmean(ms), "median": statistics.median(ms), "min": min(ms),
            "max": max(ms)}


def cpu_baseline(w, a, b, p, seconds):
    """The oracle, as it stands, on row blocks of the workload, wrapping round
    to the first row block, until `seconds` of wall time have been spent (at
    least one block).  Scaled to TFLOP/s of the GEMM part, like `value`."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    rb = max(1, min(w.M, 512))
    rows_done = 0
    blocks = 0
    t_total = 0.0
    r0 = 0
    while t_total < seconds or rows_done == 0:
        r1 = min(w.M, r0 + rb)
        t = time.perf_counter()
        oracle.gemm_reduce(a[r0:r1], b, p[:, r0:r1, :])
        t_total += time.perf_counter() - t
        rows_done += r1 - r0
        blocks += 1
        r0 = 0 if r1 >= w.M else r1
    flops = 2.0 * rows_done * w.N * w.K
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"float64 oracle (numpy/OpenBLAS, {threads} threads) on {blocks} blocks of "
                  f"{rb} rows ({rows_done} rows = {rows_done / w.M:.2f} passes over the "
                  f"{w.M}x{w.N}x{w.K} GEMM + {w.peers}-peer sum of {w.name}), {t_total:.1f} s",
        "seconds": t_total,
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


def kernel_source_hash():
    """sha256[:16] of the HIP sources that make up the fused kernel."""
    import hashlib
    h = hashlib.sha256()
    for rel in ("gemm_tile_granular_amd/csrc/mk_kernels.hip",
                "gemm_tile_granular_amd/csrc/mk_internal.hpp"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the fused kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (profiles/traffic.json), scaled by the
    plain-copy calibration stored with them.  None when the kernel sources
    changed since the counters were taken, or the workload was not profiled."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no profiles/traffic.json"
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    wrec = rec.get("workloads", {}).get(workload)
    if wrec is None:
        return None, f"{workload} not profiled"
    return float(wrec["hbm_bytes_per_launch"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def gemm_only(args, w, mk, wl, upload, np, torch):
    """The unfused baseline's GEMM kernel alone (no peers): C = A.B, timed
    with HIP events like the other legs."""
    import dataclasses
    a, b, _ = wl.make_inputs(dataclasses.replace(w, peers=0))
    A, B, P, C = upload(a, b, np.zeros((0, w.M, w.N), np.float32), "cuda:0")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def gemm():
        mk.gemm_reduce_unfused(A, B, None, C, w.tile_m, w.tile_n, w.tiles_per_chunk)

    ms, _ = time_leg(gemm, args.steps, args.warmup, None, stream, torch)
    mean = statistics.fmean(ms)
    print(json.dumps({"metric": "GEMM TFLOP/s (unfused baseline's GEMM kernel, no peers)",
                      "value": w.flops / (mean * 1e-3) / 1e12, "unit": "TFLOP/s",
                      "ms_per_step": mean, "steps": args.steps, "warmup": args.warmup,
                      "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                                 "tile": [w.tile_m, w.tile_n]}}), flush=True)


def reduce_scatter(args, w, mk, wl, upload, np, torch):
    """Rank 0's share of GEMM+ReduceScatter on the workload's shapes: the
    fused persistent launch and the two-launch baseline, timed with HIP
    events like the other legs (caches flushed between steps)."""
    a, b, p = wl.make_inputs(w)
    A, B, P, C = upload(a, b, p, "cuda:0")
    R = torch.from_numpy(wl.make_remote(w)).to("cuda:0")
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def flush():
        scratch.fill_(1)

    def fused():
        mk.gemm_reduce_scatter_local(A, B, P, C, R, w.tile_m, w.tile_n, w.tiles_per_chunk)

    def unfused():
        mk.gemm_reduce_scatter_unfused(A, B, P, C, R, w.tile_m, w.tile_n, w.tiles_per_chunk)

    mk.set_partition("adaptive", 0)
    fl = None if args.no_flush else flush
    ms_f, _ = time_leg(fused, args.steps, args.warmup, fl, stream, torch)
    st = mk.get_stats(maps=False)
    ms_u, _ = time_leg(unfused, args.steps, args.warmup, fl, stream, torch)
    mf, mu = statistics.fmean(ms_f), statistics.fmean(ms_u)
    print(json.dumps({"metric": "GEMM+ReduceScatter TFLOP/s (one rank's share, fused adaptive)",
                      "value": w.flops / (mf * 1e-3) / 1e12, "unit": "TFLOP/s",
                      "ms_per_step": mf, "unfused_ms_per_step": mu, "fused_over_unfused": mu / mf,
                      "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
                      "fused_ms": summary(ms_f), "unfused_ms": summary(ms_u),
                      "status": st["status_name"],
                      "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "ranks": w.peers + 1,
                                 "tile": [w.tile_m, w.tile_n]}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the "
              "multi-GPU GEMM+AllReduce is not part of it.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_tile_granular_amd as mk
    import workloads as wl
    from gemm_tile_granular_amd.tensors import upload

    w = wl.workload(args.workload)
    if args.gemm_only:
        gemm_only(args, w, mk, wl, upload, np, torch)
        return
    if args.reduce_scatter:
        reduce_scatter(args, w, mk, wl, upload, np, torch)
        return
    t_gen = time.perf_counter()
    a, b, p = wl.make_inputs(w)
    A, B, P, C = upload(a, b, p, "cuda:0")
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] {w.name}: {w.M}x{w.N}x{w.K}, {w.peers} peers, tile {w.tile_m}x{w.tile_n}; "
          f"inputs ready in {t_gen:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    scratch = None
    flush = None
    if not args.no_flush:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
        counter = [0]

        def flush():
            counter[0] = (counter[0] + 1) & 0xFF
            scratch.fill_(counter[0])

    def fused():
        mk.gemm_reduce_local(A, B, P, C, w.tile_m, w.tile_n, w.tiles_per_chunk)

    def unfused():
        mk.gemm_reduce_unfused(A, B, P, C, w.tile_m, w.tile_n, w.tiles_per_chunk)

    mk.set_partition("adaptive", 0)
    ms_fused, wall_fused = time_leg(fused, args.steps, args.warmup, flush, stream, torch)
    st = mk.get_stats(maps=True)
    # phase windows of the last timed launch, from the device's constant clock
    kernel_us = (st["kernel_ticks_end"] - st["kernel_ticks_start"]) / st["timer_hz"] * 1e6
    compute_us = float(np.max(st["compute_end_us"])) if len(st["compute_end_us"]) else 0.0
    reduce_us = (st["reduce_ticks_end"] - st["reduce_ticks_start"]) / st["timer_hz"] * 1e6
    reduce_bytes = 4.0 * w.M * w.N * (w.peers + 2)
    phases = {
        "kernel_us": kernel_us,
        "compute_window_us": compute_us,
        "gemm_tflops_in_compute_window": w.flops / (compute_us * 1e-6) / 1e12 if compute_us else None,
        "reduce_window_us": reduce_us,
        "reduce_GBps_in_reduce_window": reduce_bytes / (reduce_us * 1e-6) / 1e9 if reduce_us > 0 else None,
        "reduce_bytes": reduce_bytes,
        "xcd_local": st["xcd_local"],
        "n_reduce_initial": st["n_reduce_initial"],
        "n_reduce_range": [st["n_reduce_min_seen"], st["n_reduce_max_seen"]],
        "controller_cap": st["controller_cap"],
        "help_tiles": int((st["compute_owner"] >> 31).sum()),
    }
    print(f"[bench] fused adaptive: {summary(ms_fused)} (n_reduce final {st['n_reduce_final']}, "
          f"range {st['n_reduce_min_seen']}-{st['n_reduce_max_seen']})", file=sys.stderr, flush=True)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {args.copy_calibration} MiB x3", file=sys.stderr, flush=True)

    out_extra = {}
    if not args.fused_only:
        # consistency of the timed fused result with the two-kernel path, at
        # sampled positions (the oracle comparison lives in the test suite)
        C_fused = C.clone()
        unfused()
        torch.cuda.synchronize()
        g = torch.Generator(device="cpu").manual_seed(0)
        idx = torch.randint(0, w.M * w.N, (1 << 16,), generator=g).to(C.device)
        fv, uv = C_fused.view(-1)[idx].double(), C.view(-1)[idx].double()
        diff = float((fv - uv).abs().max())
        scale = float(uv.abs().max())
        out_extra["fused_matches_unfused"] = {"max_abs_diff": diff, "scale": scale,
                                              "ok": diff <= 2e-3 * scale}
        del C_fused
        ms_unf, _ = time_leg(unfused, args.steps, args.warmup, flush, stream, torch)
        print(f"[bench] unfused: {summary(ms_unf)}", file=sys.stderr, flush=True)
        out_extra["unfused_ms"] = summary(ms_unf)
        out_extra["fused_vs_unfused"] = statistics.fmean(ms_unf) / statistics.fmean(ms_fused)
        if not args.no_sweep:
            sweep = {}
            for n in STATIC_SWEEP:
                mk.set_partition("static", n)
                ms_n, _ = time_leg(fused, max(3, args.steps // 2), 1, flush, stream, torch)
                sweep[n] = statistics.fmean(ms_n)
                print(f"[bench] static {n}: {sweep[n]:.4f} ms", file=sys.stderr, flush=True)
            best_n = min(sweep, key=sweep.get)
            ext = {}
            for n in STATIC_SWEEP_EXT:
                mk.set_partition("static", n)
                ms_n, _ = time_leg(fused, max(3, args.steps // 2), 1, flush, stream, torch)
                ext[n] = statistics.fmean(ms_n)
                print(f"[bench] static {n}: {ext[n]:.4f} ms", file=sys.stderr, flush=True)
            mk.set_partition("adaptive", 0)
            best_all = min({**sweep, **ext}.items(), key=lambda kv: kv[1])
            out_extra["static_sweep_ms"] = {str(k): v for k, v in sweep.items()}
            out_extra["static_sweep_ext_ms"] = {str(k): v for k, v in ext.items()}
            out_extra["best_static"] = {"n_reduce": best_n, "ms": sweep[best_n]}
            out_extra["adaptive_vs_best_static"] = sweep[best_n] / statistics.fmean(ms_fused)
            out_extra["best_static_any"] = {"n_reduce": best_all[0], "ms": best_all[1]}
            out_extra["adaptive_vs_best_static_any"] = best_all[1] / statistics.fmean(ms_fused)

    ms = statistics.fmean(ms_fused)
    sec = ms / 1e3
    tflops = w.flops / sec / 1e12
    gbps = w.algorithmic_bytes / sec / 1e9
    t_mfma = w.flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = w.algorithmic_bytes / (HBM_PEAK_GBPS * 1e9)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": gbps / HBM_PEAK_GBPS}
    else:
        roof = {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS}
    traffic, traffic_note = measured_traffic(w.name)
    roof["traffic"] = traffic
    roof["traffic_unit"] = "bytes/launch"
    roof["traffic_note"] = traffic_note
    roof["algorithmic_bytes"] = w.algorithmic_bytes
    roof["algorithmic_flops"] = w.flops
    roof["kernel"] = (f"mk::fused_gemm_reduce_kernel<{w.tile_m}, {w.tile_n}, "
                      f"{'true' if st['xcd_local'] else 'false'}, false>")
    roof["max_roofline_frac"] = max(t_mfma, t_hbm) / sec

    result = {
        "metric": "fused GEMM+tile-reduce TFLOP/s & % roofline on 1 MI355X; speedup vs unfused",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K_local": w.K, "peers": w.peers,
                   "tile": [w.tile_m, w.tile_n], "tiles_per_chunk": w.tiles_per_chunk,
                   "partition": "adaptive", "cache_flush_between_steps": not args.no_flush},
        "roofline": roof,
        "fused_ms": summary(ms_fused),
        "hbm_GBps_algorithmic": gbps,
        "wall_s_fused_leg": wall_fused,
        "n_reduce_final": st["n_reduce_final"],
        "fused_phases": phases,
        **out_extra,
    }
    if not args.no_cpu and not args.fused_only:
        result["cpu_baseline"] = cpu_baseline(w, a, b, p, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
