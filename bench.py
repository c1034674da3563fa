"""Benchmark of the fused GEMM + tile-reduce path on one MI355X.

One step = one mk_gemm_reduce_local launch over the whole workload: the
local partial C_r = A.B on MFMA plus the tile-granular reduction of every
output tile with the R-1 peer partials, inputs resident in HBM.  Prints one
JSON line.

The headline (`value`, `roofline`, `cpu_baseline`) is the largest workload,
compute_heavy (16384x8192x8192, 7 peers, 256x128 tiles).  The same line
carries every workload of the suite under `per_config`, each with the same
legs, plus geometric means over the four full-size workloads.

Legs per workload (all on the same seeded inputs, same stream):
  fused (adaptive partition)          -> ms, TFLOP/s, roofline fraction
  unfused: GEMM kernel then reduce kernel -> fused_vs_unfused
  headline only: the GEMM kernel alone, no peers (the bound a fused launch
    cannot beat) -> fused_over_gemm_alone
  the pages' plain controller rule (start 2, no cap, no help)
  static partitions 2..64 reduce workgroups (and 96..224 beyond the pages'
    range) -> adaptive_vs_best_static_2_64, adaptive_vs_best_static_any
  chunk release lag of the last fused launch (per-chunk stamps)
Each leg runs untimed for --settle-ms first (the GPU's clock settles after
an idle spell), then its warm-up launches, then the timed ones.
Every leg ends with mk_get_stats, whose status is sticky over all the leg's
launches: a timeout or protocol violation in any launch fails the bench.
Before each timed launch a 512 MiB scratch buffer is rewritten (outside the
timed events) so the 256 MB Infinity Cache and the L2s start cold.
The CPU oracle runs on a bounded sample of the headline workload
(cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import math
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
HEADLINE = "compute_heavy"                    # the largest workload
SUITE = ("tiny", "tp_share", "reduce_heavy", "compute_heavy", "wide_many_peer")
FULL_SIZE = ("tp_share", "reduce_heavy", "compute_heavy", "wide_many_peer")


class BenchError(SystemExit):
    """A leg whose launches reported an error: the bench prints no line."""

    def __init__(self, msg: str):
        print(f"[bench] FAILED: {msg}", file=sys.stderr, flush=True)
        super().__init__(3)


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all",
                    help="'all' (default: the headline workload plus every other one under "
                         "per_config) or one workload name")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-sweep", action="store_true", help="skip the static partition sweep")
    ap.add_argument("--fused-only", action="store_true",
                    help="only the fused leg of one workload (for profiler runs)")
    ap.add_argument("--gemm-only", action="store_true",
                    help="only the GEMM kernel of the unfused baseline, no peers (for counter "
                         "runs on the MFMA core); prints its own JSON line")
    ap.add_argument("--reduce-scatter", action="store_true",
                    help="one rank's share of GEMM+ReduceScatter instead (fused and unfused legs); "
                         "prints its own JSON line")
    ap.add_argument("--allgather", default=None, metavar="WORKLOAD",
                    help="only one AllGather+GEMM workload (ag_tiny, ag_tp_share, ag_compute_heavy); "
                         "prints its own JSON line")
    ap.add_argument("--no-allgather", action="store_true",
                    help="leave the AllGather+GEMM share out of the default line")
    ap.add_argument("--ring", default=None, metavar="WORKLOAD",
                    help="only one Ring Attention workload (ra_tiny, ra_sp_share, ra_long); "
                         "prints its own JSON line")
    ap.add_argument("--no-ring", action="store_true",
                    help="leave the Ring Attention share out of the default line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_S * 1e3,
                    help="untimed run of each leg before its warm-up steps, so that it is timed "
                         "at the GPU's settled clock (0: none)")
    return ap.parse_args(argv)


SETTLE_S = 0.2


def time_leg(fn, steps, warmup, flush, stream, torch, settle_s=None):
    """Per-launch durations (ms) from HIP events recorded on the launch stream.

    Before its warm-up steps a leg runs untimed for settle_s seconds of wall
    time.  After an idle spell (input generation, a host-side check) the
    GPU's power management answers a heavy launch by cutting the shader clock
    and restores it over about ten launches: GRBM_GUI_ACTIVE per dispatch on
    the 16384x8192x8192 GEMM+AllReduce reads 1.65 GHz on the first launch,
    1.13 on the second and 1.48 on the sixth.  A leg timed in that transient
    is slower for the clock alone, so every leg is timed at its settled clock.
    """
    if settle_s is None:
        settle_s = SETTLE_S
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(4):
            if flush is not None:
                flush()
            fn()
        torch.cuda.synchronize()
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


def check_leg(mk, leg: str, maps: bool = False):
    """Stats after a leg.  mk_get_stats reports an error raised by ANY launch
    since the previous call (sticky), so one call per leg covers every timed
    and warm-up launch of it.  A non-OK status ends the bench (exit 3)."""
    st = mk.get_stats(maps=maps, raise_on_error=False)
    if st["rc"] != 0 or st["status"] != 0:
        raise BenchError(f"{leg}: {st['status_name']} (sticky error bits {st['sticky_errors']:#x})")
    return st


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
                "gemm_tile_granular_amd/csrc/mk_device.hpp",
                "gemm_tile_granular_amd/csrc/mk_internal.hpp"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic_record():
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def measured_traffic(workload):
    """HBM bytes per launch of the fused kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (profiles/traffic.json), scaled by the
    plain-copy calibration stored with them.  None when the kernel sources
    changed since the counters were taken, or the workload was not profiled."""
    rec = _traffic_record()
    if rec is None:
        return None, "no profiles/traffic.json"
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    wrec = rec.get("workloads", {}).get(workload)
    if wrec is None or "hbm_bytes_per_launch" not in wrec:
        return None, f"{workload} not profiled"
    return float(wrec["hbm_bytes_per_launch"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def counter_figures(workload):
    """Counter-derived figures of the fused kernel from the committed
    rocprofv3 passes, when they match the current kernel sources:
      - GEMM TFLOP/s: SQ_INSTS_MFMA (one v_mfma_f32_32x32x16_bf16 per count,
        32768 flops) over the kernel-trace average duration;
      - MFMA busy: SQ_INSTS_MFMA x 32 SIMD cycles over 1024 SIMDs times
        GRBM_GUI_ACTIVE / 8 (cycles of one XCD over the dispatch);
      - HBM GB/s over the launch: copy-calibrated FETCH_SIZE + WRITE_SIZE
        over the same duration (the reduce role moves nearly all of it)."""
    rec = _traffic_record()
    if rec is None or rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    wrec = rec.get("workloads", {}).get(workload)
    if not wrec or "kernel_trace_avg_us" not in wrec:
        return None
    sec = wrec["kernel_trace_avg_us"] * 1e-6
    out = {"kernel_trace_avg_us": wrec["kernel_trace_avg_us"], "source": "profiles/traffic.json"}
    if "sq_insts_mfma" in wrec:
        flops = wrec["sq_insts_mfma"] * 32768.0
        out["gemm_tflops_counters"] = flops / sec / 1e12
        out["mfma_flops_per_launch_counters"] = flops
        if wrec.get("grbm_gui_active"):
            out["mfma_busy"] = wrec["sq_insts_mfma"] * 32.0 / (1024.0 * wrec["grbm_gui_active"] / 8.0)
    if "hbm_bytes_per_launch" in wrec:
        out["hbm_GBps_counters"] = wrec["hbm_bytes_per_launch"] / sec / 1e9
    return out


def roofline(w, ms):
    """Roofline of one fused launch from its algorithmic work (2MNK flops;
    A, B, every peer once, C once) and its mean duration."""
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
    traffic, note = measured_traffic(w.name)
    roof["traffic"] = traffic
    roof["traffic_unit"] = "bytes/launch"
    roof["traffic_note"] = note
    roof["algorithmic_bytes"] = w.algorithmic_bytes
    roof["algorithmic_flops"] = w.flops
    roof["max_roofline_frac"] = max(t_mfma, t_hbm) / sec
    return roof, tflops, gbps


def release_lags(st, w, np):
    """Per-chunk lag from the end of the chunk's last reduced tile to the
    chunk's release stamp (us), from the maps of the last launch."""
    rel = st["chunk_release"].astype(np.uint32)
    rend = st["reduce_end"].astype(np.uint32)
    tpc = w.tiles_per_chunk
    lags = []
    for c in range(len(rel)):
        tiles = rend[c * tpc:min(w.tiles, (c + 1) * tpc)]
        d = (rel[c] - tiles).astype(np.uint32).view(np.int32).astype(np.int64)
        lags.append(int(d.min()))
    us = np.array(lags, dtype=np.float64) / float(st["timer_hz"]) * 1e6
    return {"median_us": float(np.median(us)), "max_us": float(us.max()), "min_us": float(us.min()),
            "chunks": int(len(us))}


def phases_of(st, w, np):
    kernel_us = (st["kernel_ticks_end"] - st["kernel_ticks_start"]) / st["timer_hz"] * 1e6
    compute_us = float(np.max(st["compute_end_us"])) if len(st["compute_end_us"]) else 0.0
    reduce_us = (st["reduce_ticks_end"] - st["reduce_ticks_start"]) / st["timer_hz"] * 1e6
    reduce_bytes = 4.0 * w.M * w.N * (w.peers + 2)
    return {
        "kernel_us": kernel_us,
        "compute_window_us": compute_us,
        "gemm_tflops_in_compute_window": w.flops / (compute_us * 1e-6) / 1e12 if compute_us else None,
        "reduce_window_us": reduce_us,
        "reduce_GBps_in_reduce_window": reduce_bytes / (reduce_us * 1e-6) / 1e9 if reduce_us > 0 else None,
        "reduce_bytes": reduce_bytes,
        "xcd_local": st["xcd_local"],
        "xcd_bands": st["xcd_bands"],
        "n_reduce_initial": st["n_reduce_initial"],
        "n_reduce_final": st["n_reduce_final"],
        "n_reduce_range": [st["n_reduce_min_seen"], st["n_reduce_max_seen"]],
        "controller_cap": st["controller_cap"],
        "help_tiles": int((st["compute_owner"] >> 31).sum()),
    }


def set_adaptive_defaults(mk):
    mk.set_partition("adaptive", 0)
    mk.set_adaptive_help(True)
    mk.set_controller_cap(0)


def measure(args, w, mk, wl, upload, np, torch, keep_host=False, headline=False):
    """Every leg of one workload.  Returns (record, host inputs or None)."""
    t_gen = time.perf_counter()
    a, b, p = wl.make_inputs(w)
    A, B, P, C = upload(a, b, p, "cuda:0")
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] {w.name}: {w.M}x{w.N}x{w.K}, {w.peers} peers, tile {w.tile_m}x{w.tile_n}; "
          f"inputs ready in {t_gen:.1f} s", file=sys.stderr, flush=True)
    host = (a, b, p) if keep_host else None
    if not keep_host:
        del a, b, p

    stream = torch.cuda.current_stream()
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

    # every workload's fused leg runs the adaptive controller; a workload
    # whose recipe fixes a partition (tiny: 2 static reducers) also times
    # that partition as a leg of its own, and skips the sweep
    fixed = w.mode != "adaptive"
    set_adaptive_defaults(mk)
    ms_fused, wall = time_leg(fused, args.steps, args.warmup, flush, stream, torch)
    st = check_leg(mk, f"{w.name} fused", maps=True)
    rec = {"partition": "adaptive", "fused_ms": summary(ms_fused), "wall_s_fused_leg": wall}
    ms = statistics.fmean(ms_fused)
    roof, tflops, gbps = roofline(w, ms)
    roof["kernel"] = (f"mk::fused_gemm_reduce_kernel<{w.tile_m}, {w.tile_n}, "
                      f"{'true' if st['xcd_local'] else 'false'}, false>")
    rec.update({"ms": ms, "tflops": tflops, "hbm_GBps_algorithmic": gbps, "roofline": roof,
                "phases": phases_of(st, w, np), "chunk_release_lag": release_lags(st, w, np)})
    cf = counter_figures(w.name)
    if cf:
        rec["counters"] = cf
    print(f"[bench] {w.name} fused: {summary(ms_fused)}", file=sys.stderr, flush=True)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] copy calibration: {args.copy_calibration} MiB x3", file=sys.stderr, flush=True)

    if args.fused_only:
        return rec, host

    # consistency of the timed fused result with the two-kernel path at
    # sampled positions (the oracle comparison lives in the test suite)
    C_fused = C.clone()
    unfused()
    torch.cuda.synchronize()
    g = torch.Generator(device="cpu").manual_seed(0)
    idx = torch.randint(0, w.M * w.N, (1 << 16,), generator=g).to(C.device)
    fv, uv = C_fused.view(-1)[idx].double(), C.view(-1)[idx].double()
    diff = float((fv - uv).abs().max())
    scale = float(uv.abs().max())
    rec["fused_matches_unfused"] = {"max_abs_diff": diff, "scale": scale, "ok": diff <= 2e-3 * scale}
    del C_fused
    if not rec["fused_matches_unfused"]["ok"]:
        raise BenchError(f"{w.name}: fused and unfused results differ ({diff} > 2e-3 * {scale})")
    ms_unf, _ = time_leg(unfused, args.steps, args.warmup, flush, stream, torch)
    rec["unfused_ms"] = summary(ms_unf)
    rec["fused_vs_unfused"] = statistics.fmean(ms_unf) / ms
    print(f"[bench] {w.name} unfused: {summary(ms_unf)}", file=sys.stderr, flush=True)

    if headline:
        # the bound a fused launch cannot beat: the same GEMM kernel with no
        # peers to reduce (the unfused baseline's first kernel alone)
        def gemm_alone():
            mk.gemm_reduce_unfused(A, B, None, C, w.tile_m, w.tile_n, w.tiles_per_chunk)

        ms_g, _ = time_leg(gemm_alone, args.steps, args.warmup, flush, stream, torch)
        rec["gemm_alone_ms"] = summary(ms_g)
        rec["fused_over_gemm_alone"] = statistics.fmean(ms_g) / ms
        print(f"[bench] {w.name} GEMM alone: {summary(ms_g)}", file=sys.stderr, flush=True)

    if fixed:
        mk.set_partition(w.mode, w.n_reduce)
        ms_fix, _ = time_leg(fused, args.steps, args.warmup, flush, stream, torch)
        check_leg(mk, f"{w.name} {w.mode} {w.n_reduce}")
        set_adaptive_defaults(mk)
        rec["recipe_partition"] = {"mode": w.mode, "n_reduce": w.n_reduce, "fused_ms": summary(ms_fix),
                                   "fused_vs_unfused": statistics.fmean(ms_unf) / statistics.fmean(ms_fix)}
        print(f"[bench] {w.name} fused, {w.mode} {w.n_reduce}: {summary(ms_fix)}", file=sys.stderr, flush=True)
    if fixed or args.no_sweep:
        set_adaptive_defaults(mk)
        return rec, host

    # the pages' rule as printed: start at the sweep floor, no cap below
    # B - keep, reducers that wait instead of helping
    mk.set_partition("adaptive", 2)
    mk.set_adaptive_help(False)
    mk.set_controller_cap(1024)
    ms_plain, _ = time_leg(fused, args.steps, args.warmup, flush, stream, torch)
    stp = check_leg(mk, f"{w.name} plain rule")
    set_adaptive_defaults(mk)
    rec["plain_rule_ms"] = summary(ms_plain)
    rec["plain_rule_n_reduce_final"] = stp["n_reduce_final"]
    rec["labelled_variants_gain"] = statistics.fmean(ms_plain) / ms
    print(f"[bench] {w.name} plain rule: {summary(ms_plain)}", file=sys.stderr, flush=True)

    sweep, ext = {}, {}
    for table, counts in ((sweep, STATIC_SWEEP), (ext, STATIC_SWEEP_EXT)):
        for n in counts:
            mk.set_partition("static", n)
            ms_n, _ = time_leg(fused, max(3, args.steps // 2), 1, flush, stream, torch)
            check_leg(mk, f"{w.name} static {n}")
            table[n] = statistics.fmean(ms_n)
            print(f"[bench] {w.name} static {n}: {table[n]:.4f} ms", file=sys.stderr, flush=True)
    set_adaptive_defaults(mk)
    best_n = min(sweep, key=sweep.get)
    best_all = min({**sweep, **ext}.items(), key=lambda kv: kv[1])
    rec["static_sweep_ms"] = {str(k): v for k, v in sweep.items()}
    rec["static_sweep_ext_ms"] = {str(k): v for k, v in ext.items()}
    rec["best_static_2_64"] = {"n_reduce": best_n, "ms": sweep[best_n]}
    rec["adaptive_vs_best_static_2_64"] = sweep[best_n] / ms
    rec["best_static_any"] = {"n_reduce": best_all[0], "ms": best_all[1]}
    rec["adaptive_vs_best_static_any"] = best_all[1] / ms
    rec["plain_rule_vs_best_static_2_64"] = sweep[best_n] / statistics.fmean(ms_plain)
    return rec, host


AG_SUITE = ("ag_tiny", "ag_tp_share", "ag_compute_heavy")


def ag_algorithmic_bytes(w):
    """One rank's share of AllGather+GEMM: every shard read once and written
    once into the gathered A, B read once, C written once."""
    R = w.peers + 1
    return 2 * R * w.M * w.K * 2 + 2 * w.K * w.N + 4 * R * w.M * w.N


def measure_allgather(args, w, mk, wl, np, torch, sweep=True):
    """One rank's share of AllGather+GEMM: fused (adaptive, and the pages'
    plain rule), unfused (gather kernel then GEMM kernel), static copy
    partitions 2..64."""
    a0, ap, b = wl.make_ag_inputs(w)
    dev = "cuda:0"
    A0 = torch.from_numpy(a0.view(np.int16)).to(dev).view(torch.bfloat16)
    AP = torch.from_numpy(ap.view(np.int16)).to(dev).view(torch.bfloat16)
    B = torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)
    R = w.peers + 1
    G = torch.empty((R * w.M, w.K), dtype=torch.bfloat16, device=dev)
    C = torch.empty((R * w.M, w.N), dtype=torch.float32, device=dev)
    del a0, ap, b
    stream = torch.cuda.current_stream()
    flush = None
    if not args.no_flush:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

        def flush():
            scratch.fill_(1)

    def fused():
        mk.allgather_gemm_local(A0, AP, G, B, C, w.tile_m, w.tile_n)

    def unfused():
        mk.allgather_gemm_unfused(A0, AP, G, B, C, w.tile_m, w.tile_n)

    fixed = w.mode != "adaptive"
    set_adaptive_defaults(mk)
    ms_f, _ = time_leg(fused, args.steps, args.warmup, flush, stream, torch)
    st = check_leg(mk, f"{w.name} fused", maps=True)
    ms = statistics.fmean(ms_f)
    M = R * w.M
    flops = 2 * M * w.N * w.K
    bytes_ = ag_algorithmic_bytes(w)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = bytes_ / (HBM_PEAK_GBPS * 1e9)
    sec = ms / 1e3
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": bytes_ / sec / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / sec / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    copy_us = (st["reduce_ticks_end"] - st["reduce_ticks_start"]) / st["timer_hz"] * 1e6
    rec = {"config": {"ranks": R, "rows_per_rank": w.M, "M": M, "N": w.N, "K": w.K,
                      "tile": [w.tile_m, w.tile_n], "chunk_rows": w.tile_m},
           "partition": "adaptive",
           "fused_ms": summary(ms_f), "ms": ms, "tflops": flops / sec / 1e12, "roofline": roof,
           "algorithmic_flops": flops, "algorithmic_bytes": bytes_,
           "copy_window_us": copy_us,
           "n_reduce_range": [st["n_reduce_min_seen"], st["n_reduce_max_seen"]],
           "help_copies": int((st["reduce_owner"][:st["num_chunks"]] >> 31).sum())}
    print(f"[bench] {w.name} fused: {summary(ms_f)}", file=sys.stderr, flush=True)
    ms_u, _ = time_leg(unfused, args.steps, args.warmup, flush, stream, torch)
    rec["unfused_ms"] = summary(ms_u)
    rec["fused_vs_unfused"] = statistics.fmean(ms_u) / ms
    print(f"[bench] {w.name} unfused: {summary(ms_u)}", file=sys.stderr, flush=True)
    if fixed:
        mk.set_partition(w.mode, w.n_reduce)
        ms_x, _ = time_leg(fused, args.steps, args.warmup, flush, stream, torch)
        check_leg(mk, f"{w.name} {w.mode} {w.n_reduce}")
        set_adaptive_defaults(mk)
        rec["recipe_partition"] = {"mode": w.mode, "n_copy": w.n_reduce, "fused_ms": summary(ms_x),
                                   "fused_vs_unfused": statistics.fmean(ms_u) / statistics.fmean(ms_x)}
    if fixed or not sweep:
        set_adaptive_defaults(mk)
        return rec
    mk.set_partition("adaptive", 2)
    mk.set_adaptive_help(False)
    mk.set_controller_cap(1024)
    ms_p, _ = time_leg(fused, args.steps, args.warmup, flush, stream, torch)
    check_leg(mk, f"{w.name} plain rule")
    set_adaptive_defaults(mk)
    rec["plain_rule_ms"] = summary(ms_p)
    rec["labelled_variants_gain"] = statistics.fmean(ms_p) / ms
    table = {}
    for n in STATIC_SWEEP:
        mk.set_partition("static", n)
        ms_n, _ = time_leg(fused, max(3, args.steps // 2), 1, flush, stream, torch)
        check_leg(mk, f"{w.name} static {n}")
        table[n] = statistics.fmean(ms_n)
    set_adaptive_defaults(mk)
    best = min(table, key=table.get)
    rec["static_sweep_ms"] = {str(k): v for k, v in table.items()}
    rec["best_static_2_64"] = {"n_copy": best, "ms": table[best]}
    rec["adaptive_vs_best_static_2_64"] = table[best] / ms
    print(f"[bench] {w.name} static sweep: {table}", file=sys.stderr, flush=True)
    return rec


RA_SUITE = ("ra_tiny", "ra_sp_share", "ra_long")


def ra_algorithmic_bytes(w):
    """One rank's share of Ring Attention: Q, K and V read once, every
    arriving K and V read once and written once into the ring buffers, O
    (fp32) and LSE written once."""
    e = w.S * w.H * w.D
    P = w.ranks - 1
    return 2 * 3 * e + 2 * 2 * 2 * P * e + 4 * e + 4 * w.S * w.H


def measure_ring(args, w, mk, wl, np, torch, sweep=True):
    """One rank's share of Ring Attention: fused (adaptive), unfused (gather
    kernel then the attention kernel), static copy partitions 2..64."""
    q, kl, vl, kp, vp = wl.make_ra_inputs(w)
    dev = "cuda:0"
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    Q, KL, VL, KP, VP = t(q), t(kl), t(vl), t(kp), t(vp)
    KR, VR = torch.empty_like(KP), torch.empty_like(VP)
    O = torch.empty(q.shape, dtype=torch.float32, device=dev)
    L = torch.empty((w.H, w.S), dtype=torch.float32, device=dev)
    del q, kl, vl, kp, vp
    stream = torch.cuda.current_stream()
    flush = None
    if not args.no_flush:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

        def flush():
            scratch.fill_(1)

    def fused():
        mk.ring_attention_local(Q, KL, VL, KP, VP, KR, VR, O, L)

    def unfused():
        mk.ring_attention_unfused(Q, KL, VL, KP, VP, KR, VR, O, L)

    fixed = w.mode != "adaptive"
    set_adaptive_defaults(mk)
    ms_f, _ = time_leg(fused, args.steps, args.warmup, flush, stream, torch)
    st = check_leg(mk, f"{w.name} fused", maps=True)
    ms = statistics.fmean(ms_f)
    flops = w.flops
    bytes_ = ra_algorithmic_bytes(w)
    sec = ms / 1e3
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = bytes_ / (HBM_PEAK_GBPS * 1e9)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": bytes_ / sec / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / sec / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    copy_us = (st["reduce_ticks_end"] - st["reduce_ticks_start"]) / st["timer_hz"] * 1e6
    rec = {"config": {"ranks": w.ranks, "tokens_per_rank": w.S, "heads": w.H, "head_dim": w.D,
                      "kv_tile_tokens": 128, "query_block": 128},
           "partition": "adaptive", "fused_ms": summary(ms_f), "ms": ms, "tflops": flops / sec / 1e12,
           "roofline": roof, "algorithmic_flops": flops, "algorithmic_bytes": bytes_,
           "copy_window_us": copy_us,
           "n_copy_range": [st["n_reduce_min_seen"], st["n_reduce_max_seen"]]}
    print(f"[bench] {w.name} fused: {summary(ms_f)}", file=sys.stderr, flush=True)
    ms_u, _ = time_leg(unfused, args.steps, args.warmup, flush, stream, torch)
    rec["unfused_ms"] = summary(ms_u)
    rec["fused_vs_unfused"] = statistics.fmean(ms_u) / ms
    print(f"[bench] {w.name} unfused: {summary(ms_u)}", file=sys.stderr, flush=True)
    if fixed:
        mk.set_partition(w.mode, w.n_copy)
        ms_x, _ = time_leg(fused, args.steps, args.warmup, flush, stream, torch)
        check_leg(mk, f"{w.name} {w.mode} {w.n_copy}")
        set_adaptive_defaults(mk)
        rec["recipe_partition"] = {"mode": w.mode, "n_copy": w.n_copy, "fused_ms": summary(ms_x),
                                   "fused_vs_unfused": statistics.fmean(ms_u) / statistics.fmean(ms_x)}
    if fixed or not sweep:
        set_adaptive_defaults(mk)
        return rec
    table = {}
    for n in STATIC_SWEEP:
        mk.set_partition("static", n)
        ms_n, _ = time_leg(fused, max(3, args.steps // 2), 1, flush, stream, torch)
        check_leg(mk, f"{w.name} static {n}")
        table[n] = statistics.fmean(ms_n)
    set_adaptive_defaults(mk)
    best = min(table, key=table.get)
    rec["static_sweep_ms"] = {str(k): v for k, v in table.items()}
    rec["best_static_2_64"] = {"n_copy": best, "ms": table[best]}
    rec["adaptive_vs_best_static_2_64"] = table[best] / ms
    print(f"[bench] {w.name} static sweep: {table}", file=sys.stderr, flush=True)
    return rec


def geomean(xs):
    xs = [x for x in xs if x]
    return math.exp(sum(math.log(x) for x in xs) / len(xs)) if xs else None


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
                      "ms_per_step": mean, "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms,
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

    set_adaptive_defaults(mk)
    fl = None if args.no_flush else flush
    ms_f, _ = time_leg(fused, args.steps, args.warmup, fl, stream, torch)
    st = check_leg(mk, f"{w.name} reduce-scatter fused")
    ms_u, _ = time_leg(unfused, args.steps, args.warmup, fl, stream, torch)
    mf, mu = statistics.fmean(ms_f), statistics.fmean(ms_u)
    print(json.dumps({"metric": "GEMM+ReduceScatter TFLOP/s (one rank's share, fused adaptive)",
                      "value": w.flops / (mf * 1e-3) / 1e12, "unit": "TFLOP/s",
                      "ms_per_step": mf, "unfused_ms_per_step": mu, "fused_over_unfused": mu / mf,
                      "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms, "dtype": "bf16", "data": "synthetic",
                      "fused_ms": summary(ms_f), "unfused_ms": summary(ms_u),
                      "status": st["status_name"],
                      "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "ranks": w.peers + 1,
                                 "tile": [w.tile_m, w.tile_n]}}), flush=True)


def main(argv=None):
    global SETTLE_S
    args = parse(argv)
    SETTLE_S = max(0.0, args.settle_ms) / 1e3
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the "
              "multi-GPU GEMM+AllReduce is not part of it.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_tile_granular_amd as mk
    import workloads as wl
    from gemm_tile_granular_amd.tensors import upload

    head_name = HEADLINE if args.workload == "all" else args.workload
    w_head = wl.workload(head_name)
    if args.gemm_only:
        gemm_only(args, w_head, mk, wl, upload, np, torch)
        return
    if args.reduce_scatter:
        reduce_scatter(args, w_head, mk, wl, upload, np, torch)
        return
    if args.ring:
        w = wl.ra_workload(args.ring)
        rec = measure_ring(args, w, mk, wl, np, torch, sweep=not (args.no_sweep or args.fused_only))
        print(json.dumps({"metric": "Ring Attention TFLOP/s (one rank's share, fused adaptive)",
                          "value": rec["tflops"], "unit": "TFLOP/s", "ms_per_step": rec["ms"],
                          "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms, "dtype": "bf16",
                          "data": "synthetic", "config": {"workload": args.ring, **rec["config"]},
                          **{k: v for k, v in rec.items() if k != "config"}}), flush=True)
        return
    if args.allgather:
        rec = measure_allgather(args, wl.ag_workload(args.allgather), mk, wl, np, torch,
                                sweep=not (args.no_sweep or args.fused_only))
        print(json.dumps({"metric": "AllGather+GEMM TFLOP/s (one rank's share, fused adaptive)",
                          "value": rec["tflops"], "unit": "TFLOP/s", "ms_per_step": rec["ms"],
                          "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms, "dtype": "bf16",
                          "data": "synthetic", "config": {"workload": args.allgather, **rec["config"]},
                          **{k: v for k, v in rec.items() if k != "config"}}), flush=True)
        return

    names = [head_name] if (args.workload != "all" or args.fused_only) else \
        [head_name] + [n for n in SUITE if n != head_name]
    per = {}
    cpu = None
    for name in names:
        w = wl.workload(name)
        want_cpu = name == head_name and not args.no_cpu and not args.fused_only
        rec, host = measure(args, w, mk, wl, upload, np, torch, keep_host=want_cpu, headline=name == head_name)
        per[name] = rec
        if want_cpu:
            cpu = cpu_baseline(w, *host, args.cpu_seconds)
            print(f"[bench] cpu oracle: {cpu['value']:.3f} TFLOP/s", file=sys.stderr, flush=True)
        del host
        torch.cuda.empty_cache()

    head = per[head_name]
    result = {
        "metric": "fused GEMM+tile-reduce TFLOP/s & % roofline on 1 MI355X; speedup vs unfused",
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": w_head.name, "M": w_head.M, "N": w_head.N, "K_local": w_head.K,
                   "peers": w_head.peers, "tile": [w_head.tile_m, w_head.tile_n],
                   "tiles_per_chunk": w_head.tiles_per_chunk, "partition": head["partition"],
                   "cache_flush_between_steps": not args.no_flush},
        "roofline": head["roofline"],
    }
    for key in ("fused_vs_unfused", "fused_over_gemm_alone", "adaptive_vs_best_static_2_64",
                "adaptive_vs_best_static_any", "labelled_variants_gain", "chunk_release_lag", "phases",
                "counters", "fused_ms", "unfused_ms", "gemm_alone_ms"):
        if key in head:
            result[key] = head[key]
    if cpu is not None:
        result["cpu_baseline"] = cpu
    full = [per[n] for n in FULL_SIZE if n in per]
    if len(full) == len(FULL_SIZE):
        result["geomean_full_size"] = {
            "workloads": list(FULL_SIZE),
            "fused_vs_unfused": geomean([r.get("fused_vs_unfused") for r in full]),
            "adaptive_vs_best_static_2_64": geomean([r.get("adaptive_vs_best_static_2_64") for r in full]),
            "adaptive_vs_best_static_any": geomean([r.get("adaptive_vs_best_static_any") for r in full]),
            "labelled_variants_gain": geomean([r.get("labelled_variants_gain") for r in full]),
            "roofline_frac": geomean([r["roofline"]["frac"] for r in full]),
        }
        result["min_fused_vs_unfused"] = min(r.get("fused_vs_unfused", float("inf")) for r in full)
    result["per_config"] = per
    if args.workload == "all" and not (args.fused_only or args.no_allgather):
        ag = {}
        for name in AG_SUITE:
            ag[name] = measure_allgather(args, wl.ag_workload(name), mk, wl, np, torch,
                                         sweep=not args.no_sweep)
            torch.cuda.empty_cache()
        result["allgather_gemm"] = ag
        result["allgather_min_fused_vs_unfused"] = min(r["fused_vs_unfused"] for r in ag.values())
    if args.workload == "all" and not (args.fused_only or args.no_ring):
        ra = {}
        for name in RA_SUITE:
            ra[name] = measure_ring(args, wl.ra_workload(name), mk, wl, np, torch, sweep=not args.no_sweep)
            torch.cuda.empty_cache()
        result["ring_attention"] = ra
        result["ring_attention_min_fused_vs_unfused"] = min(r["fused_vs_unfused"] for r in ra.values())
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
