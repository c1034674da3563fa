"""Helpers for the GPU parity tests: run the HIP path, compare with the oracle."""
from __future__ import annotations

import numpy as np

import oracle
import workloads as wl

REL_TOL = 2e-3     # max|C - C_ref| <= 2e-3 * max|C_ref|, and the same on the GEMM part
U32 = 2.0 ** -24   # unit roundoff of fp32


def run_fused(mk, w, a, b, p, mode=None, n_reduce=None, maps=True, C=None):
    from gemm_tile_granular_amd.tensors import upload
    A, B, P, C0 = upload(a, b, p)
    C = C0 if C is None else C
    mode = mode or w.mode
    mk.set_partition(mode, w.n_reduce if n_reduce is None else n_reduce)
    print(f"[gpu] fused {w.name} {w.M}x{w.N}x{w.K} P={w.peers} tile {w.tile_m}x{w.tile_n} "
          f"tpc {w.tiles_per_chunk} mode {mode} n={w.n_reduce if n_reduce is None else n_reduce}",
          flush=True)
    mk.gemm_reduce_local(A, B, P, C, w.tile_m, w.tile_n, w.tiles_per_chunk)
    st = mk.get_stats(maps=maps)
    return C.cpu().numpy(), st


def run_unfused(mk, w, a, b, p):
    from gemm_tile_granular_amd.tensors import upload
    import torch
    A, B, P, C = upload(a, b, p)
    print(f"[gpu] unfused {w.name} {w.M}x{w.N}x{w.K} P={w.peers}", flush=True)
    mk.gemm_reduce_unfused(A, B, P, C, w.tile_m, w.tile_n, w.tiles_per_chunk)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def check_full(C, a, b, p):
    """Element-by-element comparison with the float64 oracle on the whole output."""
    gemm = oracle.gemm_part(a, b)
    ps = oracle.peer_sum(p) if p.shape[0] else np.zeros_like(gemm)
    ref = gemm + ps
    Cd = C.astype(np.float64)
    err = float(np.max(np.abs(Cd - ref))) if ref.size else 0.0
    bound = REL_TOL * float(np.max(np.abs(ref))) if ref.size else 0.0
    assert err <= bound, f"max|C-C_ref| = {err:.4e} > {bound:.4e}"
    gmax = float(np.max(np.abs(gemm))) if gemm.size else 0.0
    if gmax > 0:
        gerr = float(np.max(np.abs((Cd - ps) - gemm)))
        assert gerr <= REL_TOL * gmax, f"GEMM part: {gerr:.4e} > {REL_TOL * gmax:.4e}"
    else:
        # no GEMM contribution: C is an fp32 sum of the peers
        absum = np.abs(p.astype(np.float64)).sum(axis=0) if p.shape[0] else np.zeros_like(gemm)
        assert np.all(np.abs(Cd - ps) <= p.shape[0] * U32 * absum + 1e-30)
    return err, bound


def check_sampled(C, a, b, p, rng, n_samples=4096, tiles=(), tile=(128, 128)):
    """Comparison at sampled positions and on whole tiles (oracle one element
    or one tile at a time), for outputs too large for the full oracle."""
    M, N = C.shape
    rows = rng.integers(0, M, n_samples)
    cols = rng.integers(0, N, n_samples)
    ref, gemm = oracle.gemm_reduce_at(a, b, p, rows, cols)
    got = C[rows, cols].astype(np.float64)
    ps = ref - gemm
    # scale: the largest |C_ref| seen over the samples and the checked tiles
    scale = float(np.max(np.abs(ref)))
    gscale = float(np.max(np.abs(gemm)))
    checks = [(got, ref, gemm, ps)]
    tm, tn = tile
    for (ti, tj) in tiles:
        r0, c0 = ti * tm, tj * tn
        r1, c1 = min(M, r0 + tm), min(N, c0 + tn)
        sub_p = p[:, r0:r1, c0:c1]
        g = oracle.gemm_part(a[r0:r1], b[:, c0:c1])
        s = oracle.peer_sum(np.ascontiguousarray(sub_p)) if p.shape[0] else np.zeros_like(g)
        checks.append((C[r0:r1, c0:c1].astype(np.float64).ravel(), (g + s).ravel(), g.ravel(),
                       s.ravel()))
        scale = max(scale, float(np.max(np.abs(g + s))))
        gscale = max(gscale, float(np.max(np.abs(g))))
    for got_, ref_, g_, s_ in checks:
        err = float(np.max(np.abs(got_ - ref_)))
        assert err <= REL_TOL * scale, f"max|C-C_ref| = {err:.4e} > {REL_TOL * scale:.4e}"
        if gscale > 0:
            gerr = float(np.max(np.abs((got_ - s_) - g_)))
            assert gerr <= REL_TOL * gscale, f"GEMM part {gerr:.4e} > {REL_TOL * gscale:.4e}"


def check_protocol(st, w, mode, n_reduce):
    # the task size comes from the tile shape (the oracle's reading), and the
    # device's own report must agree with it
    tpt = oracle.tiles_per_task(w.tile_m, w.tile_n)
    assert st["tiles_per_task"] == tpt, (st["tiles_per_task"], tpt)
    bad = oracle.check_state(st, w.tiles, w.tiles_per_chunk, st["epoch"], st["calls_since_reset"],
                             st["num_wg"], mode, n_reduce, tiles_n=-(-w.N // w.tile_n),
                             tiles_per_task=tpt)
    assert not bad, bad
    assert st["status"] == 0, st["status_name"]
    assert st["compute_tasks"] == w.tiles and st["reduce_tasks"] == w.tiles
    assert st["chunks_released"] == w.chunks
    assert st["invariant_violations"] == 0
