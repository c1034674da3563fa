"""GPU parity for one rank's share of AllGather+GEMM: the fused and unfused
entry points (through the C ABI) against oracle.allgather_gemm.

The gathered A: bit-exact against the shards stacked by rank.  C:
max|C - C_ref| <= 2e-3 max|C_ref| against the float64 oracle, and
bit-identical between the fused and the two-launch path (same GEMM core, same
order of additions).  Protocol state: bit-exact against its closed form
(oracle.ag_check_state), deterministic owners included.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import REL_TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mk():
    import gemm_tile_granular_amd as mk
    mk.set_num_workgroups(0)
    mk.set_timeout_us(2_000_000)
    mk.set_fault_skip_publish(-1)
    mk.set_controller_floor(2)
    mk.set_controller_cap(0)
    mk.set_adaptive_help(True)
    yield mk
    mk.set_partition("adaptive", 0)


def upload_ag(a0, ap, b):
    import torch
    dev = "cuda"
    A0 = torch.from_numpy(a0.view(np.int16)).to(dev).view(torch.bfloat16)
    AP = torch.from_numpy(ap.view(np.int16)).to(dev).view(torch.bfloat16) if ap.shape[0] else None
    B = torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)
    R, (Ms, K), N = ap.shape[0] + 1, a0.shape, b.shape[1]
    G = torch.full((R * Ms, K), 7.0, dtype=torch.bfloat16, device=dev)
    C = torch.full((R * Ms, N), -3.0, dtype=torch.float32, device=dev)
    return A0, AP, B, G, C


def run_ag(mk, fused, w, a0, ap, b, mode="adaptive", n=0):
    import torch
    A0, AP, B, G, C = upload_ag(a0, ap, b)
    print(f"[gpu] ag {'fused' if fused else 'unfused'} R={w.peers + 1} Ms={w.M} K={w.K} N={w.N} "
          f"tile {w.tile_m}x{w.tile_n} mode {mode} n={n}", flush=True)
    st = None
    if fused:
        mk.set_partition(mode, n)
        mk.allgather_gemm_local(A0, AP, G, B, C, w.tile_m, w.tile_n)
        st = mk.get_stats(maps=True)
    else:
        mk.allgather_gemm_unfused(A0, AP, G, B, C, w.tile_m, w.tile_n)
    torch.cuda.synchronize()
    g = G.cpu().view(torch.int16).numpy().view(np.uint16)
    return g, C.cpu().numpy(), st


def ag_protocol(st, w, mode, n):
    R, cps = w.peers + 1, w.M // w.tile_m
    Ch = R * cps
    tiles_n = -(-w.N // w.tile_n)
    T = Ch * tiles_n
    assert st["kind"] == 2 and st["num_tiles"] == T and st["num_chunks"] == Ch
    assert st["status"] == 0, st["status_name"]
    parts = oracle.ag_parts_per_chunk(w.tile_m, w.K, tiles_n)
    assert st["tiles_per_chunk"] == parts          # reported as copy tasks per chunk
    Q = Ch * parts
    assert st["compute_tasks"] == T and st["reduce_tasks"] == Q and st["chunks_released"] == Ch
    tpt = oracle.tiles_per_task(w.tile_m, w.tile_n)
    assert st["tiles_per_task"] == tpt
    maps = {"chunk_flag": st["chunk_flag"], "chunk_copy_cnt": st["chunk_cnt"],
            "tile_compute_cnt": st["tile_reduce_cnt"], "copy_owner": st["reduce_owner"][:Q],
            "compute_owner": st["compute_owner"]}
    bad = oracle.ag_check_state(maps, R, cps, tiles_n, st["epoch"], st["calls_since_reset"],
                                st["num_wg"], mode, n if mode != "adaptive" else st["n_reduce_initial"],
                                tpt, parts)
    assert not bad, bad
    return Q


def check_ag(g, C, a0, ap, b):
    gath, ref = oracle.allgather_gemm(a0, ap, b)
    assert np.array_equal(g, gath), "gathered A differs from the shards stacked by rank"
    err = float(np.max(np.abs(C.astype(np.float64) - ref))) if ref.size else 0.0
    bound = REL_TOL * float(np.max(np.abs(ref))) if ref.size else 0.0
    assert err <= bound, f"max|C-C_ref| = {err:.4e} > {bound:.4e}"


AG_SHAPES = [
    # R, Ms, K, N, tile_m, tile_n -- several chunks per shard, ragged N, K off the slab
    (4, 64, 256, 256, 64, 64),
    (3, 256, 200, 264, 128, 128),
    (2, 512, 512, 392, 256, 128),
    (1, 128, 64, 128, 128, 128),        # one rank: the gather is a copy of the local shard
    (8, 128, 128, 136, 64, 64),
    (5, 384, 1024, 512, 128, 128),      # K a whole number of slabs: the fast K loop
    (3, 128, 256, 1000, 64, 64),        # 16 block columns (ragged last tile): 8 bands of 2
    (4, 256, 512, 2600, 128, 128),      # 11 block columns, the last ragged: bands of 2 and 1
    (3, 256, 1784, 1024, 128, 128),     # 446 KiB chunks: 7 copy parts of unequal length
    (2, 512, 4104, 512, 256, 128),      # 2 MiB chunks, parts capped at tiles_n = 4
]


@pytest.mark.parametrize("shape", AG_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mode,n", [("adaptive", 0), ("static", 4), ("deterministic", 3)])
def test_allgather_gemm_full_oracle(mk, shape, mode, n):
    R, Ms, K, N, tm, tn = shape
    w = wl.custom(Ms, N, K, R - 1, tm, tn, 1, wid=800 + Ms % 97 + R)
    a0, ap, b = wl.make_ag_inputs(w)
    g, C, st = run_ag(mk, True, w, a0, ap, b, mode, n)
    check_ag(g, C, a0, ap, b)
    ag_protocol(st, w, mode, n)
    gu, Cu, _ = run_ag(mk, False, w, a0, ap, b)
    assert np.array_equal(g, gu)
    assert np.array_equal(C, Cu)


def test_allgather_back_to_back_epochs(mk):
    import torch
    w = wl.custom(128, 256, 256, 3, 64, 64, 1, wid=830)
    a0, ap, b = wl.make_ag_inputs(w)
    A0, AP, B, G, C = upload_ag(a0, ap, b)
    mk.set_partition("static", 5)
    for _ in range(3):
        mk.allgather_gemm_local(A0, AP, G, B, C, 64, 64)
    st = mk.get_stats(maps=True)
    assert st["calls_since_reset"] >= 3
    ag_protocol(st, w, "static", 5)
    torch.cuda.synchronize()
    check_ag(G.cpu().view(torch.int16).numpy().view(np.uint16), C.cpu().numpy(), a0, ap, b)


def test_allgather_waiting_compute_helps_copy(mk):
    """Adaptive with few copiers: compute workgroups whose chunk has not
    arrived copy meanwhile (marked on the copy owner); with help off none do."""
    w = wl.custom(256, 512, 512, 7, 64, 64, 1, wid=831)
    a0, ap, b = wl.make_ag_inputs(w)
    mk.set_controller_floor(1)
    try:
        g, C, st = run_ag(mk, True, w, a0, ap, b, "adaptive", 1)
        check_ag(g, C, a0, ap, b)
        Q = ag_protocol(st, w, "adaptive", 1)
        helped = int((st["reduce_owner"][:Q] >> 31).sum())
        print(f"[gpu] ag help: {helped} of {Q} copy tasks run by waiting compute workgroups", flush=True)
        assert helped > 0
        mk.set_adaptive_help(False)
        g, C, st = run_ag(mk, True, w, a0, ap, b, "adaptive", 1)
        check_ag(g, C, a0, ap, b)
        Q = ag_protocol(st, w, "adaptive", 1)
        assert not np.any(st["reduce_owner"][:Q] >> 31)
    finally:
        mk.set_adaptive_help(True)
        mk.set_controller_floor(2)


def test_allgather_timeout_is_reported_not_hung(mk):
    """A chunk whose arrival flag is never set: the bounded waits expire
    (20 ms), every workgroup leaves, and the launch reports MK_ERR_TIMEOUT;
    the next launch is clean."""
    w = wl.custom(128, 256, 128, 3, 64, 64, 1, wid=832)
    a0, ap, b = wl.make_ag_inputs(w)
    A0, AP, B, G, C = upload_ag(a0, ap, b)
    mk.set_timeout_us(20_000)
    mk.set_fault_skip_publish(5)       # a peer chunk (chunks 0-1 are local)
    try:
        for mode in ("deterministic", "adaptive"):
            mk.set_partition(mode, 2)
            print(f"[gpu] ag timeout case, mode {mode}", flush=True)
            mk.allgather_gemm_local(A0, AP, G, B, C, 64, 64)
            st = mk.get_stats(maps=True, raise_on_error=False)
            assert st["rc"] == mk.MK_ERR_TIMEOUT
    finally:
        mk.set_fault_skip_publish(-1)
        mk.set_timeout_us(2_000_000)
    g, C2, st = run_ag(mk, True, w, a0, ap, b, "static", 2)
    check_ag(g, C2, a0, ap, b)
    ag_protocol(st, w, "static", 2)


@pytest.mark.parametrize("name", ["ag_tp_share", "ag_compute_heavy"])
def test_allgather_full_size_sampled(mk, name):
    """The full-size shares in the launch the bench times: the gathered A
    bit-exact, C at sampled positions against the oracle one element at a
    time, fused equal to unfused everywhere."""
    w = wl.ag_workload(name)
    a0, ap, b = wl.make_ag_inputs(w)
    g, C, st = run_ag(mk, True, w, a0, ap, b, "adaptive", 0)
    ag_protocol(st, w, "adaptive", 0)
    gath = np.concatenate([a0] + [ap[p] for p in range(ap.shape[0])], axis=0)
    assert np.array_equal(g, gath)
    rng = np.random.default_rng(12)
    rows = rng.integers(0, gath.shape[0], 4096)
    cols = rng.integers(0, w.N, 4096)
    ref, _ = oracle.gemm_reduce_at(gath, b, np.zeros((0, 1, 1), np.float32), rows, cols)
    err = float(np.max(np.abs(C[rows, cols].astype(np.float64) - ref)))
    assert err <= REL_TOL * float(np.max(np.abs(ref))), err
    gu, Cu, _ = run_ag(mk, False, w, a0, ap, b)
    assert np.array_equal(C, Cu) and np.array_equal(g, gu)


@pytest.mark.parametrize("shape", [(3, 128, 256, 1000, 64, 64), (4, 256, 512, 2600, 128, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_allgather_column_bands_change_no_result(mk, shape):
    """Compute claims in 1, 2, 4 or 8 column bands (one queue per XCD) move
    blocks between workgroups only: the gathered A and C are bit-identical
    for every band count, and the protocol state matches its closed form."""
    R, Ms, K, N, tm, tn = shape
    w = wl.custom(Ms, N, K, R - 1, tm, tn, 1, wid=840 + R)
    a0, ap, b = wl.make_ag_inputs(w)
    base = None
    try:
        for bands in (1, 2, 4, 8):
            mk.set_xcd_bands(bands)
            g, C, st = run_ag(mk, True, w, a0, ap, b, "adaptive", 0)
            ag_protocol(st, w, "adaptive", 0)
            assert st["xcd_bands"] in (1, bands)
            if base is None:
                check_ag(g, C, a0, ap, b)
                base = (g, C)
            else:
                assert np.array_equal(g, base[0]) and np.array_equal(C, base[1])
    finally:
        mk.set_xcd_bands(0)


def test_allgather_same_grid_different_parts(mk):
    """Two shapes with the same tile grid and chunk count (T = 16, 4 chunks)
    but 4 and 1 copy tasks per chunk, alternated: the per-chunk counters
    restart with the part count, so every launch completes and matches its
    closed form."""
    shapes = [(2, 512, 4104, 512, 256, 128), (4, 64, 256, 256, 64, 64)]
    for i in range(4):
        R, Ms, K, N, tm, tn = shapes[i % 2]
        w = wl.custom(Ms, N, K, R - 1, tm, tn, 1, wid=850 + i % 2)
        a0, ap, b = wl.make_ag_inputs(w)
        g, C, st = run_ag(mk, True, w, a0, ap, b, "static", 2)
        check_ag(g, C, a0, ap, b)
        ag_protocol(st, w, "static", 2)


@pytest.mark.parametrize("nwg,mode,n", [(2, "adaptive", 0), (2, "static", 1), (3, "deterministic", 1),
                                        (5, "adaptive", 0), (5, "static", 2)])
def test_allgather_few_workgroups(mk, nwg, mode, n):
    """Grids of 2-5 workgroups: every chunk still arrives (a copy workgroup
    never computes while copies remain) and every block is computed once."""
    mk.set_num_workgroups(nwg)
    try:
        w = wl.custom(128, 136, 128, 2, 64, 64, 1, wid=870 + nwg)
        a0, ap, b = wl.make_ag_inputs(w)
        g, C, st = run_ag(mk, True, w, a0, ap, b, mode, n)
        assert st["num_wg"] == nwg
        check_ag(g, C, a0, ap, b)
        ag_protocol(st, w, mode, n)
    finally:
        mk.set_num_workgroups(0)
