"""GPU parity for one rank's share of GEMM+ReduceScatter: the fused and unfused
entry points (through the C ABI) against oracle.gemm_reduce_scatter.

The shard (C on this rank's tile rows) and the inbox slots (`remote` on the
other ranks' rows): max|X - X_ref| <= 2e-3 max|X_ref|, with the GEMM part of
the shard checked on its own (C - sum(peers)).  The rows each output must
leave alone (C past the shard, remote on it): bit-exact, untouched.  Fused
and unfused: bit-identical (the same GEMM core, the same order of
additions).  Protocol state:
bit-exact against its closed forms.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import REL_TOL, check_full, check_protocol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mk():
    import gemm_tile_granular_amd as mk
    mk.set_num_workgroups(0)
    mk.set_timeout_us(2_000_000)
    mk.set_fault_skip_publish(-1)
    mk.set_controller_floor(2)
    mk.set_controller_cap(0)
    mk.set_xcd_bands(0)
    yield mk
    mk.set_partition("adaptive", 0)


C_FILL = 12345.0   # C's rows outside the shard must keep this


def run_rs(mk, fused, w, a, b, p, r0, mode="adaptive", n_reduce=3):
    import torch
    from gemm_tile_granular_amd.tensors import upload
    A, B, P, C = upload(a, b, p)
    C.fill_(C_FILL)
    R = torch.from_numpy(np.ascontiguousarray(r0)).to(C.device)
    print(f"[gpu] rs {'fused' if fused else 'unfused'} {w.M}x{w.N}x{w.K} P={w.peers} "
          f"tile {w.tile_m}x{w.tile_n} tpc {w.tiles_per_chunk} mode {mode}", flush=True)
    st = None
    if fused:
        mk.set_partition(mode, n_reduce)
        mk.gemm_reduce_scatter_local(A, B, P, C, R, w.tile_m, w.tile_n, w.tiles_per_chunk)
        st = mk.get_stats(maps=True)
    else:
        mk.gemm_reduce_scatter_unfused(A, B, P, C, R, w.tile_m, w.tile_n, w.tiles_per_chunk)
    torch.cuda.synchronize()
    return C.cpu().numpy(), R.cpu().numpy(), st


def own_rows(w):
    tiles_m = -(-w.M // w.tile_m)
    return min(w.M, int(oracle.rs_shard_bounds(tiles_m, w.peers + 1)[1]) * w.tile_m)


def check_rs_protocol(st, w, mode, n_reduce):
    # the fused protocol covers the shard's tile rows; a rank that owns none
    # runs the GEMM alone, with no fused launch to check
    own = own_rows(w)
    if own:
        check_protocol(st, dataclasses.replace(w, M=own), mode, n_reduce)


def check_rs_full(C, remote, a, b, p, r0, w):
    M, N = C.shape
    own = own_rows(w)
    shard, Rref = oracle.gemm_reduce_scatter(a, b, p, r0, w.tile_m)
    assert shard.shape == (own, N)
    # both outputs against the oracle on the rows they own
    for got, ref, name in ((C[:own], shard, "shard"), (remote[own:], Rref[own:], "remote")):
        if ref.size:
            err = float(np.max(np.abs(got.astype(np.float64) - ref)))
            bound = REL_TOL * float(np.max(np.abs(ref)))
            assert err <= bound, f"max|{name}-ref| = {err:.4e} > {bound:.4e}"
    if own:
        check_full(C[:own], a[:own], b, np.ascontiguousarray(p[:, :own]))
    if own < M:
        empty = np.zeros((0, M - own, N), np.float32)
        check_full(remote[own:], a[own:], b, empty)
    # the rows each output leaves alone
    assert np.all(C[own:] == np.float32(C_FILL))
    assert np.array_equal(remote[:own], r0[:own])


RS_SHAPES = [
    # M, N, K, P, tile_m, tile_n, tpc -- R = P + 1 ranks; ragged M/N/K tails
    (200, 136, 72, 3, 64, 64, 4),        # 4 tile rows, one per rank
    (333, 264, 136, 2, 128, 128, 4),     # 3 tile rows, R = 3
    (520, 392, 200, 5, 256, 128, 3),     # 3 tile rows, R = 6: rank 0 owns none
    (1100, 264, 200, 1, 128, 128, 4),    # 9 tile rows, R = 2: own 4, ragged last row sent
    (1000, 1000, 1024, 3, 128, 128, 4),  # fast K loop, 2 of 8 tile rows own
    (600, 520, 512, 2, 256, 128, 4),
    (300, 328, 512, 7, 64, 64, 4),       # 5 tile rows, R = 8: own none
    (130, 520, 8, 1, 64, 64, 1),         # one K slab
]


@pytest.mark.parametrize("shape", RS_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mode", ["adaptive", "deterministic"])
def test_reduce_scatter_full_oracle(mk, shape, mode):
    M, N, K, P, tm, tn, tpc = shape
    w = wl.custom(M, N, K, P, tm, tn, tpc, wid=700 + M % 89)
    a, b, p = wl.make_inputs(w)
    r0 = wl.make_remote(w)
    C, R, st = run_rs(mk, True, w, a, b, p, r0, mode=mode)
    check_rs_full(C, R, a, b, p, r0, w)
    check_rs_protocol(st, w, mode, 3)
    Cu, Ru, _ = run_rs(mk, False, w, a, b, p, r0)
    assert np.array_equal(C, Cu)
    assert np.array_equal(R, Ru)


STATIC_RS_SHAPES = [(1000, 1000, 1024, 3, 128, 128, 4), (600, 520, 512, 2, 256, 128, 4),
                    (200, 136, 72, 3, 64, 64, 4)]


@pytest.mark.parametrize("shape", STATIC_RS_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("which", ["2", "8", "B-8"])
def test_reduce_scatter_static_partitions(mk, shape, which):
    """Static partitions on the reduce-scatter share: few reducers (compute
    workgroups leave for the outside rows early), one per XCD (the smallest
    XCD-local static split) and all but one per XCD (the largest)."""
    M, N, K, P, tm, tn, tpc = shape
    n = {"2": 2, "8": 8, "B-8": mk.device_cu_count() - 8}[which]
    w = wl.custom(M, N, K, P, tm, tn, tpc, wid=720 + M % 83)
    a, b, p = wl.make_inputs(w)
    r0 = wl.make_remote(w)
    C, R, st = run_rs(mk, True, w, a, b, p, r0, mode="static", n_reduce=n)
    check_rs_full(C, R, a, b, p, r0, w)
    check_rs_protocol(st, w, "static", n)
    Cu, Ru, _ = run_rs(mk, False, w, a, b, p, r0)
    assert np.array_equal(C, Cu)
    assert np.array_equal(R, Ru)


def test_reduce_scatter_one_rank_is_the_gemm(mk):
    # R = 1: rank 0 owns every row; no remote buffer
    import torch
    from gemm_tile_granular_amd.tensors import upload
    w = wl.custom(300, 200, 264, 0, 128, 128, 4, wid=790)
    a, b, p = wl.make_inputs(w)
    A, B, P, C = upload(a, b, p)
    mk.set_partition("static", 4)
    mk.gemm_reduce_scatter_local(A, B, None, C, None, 128, 128, 4)
    torch.cuda.synchronize()
    check_full(C.cpu().numpy(), a, b, p)


@pytest.mark.parametrize("name,mode,n", [("tp_share", "adaptive", 3), ("compute_heavy", "adaptive", 3),
                                         ("tp_share", "static", 2), ("tp_share", "static", 8),
                                         ("tp_share", "static", -8)])
def test_reduce_scatter_full_size_sampled(mk, name, mode, n):
    """The 4096x4096x1792 (128x128 tiles) and 16384x8192x8192 (256x128 tiles)
    8-rank shares at full size, in the launch the bench times (and the
    4096x4096x1792 share under static partitions, XCD-local at 8 and B-8):
    sampled elements against the oracle one at a time, the untouched rows
    bit-exact, and fused equal to unfused everywhere."""
    w = wl.workload(name)
    if n < 0:
        n = mk.device_cu_count() + n
    a, b, p = wl.make_inputs(w)
    r0 = wl.make_remote(w)
    C, R, st = run_rs(mk, True, w, a, b, p, r0, mode=mode, n_reduce=n)
    check_rs_protocol(st, w, mode, n)
    if mode == "static" and 8 <= n <= mk.device_cu_count() - 8:
        assert st["xcd_local"] == 1
    own = own_rows(w)
    rng = np.random.default_rng(11)
    for lo, hi, reduced in ((0, own, True), (own, w.M, False)):
        if lo == hi:
            continue
        rows = rng.integers(lo, hi, 2048)
        cols = rng.integers(0, w.N, 2048)
        ref, gemm = oracle.gemm_reduce_at(a, b, p, rows, cols)
        scale = float(np.max(np.abs(ref if reduced else gemm)))
        got = (C if reduced else R)[rows, cols].astype(np.float64)
        err = float(np.max(np.abs(got - (ref if reduced else gemm))))
        assert err <= REL_TOL * scale, (lo, hi, err, scale)
    assert np.array_equal(R[:own], r0[:own])
    assert np.all(C[own:] == np.float32(C_FILL))
    Cu, Ru, _ = run_rs(mk, False, w, a, b, p, r0)
    assert np.array_equal(C, Cu)
    assert np.array_equal(R, Ru)


@pytest.mark.parametrize("nwg,mode,n", [(2, "deterministic", 1), (2, "static", 1), (3, "static", 2),
                                        (5, "adaptive", 3)])
def test_reduce_scatter_few_workgroups(mk, nwg, mode, n):
    """Grids of 2-5 workgroups: the shard's tiles are computed and reduced
    once each and every outside row still reaches its inbox."""
    mk.set_num_workgroups(nwg)
    try:
        w = wl.custom(1100, 264, 200, 1, 128, 128, 4, wid=760 + nwg)
        a, b, p = wl.make_inputs(w)
        r0 = wl.make_remote(w)
        C, R, st = run_rs(mk, True, w, a, b, p, r0, mode=mode, n_reduce=n)
        assert st["num_wg"] == nwg
        check_rs_full(C, R, a, b, p, r0, w)
        check_rs_protocol(st, w, mode, n)
    finally:
        mk.set_num_workgroups(0)
