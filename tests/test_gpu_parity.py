"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Outputs: max|C - C_ref| <= 2e-3 max|C_ref|, and the same bound on the GEMM
part C - sum(peers) against A.B (so a dropped K slab cannot hide under the
peers).  Counters, flags and ownership maps: bit-exact against their closed
forms.  Sizes span several tiles with ragged tails; the named workloads run
at full size with sampled outputs.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import check_full, check_protocol, check_sampled, run_fused, run_unfused

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
    mk.set_num_workgroups(0)
    mk.set_xcd_bands(0)


def test_device_is_the_expected_one(mk):
    n = mk.device_cu_count()
    print(f"[gpu] compute units: {n}", flush=True)
    assert n >= 2


@pytest.mark.parametrize("mode,n", [("deterministic", 2), ("static", 2), ("adaptive", 2),
                                    ("deterministic", 7), ("static", 100)])
def test_tiny_workload_full_oracle(mk, mode, n):
    w = wl.workload("tiny")
    a, b, p = wl.make_inputs(w)
    C, st = run_fused(mk, w, a, b, p, mode=mode, n_reduce=n)
    check_full(C, a, b, p)
    check_protocol(st, w, mode, n)


SHAPES = [
    # M, N, K, P, tile_m, tile_n, tpc  -- several tiles, ragged M/N/K tails
    (200, 136, 72, 3, 64, 64, 4),
    (333, 264, 136, 2, 128, 128, 4),
    (520, 392, 200, 5, 256, 128, 3),
    (64, 64, 64, 1, 64, 64, 4),          # exactly one tile, chunk shorter than 4
    (1000, 1000, 1000, 7, 128, 128, 4),  # 64 tiles, 16 chunks
    (130, 520, 8, 1, 64, 64, 1),         # K = 8: a single partial slab
    (97, 1024, 328, 9, 64, 64, 5),       # odd peer count (not a multiple of 4)
    # 9 tile rows (XCD-local partitions, one holding two rows) and 3 tile
    # columns: the two-tile blocks of each row end in a one-tile block, whose
    # second reduce ticket is empty
    (1100, 264, 200, 3, 128, 128, 4),
    (2100, 264, 136, 2, 256, 128, 4),
    # K a multiple of the K slab and long enough for the steady-state loop:
    # interior blocks take the GEMM core's fast path (loads spread over the
    # k-steps), the ragged last row and column of blocks the checked path,
    # in the same launch
    (1000, 1000, 1024, 3, 128, 128, 4),
    (600, 520, 512, 2, 256, 128, 4),
    (300, 328, 512, 2, 64, 64, 4),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mode", ["adaptive", "deterministic"])
def test_ragged_shapes_full_oracle(mk, shape, mode):
    M, N, K, P, tm, tn, tpc = shape
    w = wl.custom(M, N, K, P, tm, tn, tpc, wid=400 + M % 97)
    a, b, p = wl.make_inputs(w)
    C, st = run_fused(mk, w, a, b, p, mode=mode, n_reduce=3)
    check_full(C, a, b, p)
    check_protocol(st, w, mode, 3)


def test_unfused_baseline_full_oracle(mk):
    for shape in SHAPES[:3] + SHAPES[-3:] + [(256, 256, 512, 1, 64, 64, 4)]:
        M, N, K, P, tm, tn, tpc = shape
        w = wl.custom(M, N, K, P, tm, tn, tpc, wid=500)
        a, b, p = wl.make_inputs(w)
        C = run_unfused(mk, w, a, b, p)
        check_full(C, a, b, p)


def test_no_peers_is_the_gemm(mk):
    w = wl.custom(300, 200, 264, 0, 128, 128, 4, wid=600)
    a, b, p = wl.make_inputs(w)
    C, st = run_fused(mk, w, a, b, p, mode="static", n_reduce=4)
    check_full(C, a, b, p)
    check_protocol(st, w, "static", 4)


def test_zero_a_gives_the_peer_sum(mk):
    w = wl.custom(256, 320, 128, 6, 64, 64, 4, wid=601, zero_rows_frac=1.0)
    a, b, p = wl.make_inputs(w)
    assert not a.any()
    C, st = run_fused(mk, w, a, b, p, mode="adaptive", n_reduce=2)
    check_full(C, a, b, p)
    check_protocol(st, w, "adaptive", 2)


def test_zero_k_gives_the_peer_sum(mk):
    w = wl.custom(192, 128, 0, 3, 64, 64, 4, wid=602)
    a, b, p = wl.make_inputs(w)
    C, st = run_fused(mk, w, a, b, p, mode="static", n_reduce=2)
    check_full(C, a, b, p)
    check_protocol(st, w, "static", 2)


def test_identity_b_gives_a_plus_peers(mk):
    n = 256
    w = wl.custom(192, n, n, 2, 64, 64, 4, wid=603)
    a, _, p = wl.make_inputs(w)
    b = wl.round_to_bf16_bits(np.eye(n, dtype=np.float32))
    C, st = run_fused(mk, w, a, b, p, mode="deterministic", n_reduce=5)
    av = oracle.bf16_bits_to_f64(a)
    want = av + p.astype(np.float64).sum(0)
    absum = np.abs(av) + np.abs(p.astype(np.float64)).sum(0)
    assert np.all(np.abs(C.astype(np.float64) - want) <= 3 * 2.0 ** -24 * absum)
    check_protocol(st, w, "deterministic", 5)


def test_back_to_back_epochs_and_counters(mk):
    w = wl.custom(512, 512, 256, 2, 128, 128, 4, wid=604)
    a, b, p = wl.make_inputs(w)
    C1, s1 = run_fused(mk, w, a, b, p, mode="adaptive", n_reduce=2)
    C2, s2 = run_fused(mk, w, a, b, p, mode="static", n_reduce=3)
    C3, s3 = run_fused(mk, w, a, b, p, mode="deterministic", n_reduce=1)
    assert s1["epoch"] < s2["epoch"] < s3["epoch"]
    assert s2["calls_since_reset"] == s1["calls_since_reset"] + 1
    assert s3["calls_since_reset"] == s1["calls_since_reset"] + 2
    for C, st, mode, n in ((C1, s1, "adaptive", 2), (C2, s2, "static", 3),
                           (C3, s3, "deterministic", 1)):
        check_full(C, a, b, p)
        check_protocol(st, w, mode, n)
    # flags never decrease between calls
    assert np.all(s2["tile_flag"] >= s1["tile_flag"]) and np.all(s3["tile_flag"] >= s2["tile_flag"])
    # a new tile count restarts the per-call counters (16 tiles before, 12 now)
    w2 = wl.custom(192, 256, 64, 1, 64, 64, 4, wid=605)
    a2, b2, p2 = wl.make_inputs(w2)
    C4, s4 = run_fused(mk, w2, a2, b2, p2, mode="static", n_reduce=2)
    assert s4["calls_since_reset"] == 1 and s4["epoch"] == s3["epoch"] + 1
    check_full(C4, a2, b2, p2)
    check_protocol(s4, w2, "static", 2)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 255])
def test_static_partition_sweep(mk, n):
    w = wl.custom(1024, 1024, 512, 3, 128, 128, 4, wid=606)
    a, b, p = wl.make_inputs(w)
    C, st = run_fused(mk, w, a, b, p, mode="static", n_reduce=n)
    check_full(C, a, b, p)
    check_protocol(st, w, "static", n)


@pytest.mark.parametrize("nwg,mode,n", [(2, "deterministic", 1), (3, "static", 2),
                                        (8, "adaptive", 2), (5, "deterministic", 3)])
def test_few_workgroups(mk, nwg, mode, n):
    mk.set_num_workgroups(nwg)
    try:
        w = wl.custom(320, 256, 128, 2, 64, 64, 4, wid=607)
        a, b, p = wl.make_inputs(w)
        C, st = run_fused(mk, w, a, b, p, mode=mode, n_reduce=n)
        assert st["num_wg"] == nwg
        check_full(C, a, b, p)
        check_protocol(st, w, mode, n)
    finally:
        mk.set_num_workgroups(0)


def test_controller_device_matches_host_closed_form(mk):
    import json, os
    rows = []
    rng = np.random.default_rng(11)
    for _ in range(4000):
        B = int(rng.integers(2, 1025))
        T = int(rng.integers(1, 1 << 22))
        cd = int(rng.integers(0, T + 1))
        rd = int(rng.integers(0, T + 1))
        sp = int(rng.integers(0, 1 << 40)) if cd else 0
        ss = int(rng.integers(0, 1 << 40)) if rd else 0
        cur = int(rng.integers(1, B + 1))
        fl = int(rng.integers(1, 70))
        kp = int(rng.choice([1, 8])) if B > 8 else 1
        cap = int(rng.choice([B, B // 2 or 1, int(rng.integers(1, B + 1))]))
        rows.append((B, T, cd, rd, sp, ss, cur, fl, kp, cap))
    # the hand-worked table, expressed as progress counters with exact means
    with open(os.path.join(os.path.dirname(__file__), "golden", "controller_table.json")) as f:
        g = json.load(f)
    for B, R_s, C_s, R_p, C_p, _, _ in g["rows"]:
        T = max(R_s, R_p) + 5
        rows.append((B, T, T - R_p, T - R_s, (T - R_p) * C_p, (T - R_s) * C_s, 7 if B > 7 else 1, 2, 1, B))
    table = np.array(rows, dtype=np.uint64)
    got = mk.controller_eval(table)
    want = np.array([oracle.controller_update(*[int(x) for x in r[:6]], current=int(r[6]),
                                              floor=int(r[7]), keep=int(r[8]), cap=int(r[9]))
                     for r in rows],
                    dtype=np.uint32)
    mism = np.nonzero(got != want)[0]
    assert mism.size == 0, [(rows[i], int(got[i]), int(want[i])) for i in mism[:5]]


def test_timeout_is_reported_not_hung(mk):
    """A compute task that never publishes its flag: the bounded waits expire
    (20 ms), the kernel ends, and the launch reports MK_ERR_TIMEOUT; the next
    launch is clean."""
    w = wl.custom(256, 256, 64, 1, 64, 64, 4, wid=608)
    a, b, p = wl.make_inputs(w)
    mk.set_timeout_us(20_000)
    mk.set_fault_skip_publish(5)
    try:
        from gemm_tile_granular_amd.tensors import upload
        A, B, P, C = upload(a, b, p)
        for mode in ("deterministic", "adaptive"):
            mk.set_partition(mode, 2)
            print(f"[gpu] timeout case, mode {mode}", flush=True)
            mk.gemm_reduce_local(A, B, P, C, 64, 64, 4)
            st = mk.get_stats(maps=True, raise_on_error=False)
            assert st["rc"] == mk.MK_ERR_TIMEOUT and st["status"] == mk.MK_ERR_TIMEOUT
            assert st["tile_flag"][5] != st["epoch"]
    finally:
        mk.set_fault_skip_publish(-1)
        mk.set_timeout_us(2_000_000)
    C2, st2 = run_fused(mk, w, a, b, p, mode="static", n_reduce=2)
    check_full(C2, a, b, p)
    check_protocol(st2, w, "static", 2)


def test_timeout_in_an_earlier_launch_is_not_lost(mk):
    """Errors are sticky: a launch that times out, then clean launches of the
    same shape with no report in between.  The next report still names the
    timeout, the clean launches' output is right, and after the report a
    launch starts from cleared counters (protocol state exact again)."""
    import torch
    from gemm_tile_granular_amd.tensors import upload
    w = wl.custom(256, 256, 64, 1, 64, 64, 4, wid=609)
    a, b, p = wl.make_inputs(w)
    A, B, P, C = upload(a, b, p)
    mk.set_partition("static", 2)
    mk.set_timeout_us(20_000)
    mk.set_fault_skip_publish(5)
    try:
        print("[gpu] sticky timeout: faulted launch", flush=True)
        mk.gemm_reduce_local(A, B, P, C, 64, 64, 4)
    finally:
        mk.set_fault_skip_publish(-1)
        mk.set_timeout_us(2_000_000)
    print("[gpu] sticky timeout: two clean launches", flush=True)
    for _ in range(2):
        mk.gemm_reduce_local(A, B, P, C, 64, 64, 4)
    st = mk.get_stats(maps=False, raise_on_error=False)
    assert st["rc"] == mk.MK_ERR_TIMEOUT and st["status"] == mk.MK_ERR_TIMEOUT, st["status_name"]
    assert st["sticky_errors"] & 1
    torch.cuda.synchronize()
    check_full(C.cpu().numpy(), a, b, p)
    C2, st2 = run_fused(mk, w, a, b, p, mode="static", n_reduce=2)
    check_full(C2, a, b, p)
    check_protocol(st2, w, "static", 2)
    assert st2["sticky_errors"] == 0


def check_release_order(st, w):
    """Each chunk's release stamp is no earlier than the end of every tile in
    it (the last reduced tile lets the chunk go), and follows it closely."""
    T, tpc = w.tiles, w.tiles_per_chunk
    rel = st["chunk_release"].astype(np.uint32)
    rend = st["reduce_end"].astype(np.uint32)
    lags = []
    for c in range(w.chunks):
        tiles = np.arange(c * tpc, min(T, (c + 1) * tpc))
        d = (rel[c] - rend[tiles]).astype(np.uint32).view(np.int32).astype(np.int64)
        assert np.all(d >= 0), (c, d)
        lags.append(int(d.min()))
    hz = float(st["timer_hz"])
    lags_us = np.array(lags) / hz * 1e6
    # the release follows its last tile by about one atomic round trip
    assert float(np.max(lags_us)) < 1000.0, float(np.max(lags_us))
    return lags_us


@pytest.mark.parametrize("mode", ["adaptive", "static", "deterministic"])
def test_chunk_release_follows_its_last_tile(mk, mode):
    w = wl.custom(1000, 1000, 512, 3, 128, 128, 4, wid=611)
    a, b, p = wl.make_inputs(w)
    C, st = run_fused(mk, w, a, b, p, mode=mode, n_reduce=5)
    check_full(C, a, b, p)
    check_protocol(st, w, mode, 5)
    lags = check_release_order(st, w)
    print(f"[gpu] {mode}: release lag median {np.median(lags):.2f} us, max {lags.max():.2f} us",
          flush=True)


def test_plain_controller_rule(mk):
    """The pages' rule without this library's labelled variants: initial
    target 2, no cap below B - keep, and reducers that wait instead of
    helping.  Output against the oracle, protocol exact, no help marks."""
    w = wl.custom(1000, 1000, 1024, 7, 128, 128, 4, wid=612)
    a, b, p = wl.make_inputs(w)
    mk.set_adaptive_help(False)
    mk.set_controller_cap(1024)
    try:
        C, st = run_fused(mk, w, a, b, p, mode="adaptive", n_reduce=2)
    finally:
        mk.set_adaptive_help(True)
        mk.set_controller_cap(0)
    check_full(C, a, b, p)
    check_protocol(st, w, "adaptive", 2)
    assert st["adaptive_help"] == 0
    assert not np.any(st["compute_owner"] >> 31)
    assert st["controller_cap"] == st["num_wg"] - st["keep_compute"]


FULL = ["tp_share", "reduce_heavy", "compute_heavy", "wide_many_peer"]


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size_workload_sampled(mk, name):
    w = wl.workload(name)
    a, b, p = wl.make_inputs(w)
    # the launch configuration the benchmark times: the library's default
    # initial target (the controller cap) and cap
    C, st = run_fused(mk, w, a, b, p, mode="adaptive", n_reduce=0)
    check_protocol(st, w, "adaptive", 0)
    check_release_order(st, w)
    tiles_m, tiles_n = oracle.tile_grid(w.M, w.N, w.tile_m, w.tile_n)
    rng = np.random.default_rng(7)
    check_sampled(C, a, b, p, rng, tiles=[(0, 0), (tiles_m - 1, tiles_n - 1),
                                          (tiles_m // 2, tiles_n // 3)],
                  tile=(w.tile_m, w.tile_n))
    if w.zero_rows_frac:
        nz = int(np.floor(w.zero_rows_frac * w.M))
        ps = p[:, :nz].astype(np.float64).sum(0)
        absum = np.abs(p[:, :nz].astype(np.float64)).sum(0)
        assert np.all(np.abs(C[:nz].astype(np.float64) - ps) <= w.peers * 2.0 ** -24 * absum + 1e-30)
    print(f"[gpu] {name}: n_reduce initial {st['n_reduce_initial']} final {st['n_reduce_final']} "
          f"range [{st['n_reduce_min_seen']}, {st['n_reduce_max_seen']}] "
          f"switches {st['role_switches']} cap {st['controller_cap']} "
          f"help tiles {int((st['compute_owner'] >> 31).sum())}", flush=True)


def test_adaptive_reducers_help_compute_while_waiting(mk):
    # 16 workgroups (8 per role at the start), 32 blocks of 128x256 with
    # K = 4096: no block can be published before every reducer's first
    # readiness check, so reducers take compute blocks (marked as help) and
    # keep their tickets; the result and the protocol must not change.
    mk.set_num_workgroups(16)
    mk.set_controller_cap(8)
    try:
        w = wl.custom(1024, 1024, 4096, 3, 128, 128, 4, wid=611)
        a, b, p = wl.make_inputs(w)
        C, st = run_fused(mk, w, a, b, p, mode="adaptive", n_reduce=8)
        check_full(C, a, b, p)
        check_protocol(st, w, "adaptive", 8)
        help_tiles = int((st["compute_owner"] >> 31).sum())
        print(f"[gpu] help tiles {help_tiles} cap {st['controller_cap']} local {st['xcd_local']}",
              flush=True)
        assert st["controller_cap"] == 8
        assert help_tiles >= 1
    finally:
        mk.set_num_workgroups(0)
        mk.set_controller_cap(0)


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size_static_and_unfused_sampled(mk, name):
    w = wl.workload(name)
    a, b, p = wl.make_inputs(w)
    C, st = run_fused(mk, w, a, b, p, mode="static", n_reduce=16)
    check_protocol(st, w, "static", 16)
    rng = np.random.default_rng(8)
    check_sampled(C, a, b, p, rng, n_samples=2048)
    Cu = run_unfused(mk, w, a, b, p)
    check_sampled(Cu, a, b, p, rng, n_samples=2048)


def test_alternating_inputs_same_output_buffer(mk):
    """Two input sets through one C buffer, back to back: a reducer that read a
    stale copy of a partial tile (the previous call's values at the same
    addresses) would fail the comparison."""
    import torch
    from gemm_tile_granular_amd.tensors import upload
    w1 = wl.custom(2048, 2048, 512, 7, 128, 128, 4, wid=700, dist_peer=("normal", 0.5))
    w2 = wl.custom(2048, 2048, 512, 7, 128, 128, 4, wid=701, dist_peer=("normal", 3.0))
    sets = []
    for w in (w1, w2):
        a, b, p = wl.make_inputs(w)
        A, B, P, _ = upload(a, b, p)
        sets.append((w, a, b, p, A, B, P))
    C = torch.empty((2048, 2048), dtype=torch.float32, device="cuda:0")
    for i, mode in enumerate(["adaptive", "static", "adaptive", "deterministic", "adaptive", "static"]):
        w, a, b, p, A, B, P = sets[i % 2]
        mk.set_partition(mode, 64 if mode != "adaptive" else 2)
        print(f"[gpu] alternating call {i}: input set {i % 2}, mode {mode}", flush=True)
        mk.gemm_reduce_local(A, B, P, C, 128, 128, 4)
        st = mk.get_stats(maps=True)
        check_full(C.cpu().numpy(), a, b, p)
        check_protocol(st, w, mode, 64 if mode != "adaptive" else 2)


# XCD-local partitions as row groups x column bands of whole chunks, forced to
# each split the shape allows.  (M, N, K, P, bands, expected bands): 8 tile
# rows by 8 chunk columns allow every split; 9 tile rows by 5 chunk columns
# give ragged row groups and bands of unequal width (5 chunks over 4 bands),
# and 8 bands fall back to the most the shape allows (4).
BAND_CASES = [
    (1024, 4096, 256, 2, 1, 1), (1024, 4096, 256, 2, 2, 2),
    (1024, 4096, 256, 2, 4, 4), (1024, 4096, 256, 2, 8, 8),
    (1100, 2560, 192, 3, 2, 2), (1100, 2560, 192, 3, 4, 4), (1100, 2560, 192, 3, 8, 4),
]


@pytest.mark.parametrize("case", BAND_CASES, ids=lambda c: "x".join(map(str, c)))
def test_xcd_column_bands_full_oracle(mk, case):
    M, N, K, P, bands, used = case
    w = wl.custom(M, N, K, P, 128, 128, 4, wid=700 + bands)
    a, b, p = wl.make_inputs(w)
    mk.set_xcd_bands(bands)
    try:
        C, st = run_fused(mk, w, a, b, p, mode="adaptive", n_reduce=0)
        print(f"[gpu] bands forced {bands}: used {st['xcd_bands']} local {st['xcd_local']}", flush=True)
        if st["xcd_local"]:
            assert st["xcd_bands"] == used
        check_full(C, a, b, p)
        check_protocol(st, w, "adaptive", 0)
        # the split moves work between XCDs, not the order of any sum
        mk.set_xcd_bands(1)
        C1, _ = run_fused(mk, w, a, b, p, mode="adaptive", n_reduce=0, maps=False)
        assert np.array_equal(C, C1)
        Cu = run_unfused(mk, w, a, b, p)
        assert np.array_equal(C, Cu)
    finally:
        mk.set_xcd_bands(0)
