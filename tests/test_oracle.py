"""Pins for the CPU oracle: each function is tied to something other than itself.

* result definition: a hand-worked fixture, closed forms (no peers, A = 0,
  B = I, all-ones, rank-1, integer operands against exact integer arithmetic)
  and an independent C brute force;
* controller: a hand-worked table and the defining equal-finish-time
  condition of the adaptive partition rule;
* protocol checker: the closed-form state is accepted, every kind of
  corruption is rejected;
* mutation checks: a planted mistake in the oracle (dropped term, wrong sign,
  transposed operand, wrong index, wrong rounding, missing clamp) fails at
  least one pin.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits_of(values):
    return wl.round_to_bf16_bits(np.asarray(values, dtype=np.float32))


# ---------------------------------------------------------------------------
# result pins, written so that any implementation can be checked
# ---------------------------------------------------------------------------

def pin_golden(fn):
    g = _load("tiny_gemm_reduce.json")
    a = np.array(g["A_bits"], dtype=np.uint16)
    b = np.array(g["B_bits"], dtype=np.uint16)
    peers = np.array(g["peers"], dtype=np.float32)
    np.testing.assert_array_equal(_bits_of(g["A_values"]), a)
    np.testing.assert_array_equal(_bits_of(g["B_values"]), b)
    got = fn(a, b, peers)
    return np.array_equal(got, np.array(g["C"]))


def pin_no_peers_is_integer_matmul(fn):
    # integer-valued bf16 operands: the product is exact in float64 and equals
    # exact integer arithmetic
    rng = np.random.default_rng(3)
    ai = rng.integers(-8, 9, size=(5, 7))
    bi = rng.integers(-8, 9, size=(7, 6))
    got = fn(_bits_of(ai), _bits_of(bi), np.zeros((0, 5, 6), np.float32))
    want = np.array([[sum(int(ai[i, k]) * int(bi[k, j]) for k in range(7)) for j in range(6)]
                     for i in range(5)])
    return got.shape == want.shape and np.array_equal(got, want)


def pin_zero_a_is_peer_sum(fn):
    peers = np.array([[[1.5, -2.0, 0.25]], [[4.0, 0.5, -0.75]], [[-1.0, 1.0, 2.0]]],
                     dtype=np.float32)               # [3, 1, 3]
    a = np.zeros((1, 4), np.uint16)
    b = _bits_of(np.arange(12, dtype=np.float32).reshape(4, 3))
    got = fn(a, b, peers)
    return np.array_equal(got, np.array([[4.5, -0.5, 1.5]]))


def pin_identity_b(fn):
    rng = np.random.default_rng(4)
    a = _bits_of(rng.uniform(-3, 3, size=(4, 6)).astype(np.float32))
    b = _bits_of(np.eye(6, dtype=np.float32))
    peers = rng.standard_normal((2, 4, 6)).astype(np.float32)
    got = fn(a, b, peers)
    av = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = av + peers[0].astype(np.float64) + peers[1].astype(np.float64)
    return np.allclose(got, want, rtol=0, atol=1e-12)


def pin_all_ones(fn):
    K = 37
    a = _bits_of(np.ones((3, K), np.float32))
    b = _bits_of(np.ones((K, 2), np.float32))
    peers = np.full((4, 3, 2), 0.5, np.float32)
    got = fn(a, b, peers)
    return np.array_equal(got, np.full((3, 2), K + 2.0))


def pin_rank_one(fn):
    u = np.array([[1.0], [-2.0], [0.5]], np.float32)      # [3,1]
    v = np.array([[3.0, -1.0, 0.25, 8.0]], np.float32)     # [1,4]
    got = fn(_bits_of(u), _bits_of(v), np.zeros((0, 3, 4), np.float32))
    return np.array_equal(got, (u.astype(np.float64) @ v.astype(np.float64)))


def pin_brute_force(fn):
    for seed, (M, N, K, P) in enumerate([(3, 5, 7, 2), (8, 4, 16, 1), (2, 9, 3, 0), (6, 6, 6, 3)]):
        w = wl.custom(M, N, K, P, wid=200 + seed)
        a, b, p = wl.make_inputs(w, seed=seed)
        got = fn(a, b, p)
        want = oracle.gemm_reduce_brute(a, b, p)
        if got.shape != want.shape or not np.allclose(got, want, rtol=1e-12, atol=1e-12):
            return False
    return True


RESULT_PINS = [pin_golden, pin_no_peers_is_integer_matmul, pin_zero_a_is_peer_sum,
               pin_identity_b, pin_all_ones, pin_rank_one, pin_brute_force]


@pytest.mark.parametrize("pin", RESULT_PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin):
    assert pin(oracle.gemm_reduce)


def test_brute_force_meets_closed_form_pins():
    # the C brute force is itself held to the hand-worked and closed-form pins
    for pin in RESULT_PINS[:-1]:
        assert pin(oracle.gemm_reduce_brute), pin.__name__


def test_elementwise_oracle_agrees_with_full_oracle():
    w = wl.custom(50, 70, 90, 3, wid=300)
    a, b, p = wl.make_inputs(w)
    full = oracle.gemm_reduce(a, b, p)
    gemm = oracle.gemm_part(a, b)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, 50, 200)
    cols = rng.integers(0, 70, 200)
    v, g = oracle.gemm_reduce_at(a, b, p, rows, cols)
    np.testing.assert_allclose(v, full[rows, cols], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(g, gemm[rows, cols], rtol=1e-13, atol=1e-13)


def test_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.gemm_reduce(np.zeros((2, 3), np.uint16), np.zeros((4, 2), np.uint16), None)


# ---------------------------------------------------------------------------
# mutation checks: plausible mistakes must fail a pin
# ---------------------------------------------------------------------------

def _dec(bits):
    return oracle.bf16_bits_to_f64(bits)


MUTANTS = {
    "dropped_peer_sum": lambda a, b, p: _dec(a) @ _dec(b),
    "peers_subtracted": lambda a, b, p: _dec(a) @ _dec(b) - p.astype(np.float64).sum(0),
    "only_first_peer": lambda a, b, p: _dec(a) @ _dec(b) + (p[0].astype(np.float64) if p.shape[0] else 0),
    # row-major [K,N] buffer read as if it were [N,K] column-major
    "b_layout_transposed": lambda a, b, p: (_dec(a) @ _dec(b).reshape(b.shape[1], b.shape[0]).T
                                            + p.astype(np.float64).sum(0)),
    "last_k_dropped": lambda a, b, p: _dec(a)[:, :-1] @ _dec(b)[:-1] + p.astype(np.float64).sum(0),
    "bf16_low_half": lambda a, b, p: ((a.astype(np.uint32)).view(np.float32).astype(np.float64)
                                      @ (b.astype(np.uint32)).view(np.float32).astype(np.float64)
                                      + p.astype(np.float64).sum(0)),
    "peers_counted_twice": lambda a, b, p: _dec(a) @ _dec(b) + 2 * p.astype(np.float64).sum(0),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_result_mistake_fails_a_pin(name):
    fn = MUTANTS[name]
    failed = []
    for pin in RESULT_PINS[:-1]:
        try:
            ok = pin(fn)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


# ---------------------------------------------------------------------------
# peer_sum's row blocking: the blocked loop must cover every row exactly once
# ---------------------------------------------------------------------------

def _peer_sum_reference(peers):
    """The peer sum from the C brute force with A = 0 (a path with no row
    blocking at all): C = 0.B + sum_p peers[p]."""
    P, M, N = peers.shape
    return oracle.gemm_reduce_brute(np.zeros((M, 1), np.uint16), np.zeros((1, N), np.uint16), peers)


def pin_peer_sum_blocked(fn):
    rng = np.random.default_rng(11)
    for (P, M, N, rb) in [(3, 10, 4, 3), (2, 7, 5, 7), (4, 9, 3, 2), (1, 5, 6, 1), (5, 8, 2, 4)]:
        peers = rng.standard_normal((P, M, N)).astype(np.float32)
        got = fn(peers, rb)
        want = _peer_sum_reference(peers)
        if got.shape != want.shape or not np.allclose(got, want, rtol=1e-12, atol=1e-12):
            return False
    return True


def test_peer_sum_blocked_path_meets_brute_force():
    # row blocks smaller than M (several blocks, a ragged last one, one-row
    # blocks) against the unblocked brute force
    assert pin_peer_sum_blocked(lambda p, rb: oracle.peer_sum(p, row_block=rb))


def _peer_sum_mutant(drop_last=False, short_block=False, skip_first_peer=False):
    def fn(peers, row_block):
        P, M, N = peers.shape
        out = np.zeros((M, N), dtype=np.float64)
        stop = M - row_block if drop_last else M
        for r0 in range(0, max(stop, 0), row_block):
            r1 = min(M, r0 + row_block - (1 if short_block else 0))
            for p in range(1 if skip_first_peer else 0, P):
                out[r0:r1] += peers[p, r0:r1].astype(np.float64)
        return out
    return fn


@pytest.mark.parametrize("kw", [{"drop_last": True}, {"short_block": True},
                                {"skip_first_peer": True}], ids=lambda k: next(iter(k)))
def test_planted_peer_sum_mistake_fails_the_pin(kw):
    assert not pin_peer_sum_blocked(_peer_sum_mutant(**kw))


def test_tiles_per_task_reading():
    # two 128-wide tiles per task for the 128x128 and 256x128 tiles, one 64x64
    assert oracle.tiles_per_task(64, 64) == 1
    assert oracle.tiles_per_task(128, 128) == 2
    assert oracle.tiles_per_task(256, 128) == 2
    with pytest.raises(ValueError):
        oracle.tiles_per_task(32, 32)


# ---------------------------------------------------------------------------
# controller
# ---------------------------------------------------------------------------

def test_controller_hand_table():
    g = _load("controller_table.json")
    for B, R_s, C_s, R_p, C_p, exact, n in g["rows"]:
        if R_p:
            assert oracle.controller_exact(B, R_s, C_s, R_p, C_p) == Fraction(exact)
        assert oracle.controller_target(B, R_s, C_s, R_p, C_p, current=7) == n, (B, R_s, C_s, R_p, C_p)


@settings(max_examples=300, deadline=None)
@given(B=st.integers(4, 1024), R_s=st.integers(1, 1 << 20), C_s=st.integers(1, (1 << 26) - 1),
       R_p=st.integers(1, 1 << 20), C_p=st.integers(1, (1 << 26) - 1))
def test_controller_equalises_predicted_finish_times(B, R_s, C_s, R_p, C_p):
    x = oracle.controller_exact(B, R_s, C_s, R_p, C_p)
    # defining condition: R_s C_s / n == R_p C_p / (B - n) at the exact n
    assert 0 < x < B
    assert Fraction(R_s * C_s) / x == Fraction(R_p * C_p) / (B - x)
    n = oracle.controller_target(B, R_s, C_s, R_p, C_p, current=2)
    lo, hi = min(2, B - 1), B - 1
    if lo <= x <= hi:
        assert abs(Fraction(n) - x) <= Fraction(1, 2)
        if abs(Fraction(n) - x) == Fraction(1, 2):
            assert n > x          # ties round up
    assert lo <= n <= hi


@settings(max_examples=200, deadline=None)
@given(B=st.integers(4, 512), R_s=st.integers(1, 5000), C_s=st.integers(1, 100000),
       R_p=st.integers(1, 5000), C_p=st.integers(1, 100000))
def test_controller_monotone_in_reduce_cost(B, R_s, C_s, R_p, C_p):
    n1 = oracle.controller_target(B, R_s, C_s, R_p, C_p, 2)
    n2 = oracle.controller_target(B, R_s, C_s + 1000, R_p, C_p, 2)
    n3 = oracle.controller_target(B, R_s, C_s, R_p, C_p + 1000, 2)
    assert n2 >= n1 >= n3


def test_controller_keeps_one_compute_workgroup_per_partition():
    # R_s C_s dominates: the formula asks for ~B, the clamp keeps `keep` computing
    assert oracle.controller_target(256, 1000, 10 ** 6, 10, 1, current=2) == 255
    assert oracle.controller_target(256, 1000, 10 ** 6, 10, 1, current=2, keep=8) == 248
    # the clamp does not apply once compute is done (the drain target is B)
    assert oracle.controller_target(256, 1000, 5, 0, 5, current=2, keep=8) == 256
    # and a balanced case is unaffected: 256 * 1/2 = 128
    assert oracle.controller_target(256, 100, 100, 100, 100, current=2, keep=8) == 128
    assert oracle.controller_update(256, 100, 0, 0, 0, 0, current=300, keep=8) == 248


def test_controller_cap_bounds_reducers_while_compute_remains():
    # hand-worked: 256 * (300*30) / (100*10 + 300*30) = 256 * 9000/10000 = 230.4 -> 230
    assert oracle.controller_target(256, 300, 30, 100, 10, current=2) == 230
    assert oracle.controller_target(256, 300, 30, 100, 10, current=2, cap=128) == 128
    # the tighter of B - keep and the cap wins
    assert oracle.controller_target(256, 300, 30, 100, 10, current=2, keep=200, cap=128) == 56
    # a value under the cap is untouched; so is the drain target B
    assert oracle.controller_target(256, 100, 10, 300, 30, current=2, cap=128) == 26
    assert oracle.controller_target(256, 300, 30, 0, 10, current=2, cap=128) == 256
    # a cap below the floor wins over the floor (liveness of compute first)
    assert oracle.controller_target(256, 1, 1, 10 ** 6, 10 ** 6, current=2, floor=8, cap=4) == 4
    # without samples the current target is clamped to the cap as well
    assert oracle.controller_update(256, 100, 0, 0, 0, 0, current=200, cap=128) == 128
    with pytest.raises(ValueError):
        oracle.controller_target(256, 1, 1, 1, 1, current=2, cap=0)


def test_controller_update_keeps_target_without_samples():
    assert oracle.controller_update(256, 100, 0, 0, 0, 0, current=9) == 9
    assert oracle.controller_update(256, 100, 5, 0, 500, 0, current=9) == 9
    assert oracle.controller_update(256, 100, 0, 0, 0, 0, current=1) == 2      # clamped
    assert oracle.controller_update(256, 100, 0, 0, 0, 0, current=300) == 255  # clamped
    assert oracle.controller_update(256, 100, 100, 3, 10, 10, current=9) == 256  # drain
    # with samples: cumulative means, then the closed form
    got = oracle.controller_update(256, 1024, 24, 8, 24 * 1000, 8 * 3000, current=2)
    assert got == oracle.controller_target(256, 1016, 3000, 1000, 1000, 2)


def test_cycle_mean_saturates():
    assert oracle.cycle_mean(10, 3) == 3
    assert oracle.cycle_mean(1 << 40, 1) == oracle.COST_CAP


CONTROLLER_MUTANTS = {
    "roles_swapped": lambda B, R_s, C_s, R_p, C_p, cur: (
        B if R_p == 0 else min(max((2 * B * R_p * C_p + R_p * C_p + R_s * C_s)
                                   // (2 * (R_p * C_p + R_s * C_s)), 2), B - 1)),
    "floor_rounding": lambda B, R_s, C_s, R_p, C_p, cur: (
        B if R_p == 0 else min(max(B * R_s * C_s // (R_p * C_p + R_s * C_s), 2), B - 1)),
    "no_upper_clamp": lambda B, R_s, C_s, R_p, C_p, cur: (
        B if R_p == 0 else max((2 * B * R_s * C_s + R_p * C_p + R_s * C_s)
                               // (2 * (R_p * C_p + R_s * C_s)), 2)),
    "no_drain": lambda B, R_s, C_s, R_p, C_p, cur: (
        min(max((2 * B * R_s * C_s + R_p * C_p + R_s * C_s)
                // (2 * (R_p * C_p + R_s * C_s)), 2), B - 1)),
}


@pytest.mark.parametrize("name", sorted(CONTROLLER_MUTANTS))
def test_planted_controller_mistake_fails_the_table(name):
    fn = CONTROLLER_MUTANTS[name]
    g = _load("controller_table.json")
    mismatches = [r for r in g["rows"] if fn(*r[:5], 7) != r[6]]
    assert mismatches, f"controller mutant {name} matched the whole table"


# ---------------------------------------------------------------------------
# tiles, chunks and the protocol checker
# ---------------------------------------------------------------------------

def test_chunk_sizes_and_grid():
    assert oracle.tile_grid(256, 256, 64, 64) == (4, 4)
    assert oracle.tile_grid(300, 130, 128, 128) == (3, 2)
    np.testing.assert_array_equal(oracle.chunk_sizes(16, 4), [4, 4, 4, 4])
    np.testing.assert_array_equal(oracle.chunk_sizes(10, 4), [4, 4, 2])
    assert oracle.chunk_sizes(0, 4).shape == (0,)


def test_deterministic_owners_partition_tiles():
    T, B, ns = 1000, 256, 6
    co, ro = oracle.deterministic_owners(T, B, ns)
    assert np.all((co >= ns) & (co < B)) and np.all((ro >= 0) & (ro < ns))
    # each workgroup's tiles, taken in increasing order, are round-robin
    for w in range(ns, B):
        ts = np.nonzero(co == w)[0]
        np.testing.assert_array_equal(ts, np.arange(w - ns, T, B - ns))
    for w in range(ns):
        np.testing.assert_array_equal(np.nonzero(ro == w)[0], np.arange(w, T, ns))


def test_compute_task_of_tile_hand_example():
    # 2 tile rows of 5 tiles, 2 tiles per task: the last task of a row is short
    np.testing.assert_array_equal(oracle.compute_task_of_tile(10, 5, 2),
                                  [0, 0, 1, 1, 2, 3, 3, 4, 4, 5])
    np.testing.assert_array_equal(oracle.compute_task_of_tile(6, 3, 1), np.arange(6))


def test_deterministic_owners_with_blocks():
    tiles_n, tiles_m, B, ns = 6, 4, 5, 2
    T = tiles_n * tiles_m
    co, ro = oracle.deterministic_owners(T, B, ns, tiles_n, 2)
    # tasks (0..11, three per row) go round-robin to workgroups 2, 3, 4
    want = [2, 2, 3, 3, 4, 4, 2, 2, 3, 3, 4, 4, 2, 2, 3, 3, 4, 4, 2, 2, 3, 3, 4, 4]
    np.testing.assert_array_equal(co, want)
    # reduce tasks are single tiles, round-robin over workgroups 0, 1
    np.testing.assert_array_equal(ro, [0, 1] * 12)


def test_check_state_rejects_split_task_owner():
    T, tiles_n, B, ns = 12, 4, 8, 2
    exp = oracle.expected_state(T, 4, 1, 1)
    co, ro = oracle.deterministic_owners(T, B, ns, tiles_n, 2)
    maps = {k: v.copy() for k, v in exp.items()}
    maps["compute_owner"] = co | (ns << 16)
    maps["reduce_owner"] = ro | (ns << 16)
    assert oracle.check_state(maps, T, 4, 1, 1, B, "static", ns, tiles_n, 2) == []
    assert oracle.check_state(maps, T, 4, 1, 1, B, "deterministic", ns, tiles_n, 2) == []
    split = {k: v.copy() for k, v in maps.items()}
    split["compute_owner"][5] = (ns << 16) | 7    # the other tile of its task stays with 4
    assert oracle.check_state(split, T, 4, 1, 1, B, "static", ns, tiles_n, 2)
    # reduce tasks are single tiles: in a dynamic schedule any reducer may take
    # tile 3 whatever took tile 2; the deterministic schedule fixes which
    split = {k: v.copy() for k, v in maps.items()}
    split["reduce_owner"][3] = (ns << 16) | (1 - int(ro[3]))
    assert oracle.check_state(split, T, 4, 1, 1, B, "static", ns, tiles_n, 2) == []
    assert oracle.check_state(split, T, 4, 1, 1, B, "deterministic", ns, tiles_n, 2)


def _good_maps(T, tpc, epoch, calls, B, ns):
    exp = oracle.expected_state(T, tpc, epoch, calls)
    co, ro = oracle.deterministic_owners(T, B, ns)
    maps = {k: v.copy() for k, v in exp.items()}
    maps["compute_owner"] = co | (ns << 16)
    maps["reduce_owner"] = ro | (ns << 16)
    return maps


def test_check_state_accepts_the_closed_form():
    maps = _good_maps(18, 4, 5, 3, 16, 3)
    assert oracle.check_state(maps, 18, 4, 5, 3, 16, "deterministic", 3) == []
    assert oracle.check_state(maps, 18, 4, 5, 3, 16, "static", 3) == []


@pytest.mark.parametrize("corrupt", [
    ("tile_flag", 3, 4), ("tile_reduce_cnt", 0, 4), ("tile_reduce_cnt", 7, 2),
    ("chunk_cnt", 1, 11), ("chunk_cnt", 4, 7), ("chunk_flag", 2, 0),
    ("compute_owner", 5, 1 | (3 << 16)), ("reduce_owner", 6, 2 | (3 << 16)),
    ("compute_owner", 0, 20 | (3 << 16)), ("reduce_owner", 1, 1 | (4 << 16)),
])
def test_check_state_rejects_corruption(corrupt):
    key, i, v = corrupt
    maps = _good_maps(18, 4, 5, 3, 16, 3)
    maps[key][i] = v
    assert oracle.check_state(maps, 18, 4, 5, 3, 16, "deterministic", 3)


def test_check_state_role_log_in_adaptive_mode():
    T, B = 8, 8
    maps = _good_maps(T, 4, 1, 1, B, 2)
    maps["compute_owner"][:] = 5 | (3 << 16)      # index 5 >= target 3: compute ok
    maps["reduce_owner"][:] = 1 | (3 << 16)       # index 1 < target 3: reduce ok
    assert oracle.check_state(maps, T, 4, 1, 1, B, "adaptive", 2) == []
    maps["reduce_owner"][4] = 6 | (3 << 16)       # reduced while in the compute role
    assert oracle.check_state(maps, T, 4, 1, 1, B, "adaptive", 2)


def test_check_state_help_mark():
    T, B = 8, 8
    maps = _good_maps(T, 4, 1, 1, B, 2)
    maps["compute_owner"][:] = 5 | (3 << 16)
    maps["reduce_owner"][:] = 1 | (3 << 16)
    # workgroup 1 (reduce role under target 3) computed tile 2 while its
    # reduce ticket was not ready: legal only with the help mark, only in
    # adaptive mode, and never on a reduce owner
    maps["compute_owner"][2] = 1 | (3 << 16)
    assert oracle.check_state(maps, T, 4, 1, 1, B, "adaptive", 2)
    maps["compute_owner"][2] = oracle.OWNER_HELP | 1 | (3 << 16)
    assert oracle.check_state(maps, T, 4, 1, 1, B, "adaptive", 2) == []
    assert oracle.check_state(maps, T, 4, 1, 1, B, "static", 2)
    maps["reduce_owner"][3] = oracle.OWNER_HELP | 1 | (3 << 16)
    assert oracle.check_state(maps, T, 4, 1, 1, B, "adaptive", 2)


def test_brute_library_builds():
    path = oracle.build_brute()
    assert os.path.exists(path)
