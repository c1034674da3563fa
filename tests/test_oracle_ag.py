"""Pins for the oracle of one rank's share of AllGather+GEMM (CPU only).

* result: a hand-worked two-rank example (tests/golden/tiny_allgather_gemm.json),
  the C triple loop on the gathered A, the block structure (each rank's rows of
  C are its own shard times B), the gathered A bit-exact against the shards,
  one rank (the plain GEMM), integer operands against exact arithmetic;
* protocol: the copy order and the deterministic owner maps worked by hand,
  the closed-form state accepted, corruptions and role violations rejected;
* mutants: shards out of rank order, the local shard placed last, a dropped
  shard, a transposed B each fail a pin.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    return wl.round_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _dec(bits):
    return oracle.bf16_bits_to_f64(bits)


# ---------------------------------------------------------------------------
# result pins (fn(a_local, a_peers, b) -> (gathered, C))
# ---------------------------------------------------------------------------

def pin_golden(fn):
    with open(os.path.join(GOLDEN, "tiny_allgather_gemm.json")) as f:
        g = json.load(f)
    a0, ap, b = _bits(g["A_local_values"]), _bits(g["A_peers_values"]), _bits(g["B_values"])
    gathered, C = fn(a0, ap, b)
    return (np.array_equal(_dec(gathered), np.array(g["gathered_values"]))
            and np.array_equal(C, np.array(g["C"])))


def pin_brute_force(fn):
    for seed, (R, Ms, K, N) in enumerate([(3, 2, 5, 4), (2, 4, 3, 6), (4, 1, 7, 2), (1, 3, 4, 5)]):
        rng = np.random.default_rng(40 + seed)
        a0 = _bits(rng.uniform(-2, 2, (Ms, K)))
        ap = _bits(rng.uniform(-2, 2, (R - 1, Ms, K)))
        b = _bits(rng.uniform(-2, 2, (K, N)))
        gathered, C = fn(a0, ap, b)
        stacked = np.concatenate([a0] + [ap[p] for p in range(R - 1)], axis=0)
        want = oracle.gemm_reduce_brute(stacked, b, np.zeros((0, R * Ms, N), np.float32))
        if C.shape != want.shape or not np.allclose(C, want, rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_rows_by_rank(fn):
    # rank r's rows of the gathered A are its shard, bit for bit, and its
    # rows of C are that shard times B (integer operands: exact)
    rng = np.random.default_rng(5)
    R, Ms, K, N = 4, 3, 6, 5
    ai = rng.integers(-6, 7, (R, Ms, K))
    bi = rng.integers(-6, 7, (K, N))
    gathered, C = fn(_bits(ai[0]), _bits(ai[1:]), _bits(bi))
    for r in range(R):
        if not np.array_equal(gathered[r * Ms:(r + 1) * Ms], _bits(ai[r])):
            return False
        want = np.array([[sum(int(ai[r, i, k]) * int(bi[k, j]) for k in range(K)) for j in range(N)]
                         for i in range(Ms)])
        if not np.array_equal(C[r * Ms:(r + 1) * Ms], want):
            return False
    return True


def pin_one_rank(fn):
    u = np.array([[1.0, -2.0], [0.5, 3.0]], np.float32)
    v = np.array([[3.0, -1.0, 0.25], [2.0, 0.5, -4.0]], np.float32)
    gathered, C = fn(_bits(u), np.zeros((0, 2, 2), np.uint16), _bits(v))
    return np.array_equal(gathered, _bits(u)) and np.array_equal(C, u.astype(np.float64) @ v)


AG_PINS = [pin_golden, pin_brute_force, pin_rows_by_rank, pin_one_rank]


@pytest.mark.parametrize("pin", AG_PINS, ids=lambda p: p.__name__)
def test_allgather_oracle_meets_pin(pin):
    assert pin(oracle.allgather_gemm)


def _stack(a0, ap, order):
    shards = [a0] + [ap[p] for p in range(ap.shape[0])]
    return np.concatenate([shards[r] for r in order], axis=0) if shards else a0


AG_MUTANTS = {
    "peers_reversed": lambda a0, ap, b: (lambda g: (g, _dec(g) @ _dec(b)))(
        _stack(a0, ap, [0] + list(range(ap.shape[0], 0, -1)))),
    "local_last": lambda a0, ap, b: (lambda g: (g, _dec(g) @ _dec(b)))(
        _stack(a0, ap, list(range(1, ap.shape[0] + 1)) + [0])),
    "last_peer_dropped": lambda a0, ap, b: (lambda g: (g, _dec(g) @ _dec(b)))(
        _stack(a0, ap, list(range(ap.shape[0])) + ([ap.shape[0] - 1] if ap.shape[0] else []))),
    "b_transposed_layout": lambda a0, ap, b: (lambda g: (g, _dec(g) @ _dec(b).reshape(b.shape[1], b.shape[0]).T))(
        _stack(a0, ap, list(range(ap.shape[0] + 1)))),
}


@pytest.mark.parametrize("name", sorted(AG_MUTANTS))
def test_planted_allgather_mistake_fails_a_pin(name):
    fn = AG_MUTANTS[name]
    failed = []
    for pin in AG_PINS:
        try:
            ok = pin(fn)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_allgather_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.allgather_gemm(np.zeros((2, 3), np.uint16), np.zeros((1, 2, 4), np.uint16),
                              np.zeros((3, 2), np.uint16))


# ---------------------------------------------------------------------------
# protocol
# ---------------------------------------------------------------------------

def test_copy_order_hand_example():
    # three ranks of two chunks: the other ranks' chunks first, then ours
    np.testing.assert_array_equal(oracle.ag_copy_order(3, 2), [2, 3, 4, 5, 0, 1])
    np.testing.assert_array_equal(oracle.ag_copy_order(1, 3), [0, 1, 2])


def test_deterministic_owners_hand_example():
    # 2 ranks x 2 chunks, 3 tile columns, 2-tile tasks, B = 5, 2 copiers
    co, po = oracle.ag_deterministic_owners(2, 2, 3, 5, 2, 2)
    # copy order [2, 3, 0, 1] dealt to workgroups 0, 1, 0, 1
    np.testing.assert_array_equal(co, [0, 1, 0, 1])
    # tasks per tile row: [0,0,1] [2,2,3] [4,4,5] [6,6,7] -> 2 + task mod 3
    np.testing.assert_array_equal(po, [2, 2, 3, 4, 4, 2, 3, 3, 4, 2, 2, 3])


def _good(ranks=2, cps=2, tn=3, B=5, n=2, tpt=2):
    exp = oracle.ag_expected_state(ranks * cps, ranks * cps * tn, 3, 2)
    co, po = oracle.ag_deterministic_owners(ranks, cps, tn, B, n, tpt)
    maps = {k: v.copy() for k, v in exp.items()}
    maps["copy_owner"] = co | (n << 16)
    maps["compute_owner"] = po | (n << 16)
    return maps


def test_ag_check_state_accepts_the_closed_form():
    maps = _good()
    for mode in ("deterministic", "static", "adaptive"):
        assert oracle.ag_check_state(maps, 2, 2, 3, 3, 2, 5, mode, 2, 2) == []


@pytest.mark.parametrize("corrupt", [
    lambda m: m["chunk_flag"].__setitem__(1, 2),
    lambda m: m["chunk_copy_cnt"].__setitem__(3, 1),
    lambda m: m["tile_compute_cnt"].__setitem__(7, 3),
    lambda m: m["copy_owner"].__setitem__(0, 1 | (2 << 16)),
    lambda m: m["compute_owner"].__setitem__(5, 4 | (2 << 16)),
])
def test_ag_check_state_rejects_corruption(corrupt):
    maps = _good()
    corrupt(maps)
    assert oracle.ag_check_state(maps, 2, 2, 3, 3, 2, 5, "deterministic", 2, 2)


def test_ag_check_state_roles_and_help_mark():
    maps = _good()
    # workgroup 3 (compute role under target 2) copied chunk 2 while waiting
    # for its input: legal only with the mark, only in adaptive mode
    maps["copy_owner"][2] = 3 | (2 << 16)
    assert oracle.ag_check_state(maps, 2, 2, 3, 3, 2, 5, "adaptive", 2, 2)
    maps["copy_owner"][2] = oracle.OWNER_HELP | 3 | (2 << 16)
    assert oracle.ag_check_state(maps, 2, 2, 3, 3, 2, 5, "adaptive", 2, 2) == []
    assert oracle.ag_check_state(maps, 2, 2, 3, 3, 2, 5, "static", 2, 2)
    # a compute task by a copy-role workgroup is never legal
    maps = _good()
    maps["compute_owner"][0:2] = 1 | (2 << 16)
    assert oracle.ag_check_state(maps, 2, 2, 3, 3, 2, 5, "adaptive", 2, 2)


def test_parts_per_chunk_hand_values():
    # ceil(2 tile_m K / 64 KiB), at least 1, at most min(tiles_n, 64)
    assert oracle.ag_parts_per_chunk(64, 256, 4) == 1          # 32 KiB chunk
    assert oracle.ag_parts_per_chunk(64, 512, 4) == 1          # exactly 64 KiB
    assert oracle.ag_parts_per_chunk(64, 520, 4) == 2          # just over
    assert oracle.ag_parts_per_chunk(128, 1792, 32) == 7       # 448 KiB
    assert oracle.ag_parts_per_chunk(256, 8192, 64) == 64      # 4 MiB
    assert oracle.ag_parts_per_chunk(256, 16384, 64) == 64     # capped at 64
    assert oracle.ag_parts_per_chunk(128, 4096, 2) == 2        # capped at tiles_n


def test_deterministic_owners_with_parts_hand_example():
    # 2 ranks x 1 chunk, 2 parts, 3 copiers: copy order [1, 0]; tasks in
    # order (1,0) (1,1) (0,0) (0,1) dealt to 0 1 2 0; indexed chunk*2 + part
    co, _ = oracle.ag_deterministic_owners(2, 1, 1, 5, 3, 1, parts=2)
    np.testing.assert_array_equal(co, [2, 0, 0, 1])


def test_ag_check_state_with_parts():
    exp = oracle.ag_expected_state(4, 12, 3, 2, parts=3)
    np.testing.assert_array_equal(exp["chunk_copy_cnt"], [6, 6, 6, 6])
    co, po = oracle.ag_deterministic_owners(2, 2, 3, 5, 2, 2, parts=3)
    maps = {k: v.copy() for k, v in exp.items()}
    maps["copy_owner"] = co | (2 << 16)
    maps["compute_owner"] = po | (2 << 16)
    assert oracle.ag_check_state(maps, 2, 2, 3, 3, 2, 5, "deterministic", 2, 2, parts=3) == []
    # one part short of a chunk, or a map of one owner per chunk, is caught
    bad = {k: v.copy() for k, v in maps.items()}
    bad["chunk_copy_cnt"][2] = 5
    assert oracle.ag_check_state(bad, 2, 2, 3, 3, 2, 5, "deterministic", 2, 2, parts=3)
    bad = {k: v.copy() for k, v in maps.items()}
    bad["copy_owner"] = bad["copy_owner"][:4]
    assert oracle.ag_check_state(bad, 2, 2, 3, 3, 2, 5, "deterministic", 2, 2, parts=3)
    # swapping two parts' owners breaks the deterministic deal
    bad = {k: v.copy() for k, v in maps.items()}
    bad["copy_owner"][[0, 1]] = bad["copy_owner"][[1, 0]]
    assert oracle.ag_check_state(bad, 2, 2, 3, 3, 2, 5, "deterministic", 2, 2, parts=3)
