"""Pins for the oracle of one rank's share of GEMM+ReduceScatter.

Rank 0 of R = P + 1 ranks: tile rows are cut into R shards (rank o owns tile
rows [floor(o T_m / R), floor((o+1) T_m / R))); rank 0's output is its shard,
A.B plus the other ranks' partials (the peers, its inbox) on its rows; every
other tile of A.B is stored into this rank's inbox slot at its owner (a
stand-in buffer).  Pins: hand-worked shard bounds, an
integer hand example checked with exact integer arithmetic, closed forms (one
rank, A = 0), the independent C brute force, the shard cover invariant, and
planted mistakes that must each fail a pin.
"""
import numpy as np
import pytest

import oracle
import workloads as wl


def _bits_of(values):
    return wl.round_to_bf16_bits(np.asarray(values, dtype=np.float32))


def test_shard_bounds_hand_cases():
    assert oracle.rs_shard_bounds(5, 3).tolist() == [0, 1, 3, 5]
    assert oracle.rs_shard_bounds(2, 4).tolist() == [0, 0, 1, 1, 2]      # empty shards
    assert oracle.rs_shard_bounds(8, 8).tolist() == list(range(9))
    assert oracle.rs_shard_bounds(32, 1).tolist() == [0, 32]
    with pytest.raises(ValueError):
        oracle.rs_shard_bounds(4, 0)


@pytest.mark.parametrize("tiles_m", [0, 1, 3, 7, 32, 33])
@pytest.mark.parametrize("ranks", [1, 2, 3, 8, 16])
def test_shards_cover_every_tile_row_once(tiles_m, ranks):
    b = oracle.rs_shard_bounds(tiles_m, ranks)
    owner = np.concatenate([np.full(b[o + 1] - b[o], o) for o in range(ranks)])
    assert owner.tolist() == sorted(owner.tolist()) and len(owner) == tiles_m
    sizes = np.diff(b)
    assert sizes.max() - sizes.min() <= 1


# ---------------------------------------------------------------------------
# result pins: fn(a_bits, b_bits, peers, remote_init, tile_m) -> (shard, remote)
# ---------------------------------------------------------------------------

def pin_rs_hand_example(fn):
    # M = 6 rows in tiles of 2 (3 tile rows), P = 2: ranks own tile rows
    # {0}, {1}, {2} -> rank 0 owns rows 0-1.  Integer operands: the float64
    # results must equal exact integer arithmetic.
    rng = np.random.default_rng(11)
    ai = rng.integers(-6, 7, size=(6, 5))
    bi = rng.integers(-6, 7, size=(5, 4))
    pi = rng.integers(-9, 10, size=(2, 6, 4))
    ri = rng.integers(-9, 10, size=(6, 4))
    C, R = fn(_bits_of(ai), _bits_of(bi), pi.astype(np.float32), ri.astype(np.float32), 2)
    ab = [[sum(int(ai[i, k]) * int(bi[k, j]) for k in range(5)) for j in range(4)] for i in range(6)]
    wantC = [[ab[i][j] + (int(pi[0, i, j]) + int(pi[1, i, j]) if i < 2 else 0) for j in range(4)]
             for i in range(6)]
    wantR = [[ab[i][j] if i >= 2 else int(ri[i, j]) for j in range(4)] for i in range(6)]
    return np.array_equal(C, np.array(wantC)[:2]) and np.array_equal(R, np.array(wantR))


def pin_rs_one_rank_is_the_gemm(fn):
    rng = np.random.default_rng(12)
    a = _bits_of(rng.uniform(-2, 2, (7, 9)).astype(np.float32))
    b = _bits_of(rng.uniform(-2, 2, (9, 3)).astype(np.float32))
    init = rng.standard_normal((7, 3)).astype(np.float32)
    C, R = fn(a, b, np.zeros((0, 7, 3), np.float32), init, 4)
    ab = oracle.bf16_bits_to_f64(a) @ oracle.bf16_bits_to_f64(b)
    return np.allclose(C, ab, rtol=0, atol=1e-12) and np.array_equal(R, init.astype(np.float64))


def pin_rs_zero_a(fn):
    rng = np.random.default_rng(13)
    peers = rng.standard_normal((3, 8, 5)).astype(np.float32)   # R = 4, tile_m 2: 4 tile rows
    init = rng.standard_normal((8, 5)).astype(np.float32)
    b = _bits_of(rng.uniform(-1, 1, (6, 5)).astype(np.float32))
    C, R = fn(np.zeros((8, 6), np.uint16), b, peers, init, 2)
    want = peers[:, :2].astype(np.float64).sum(0)
    wantR = np.zeros((8, 5))
    wantR[:2] = init[:2]
    return np.allclose(C, want, rtol=0, atol=1e-12) and np.array_equal(R, wantR)


def pin_rs_brute_force(fn):
    for seed, (M, N, K, P, tm) in enumerate([(12, 8, 16, 3, 2), (20, 6, 9, 2, 4), (5, 4, 7, 7, 1)]):
        w = wl.custom(M, N, K, P, wid=220 + seed)
        a, b, p = wl.make_inputs(w, seed=seed)
        init = np.random.default_rng(seed).standard_normal((M, N)).astype(np.float32)
        C, R = fn(a, b, p, init, tm)
        full = oracle.gemm_reduce_brute(a, b, p)
        ab = oracle.gemm_reduce_brute(a, b, np.zeros((0, M, N), np.float32))
        own = int(oracle.rs_shard_bounds(-(-M // tm), P + 1)[1]) * tm
        wantC = ab.copy()
        wantC[:own] = full[:own]
        wantR = init.astype(np.float64)
        wantR[own:] = ab[own:]
        if C.shape != (min(M, own), N):
            return False
        if not (np.allclose(C, wantC[:own], rtol=1e-12, atol=1e-12)
                and np.allclose(R, wantR, rtol=1e-12, atol=1e-12)):
            return False
    return True


RS_PINS = [pin_rs_hand_example, pin_rs_one_rank_is_the_gemm, pin_rs_zero_a, pin_rs_brute_force]


@pytest.mark.parametrize("pin", RS_PINS, ids=lambda p: p.__name__)
def test_rs_oracle_meets_pin(pin):
    assert pin(oracle.gemm_reduce_scatter)


def _rs_mutant(own_shard=0, init=True, remote_everywhere=False, skip_peers=False, ceil=False,
               add=False):
    def fn(a, b, p, r0, tm):
        M = a.shape[0]
        P = p.shape[0]
        tiles_m = -(-M // tm)
        R = P + 1
        if ceil:
            bounds = [-(-(o * tiles_m) // R) for o in range(R + 1)]
        else:
            bounds = oracle.rs_shard_bounds(tiles_m, R).tolist()
        lo, hi = bounds[own_shard] * tm, min(M, bounds[own_shard + 1] * tm)
        ab = oracle.bf16_bits_to_f64(a) @ oracle.bf16_bits_to_f64(b)
        ps = p.astype(np.float64).sum(0) if P else np.zeros_like(ab)
        C = ab.copy()
        if not skip_peers:
            C[lo:hi] += ps[lo:hi]
        Rm = r0.astype(np.float64).copy() if init else np.zeros_like(ab)
        mask = np.ones(M, bool)
        if not remote_everywhere:
            mask[lo:hi] = False
        if add:
            Rm[mask] += ab[mask]
        else:
            Rm[mask] = ab[mask]
        return C[lo:hi], Rm
    return fn


RS_MUTANTS = {
    "owns_the_last_shard": lambda a, b, p, r0, tm: _rs_mutant(own_shard=max(0, p.shape[0]))(a, b, p, r0, tm),
    "own_rows_of_remote_cleared": _rs_mutant(init=False),
    "partial_added_into_remote": _rs_mutant(add=True),
    "own_rows_also_sent": _rs_mutant(remote_everywhere=True),
    "shard_without_the_peer_sum": _rs_mutant(skip_peers=True),
    "shard_bounds_rounded_up": _rs_mutant(ceil=True),
}


@pytest.mark.parametrize("name", sorted(RS_MUTANTS))
def test_planted_rs_mistake_fails_a_pin(name):
    fn = RS_MUTANTS[name]
    assert fn is not None
    ok = [pin(fn) for pin in RS_PINS]
    assert not all(ok), f"mutant {name} passed every pin"


def test_rs_oracle_rejects_bad_shapes():
    z = np.zeros
    with pytest.raises(ValueError):
        oracle.gemm_reduce_scatter(z((2, 3), np.uint16), z((4, 2), np.uint16), None, z((2, 2), np.float32), 1)
    with pytest.raises(ValueError):
        oracle.gemm_reduce_scatter(z((2, 3), np.uint16), z((3, 2), np.uint16), z((1, 2, 3), np.float32),
                                   z((2, 2), np.float32), 1)
    with pytest.raises(ValueError):
        oracle.gemm_reduce_scatter(z((2, 3), np.uint16), z((3, 2), np.uint16), None, z((3, 2), np.float32), 1)
