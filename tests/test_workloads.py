"""Seeded input generator: determinism, bfloat16 rounding, recipe."""
import numpy as np
import pytest

import workloads as wl


def test_bf16_round_to_nearest_even_hand_cases():
    x = np.array([
        1.0,                      # exact
        1.0 + 2.0 ** -8,          # halfway between 1.0 and 1+2^-7: ties to even -> 1.0
        1.0 + 1.5 * 2.0 ** -8,    # above halfway -> 1+2^-7
        1.0 + 2.0 ** -7 + 2.0 ** -8,  # halfway, odd lower neighbour -> 1+2^-6
        -2.5,
        0.0,
        -0.0,
        3.0e-41,                  # subnormal binary32: keeps its high half
    ], dtype=np.float32)
    got = wl.round_to_bf16_bits(x)
    want = np.array([0x3F80, 0x3F80, 0x3F81, 0x3F82, 0xC020, 0x0000, 0x8000,
                     (np.float32(3.0e-41).view(np.uint32) + 0x7FFF
                      + ((np.float32(3.0e-41).view(np.uint32) >> 16) & 1)) >> 16],
                    dtype=np.uint16)
    assert got.dtype == np.uint16
    np.testing.assert_array_equal(got, want)


def test_bf16_rounding_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100000).astype(np.float32)
    bits = wl.round_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # bfloat16 keeps 8 significant bits: |x - rne(x)| <= 2^-8 |x| (half an ulp)
    assert np.all(np.abs(back.astype(np.float64) - x) <= 2.0 ** -8 * np.abs(x) + 1e-45)


def test_generator_is_deterministic_and_threads_do_not_matter():
    w = wl.custom(64, 96, 32, 3, wid=7)
    a1, b1, p1 = wl.make_inputs(w, seed=5, threads=1)
    a2, b2, p2 = wl.make_inputs(w, seed=5, threads=3)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(b1, b2)
    np.testing.assert_array_equal(p1, p2)
    a3, _, _ = wl.make_inputs(w, seed=6)
    assert not np.array_equal(a1, a3)
    assert a1.shape == (64, 32) and b1.shape == (32, 96) and p1.shape == (3, 64, 96)
    assert a1.dtype == np.uint16 and p1.dtype == np.float32


def test_streams_are_independent_per_buffer():
    # peer p's values do not depend on how many peers are drawn
    w3 = wl.custom(32, 32, 16, 3, wid=9)
    w5 = wl.custom(32, 32, 16, 5, wid=9)
    _, _, p3 = wl.make_inputs(w3)
    _, _, p5 = wl.make_inputs(w5)
    np.testing.assert_array_equal(p3, p5[:3])


def test_distributions_and_zero_rows():
    w = wl.custom(400, 64, 256, 2, wid=11, dist_ab=("normal", 0.02),
                  dist_peer=("uniform", -0.5, 0.5), zero_rows_frac=0.1)
    a, b, p = wl.make_inputs(w)
    av = (a.astype(np.uint32) << 16).view(np.float32)
    bv = (b.astype(np.uint32) << 16).view(np.float32)
    assert np.all(a[:40] == 0) and np.any(a[40] != 0)
    assert abs(bv.std() - 0.02) < 0.001
    assert abs(av[40:].std() - 0.02) < 0.001
    assert p.min() >= -0.5 and p.max() < 0.5 and abs(p.mean()) < 0.01


def test_named_workloads_match_their_descriptions():
    W = wl.WORKLOADS
    assert (W["tiny"].M, W["tiny"].N, W["tiny"].K, W["tiny"].peers) == (256, 256, 512, 1)
    assert W["tiny"].tiles == 16 and W["tiny"].chunks == 4
    assert W["tp_share"].tiles == 1024 and W["tp_share"].chunks == 256
    assert W["reduce_heavy"].tiles == 4096
    assert (W["compute_heavy"].tile_m, W["compute_heavy"].tile_n) == (256, 128)
    assert W["compute_heavy"].tiles == 4096 and W["compute_heavy"].chunks == 1024
    assert W["wide_many_peer"].peers == 15 and W["wide_many_peer"].tiles == 1536
    assert int(np.floor(W["wide_many_peer"].zero_rows_frac * 2048)) == 204
    # algorithmic bytes: A + B once, peers once, C once
    tp = W["tp_share"]
    assert tp.algorithmic_bytes == 2 * 4096 * 1792 * 2 + 4 * 7 * 4096 * 4096 + 4 * 4096 * 4096


def test_ring_attention_inputs_are_seeded_and_shaped():
    w = wl.ra_custom(3, 130, 2, 128, wid=201)
    a = wl.make_ra_inputs(w)
    b = wl.make_ra_inputs(w)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert a[0].shape == (130, 2, 128) and a[3].shape == (2, 130, 2, 128)
    assert all(x.dtype == np.uint16 for x in a)
    # every buffer its own stream: Q, K, V and each peer's K and V differ
    flat = [a[0], a[1], a[2], a[3][0], a[4][0], a[3][1], a[4][1]]
    assert len({x.tobytes() for x in flat}) == len(flat)
    c = wl.make_ra_inputs(w, seed=1)
    assert not np.array_equal(a[0], c[0])


def test_ring_attention_workload_sizes():
    W = wl.RA_WORKLOADS
    assert (W["ra_sp_share"].ranks, W["ra_sp_share"].S, W["ra_sp_share"].H, W["ra_sp_share"].D) == (8, 4096, 32, 128)
    assert W["ra_sp_share"].tasks == 1024 and W["ra_sp_share"].kv_tiles == 7 * 32
    assert W["ra_sp_share"].flops == 4 * 4096 * 32768 * 128 * 32
