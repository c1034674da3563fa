"""Pins for the oracle of one rank's share of Ring Attention (CPU only).

* result: a hand-worked two-rank example (tests/golden/tiny_ring_attention.json),
  a pure-Python brute force on tiny shapes, one rank against torch's
  scaled_dot_product_attention (float64, CPU), zero queries (uniform weights:
  the mean of every rank's V, LSE = log of the key count), the ring order not
  mattering (no causal mask), and the log-sum-exp merge of two key sets (how
  a ring step combines partial results);
* protocol: the split rule and the deterministic owner maps worked by hand,
  the closed-form state accepted, corruptions and role violations rejected;
* mutants: a missing or inverted 1/sqrt(D), a dropped peer, heads mixed up,
  LSE in base 2, K used for V, and a [H, S, D] reading of the layout each
  fail a pin.
"""
import json
import math
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


def _rand(rng, shape, lo=-1.5, hi=1.5):
    return _bits(rng.uniform(lo, hi, shape))


def _inputs(seed, R, S, H, D):
    rng = np.random.default_rng(seed)
    return (_rand(rng, (S, H, D)), _rand(rng, (S, H, D)), _rand(rng, (S, H, D)),
            _rand(rng, (R - 1, S, H, D)), _rand(rng, (R - 1, S, H, D)))


# ---------------------------------------------------------------------------
# result pins (fn(q, k_local, v_local, k_peers, v_peers) -> (O, LSE))
# ---------------------------------------------------------------------------

def pin_golden(fn):
    with open(os.path.join(GOLDEN, "tiny_ring_attention.json")) as f:
        g = json.load(f)
    O, L = fn(_bits(g["q"]), _bits(g["k_local"]), _bits(g["v_local"]), _bits(g["k_peers"]), _bits(g["v_peers"]))
    return np.allclose(O, np.array(g["O"]), rtol=1e-13, atol=0) and \
        np.allclose(L, np.array(g["LSE"]), rtol=1e-13, atol=0)


def _brute(q, kl, vl, kp, vp):
    S, H, D = q.shape
    keys = [(_dec(kl[j]), _dec(vl[j])) for j in range(S)]
    for p in range(kp.shape[0]):
        keys += [(_dec(kp[p, j]), _dec(vp[p, j])) for j in range(S)]
    O = np.zeros((S, H, D))
    L = np.zeros((H, S))
    for h in range(H):
        for i in range(S):
            qi = [float(x) for x in _dec(q[i, h])]
            sc = [sum(qi[d] * float(k[h, d]) for d in range(D)) / math.sqrt(D) for k, _ in keys]
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            tot = sum(w)
            for d in range(D):
                O[i, h, d] = sum(w[j] * float(keys[j][1][h, d]) for j in range(len(keys))) / tot
            L[h, i] = m + math.log(tot)
    return O, L


def pin_brute_force(fn):
    for seed, (R, S, H, D) in enumerate([(3, 2, 2, 3), (2, 3, 1, 4), (1, 2, 3, 2), (4, 1, 2, 5)]):
        args = _inputs(60 + seed, R, S, H, D)
        O, L = fn(*args)
        Ob, Lb = _brute(*args)
        if O.shape != Ob.shape or L.shape != Lb.shape:
            return False
        if not (np.allclose(O, Ob, rtol=1e-12, atol=1e-13) and np.allclose(L, Lb, rtol=1e-12, atol=1e-13)):
            return False
    return True


def pin_one_rank_is_sdpa(fn):
    import torch
    S, H, D = 5, 3, 8
    q, kl, vl, _, _ = _inputs(70, 1, S, H, D)
    O, L = fn(q, kl, vl, np.zeros((0, S, H, D), np.uint16), np.zeros((0, S, H, D), np.uint16))
    t = lambda b: torch.from_numpy(_dec(b)).permute(1, 0, 2)          # [H, S, D]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(kl), t(vl)).permute(1, 0, 2).numpy()
    lse = torch.logsumexp(t(q) @ t(kl).transpose(1, 2) / math.sqrt(D), dim=-1).numpy()
    return np.allclose(O, ref, rtol=1e-12, atol=1e-13) and np.allclose(L, lse, rtol=1e-12, atol=1e-13)


def pin_zero_queries(fn):
    # every score 0: uniform weights over all R S keys
    R, S, H, D = 3, 4, 2, 3
    _, kl, vl, kp, vp = _inputs(71, R, S, H, D)
    q = np.zeros((S, H, D), np.uint16)
    O, L = fn(q, kl, vl, kp, vp)
    allv = np.concatenate([_dec(vl)[None], _dec(vp)], axis=0).reshape(-1, H, D)
    return np.allclose(O, np.broadcast_to(allv.mean(axis=0), O.shape), rtol=1e-13, atol=1e-14) and \
        np.allclose(L, math.log(R * S), rtol=1e-14, atol=0)


def pin_ring_order_free(fn):
    # no causal mask: relabelling the ranks (peers reversed, or a peer's KV
    # taken as the local one) changes nothing but rounding
    R, S, H, D = 4, 3, 2, 4
    q, kl, vl, kp, vp = _inputs(72, R, S, H, D)
    O, L = fn(q, kl, vl, kp, vp)
    O2, L2 = fn(q, kl, vl, kp[::-1].copy(), vp[::-1].copy())
    kp3 = np.concatenate([kl[None], kp[1:]], axis=0)
    vp3 = np.concatenate([vl[None], vp[1:]], axis=0)
    O3, L3 = fn(q, kp[0], vp[0], kp3, vp3)
    return all(np.allclose(a, b, rtol=1e-12, atol=1e-13) for a, b in ((O, O2), (L, L2), (O, O3), (L, L3)))


def pin_lse_merge(fn):
    # what a ring step relies on: attention over keys X u Y from the parts'
    # outputs, weighted by exp(LSE)
    R, S, H, D = 3, 3, 2, 4
    q, kl, vl, kp, vp = _inputs(73, R, S, H, D)
    O, L = fn(q, kl, vl, kp, vp)
    Oa, La = fn(q, kl, vl, kp[:0], vp[:0])
    Ob, Lb = fn(q, kp[0], vp[0], kp[1:], vp[1:])
    m = np.maximum(La, Lb)
    wa, wb = np.exp(La - m), np.exp(Lb - m)
    Om = (wa.T[..., None] * Oa + wb.T[..., None] * Ob) / (wa + wb).T[..., None]
    Lm = m + np.log(wa + wb)
    return np.allclose(O, Om, rtol=1e-12, atol=1e-13) and np.allclose(L, Lm, rtol=1e-12, atol=1e-13)


RA_PINS = [pin_golden, pin_brute_force, pin_one_rank_is_sdpa, pin_zero_queries, pin_ring_order_free,
           pin_lse_merge]


@pytest.mark.parametrize("pin", RA_PINS, ids=lambda p: p.__name__)
def test_ring_oracle_meets_pin(pin):
    assert pin(oracle.ring_attention)


def test_sampled_form_matches_the_full_form():
    R, S, H, D = 3, 5, 3, 4
    args = _inputs(74, R, S, H, D)
    O, L = oracle.ring_attention(*args, row_block=2)
    rows, heads = np.array([0, 4, 2, 4, 1]), np.array([2, 0, 1, 2, 0])
    Os, Ls = oracle.ring_attention_at(*args, rows, heads)
    assert np.allclose(Os, O[rows, heads], rtol=1e-13, atol=1e-14)
    assert np.allclose(Ls, L[heads, rows], rtol=1e-13, atol=1e-14)


def _reference_with(q, kl, vl, kp, vp, *, scale_pow=-0.5, drop_last=False, head0_v=False,
                    log_base=math.e, v_is_k=False, hsd=False):
    """A deliberately wrong variant of the definition, for the mutants."""
    if hsd:   # read [S, H, D] buffers as if they were [H, S, D]
        q, kl, vl = (x.reshape(x.shape[1], x.shape[0], x.shape[2]).transpose(1, 0, 2) for x in (q, kl, vl))
        kp, vp = (x.reshape(x.shape[0], x.shape[2], x.shape[1], x.shape[3]).transpose(0, 2, 1, 3) for x in (kp, vp))
    S, H, D = q.shape
    if drop_last and kp.shape[0]:
        kp, vp = kp[:-1], vp[:-1]
    K = _dec(np.concatenate([kl[None], kp], axis=0).reshape(-1, H, D))
    V = _dec(np.concatenate([vl[None], vp], axis=0).reshape(-1, H, D))
    if v_is_k:
        V = K
    Q = _dec(q)
    O = np.zeros((S, H, D))
    L = np.zeros((H, S))
    for h in range(H):
        s_ = Q[:, h] @ K[:, h].T * D ** scale_pow
        m = s_.max(axis=1, keepdims=True)
        w = np.exp(s_ - m)
        O[:, h] = (w @ V[:, 0 if head0_v else h]) / w.sum(axis=1, keepdims=True)
        L[h] = (m + np.log(w.sum(axis=1, keepdims=True)))[:, 0] / math.log(log_base)
    return O, L


RA_MUTANTS = {
    "no_scale": lambda *a: _reference_with(*a, scale_pow=0.0),
    "scale_inverted": lambda *a: _reference_with(*a, scale_pow=0.5),
    "last_peer_dropped": lambda *a: _reference_with(*a, drop_last=True),
    "v_of_head_0": lambda *a: _reference_with(*a, head0_v=True),
    "lse_base_2": lambda *a: _reference_with(*a, log_base=2.0),
    "k_used_as_v": lambda *a: _reference_with(*a, v_is_k=True),
    "layout_h_s_d": lambda *a: _reference_with(*a, hsd=True),
}


def test_unmutated_variant_meets_every_pin():
    for pin in RA_PINS:
        assert pin(lambda *a: _reference_with(*a)), pin.__name__


@pytest.mark.parametrize("name", sorted(RA_MUTANTS))
def test_planted_ring_mistake_fails_a_pin(name):
    fn = RA_MUTANTS[name]
    failed = []
    for pin in RA_PINS:
        try:
            ok = pin(fn)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_ring_oracle_rejects_bad_shapes():
    z = np.zeros((2, 1, 4), np.uint16)
    with pytest.raises(ValueError):
        oracle.ring_attention(z, z, z, np.zeros((1, 2, 1, 3), np.uint16), np.zeros((1, 2, 1, 3), np.uint16))
    with pytest.raises(ValueError):
        oracle.ring_attention(z, z[:1], z, np.zeros((1, 2, 1, 4), np.uint16), np.zeros((1, 2, 1, 4), np.uint16))


# ---------------------------------------------------------------------------
# protocol
# ---------------------------------------------------------------------------

def test_split_rule_hand_values():
    assert oracle.ra_kv_tiles(4096) == 32 and oracle.ra_kv_tiles(200) == 2 and oracle.ra_kv_tiles(128) == 1
    # 2 (K, V) x 128 rows x H x D x 2 bytes over 64 KiB
    assert oracle.ra_parts_per_tile(32, 128) == 32
    assert oracle.ra_parts_per_tile(2, 128) == 2
    assert oracle.ra_parts_per_tile(1, 128) == 1
    assert oracle.ra_parts_per_tile(3, 128) == 3
    assert oracle.ra_parts_per_tile(128, 128) == 64


def test_deterministic_owners_hand_example():
    co, po = oracle.ra_deterministic_owners(3, 4, 6, 2, parts=2)
    np.testing.assert_array_equal(co, [0, 1, 0, 1, 0, 1])
    np.testing.assert_array_equal(po, [2, 3, 4, 5])
    co, po = oracle.ra_deterministic_owners(2, 5, 4, 3, parts=1)
    np.testing.assert_array_equal(co, [0, 1])
    np.testing.assert_array_equal(po, [3, 3, 3, 3, 3])


def _good(n_tiles=3, n_tasks=5, B=6, n=2, parts=2):
    exp = oracle.ra_expected_state(n_tiles, n_tasks, 4, 3, parts)
    co, po = oracle.ra_deterministic_owners(n_tiles, n_tasks, B, n, parts)
    maps = {k: v.copy() for k, v in exp.items()}
    maps["copy_owner"] = co | (n << 16)
    maps["compute_owner"] = po | (n << 16)
    return maps


def test_ra_check_state_accepts_the_closed_form():
    np.testing.assert_array_equal(oracle.ra_expected_state(3, 5, 4, 3, 2)["tile_copy_cnt"], [6, 6, 6])
    for mode in ("deterministic", "static", "adaptive"):
        assert oracle.ra_check_state(_good(), 3, 5, 4, 3, 6, mode, 2, 2) == []


@pytest.mark.parametrize("corrupt", [
    lambda m: m["tile_flag"].__setitem__(1, 3),
    lambda m: m["tile_copy_cnt"].__setitem__(2, 5),
    lambda m: m["task_compute_cnt"].__setitem__(4, 2),
    lambda m: m["copy_owner"].__setitem__(0, 1 | (2 << 16)),
    lambda m: m["compute_owner"].__setitem__(3, 2 | (2 << 16)),
    lambda m: m.__setitem__("copy_owner", m["copy_owner"][:3]),
])
def test_ra_check_state_rejects_corruption(corrupt):
    maps = _good()
    corrupt(maps)
    assert oracle.ra_check_state(maps, 3, 5, 4, 3, 6, "deterministic", 2, 2)


def test_ra_check_state_roles_and_help_mark():
    maps = _good()
    maps["copy_owner"][1] = 4 | (2 << 16)          # a compute workgroup copied, unmarked
    assert oracle.ra_check_state(maps, 3, 5, 4, 3, 6, "adaptive", 2, 2)
    maps["copy_owner"][1] = oracle.OWNER_HELP | 4 | (2 << 16)
    assert oracle.ra_check_state(maps, 3, 5, 4, 3, 6, "adaptive", 2, 2) == []
    assert oracle.ra_check_state(maps, 3, 5, 4, 3, 6, "static", 2, 2)
    maps = _good()
    maps["compute_owner"][0] = 1 | (2 << 16)       # a copy workgroup computed
    assert oracle.ra_check_state(maps, 3, 5, 4, 3, 6, "adaptive", 2, 2)
