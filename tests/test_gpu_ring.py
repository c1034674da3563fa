"""GPU parity for one rank's share of Ring Attention: the fused and unfused
entry points (through the C ABI) against oracle.ring_attention.

Tolerance, from the arithmetic: the kernel rounds each exponentiated score
p_j to bfloat16 (relative error at most 2^-9) before P.V, and everything else
is fp32 on exact bf16 inputs.  With weights w_j = p_j / sum p, the error of
O_i is then at most 2^-9 sum_j w_ij |v_j|, i.e. 2^-9 times the attention
output of |V| (the oracle on the sign-cleared V), plus fp32 rounding; the test
allows 1.1 times that plus 1e-5.  LSE comes from fp32 sums of unrounded p:
|LSE - LSE_ref| <= 1e-3.  The ring buffers are bit-exact copies; the fused
and unfused launches (same core, same order of operations) agree bit for bit;
the protocol state matches its closed form (oracle.ra_check_state).
"""
import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def mk():
    import gemm_tile_granular_amd as mk
    mk.set_num_workgroups(0)
    mk.set_timeout_us(2_000_000)
    mk.set_fault_skip_publish(-1)
    mk.set_controller_floor(2)
    mk.set_controller_cap(0)
    yield mk
    mk.set_partition("adaptive", 0)


def _t(x, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)


def run_ring(mk, fused, w, inp, mode="adaptive", n=0):
    import torch
    q, kl, vl, kp, vp = inp
    P = kp.shape[0]
    Q, KL, VL = _t(q), _t(kl), _t(vl)
    KP = _t(kp) if P else None
    VP = _t(vp) if P else None
    KR = torch.full(kp.shape, 3.0, dtype=torch.bfloat16, device="cuda") if P else None
    VR = torch.full(vp.shape, 3.0, dtype=torch.bfloat16, device="cuda") if P else None
    O = torch.full(q.shape, -7.0, dtype=torch.float32, device="cuda")
    L = torch.full((w.H, w.S), -7.0, dtype=torch.float32, device="cuda")
    print(f"[gpu] ring {'fused' if fused else 'unfused'} R={w.ranks} S={w.S} H={w.H} mode {mode} n={n}", flush=True)
    st = None
    if fused:
        mk.set_partition(mode, n)
        mk.ring_attention_local(Q, KL, VL, KP, VP, KR, VR, O, L)
        st = mk.get_stats(maps=True)
    else:
        mk.ring_attention_unfused(Q, KL, VL, KP, VP, KR, VR, O, L)
    torch.cuda.synchronize()
    kr = KR.cpu().view(torch.int16).numpy().view(np.uint16) if P else kp
    vr = VR.cpu().view(torch.int16).numpy().view(np.uint16) if P else vp
    return O.cpu().numpy(), L.cpu().numpy(), kr, vr, st


def o_bound(inp, O_abs):
    return 1.1 * 2.0 ** -9 * O_abs + 1e-5


def abs_v(bits):
    return (np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)).astype(np.uint16)


def check_ring(O, L, kr, vr, inp):
    q, kl, vl, kp, vp = inp
    assert np.array_equal(kr, kp) and np.array_equal(vr, vp), "ring buffers differ from the arriving K, V"
    O_ref, L_ref = oracle.ring_attention(*inp)
    O_abs, _ = oracle.ring_attention(q, kl, abs_v(vl), kp, abs_v(vp))
    err = np.abs(O.astype(np.float64) - O_ref)
    bound = o_bound(inp, O_abs)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"O off at {bad[:4].tolist()}: err {err[tuple(bad[0])]:.3e} > {bound[tuple(bad[0])]:.3e}"
    lerr = float(np.max(np.abs(L.astype(np.float64) - L_ref)))
    assert lerr <= LSE_TOL, f"max|LSE - LSE_ref| = {lerr:.3e}"


def ring_protocol(st, w, mode, n):
    nkv = -(-w.S // 128)
    Ch = (w.ranks - 1) * nkv
    NTk = w.H * nkv
    parts = oracle.ra_parts_per_tile(w.H, w.D)
    Qc = Ch * parts
    assert st["kind"] == 3 and st["status"] == 0, st["status_name"]
    assert st["num_chunks"] == Ch and st["tiles_per_chunk"] == parts
    assert st["num_tiles"] == max(NTk, Qc)
    assert st["compute_tasks"] == NTk and st["reduce_tasks"] == Qc and st["chunks_released"] == Ch
    maps = {"tile_flag": st["chunk_flag"], "tile_copy_cnt": st["chunk_cnt"],
            "task_compute_cnt": st["tile_reduce_cnt"][:NTk], "copy_owner": st["reduce_owner"][:Qc],
            "compute_owner": st["compute_owner"][:NTk]}
    bad = oracle.ra_check_state(maps, Ch, NTk, st["epoch"], st["calls_since_reset"], st["num_wg"], mode,
                                n if mode != "adaptive" else st["n_reduce_initial"], parts)
    assert not bad, bad


RING_SHAPES = [
    # R, S, H -- ragged token counts, one rank, S below one tile, H >= 8 (head bands)
    (2, 256, 2),
    (3, 200, 3),
    (1, 128, 1),
    (4, 130, 2),
    (2, 64, 5),
    (8, 128, 9),
    (3, 384, 8),
]


@pytest.mark.parametrize("shape", RING_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mode,n", [("adaptive", 0), ("static", 3), ("deterministic", 2)])
def test_ring_attention_full_oracle(mk, shape, mode, n):
    R, S, H = shape
    w = wl.ra_custom(R, S, H, 128, wid=300 + R * 7 + S % 61 + H)
    inp = wl.make_ra_inputs(w)
    O, L, kr, vr, st = run_ring(mk, True, w, inp, mode, n)
    check_ring(O, L, kr, vr, inp)
    ring_protocol(st, w, mode, n)
    Ou, Lu, kru, vru, _ = run_ring(mk, False, w, inp)
    assert np.array_equal(O, Ou) and np.array_equal(L, Lu)
    assert np.array_equal(kru, kr) and np.array_equal(vru, vr)


def test_ring_back_to_back_epochs(mk):
    import torch
    w = wl.ra_custom(3, 256, 2, 128, wid=330)
    inp = wl.make_ra_inputs(w)
    q, kl, vl, kp, vp = inp
    KR = torch.empty(kp.shape, dtype=torch.bfloat16, device="cuda")
    VR = torch.empty(vp.shape, dtype=torch.bfloat16, device="cuda")
    O = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    L = torch.empty((w.H, w.S), dtype=torch.float32, device="cuda")
    mk.set_partition("static", 4)
    for _ in range(3):
        mk.ring_attention_local(_t(q), _t(kl), _t(vl), _t(kp), _t(vp), KR, VR, O, L)
    st = mk.get_stats(maps=True)
    assert st["calls_since_reset"] >= 3
    ring_protocol(st, w, "static", 4)
    torch.cuda.synchronize()
    check_ring(O.cpu().numpy(), L.cpu().numpy(), KR.cpu().view(torch.int16).numpy().view(np.uint16),
               VR.cpu().view(torch.int16).numpy().view(np.uint16), inp)


def test_ring_timeout_is_reported_not_hung(mk):
    """An arriving tile whose flag is never set: every wait on it expires
    (20 ms), every workgroup leaves, the launch reports MK_ERR_TIMEOUT, and
    the next launch is clean."""
    import torch
    w = wl.ra_custom(3, 256, 2, 128, wid=331)
    inp = wl.make_ra_inputs(w)
    q, kl, vl, kp, vp = inp
    KR = torch.empty(kp.shape, dtype=torch.bfloat16, device="cuda")
    VR = torch.empty(vp.shape, dtype=torch.bfloat16, device="cuda")
    O = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    L = torch.empty((w.H, w.S), dtype=torch.float32, device="cuda")
    mk.set_timeout_us(20_000)
    mk.set_fault_skip_publish(1)
    try:
        for mode in ("deterministic", "adaptive"):
            mk.set_partition(mode, 2)
            print(f"[gpu] ring timeout case, mode {mode}", flush=True)
            mk.ring_attention_local(_t(q), _t(kl), _t(vl), _t(kp), _t(vp), KR, VR, O, L)
            st = mk.get_stats(maps=True, raise_on_error=False)
            assert st["rc"] == mk.MK_ERR_TIMEOUT
    finally:
        mk.set_fault_skip_publish(-1)
        mk.set_timeout_us(2_000_000)
    Ok, Lk, kr, vr, st = run_ring(mk, True, w, inp, "static", 2)
    check_ring(Ok, Lk, kr, vr, inp)
    ring_protocol(st, w, "static", 2)


def test_ring_head_bands_change_no_result(mk):
    """Compute claims in 1, 2, 4 or 8 head bands move tasks between
    workgroups only: outputs bit-identical, protocol state closed-form."""
    w = wl.ra_custom(3, 256, 8, 128, wid=332)
    inp = wl.make_ra_inputs(w)
    base = None
    try:
        for bands in (1, 2, 4, 8):
            mk.set_xcd_bands(bands)
            O, L, kr, vr, st = run_ring(mk, True, w, inp, "adaptive", 0)
            ring_protocol(st, w, "adaptive", 0)
            assert st["xcd_bands"] in (1, bands)
            if base is None:
                check_ring(O, L, kr, vr, inp)
                base = (O, L)
            else:
                assert np.array_equal(O, base[0]) and np.array_equal(L, base[1])
    finally:
        mk.set_xcd_bands(0)


@pytest.mark.parametrize("name", ["ra_sp_share", "ra_long"])
def test_ring_full_size_sampled(mk, name):
    """The full-size shares in the launch the bench times: ring buffers
    bit-exact, O and LSE at sampled (query, head) pairs against the oracle
    one at a time, fused equal to unfused everywhere."""
    w = wl.ra_workload(name)
    inp = wl.make_ra_inputs(w)
    q, kl, vl, kp, vp = inp
    O, L, kr, vr, st = run_ring(mk, True, w, inp, "adaptive", 0)
    ring_protocol(st, w, "adaptive", 0)
    assert np.array_equal(kr, kp) and np.array_equal(vr, vp)
    rng = np.random.default_rng(13)
    rows = rng.integers(0, w.S, 48)
    heads = rng.integers(0, w.H, 48)
    Oref, Lref = oracle.ring_attention_at(*inp, rows, heads)
    Oabs, _ = oracle.ring_attention_at(q, kl, abs_v(vl), kp, abs_v(vp), rows, heads)
    err = np.abs(O[rows, heads].astype(np.float64) - Oref)
    assert np.all(err <= 1.1 * 2.0 ** -9 * Oabs + 1e-5), float(np.max(err))
    assert float(np.max(np.abs(L[heads, rows] - Lref))) <= LSE_TOL
    Ou, Lu, _, _, _ = run_ring(mk, False, w, inp)
    assert np.array_equal(O, Ou) and np.array_equal(L, Lu)


@pytest.mark.parametrize("nwg,mode,n", [(2, "adaptive", 0), (2, "static", 1), (3, "deterministic", 1),
                                        (5, "adaptive", 0), (5, "static", 2)])
def test_ring_few_workgroups(mk, nwg, mode, n):
    """Grids of 2-5 workgroups: the copy role keeps at least one workgroup
    while tiles remain to copy, so every compute task completes."""
    mk.set_num_workgroups(nwg)
    try:
        w = wl.ra_custom(3, 200, 2, 128, wid=340 + nwg)
        inp = wl.make_ra_inputs(w)
        O, L, kr, vr, st = run_ring(mk, True, w, inp, mode, n)
        assert st["num_wg"] == nwg
        check_ring(O, L, kr, vr, inp)
        ring_protocol(st, w, mode, n)
    finally:
        mk.set_num_workgroups(0)
