"""GPU: every fused share, one after another, on the one per-device
workspace.  GEMM+AllReduce, AllGather+GEMM, Ring Attention,
GEMM+ReduceScatter, then GEMM+AllReduce again on its first shape: each launch
takes the next epoch, its counters restart for the new shape, its result
matches the oracle and its protocol state matches the closed form of a
first call on that shape.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_util import check_full, check_protocol, run_fused
from test_gpu_ag import ag_protocol, check_ag, run_ag
from test_gpu_ring import check_ring, ring_protocol, run_ring
from test_gpu_rs import check_rs_full, check_rs_protocol, run_rs

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
    mk.set_adaptive_help(True)
    yield mk
    mk.set_partition("adaptive", 0)


def test_every_share_back_to_back_on_one_workspace(mk):
    epochs = []

    w1 = wl.custom(320, 256, 128, 2, 64, 64, 4, wid=880)
    a1, b1, p1 = wl.make_inputs(w1)
    C, st = run_fused(mk, w1, a1, b1, p1, mode="adaptive", n_reduce=0)
    check_full(C, a1, b1, p1)
    check_protocol(st, w1, "adaptive", 0)
    epochs.append(st["epoch"])

    w2 = wl.custom(128, 136, 256, 2, 64, 64, 1, wid=881)
    a0, ap, b2 = wl.make_ag_inputs(w2)
    g, C2, st = run_ag(mk, True, w2, a0, ap, b2, "adaptive", 0)
    check_ag(g, C2, a0, ap, b2)
    ag_protocol(st, w2, "adaptive", 0)
    assert st["calls_since_reset"] == 1
    epochs.append(st["epoch"])

    w3 = wl.ra_custom(3, 200, 2, 128, wid=882)
    inp = wl.make_ra_inputs(w3)
    O, L, kr, vr, st = run_ring(mk, True, w3, inp, "adaptive", 0)
    check_ring(O, L, kr, vr, inp)
    ring_protocol(st, w3, "adaptive", 0)
    assert st["calls_since_reset"] == 1
    epochs.append(st["epoch"])

    w4 = wl.custom(1100, 264, 200, 1, 128, 128, 4, wid=883)
    a4, b4, p4 = wl.make_inputs(w4)
    r4 = wl.make_remote(w4)
    C4, R4, st = run_rs(mk, True, w4, a4, b4, p4, r4, mode="adaptive", n_reduce=0)
    check_rs_full(C4, R4, a4, b4, p4, r4, w4)
    check_rs_protocol(st, w4, "adaptive", 0)
    assert st["calls_since_reset"] == 1
    epochs.append(st["epoch"])

    C, st = run_fused(mk, w1, a1, b1, p1, mode="adaptive", n_reduce=0)
    check_full(C, a1, b1, p1)
    check_protocol(st, w1, "adaptive", 0)
    assert st["calls_since_reset"] == 1
    epochs.append(st["epoch"])

    assert all(np.diff(epochs) > 0), epochs
