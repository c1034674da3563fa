"""The allocation-free entry point (mk_gemm_reduce_local_noalloc) through the
C ABI, against the allocating one (mk_gemm_reduce_local) and the oracle.

The two share their kernels and the order of every addition, so their outputs
must agree bit for bit; each is also held to the oracle's tolerance and its
protocol state to the closed form.  Two calls of the new entry point run in a
row, the second on a smaller input, so the static workspace is reused across
a change of tile grid.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_util import check_full, check_protocol

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


def _launch(mk, fn, w, a, b, p, mode, n):
    from gemm_tile_granular_amd.tensors import upload
    A, B, P, C = upload(a, b, p)
    mk.set_partition(mode, n)
    print(f"[gpu] {fn.__name__} {w.M}x{w.N}x{w.K} P={w.peers} tile {w.tile_m}x{w.tile_n} "
          f"mode {mode} n={n}", flush=True)
    fn(A, B, P, C, w.tile_m, w.tile_n, w.tiles_per_chunk)
    st = mk.get_stats(maps=True)
    return C.cpu().numpy(), st


SHAPES = [((1000, 1000, 512, 3, 128, 128, 4), 901),   # 64 tiles, XCD-local partitions
          ((200, 136, 72, 2, 64, 64, 4), 902)]        # smaller: 12 tiles, ragged edges


@pytest.mark.parametrize("mode,n", [("adaptive", 0), ("static", 4), ("deterministic", 3)])
def test_noalloc_matches_the_allocating_entry_point(mk, mode, n):
    cases = []
    for shape, wid in SHAPES:
        w = wl.custom(*shape, wid=wid)
        a, b, p = wl.make_inputs(w)
        C_ref, _ = _launch(mk, mk.gemm_reduce_local, w, a, b, p, mode, n)
        cases.append((w, a, b, p, C_ref))
    # the new entry point twice in a row, the second call on the smaller grid
    for w, a, b, p, C_ref in cases:
        C, st = _launch(mk, mk.gemm_reduce_local_noalloc, w, a, b, p, mode, n)
        check_full(C, a, b, p)
        check_protocol(st, w, mode, n)
        assert np.array_equal(C, C_ref)


def test_noalloc_back_to_back_epochs(mk):
    """Repeated calls on one grid: epochs advance, counters count every call."""
    w = wl.custom(520, 392, 200, 5, 256, 128, 3, wid=903)
    a, b, p = wl.make_inputs(w)
    from gemm_tile_granular_amd.tensors import upload
    A, B, P, C = upload(a, b, p)
    mk.set_partition("static", 6)
    print("[gpu] noalloc back to back", flush=True)
    for _ in range(3):
        mk.gemm_reduce_local_noalloc(A, B, P, C, w.tile_m, w.tile_n, w.tiles_per_chunk)
    st = mk.get_stats(maps=True)
    assert st["calls_since_reset"] >= 3
    check_protocol(st, w, "static", 6)
    check_full(C.cpu().numpy(), a, b, p)


def test_noalloc_rejects_a_grid_beyond_its_workspace(mk):
    """91 x 91 tiles of 64x64 (8281 > 8192): refused before any launch."""
    import torch
    w = wl.custom(64 * 91, 64 * 91, 8, 0, 64, 64, 4, wid=904)
    A = torch.zeros((w.M, w.K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((w.K, w.N), dtype=torch.bfloat16, device="cuda")
    C = torch.full((w.M, w.N), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(mk.MkError) as e:
        mk.gemm_reduce_local_noalloc(A, B, None, C, 64, 64, 4)
    assert e.value.code == mk.MK_ERR_SHAPE
    assert "8192" in str(e.value)
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())
