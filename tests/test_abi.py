"""The C ABI without a GPU: the library loads, exports every symbol that
include/mk.h declares, its stats struct matches the binding, and argument
checks answer before any HIP call (no compute is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")


@pytest.fixture(scope="module")
def mk():
    # build.py by path: importing the package first would load a stale library
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_mk_build", os.path.join(ROOT, "gemm_tile_granular_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    if build.is_stale():
        build.build()
    import gemm_tile_granular_amd as mk
    return mk


def _header():
    with open(HEADER) as f:
        return f.read()


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header(), flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_0-9]+)\s*\(", text)))


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_every_declared_symbol_is_exported(mk):
    names = _declared_functions()
    assert "mk_gemm_reduce_local" in names and "mk_get_stats" in names
    lib = ctypes.CDLL(mk.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding declares a signature for each one
    assert sorted(mk.SIGNATURES) == names


def test_stats_struct_matches_header(mk):
    text = _header()
    body = re.search(r"typedef struct mk_stats \{(.*?)\} mk_stats;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        ctype, names = decl.split(None, 1)
        for n in names.split(","):
            fields.append((n.strip(), ctype))
    want = {"uint32_t": ctypes.c_uint32, "int32_t": ctypes.c_int32, "uint64_t": ctypes.c_uint64}
    got = [(n, t) for n, t in mk.Stats._fields_]
    assert [n for n, _ in got] == [n for n, _ in fields]
    assert all(t == want[c] for (_, t), (_, c) in zip(got, fields))
    assert ctypes.sizeof(mk.Stats) == 176


def test_abi_version_and_trace_cap(mk):
    assert mk.abi_version() == int(re.search(r"#define MK_ABI_VERSION (\d+)", _header()).group(1))
    assert mk.TRACE_CAP == int(re.search(r"#define MK_TRACE_CAP (\d+)", _header()).group(1))


# fake, never dereferenced addresses (16-byte aligned unless stated)
A, B, P, C = 0x1000000, 0x2000000, 0x3000000, 0x4000000


def _call(mk, **kw):
    args = dict(A=A, B=B, peers=P, num_peers=3, C=C, M=256, N=256, K=512, tm=64, tn=64, tpc=4)
    args.update(kw)
    return mk.lib.mk_gemm_reduce_local(args["A"], args["B"], args["peers"], args["num_peers"],
                                       args["C"], args["M"], args["N"], args["K"], args["tm"],
                                       args["tn"], args["tpc"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), -1), (dict(K=-8), -1), (dict(num_peers=-1), -1),
    (dict(tm=32, tn=32), -1), (dict(tm=128, tn=64), -1), (dict(tpc=0), -1), (dict(tpc=65), -1),
    (dict(N=260), -2), (dict(K=100), -2), (dict(M=1 << 31), -2),
    (dict(M=1 << 22, N=1 << 16), -2),
    (dict(C=0), -1), (dict(A=0), -1), (dict(B=0), -1), (dict(peers=0), -1),
    (dict(num_peers=0), -1),                 # peers given but num_peers == 0
    (dict(A=A + 8), -1), (dict(C=C + 4), -1), (dict(peers=P + 2), -1),
    (dict(C=A + 4096), -1), (dict(C=B), -1), (dict(C=P + 65536), -1),   # C overlaps an input
])
def test_argument_errors_before_any_gpu_call(mk, kw, code):
    assert _call(mk, **kw) == code
    assert mk.lib.mk_last_error().decode()
    # the unfused entry point applies the same checks
    args = dict(A=A, B=B, peers=P, num_peers=3, C=C, M=256, N=256, K=512, tm=64, tn=64, tpc=4)
    args.update(kw)
    assert mk.lib.mk_gemm_reduce_unfused(args["A"], args["B"], args["peers"], args["num_peers"],
                                         args["C"], args["M"], args["N"], args["K"], args["tm"],
                                         args["tn"], args["tpc"], None) == code


R = 0x5000000   # fake remote output


def _call_rs(mk, fused=True, **kw):
    args = dict(A=A, B=B, peers=P, num_peers=3, C=C, remote=R, M=256, N=256, K=512, tm=64, tn=64, tpc=4)
    args.update(kw)
    fn = mk.lib.mk_gemm_reduce_scatter_local if fused else mk.lib.mk_gemm_reduce_scatter_unfused
    return fn(args["A"], args["B"], args["peers"], args["num_peers"], args["C"], args["remote"], args["M"],
              args["N"], args["K"], args["tm"], args["tn"], args["tpc"], None)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), -1), (dict(tm=128, tn=64), -1), (dict(tpc=0), -1), (dict(N=260), -2),
    (dict(C=0), -1), (dict(peers=0), -1), (dict(A=A + 8), -1),
    (dict(remote=0), -1),                     # other ranks own tile rows: remote is needed
    (dict(remote=R + 4), -1),                 # misaligned
    (dict(remote=C + 1024), -1),              # overlaps C
    (dict(remote=P + 4096), -1),              # overlaps the peers
])
def test_reduce_scatter_argument_errors(mk, fused, kw, code):
    assert _call_rs(mk, fused, **kw) == code
    assert mk.lib.mk_last_error().decode()


def test_reduce_scatter_empty_output_is_a_no_op(mk):
    assert _call_rs(mk, M=0, remote=0) == 0
    assert _call_rs(mk, fused=False, N=0, remote=0) == 0


@pytest.mark.skipif(_gpu_present(), reason="fake pointers must never reach a real GPU")
def test_reduce_scatter_one_rank_needs_no_remote(mk):
    # R = 1: rank 0 owns every row, so remote may be NULL; the call gets as
    # far as looking for a device
    assert _call_rs(mk, peers=0, num_peers=0, remote=0) == mk.MK_ERR_NO_DEVICE
    assert _call_rs(mk) == mk.MK_ERR_NO_DEVICE


def test_empty_output_is_a_no_op(mk):
    assert _call(mk, M=0) == 0
    assert _call(mk, N=0) == 0
    assert _call(mk, M=0, A=0, B=0, C=0, peers=0, num_peers=0) == 0


@pytest.mark.skipif(_gpu_present(), reason="fake pointers must never reach a real GPU")
def test_valid_arguments_without_a_device_report_no_device(mk):
    assert _call(mk) == mk.MK_ERR_NO_DEVICE
    assert mk.lib.mk_device_cu_count() == mk.MK_ERR_NO_DEVICE


def test_setting_calls_validate(mk):
    lib = mk.lib
    assert lib.mk_set_partition(7, 2) == -1
    assert lib.mk_set_partition(mk.PART_STATIC, 0) == -1
    assert lib.mk_set_partition(mk.PART_STATIC, -3) == -1
    assert lib.mk_set_partition(mk.PART_ADAPTIVE, 0) == 0
    assert lib.mk_set_num_workgroups(1) == -1
    assert lib.mk_set_num_workgroups(4096) == -1
    assert lib.mk_set_num_workgroups(0) == 0
    assert lib.mk_set_timeout_us(0) == -1
    assert lib.mk_set_timeout_us(2000000) == 0
    assert lib.mk_set_fault_skip_publish(-2) == -1
    assert lib.mk_set_fault_skip_publish(-1) == 0
    assert lib.mk_set_controller_floor(0) == -1
    assert lib.mk_set_controller_floor(2) == 0
    assert lib.mk_set_controller_cap(-1) == -1
    assert lib.mk_set_controller_cap(1025) == -1
    assert lib.mk_set_controller_cap(0) == 0
    for bad in (-1, 3, 5, 16):
        assert lib.mk_set_xcd_bands(bad) == -1
    for ok in (1, 2, 4, 8, 0):
        assert lib.mk_set_xcd_bands(ok) == 0
    assert lib.mk_controller_eval(None, None, -1, None) == -1
    assert lib.mk_controller_eval(None, None, 0, None) == 0


def test_get_stats_rejects_bad_struct(mk):
    assert mk.lib.mk_get_stats(None, None, 0) == -1
    st = mk.Stats()
    st.struct_size = 12
    assert mk.lib.mk_get_stats(ctypes.byref(st), None, 0) == -1


def test_binding_rejects_wrong_tensor_types(mk):
    torch = pytest.importorskip("torch")
    a = torch.zeros(4, 8, dtype=torch.float32)
    with pytest.raises(ValueError):
        mk.gemm_reduce_local(a, a, None, a, 64, 64)


def test_kernels_fit_their_register_and_lds_budget(mk):
    """The compiler's resource report of the last build: every kernel keeps
    its state in registers (no scratch: a reload in a K loop would make the
    compiler wait for every load in flight, the operand ring included), the
    256x128 fused kernel keeps two 8-wave blocks per CU, and no kernel asks
    for more LDS than a CU has (160 KiB)."""
    import json
    lib = os.path.join(ROOT, "gemm_tile_granular_amd", "libmk.so")
    path = os.path.join(ROOT, "gemm_tile_granular_amd", "libmk.resources.json")
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(lib):
        pytest.skip("library built without a resource report")
    with open(path) as f:
        res = json.load(f)
    fused = {k: v for k, v in res.items() if "fused_gemm_reduce_kernel" in k}
    ag = {k: v for k, v in res.items() if "allgather_gemm_kernel" in k}
    gemm = {k: v for k, v in res.items() if "gemm_kernel" in k and k not in fused and k not in ag}
    assert len(fused) == 12 and len(gemm) == 3 and len(ag) == 3, sorted(res)
    for name, r in ag.items():
        if "ILi256ELi128E" in name:
            assert r["Occupancy"] == 2, (name, r)
    for name, r in res.items():
        assert r["LDS Size"] <= 160 * 1024, name
        assert r["ScratchSize"] == 0, (name, r)
        # no vector register spills either (SGPR spills land in VGPR lanes,
        # which costs no memory traffic)
        assert r.get("VGPRs Spill", 0) == 0, (name, r)
    for name, r in fused.items():
        if "ILi256ELi128E" in name:
            assert r["Occupancy"] == 2, (name, r)
