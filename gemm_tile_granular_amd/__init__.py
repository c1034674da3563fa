"""Python binding of libmk.so, the fused GEMM + tile-reduce library for MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels of
libmk.so (C ABI in include/mk.h).  PyTorch supplies device memory and the
current stream; nothing here computes.  If the library is not built, import
fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmk.so")

MK_OK = 0
MK_ERR_INVALID_ARG = -1
MK_ERR_SHAPE = -2
MK_ERR_HIP = -3
MK_ERR_TIMEOUT = -4
MK_ERR_NO_DEVICE = -5
MK_ERR_PROTOCOL = -6
STATUS_NAMES = {0: "MK_OK", -1: "MK_ERR_INVALID_ARG", -2: "MK_ERR_SHAPE", -3: "MK_ERR_HIP",
                -4: "MK_ERR_TIMEOUT", -5: "MK_ERR_NO_DEVICE", -6: "MK_ERR_PROTOCOL"}

PART_ADAPTIVE = 0
PART_STATIC = 1
PART_STATIC_DETERMINISTIC = 2
MODES = {"adaptive": PART_ADAPTIVE, "static": PART_STATIC,
         "deterministic": PART_STATIC_DETERMINISTIC}
TRACE_CAP = 1024
SUPPORTED_TILES = ((64, 64), (128, 128), (256, 128))


class MkError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


class Stats(ctypes.Structure):
    """Mirror of struct mk_stats in include/mk.h (same order and types)."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("status", ctypes.c_int32),
        ("epoch", ctypes.c_uint32),
        ("calls_since_reset", ctypes.c_uint32),
        ("num_wg", ctypes.c_uint32),
        ("num_tiles", ctypes.c_uint32),
        ("num_chunks", ctypes.c_uint32),
        ("tiles_per_chunk", ctypes.c_uint32),
        ("tile_m", ctypes.c_uint32),
        ("tile_n", ctypes.c_uint32),
        ("mode", ctypes.c_uint32),
        ("n_reduce_initial", ctypes.c_uint32),
        ("n_reduce_final", ctypes.c_uint32),
        ("n_reduce_min_seen", ctypes.c_uint32),
        ("n_reduce_max_seen", ctypes.c_uint32),
        ("role_switches", ctypes.c_uint32),
        ("compute_tasks", ctypes.c_uint32),
        ("reduce_tasks", ctypes.c_uint32),
        ("chunks_released", ctypes.c_uint32),
        ("invariant_violations", ctypes.c_uint32),
        ("ns_trace_len", ctypes.c_uint32),
        ("tiles_per_task", ctypes.c_uint32),
        ("sum_cycles_compute", ctypes.c_uint64),
        ("sum_cycles_reduce", ctypes.c_uint64),
        ("kernel_ticks_start", ctypes.c_uint64),
        ("kernel_ticks_end", ctypes.c_uint64),
        ("reduce_ticks_start", ctypes.c_uint64),
        ("reduce_ticks_end", ctypes.c_uint64),
        ("timer_hz", ctypes.c_uint64),
        ("xcd_local", ctypes.c_uint32),
        ("keep_compute", ctypes.c_uint32),
        ("controller_cap", ctypes.c_uint32),
        ("xcd_bands", ctypes.c_uint32),
        ("adaptive_help", ctypes.c_uint32),
        ("sticky_errors", ctypes.c_uint32),
        ("kind", ctypes.c_uint32),
    ]


_vp, _i32, _i64, _u32p = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.POINTER(ctypes.c_uint32)

SIGNATURES = {
    "mk_gemm_reduce_local": (_i32, [_vp, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp]),
    "mk_gemm_reduce_local_noalloc": (_i32, [_vp, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _i32, _i32, _i32,
                                             _vp]),
    "mk_gemm_reduce_unfused": (_i32, [_vp, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp]),
    "mk_gemm_reduce_scatter_local": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32,
                                             _vp]),
    "mk_gemm_reduce_scatter_unfused": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32,
                                               _vp]),
    "mk_allgather_gemm_local": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp]),
    "mk_allgather_gemm_unfused": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp]),
    "mk_ring_attention_local": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _vp]),
    "mk_ring_attention_unfused": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _i32, _i32,
                                         _vp]),
    "mk_set_partition": (_i32, [_i32, _i32]),
    "mk_set_controller_floor": (_i32, [_i32]),
    "mk_set_controller_cap": (_i32, [_i32]),
    "mk_set_xcd_bands": (_i32, [_i32]),
    "mk_set_num_workgroups": (_i32, [_i32]),
    "mk_set_adaptive_help": (_i32, [_i32]),
    "mk_set_timeout_us": (_i32, [ctypes.c_uint64]),
    "mk_set_fault_skip_publish": (_i32, [_i64]),
    "mk_get_stats": (_i32, [ctypes.POINTER(Stats), _u32p, ctypes.c_size_t]),
    "mk_controller_eval": (_i32, [_vp, _vp, _i32, _vp]),
    "mk_device_cu_count": (_i32, []),
    "mk_release_workspace": (_i32, []),
    "mk_last_error": (ctypes.c_char_p, []),
    "mk_abi_version": (_i32, []),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python gemm_tile_granular_amd/build.py` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(rc: int) -> None:
    if rc != MK_OK:
        raise MkError(rc, lib.mk_last_error().decode(errors="replace"))


def _torch():
    import torch
    return torch


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_tensors(A, B, peers, C):
    torch = _torch()
    for name, t, dt in (("A", A, torch.bfloat16), ("B", B, torch.bfloat16), ("C", C, torch.float32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
            raise ValueError(f"{name} must be a contiguous 2-D {dt} CUDA tensor")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    P = 0
    if peers is not None:
        if (peers.dtype != torch.float32 or not peers.is_cuda or not peers.is_contiguous()
                or peers.dim() != 3 or tuple(peers.shape[1:]) != (M, N)):
            raise ValueError("peers must be a contiguous [P, M, N] float32 CUDA tensor")
        P = peers.shape[0]
    return M, N, K, P


def _call(fn, A, B, peers, C, tile_m, tile_n, tiles_per_chunk, stream):
    M, N, K, P = _check_tensors(A, B, peers, C)
    pp = peers.data_ptr() if (peers is not None and P > 0) else None
    _check(fn(A.data_ptr(), B.data_ptr(), pp, P, C.data_ptr(), M, N, K,
              tile_m, tile_n, tiles_per_chunk, _stream_handle(stream)))


def gemm_reduce_local(A, B, peers, C, tile_m: int, tile_n: int, tiles_per_chunk: int = 4,
                      stream=None) -> None:
    """C = A.B + sum_p peers[p] in one persistent launch (mk_gemm_reduce_local)."""
    _call(lib.mk_gemm_reduce_local, A, B, peers, C, tile_m, tile_n, tiles_per_chunk, stream)


def gemm_reduce_local_noalloc(A, B, peers, C, tile_m: int, tile_n: int, tiles_per_chunk: int = 4,
                              stream=None) -> None:
    """The same launch on the library's static workspace: the call allocates
    no device memory (mk_gemm_reduce_local_noalloc; at most 8192 tiles)."""
    _call(lib.mk_gemm_reduce_local_noalloc, A, B, peers, C, tile_m, tile_n, tiles_per_chunk, stream)


def gemm_reduce_unfused(A, B, peers, C, tile_m: int, tile_n: int, tiles_per_chunk: int = 4,
                        stream=None) -> None:
    """Same result from two launches: GEMM, then reduce (mk_gemm_reduce_unfused)."""
    _call(lib.mk_gemm_reduce_unfused, A, B, peers, C, tile_m, tile_n, tiles_per_chunk, stream)


def _call_rs(fn, A, B, peers, C, remote, tile_m, tile_n, tiles_per_chunk, stream):
    M, N, K, P = _check_tensors(A, B, peers, C)
    rp = None
    if remote is not None:
        torch = _torch()
        if (remote.dtype != torch.float32 or not remote.is_cuda or not remote.is_contiguous()
                or tuple(remote.shape) != (M, N)):
            raise ValueError("remote must be a contiguous [M, N] float32 CUDA tensor")
        rp = remote.data_ptr()
    pp = peers.data_ptr() if (peers is not None and P > 0) else None
    _check(fn(A.data_ptr(), B.data_ptr(), pp, P, C.data_ptr(), rp, M, N, K,
              tile_m, tile_n, tiles_per_chunk, _stream_handle(stream)))


def gemm_reduce_scatter_local(A, B, peers, C, remote, tile_m: int, tile_n: int, tiles_per_chunk: int = 4,
                              stream=None) -> None:
    """Rank 0's share of GEMM+ReduceScatter in one persistent launch
    (mk_gemm_reduce_scatter_local): C = A.B + sum_p peers[p] on rank 0's tile
    rows (its shard); the other ranks' rows of A.B are stored into remote (this
    rank's inbox slots at their owners); C's other rows and remote's shard rows
    are left untouched."""
    _call_rs(lib.mk_gemm_reduce_scatter_local, A, B, peers, C, remote, tile_m, tile_n, tiles_per_chunk,
             stream)


def gemm_reduce_scatter_unfused(A, B, peers, C, remote, tile_m: int, tile_n: int, tiles_per_chunk: int = 4,
                                stream=None) -> None:
    """Same result from two launches (mk_gemm_reduce_scatter_unfused)."""
    _call_rs(lib.mk_gemm_reduce_scatter_unfused, A, B, peers, C, remote, tile_m, tile_n, tiles_per_chunk,
             stream)


def _call_ag(fn, A_local, A_peers, A_gathered, B, C, tile_m, tile_n, stream):
    torch = _torch()
    for name, t, dt in (("A_local", A_local, torch.bfloat16), ("A_gathered", A_gathered, torch.bfloat16),
                        ("B", B, torch.bfloat16), ("C", C, torch.float32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
            raise ValueError(f"{name} must be a contiguous 2-D {dt} CUDA tensor")
    Ms, K = A_local.shape
    K2, N = B.shape
    P = 0
    if A_peers is not None:
        if (A_peers.dtype != torch.bfloat16 or not A_peers.is_cuda or not A_peers.is_contiguous()
                or A_peers.dim() != 3 or tuple(A_peers.shape[1:]) != (Ms, K)):
            raise ValueError("A_peers must be a contiguous [P, Ms, K] bfloat16 CUDA tensor")
        P = A_peers.shape[0]
    M = (P + 1) * Ms
    if K2 != K or tuple(A_gathered.shape) != (M, K) or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch: A_local [Ms,K], A_peers [P,Ms,K], A_gathered [(P+1)Ms,K], "
                         "B [K,N], C [(P+1)Ms,N]")
    pp = A_peers.data_ptr() if (A_peers is not None and P > 0) else None
    _check(fn(A_local.data_ptr(), pp, P, A_gathered.data_ptr(), B.data_ptr(), C.data_ptr(), Ms, N, K,
              tile_m, tile_n, _stream_handle(stream)))


def allgather_gemm_local(A_local, A_peers, A_gathered, B, C, tile_m: int, tile_n: int, stream=None) -> None:
    """Rank 0's share of AllGather+GEMM in one persistent launch
    (mk_allgather_gemm_local): A_gathered = the shards stacked by rank,
    C = A_gathered . B."""
    _call_ag(lib.mk_allgather_gemm_local, A_local, A_peers, A_gathered, B, C, tile_m, tile_n, stream)


def allgather_gemm_unfused(A_local, A_peers, A_gathered, B, C, tile_m: int, tile_n: int, stream=None) -> None:
    """The same from two launches: gather, then GEMM (mk_allgather_gemm_unfused)."""
    _call_ag(lib.mk_allgather_gemm_unfused, A_local, A_peers, A_gathered, B, C, tile_m, tile_n, stream)


def _call_ring(fn, q, k_local, v_local, k_peers, v_peers, k_ring, v_ring, O, lse, stream):
    torch = _torch()
    for name, t, dt in (("q", q, torch.bfloat16), ("k_local", k_local, torch.bfloat16),
                        ("v_local", v_local, torch.bfloat16), ("O", O, torch.float32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D {dt} CUDA tensor [S, H, D]")
    S, H, D = q.shape
    if tuple(k_local.shape) != (S, H, D) or tuple(v_local.shape) != (S, H, D) or tuple(O.shape) != (S, H, D):
        raise ValueError("q, k_local, v_local and O must all be [S, H, D]")
    if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() or tuple(lse.shape) != (H, S):
        raise ValueError("lse must be a contiguous [H, S] float32 CUDA tensor")
    P = 0
    if k_peers is not None:
        P = k_peers.shape[0]
        for name, t in (("k_peers", k_peers), ("v_peers", v_peers), ("k_ring", k_ring), ("v_ring", v_ring)):
            if (t is None or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous()
                    or tuple(t.shape) != (P, S, H, D)):
                raise ValueError(f"{name} must be a contiguous [P, S, H, D] bfloat16 CUDA tensor")
    ptr = lambda t: t.data_ptr() if (t is not None and P > 0) else None
    _check(fn(q.data_ptr(), k_local.data_ptr(), v_local.data_ptr(), ptr(k_peers), ptr(v_peers), P,
              ptr(k_ring), ptr(v_ring), O.data_ptr(), lse.data_ptr(), S, H, D, _stream_handle(stream)))


def ring_attention_local(q, k_local, v_local, k_peers, v_peers, k_ring, v_ring, O, lse, stream=None) -> None:
    """Rank 0's share of Ring Attention in one persistent launch
    (mk_ring_attention_local): O [S,H,D] and lse [H,S] of attention over
    every rank's keys (no mask, scale 1/sqrt(D)); k_ring / v_ring receive the
    arriving K and V.  k_peers / v_peers are [P,S,H,D] in arrival order, or
    None for one rank."""
    _call_ring(lib.mk_ring_attention_local, q, k_local, v_local, k_peers, v_peers, k_ring, v_ring, O, lse, stream)


def ring_attention_unfused(q, k_local, v_local, k_peers, v_peers, k_ring, v_ring, O, lse, stream=None) -> None:
    """The same from two launches: gather, then attention (mk_ring_attention_unfused)."""
    _call_ring(lib.mk_ring_attention_unfused, q, k_local, v_local, k_peers, v_peers, k_ring, v_ring, O, lse,
               stream)


def set_partition(mode, n_reduce: int = 0) -> None:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    _check(lib.mk_set_partition(m, int(n_reduce)))


def set_controller_floor(floor: int) -> None:
    _check(lib.mk_set_controller_floor(int(floor)))


def set_controller_cap(cap: int) -> None:
    """Most reduce workgroups the adaptive controller sets while compute remains (0: 5B/8)."""
    _check(lib.mk_set_controller_cap(int(cap)))


def set_xcd_bands(bands: int) -> None:
    """Column bands of the XCD-local partitions (0: least operand traffic; 1, 2, 4, 8)."""
    _check(lib.mk_set_xcd_bands(int(bands)))


def set_adaptive_help(on: bool) -> None:
    """Adaptive mode: a reducer whose ticket is not ready computes meanwhile (default on)."""
    _check(lib.mk_set_adaptive_help(1 if on else 0))


def set_num_workgroups(num_wg: int) -> None:
    _check(lib.mk_set_num_workgroups(int(num_wg)))


def set_timeout_us(us: int) -> None:
    _check(lib.mk_set_timeout_us(int(us)))


def set_fault_skip_publish(tile: int) -> None:
    _check(lib.mk_set_fault_skip_publish(int(tile)))


def device_cu_count() -> int:
    rc = lib.mk_device_cu_count()
    if rc < 0:
        _check(rc)
    return rc


def release_workspace() -> None:
    _check(lib.mk_release_workspace())


def abi_version() -> int:
    return lib.mk_abi_version()


def get_stats(maps: bool = False, raise_on_error: bool = True) -> Dict:
    """Stats of the last fused launch (synchronizes).  With maps=True also the
    tile/chunk maps and the controller trace as numpy arrays.  The status is
    sticky: it reports an error raised by any fused launch since the previous
    call, not only by the last launch."""
    st = Stats()
    st.struct_size = ctypes.sizeof(Stats)
    buf = None
    n = 0
    if maps:
        # sized from a first call without maps
        rc0 = lib.mk_get_stats(ctypes.byref(st), None, 0)
        if rc0 not in (MK_OK, MK_ERR_TIMEOUT, MK_ERR_PROTOCOL):
            _check(rc0)
        T, Ch = st.num_tiles, st.num_chunks
        n = 10 * T + 3 * Ch + 2 * TRACE_CAP
        buf = np.zeros(n, dtype=np.uint32)
        st = Stats()
        st.struct_size = ctypes.sizeof(Stats)
    rc = lib.mk_get_stats(ctypes.byref(st), buf.ctypes.data_as(_u32p) if buf is not None else None, n)
    out = {name: getattr(st, name) for name, _ in Stats._fields_}
    out["status_name"] = STATUS_NAMES.get(st.status, str(st.status))
    if maps:
        T, Ch = st.num_tiles, st.num_chunks
        o = 0
        for key, cnt in (("tile_flag", T), ("tile_reduce_cnt", T), ("chunk_cnt", Ch),
                         ("chunk_flag", Ch), ("compute_owner", T), ("reduce_owner", T),
                         ("ns_trace", 2 * TRACE_CAP), ("compute_start", T), ("compute_end", T),
                         ("reduce_start", T), ("reduce_end", T), ("compute_choice_ticks", T),
                         ("reduce_choice_ticks", T), ("chunk_release", Ch)):
            out[key] = buf[o:o + cnt].copy()
            o += cnt
        out["ns_trace"] = out["ns_trace"].reshape(TRACE_CAP, 2)[: st.ns_trace_len]
        # timeline in microseconds since the kernel started
        t0 = np.uint32(st.kernel_ticks_start & 0xFFFFFFFF)
        us = 1e6 / float(st.timer_hz or 100_000_000)
        for key in ("compute_start", "compute_end", "reduce_start", "reduce_end", "chunk_release"):
            out[key + "_us"] = (out[key] - t0).astype(np.uint32).astype(np.float64) * us
        out["ns_trace_us"] = (out["ns_trace"][:, 0] - t0).astype(np.uint32).astype(np.float64) * us
        out["compute_choice_us"] = out["compute_choice_ticks"].astype(np.float64) * us
        out["reduce_choice_us"] = out["reduce_choice_ticks"].astype(np.float64) * us
    if raise_on_error and rc not in (MK_OK,):
        _check(rc)
    out["rc"] = rc
    return out


def controller_eval(rows: np.ndarray) -> np.ndarray:
    """Runs the device controller step on each row (B, T, compute_done,
    reduce_done, sum_cycles_compute, sum_cycles_reduce, current, floor, keep, cap)."""
    torch = _torch()
    rows = np.ascontiguousarray(rows, dtype=np.uint64)
    assert rows.ndim == 2 and rows.shape[1] == 10
    n = rows.shape[0]
    dev_in = torch.from_numpy(rows.view(np.int64)).cuda()
    dev_out = torch.zeros(n, dtype=torch.int32, device=dev_in.device)
    _check(lib.mk_controller_eval(dev_in.data_ptr(), dev_out.data_ptr(), n, _stream_handle(None)))
    torch.cuda.synchronize()
    return dev_out.cpu().numpy().view(np.uint32)
