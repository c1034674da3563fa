"""CPU oracle for the fused GEMM + tile-reduce path.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or run anything in this package.  The product path
(gemm_tile_granular_amd) never imports it, and it imports nothing from there.
It shares no code with the HIP path; the only common module is `workloads`,
which draws the seeded inputs and does none of the method's arithmetic.

What it computes, and from which passage:

* `gemm_reduce` -- the result of GEMM+AllReduce for one rank's output:
  C = A.B (this rank's partial) plus the sum of the other ranks' partial
  outputs.  The method computes C = A @ B and reduces the partial outputs
  across ranks (abstract of "mKernel: Fast Multi-GPU, Multi-Node Fused
  Kernels"; GEMM + AllReduce row of the five-kernel table on the MarkTechPost
  and chathome pages).  Fusion only reorders and overlaps this sum, so the
  oracle is the definition itself, in float64, on the exact bfloat16 input
  values.  The reduction operator is addition (partial sums of a row-parallel
  product).
* `gemm_reduce_scatter` / `rs_shard_bounds` -- one rank's share of
  GEMM+ReduceScatter (GEMM + ReduceScatter row of the five-kernel table on the
  MarkTechPost page: C = A @ B is computed and each output tile is reduced and
  sent to the rank that owns it as soon as it exists; "【学习】mKernel 分析"
  section 2.6, Table 3: tiles reach their rank in chunks of 2 to 32 tiles).
  The pages fix no shard layout.  The reading used: R = P + 1 ranks, this
  rank is rank 0, and rank o owns tile rows [floor(o T_m / R),
  floor((o+1) T_m / R)) of the T_m tile rows.  Each owner keeps an inbox with
  one slot per other rank; a rank stores each finished tile it does not own
  into its slot at the owner, and the owner sums its own partial and its
  inbox.  Here rank 0's inbox is the peers (its own rows receive their sum),
  and a buffer in local memory stands in for rank 0's slots at the other
  owners: every tile of this rank's partial outside its rows is stored
  there.  A rank's output is its shard only; its partial of the other rows
  is not kept.  (The analysis page delivers tiles by atomic add into the
  owner's output instead; the owner's reduced shard is the same sum either
  way.)
* `controller_update` / `controller_target` -- the adaptive partition rule of
  "【学习】mKernel 分析" section 2.4: the target number of communication
  (here: reduce) workgroups n_s* = B (R_s C_s) / (R_p C_p + R_s C_s), the value
  that makes both roles' predicted finish times equal.  The page leaves the
  symbols, rounding and clamping open; the readings used are written next to
  each line below.
* `expected_state` / `check_state` / `deterministic_owners` -- the integer
  protocol: per-tile readiness flags (section 2.2, Figure 2), per-chunk
  counters where the last tile of a 4-tile chunk releases it (section 2.3),
  roles chosen by workgroup index and re-checked at task boundaries
  (sections 2.4 and 4.1); under the adaptive controller a reduce-role
  workgroup whose next tile is not ready yet may compute meanwhile (the
  section 2.4 rule that a block waiting for its input helps the other role,
  read in the direction this kernel's data flows), which its owner word
  marks.

* `ring_attention` / `ring_attention_at` and the `ra_*` protocol forms -- one
  rank's share of Ring Attention (Ring Attention row of the MarkTechPost
  page's five-kernel table: sequence-parallel attention, each step passes a
  KV chunk around the ring while the local FlashAttention consumes the chunk
  received before; compute and ring send/receive run together in one
  persistent kernel.  "【学习】mKernel 分析" section 2.6, Table 3: 128-row KV
  tiles).  The result is the definition of attention over every rank's keys,
  in float64; the readings are written at that section below.

Parity pins (tests/test_oracle.py) tie each function to something other than
itself: hand-worked fixtures, closed forms (A = 0, no peers, B = I, all-ones,
rank-1), an independent C brute force on tiny shapes, the controller's
defining equal-finish-time condition, and mutation checks that a planted
mistake in the oracle fails a pin.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

# ---------------------------------------------------------------------------
# Inputs: bfloat16 bit patterns -> exact values
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of each bfloat16 bit pattern, as float64.

    A bfloat16 pattern is the upper half of an IEEE binary32 pattern, so the
    value is the binary32 number whose low 16 bits are zero.
    """
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Result definition
# ---------------------------------------------------------------------------


def gemm_part(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """This rank's partial product A.B in float64 (A [M,K], B [K,N])."""
    return bf16_bits_to_f64(a_bits) @ bf16_bits_to_f64(b_bits)


def peer_sum(peers: np.ndarray, row_block: int = 1024) -> np.ndarray:
    """Sum over the P peer partials (float32 [P,M,N]) in float64."""
    P, M, N = peers.shape
    out = np.zeros((M, N), dtype=np.float64)
    for r0 in range(0, M, row_block):
        r1 = min(M, r0 + row_block)
        for p in range(P):
            out[r0:r1] += peers[p, r0:r1].astype(np.float64)
    return out


def gemm_reduce(a_bits: np.ndarray, b_bits: np.ndarray, peers: np.ndarray) -> np.ndarray:
    """C_ref = A.B + sum_p peers[p], float64, exact bfloat16 operands."""
    a = np.asarray(a_bits)
    b = np.asarray(b_bits)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("A must be [M,K] and B must be [K,N]")
    out = gemm_part(a, b)
    if peers is not None and peers.shape[0]:
        if peers.shape[1:] != out.shape:
            raise ValueError("peers must be [P,M,N]")
        out += peer_sum(peers)
    return out


def gemm_reduce_at(a_bits: np.ndarray, b_bits: np.ndarray, peers: np.ndarray,
                   rows: Sequence[int], cols: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """C_ref at the listed (row, col) positions, one element at a time.

    Returns (full value, GEMM part) in float64.  Used where the whole product
    is too large for the CPU in a test's time budget.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    a_rows = bf16_bits_to_f64(a_bits[rows, :])            # [S, K]
    b_cols = bf16_bits_to_f64(b_bits[:, cols]).T          # [S, K]
    gemm = np.einsum("sk,sk->s", a_rows, b_cols)
    full = gemm.copy()
    if peers is not None and peers.shape[0]:
        full += peers[:, rows, cols].astype(np.float64).sum(axis=0)
    return full, gemm


def rs_shard_bounds(tiles_m: int, ranks: int) -> np.ndarray:
    """Tile-row bounds of the R row shards: rank o owns tile rows
    [bounds[o], bounds[o+1]), bounds[o] = floor(o * tiles_m / R).  Shards are
    as even as whole tile rows allow; with fewer tile rows than ranks some
    shards are empty."""
    if tiles_m < 0 or ranks < 1:
        raise ValueError("tiles_m >= 0 and ranks >= 1")
    return np.array([(o * tiles_m) // ranks for o in range(ranks + 1)], dtype=np.int64)


def gemm_reduce_scatter(a_bits: np.ndarray, b_bits: np.ndarray, peers: np.ndarray,
                        remote_init: np.ndarray, tile_m: int) -> Tuple[np.ndarray, np.ndarray]:
    """Rank 0's share of GEMM+ReduceScatter with R = P + 1 ranks, float64.

    Returns (shard, remote):
    - shard [own, N], own = min(M, floor(T_m / R) tile_m): rows [0, own) of
      A.B + sum_p peers[p], rank 0's reduced shard;
    - remote [M, N]: A.B on the rows of ranks 1..R-1 (this rank's inbox slot
      at each owner receives its partial of that owner's tiles), remote_init
      on rank 0's rows (never written).
    """
    a = np.asarray(a_bits)
    b = np.asarray(b_bits)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("A must be [M,K] and B must be [K,N]")
    M, N = a.shape[0], b.shape[1]
    P = 0 if peers is None else peers.shape[0]
    if P and peers.shape[1:] != (M, N):
        raise ValueError("peers must be [P,M,N]")
    if remote_init.shape != (M, N):
        raise ValueError("remote_init must be [M,N]")
    tiles_m = -(-M // tile_m)
    bounds = rs_shard_bounds(tiles_m, P + 1)
    own_rows = slice(0, min(M, int(bounds[1]) * tile_m))
    part = gemm_part(a, b)
    shard = part[own_rows].copy()
    if P:
        shard += peer_sum(peers[:, own_rows, :])
    remote = remote_init.astype(np.float64).copy()
    remote[own_rows.stop:] = part[own_rows.stop:]
    return shard, remote


# ---------------------------------------------------------------------------
# Independent brute force (C, single thread) for tiny shapes
# ---------------------------------------------------------------------------

_brute_lib = None


def brute_library_path() -> str:
    return os.path.join(_HERE, "libmkbrute.so")


def build_brute(force: bool = False) -> str:
    """Compile oracle/brute.c with the host C compiler."""
    out = brute_library_path()
    src = os.path.join(_HERE, "brute.c")
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", "-o", tmp, src])
        os.replace(tmp, out)
    return out


def _brute():
    global _brute_lib
    if _brute_lib is None:
        lib = ctypes.CDLL(build_brute())
        lib.mk_brute_gemm_reduce.restype = None
        lib.mk_brute_gemm_reduce.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        _brute_lib = lib
    return _brute_lib


def gemm_reduce_brute(a_bits: np.ndarray, b_bits: np.ndarray, peers: np.ndarray) -> np.ndarray:
    """Triple-loop float64 brute force in C (tiny shapes only)."""
    a = np.ascontiguousarray(a_bits, dtype=np.uint16)
    b = np.ascontiguousarray(b_bits, dtype=np.uint16)
    M, K = a.shape
    K2, N = b.shape
    assert K == K2
    P = 0 if peers is None else peers.shape[0]
    pe = np.ascontiguousarray(peers if P else np.zeros((1, 1, 1), np.float32), dtype=np.float32)
    out = np.empty((M, N), dtype=np.float64)
    _brute().mk_brute_gemm_reduce(a.ctypes.data, b.ctypes.data, pe.ctypes.data, P,
                                  M, N, K, out.ctypes.data)
    return out


# ---------------------------------------------------------------------------
# Adaptive partition controller (section 2.4 of the analysis page)
# ---------------------------------------------------------------------------

U64 = (1 << 64) - 1
COST_CAP = (1 << 26) - 1     # per-task cycle means saturate here (keeps the u64 math exact)


def controller_target(B: int, R_s: int, C_s: int, R_p: int, C_p: int,
                      current: int, floor: int = 2, keep: int = 1,
                      cap: Optional[int] = None) -> int:
    """Target reduce-workgroup count n_s*.

    Readings of the page's undefined symbols (applied here and on the GPU):
      B   -- persistent workgroups sharing the two roles;
      s   -- the communication role (here: tile-reduce); p -- compute;
      R_x -- tasks of role x not yet finished; C_x -- mean cycles per task.
    n_s* = B R_s C_s / (R_p C_p + R_s C_s) is the n at which the two roles'
    predicted finish times R_s C_s / n and R_p C_p / (B - n) are equal.
    Rounding: nearest, ties up, in unsigned 64-bit integers.
    Clamp: while compute remains (R_p > 0) keep at least `keep` compute
    workgroups (n <= B - keep; one, or one per tile partition when every
    partition is worked only by its own XCD's workgroups -- otherwise a
    partition could be left without a producer) and at least `floor` reducers
    (2, the low end of the page's static sweep); with no compute left the
    formula itself gives B.  `cap` (None: none) is the most reducers while
    compute remains: the count at which the reduce role already saturates the
    memory system, past which more reducers only stretch every reduce task and
    take compute units from the tiles the reducers wait for.
    A zero denominator carries no information: the current target stays.
    """
    if B < 2:
        raise ValueError("need at least two workgroups")
    if R_p == 0:
        return B
    hi = _upper(B, keep, cap)
    lo = min(floor, hi)
    num = B * R_s * C_s
    den = R_p * C_p + R_s * C_s
    if den == 0:
        n = current
    else:
        if 2 * num + den > U64:
            raise OverflowError("controller operands exceed the unsigned 64-bit range")
        n = (2 * num + den) // (2 * den)
    return min(max(n, lo), hi)


def _upper(B: int, keep: int, cap: Optional[int]) -> int:
    """Upper clamp while compute remains: B - keep, and at most `cap`."""
    hi = B - keep
    if cap is not None:
        if cap < 1:
            raise ValueError("cap must be at least 1")
        hi = min(hi, cap)
    return hi


def cycle_mean(total_cycles: int, tasks: int) -> int:
    """Cumulative mean cost per task since launch (integer, saturating)."""
    return min(total_cycles // tasks, COST_CAP)


def controller_update(B: int, T: int, compute_done: int, reduce_done: int,
                      sum_cycles_compute: int, sum_cycles_reduce: int,
                      current: int, floor: int = 2, keep: int = 1,
                      cap: Optional[int] = None) -> int:
    """One controller step from the progress counters.

    R_p counts compute tasks not yet finished (claimed-but-running tasks count
    as remaining); R_s counts tiles not yet reduced, ready or not.  Until both
    roles have finished a task there is no cost estimate and the current
    target stays (clamped).
    """
    R_p = T - compute_done
    R_s = T - reduce_done
    if R_p == 0:
        return B
    if compute_done == 0 or reduce_done == 0:
        hi = _upper(B, keep, cap)
        return min(max(current, min(floor, hi)), hi)
    C_p = cycle_mean(sum_cycles_compute, compute_done)
    C_s = cycle_mean(sum_cycles_reduce, reduce_done)
    return controller_target(B, R_s, C_s, R_p, C_p, current, floor, keep, cap)


def controller_exact(B: int, R_s: int, C_s: int, R_p: int, C_p: int) -> Fraction:
    """Unrounded, unclamped n_s* as an exact rational."""
    return Fraction(B * R_s * C_s, R_p * C_p + R_s * C_s)


# ---------------------------------------------------------------------------
# Tiles, chunks and the integer protocol
# ---------------------------------------------------------------------------


def tile_grid(M: int, N: int, tile_m: int, tile_n: int) -> Tuple[int, int]:
    """Tile rows and tile columns; ragged edges make a partial last tile."""
    return -(-M // tile_m), -(-N // tile_n)


def chunk_sizes(T: int, tiles_per_chunk: int) -> np.ndarray:
    """Tiles in each chunk.  Chunk c holds tiles [c*tpc, (c+1)*tpc) in row-major
    tile order; only the last chunk may be short."""
    Ch = -(-T // tiles_per_chunk)
    sizes = np.full(Ch, tiles_per_chunk, dtype=np.int64)
    if Ch and T % tiles_per_chunk:
        sizes[-1] = T % tiles_per_chunk
    return sizes


def tiles_per_task(tile_m: int, tile_n: int) -> int:
    """Output tiles one compute task covers, from the tile shape alone.

    The pages make the tile the unit of compute, flags and reduce
    ("【学习】mKernel 分析" sections 2.2-2.3) and leave open how many tiles one
    workgroup computes at once.  The reading taken: two adjacent tiles of one
    tile row for the 128x128 and 256x128 tiles (two tiles share their A rows,
    halving the operand bytes per flop), one for 64x64 tiles.  The protocol
    checker builds its expectations from this value, never from what the
    device reports.
    """
    if (tile_m, tile_n) == (64, 64):
        return 1
    if (tile_m, tile_n) in ((128, 128), (256, 128)):
        return 2
    raise ValueError(f"no task size for {tile_m}x{tile_n} tiles")


def compute_task_of_tile(T: int, tiles_n: Optional[int], tiles_per_task: int) -> np.ndarray:
    """Index of the compute task that produces each tile.

    A compute task covers `tiles_per_task` adjacent tiles of one tile row
    (the last task of a row may hold fewer); tasks are numbered row by row.
    With one tile per task this is the tile index itself.
    """
    t = np.arange(T, dtype=np.int64)
    if tiles_per_task == 1:
        return t
    tn = int(tiles_n)
    per_row = -(-tn // tiles_per_task)
    return (t // tn) * per_row + (t % tn) // tiles_per_task


def deterministic_owners(T: int, B: int, n_reduce: int, tiles_n: Optional[int] = None,
                         tiles_per_task: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Owner maps of the deterministic static schedule.

    Workgroups [0, n_reduce) reduce and the rest compute (roles by workgroup
    index).  A compute task covers the tiles of one block (`tiles_per_task`
    adjacent tiles of a tile row); a reduce task is one tile, the unit the
    pages reduce.  Each workgroup takes its tasks round-robin in increasing
    task order, and every tile of a compute task has that task's owner.
    """
    task = compute_task_of_tile(T, tiles_n, tiles_per_task)
    return n_reduce + task % (B - n_reduce), np.arange(T, dtype=np.int64) % n_reduce


OWNER_WG_MASK = 0xFFFF
OWNER_NS_MASK = 0x7FFF        # bits 16..30: the reduce target the task was taken under
OWNER_HELP = 1 << 31          # compute task taken by a workgroup waiting on a reduce ticket


def expected_state(T: int, tiles_per_chunk: int, epoch: int, calls: int) -> Dict[str, np.ndarray]:
    """Integer state after `calls` complete launches of one shape since the
    counters were last cleared; `epoch` is the last launch's epoch."""
    sizes = chunk_sizes(T, tiles_per_chunk)
    return {
        "tile_flag": np.full(T, epoch, dtype=np.int64),
        "tile_reduce_cnt": np.full(T, calls, dtype=np.int64),
        "chunk_cnt": sizes * calls,
        "chunk_flag": np.full(sizes.shape[0], epoch, dtype=np.int64),
    }


def check_state(maps: Dict[str, np.ndarray], T: int, tiles_per_chunk: int, epoch: int,
                calls: int, B: int, mode: str, n_reduce: int, tiles_n: Optional[int] = None,
                tiles_per_task: int = 1) -> List[str]:
    """Compare the protocol state against its closed form.

    Returns a list of human-readable violations (empty when all holds).
    `mode` is "deterministic", "static" or "adaptive"; `tiles_n` (tiles per
    tile row) and `tiles_per_task` describe the compute tasks.
    """
    bad: List[str] = []
    exp = expected_state(T, tiles_per_chunk, epoch, calls)
    for key, want in exp.items():
        got = np.asarray(maps[key], dtype=np.int64)
        if got.shape != want.shape:
            bad.append(f"{key}: shape {got.shape} != {want.shape}")
            continue
        idx = np.nonzero(got != want)[0]
        if idx.size:
            i = int(idx[0])
            bad.append(f"{key}[{i}] = {int(got[i])}, expected {int(want[i])} "
                       f"({idx.size} mismatches)")
    co = np.asarray(maps["compute_owner"], dtype=np.int64)
    ro = np.asarray(maps["reduce_owner"], dtype=np.int64)
    co_wg, co_ns, co_help = co & OWNER_WG_MASK, (co >> 16) & OWNER_NS_MASK, (co & OWNER_HELP) != 0
    ro_wg, ro_ns, ro_help = ro & OWNER_WG_MASK, (ro >> 16) & OWNER_NS_MASK, (ro & OWNER_HELP) != 0
    if mode == "deterministic":
        dc, dr = deterministic_owners(T, B, n_reduce, tiles_n, tiles_per_task)
        if not np.array_equal(co_wg, dc):
            i = int(np.nonzero(co_wg != dc)[0][0])
            bad.append(f"compute_owner[{i}] = {int(co_wg[i])}, expected {int(dc[i])}")
        if not np.array_equal(ro_wg, dr):
            i = int(np.nonzero(ro_wg != dr)[0][0])
            bad.append(f"reduce_owner[{i}] = {int(ro_wg[i])}, expected {int(dr[i])}")
    if tiles_per_task > 1 and T:
        # reduce tasks are single tiles; a compute task's tiles share one owner
        task = compute_task_of_tile(T, tiles_n, tiles_per_task)
        first = np.zeros(int(task.max()) + 1, dtype=np.int64)
        first[task[::-1]] = co[::-1]
        if np.any(co != first[task]):
            i = int(np.nonzero(co != first[task])[0][0])
            bad.append(f"tile {i}: compute owner differs from the rest of its task")
    if np.any(co_wg >= B):
        bad.append("compute owner outside [0, B)")
    if np.any(ro_wg >= B):
        bad.append("reduce owner outside [0, B)")
    # role at the time of the task: compute iff index >= target, reduce iff
    # index < target; a compute task marked as help may come from either
    if np.any(ro_help):
        bad.append(f"tile {int(np.nonzero(ro_help)[0][0])}: reduce owner carries the help mark")
    if mode != "adaptive" and np.any(co_help):
        bad.append(f"tile {int(np.nonzero(co_help)[0][0])}: help task outside adaptive mode")
    if np.any((co_wg < co_ns) & ~co_help):
        i = int(np.nonzero((co_wg < co_ns) & ~co_help)[0][0])
        bad.append(f"tile {i} computed by workgroup {int(co_wg[i])} while the reduce "
                   f"target was {int(co_ns[i])}")
    if np.any(ro_wg >= ro_ns):
        i = int(np.nonzero(ro_wg >= ro_ns)[0][0])
        bad.append(f"tile {i} reduced by workgroup {int(ro_wg[i])} while the reduce "
                   f"target was {int(ro_ns[i])}")
    if mode in ("static", "deterministic"):
        if np.any(co_ns != n_reduce):
            bad.append("static partition changed during the launch (compute side)")
        if np.any(ro_ns != n_reduce):
            bad.append("static partition changed during the launch (reduce side)")
    return bad


# ---------------------------------------------------------------------------
# AllGather+GEMM, one rank's share
# ---------------------------------------------------------------------------
#
# AllGather + GEMM row of the MarkTechPost page's five-kernel table: every
# rank holds a shard of A; while the shards of the other ranks are gathered,
# the local GEMM consumes A's tiles as they arrive.  "【学习】mKernel 分析"
# section 2.6, Table 3: the dependency runs from communication to compute,
# the transfer unit is 128 rows, input shards are submitted at launch, and
# compute tiles are taken in order of input availability (local first);
# section 2.4: when communication feeds compute, a compute block waiting for
# its input helps communication.
#
# The readings used (the pages fix no layout):
# - R = P + 1 ranks, this rank is rank 0; every shard has Ms rows, and the
#   gathered A stacks the shards by rank: rank r's rows are
#   [r Ms, (r + 1) Ms).  The result is C = A_gathered . B over all R Ms rows
#   (a column-parallel layer whose input is sequence-sharded), and the
#   gathered A itself, which every rank holds after an AllGather.
# - A chunk is one tile row of A: tile_m rows (128 on the pages), K columns.
# - Copy order: the other ranks' chunks first, by rank and row (they gate
#   compute), then this rank's own (nothing waits for them: the local rows
#   are computed from the local shard directly).  Compute order: local tile
#   rows first, then the other ranks' rows in the order they are copied,
#   which is plain row order; blocks left to right inside a tile row.


def allgather_gemm(a_local_bits: np.ndarray, a_peers_bits: np.ndarray,
                   b_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Rank 0's share of AllGather+GEMM.

    a_local_bits [Ms, K] (uint16 bfloat16 patterns), a_peers_bits [P, Ms, K]
    (the other ranks' shards, rank 1 first), b_bits [K, N].  Returns
    (gathered, C): gathered [R Ms, K] uint16 is the shards stacked by rank,
    C [R Ms, N] float64 is gathered . B on the exact bfloat16 values."""
    a0 = np.asarray(a_local_bits, dtype=np.uint16)
    ap = np.asarray(a_peers_bits, dtype=np.uint16)
    b = np.asarray(b_bits, dtype=np.uint16)
    if a0.ndim != 2 or ap.ndim != 3 or b.ndim != 2:
        raise ValueError("A_local [Ms,K], A_peers [P,Ms,K], B [K,N]")
    if ap.shape[0] and ap.shape[1:] != a0.shape:
        raise ValueError("every shard must have the local shard's shape")
    if a0.shape[1] != b.shape[0]:
        raise ValueError("A's columns must match B's rows")
    gathered = np.concatenate([a0] + [ap[p] for p in range(ap.shape[0])], axis=0)
    return gathered, gemm_part(gathered, b)


def ag_copy_order(ranks: int, chunks_per_shard: int) -> np.ndarray:
    """Chunk ids (tile rows of the gathered A) in copy-claim order: the other
    ranks' chunks by rank and row, then this rank's own."""
    if ranks < 1 or chunks_per_shard < 0:
        raise ValueError("ranks >= 1, chunks_per_shard >= 0")
    peers = np.arange(chunks_per_shard, ranks * chunks_per_shard, dtype=np.int64)
    local = np.arange(0, chunks_per_shard, dtype=np.int64)
    return np.concatenate([peers, local])


def ag_parts_per_chunk(tile_m: int, K: int, tiles_n: int) -> int:
    """Copy tasks one chunk is split into.  The pages fix the chunk (the
    arrival unit, one tile row of A) but not how many movers share it; here
    one copy task moves at most 64 KiB of the chunk's tile_m x K bf16 bytes:
    ceil(2 tile_m K / 65536) parts, at least 1 and at most min(tiles_n, 64)."""
    parts = -(-(2 * tile_m * K) // 65536)
    return int(max(1, min(parts, tiles_n, 64)))


def ag_expected_state(n_chunks: int, n_tiles: int, epoch: int, calls: int,
                      parts: int = 1) -> Dict[str, np.ndarray]:
    """Integer state after `calls` complete launches of one shape: every
    chunk's arrival flag holds the last epoch, each of a chunk's `parts`
    copy tasks ran and every tile was computed exactly once per call."""
    return {
        "chunk_flag": np.full(n_chunks, epoch, dtype=np.int64),
        "chunk_copy_cnt": np.full(n_chunks, parts * calls, dtype=np.int64),
        "tile_compute_cnt": np.full(n_tiles, calls, dtype=np.int64),
    }


def ag_deterministic_owners(ranks: int, chunks_per_shard: int, tiles_n: int, B: int, n_copy: int,
                            tiles_per_task: int = 1, parts: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Owner maps of the deterministic static schedule: workgroups
    [0, n_copy) copy, the others compute.  Copy tasks are the chunks in copy
    order, each split into `parts` consecutive tasks; copy task i goes to
    workgroup i mod n_copy.  Compute task j (blocks of `tiles_per_task`
    adjacent tiles, row by row) goes to n_copy + j mod (B - n_copy).
    Returns (copy owner per copy task, indexed chunk id * parts + part;
    compute owner per tile)."""
    order = ag_copy_order(ranks, chunks_per_shard)
    n_tasks = order.shape[0] * parts
    i = np.arange(n_tasks, dtype=np.int64)
    copy_owner = np.zeros(n_tasks, dtype=np.int64)
    copy_owner[order[i // parts] * parts + i % parts] = i % n_copy
    T = ranks * chunks_per_shard * tiles_n
    task = compute_task_of_tile(T, tiles_n, tiles_per_task)
    return copy_owner, n_copy + task % (B - n_copy)


def ag_check_state(maps: Dict[str, np.ndarray], ranks: int, chunks_per_shard: int, tiles_n: int,
                   epoch: int, calls: int, B: int, mode: str, n_copy: int,
                   tiles_per_task: int = 1, parts: int = 1) -> List[str]:
    """Compare an AllGather+GEMM launch's protocol state with its closed form.

    Owner words are (mark << 31) | (copy target seen << 16) | workgroup.  A
    copy task by a workgroup at or above the copy target is legal only with
    the mark (a compute-role workgroup waiting for its input helped copy),
    and only in adaptive mode; a compute task needs an index at or above the
    target and never carries the mark."""
    bad: List[str] = []
    n_chunks = ranks * chunks_per_shard
    T = n_chunks * tiles_n
    for key, want in ag_expected_state(n_chunks, T, epoch, calls, parts).items():
        got = np.asarray(maps[key], dtype=np.int64)
        if got.shape != want.shape:
            bad.append(f"{key}: shape {got.shape} != {want.shape}")
            continue
        idx = np.nonzero(got != want)[0]
        if idx.size:
            i = int(idx[0])
            bad.append(f"{key}[{i}] = {int(got[i])}, expected {int(want[i])} ({idx.size} mismatches)")
    co = np.asarray(maps["copy_owner"], dtype=np.int64)
    po = np.asarray(maps["compute_owner"], dtype=np.int64)
    if co.shape != (n_chunks * parts,):
        return bad + [f"copy_owner: shape {co.shape} != ({n_chunks * parts},)"]
    co_wg, co_ns, co_help = co & OWNER_WG_MASK, (co >> 16) & OWNER_NS_MASK, (co & OWNER_HELP) != 0
    po_wg, po_ns, po_mark = po & OWNER_WG_MASK, (po >> 16) & OWNER_NS_MASK, (po & OWNER_HELP) != 0
    if np.any(co_wg >= B) or np.any(po_wg >= B):
        bad.append("owner outside [0, B)")
    if mode == "deterministic":
        dc, dp = ag_deterministic_owners(ranks, chunks_per_shard, tiles_n, B, n_copy, tiles_per_task, parts)
        if not np.array_equal(co_wg, dc):
            i = int(np.nonzero(co_wg != dc)[0][0])
            bad.append(f"copy_owner[{i}] = {int(co_wg[i])}, expected {int(dc[i])}")
        if not np.array_equal(po_wg, dp):
            i = int(np.nonzero(po_wg != dp)[0][0])
            bad.append(f"compute_owner[{i}] = {int(po_wg[i])}, expected {int(dp[i])}")
    if tiles_per_task > 1 and T:
        task = compute_task_of_tile(T, tiles_n, tiles_per_task)
        first = np.zeros(int(task.max()) + 1, dtype=np.int64)
        first[task[::-1]] = po[::-1]
        if np.any(po != first[task]):
            i = int(np.nonzero(po != first[task])[0][0])
            bad.append(f"tile {i}: compute owner differs from the rest of its task")
    if np.any(po_mark):
        bad.append(f"tile {int(np.nonzero(po_mark)[0][0])}: compute owner carries the help mark")
    if mode != "adaptive" and np.any(co_help):
        bad.append(f"copy task {int(np.nonzero(co_help)[0][0])}: help copy outside adaptive mode")
    if np.any((co_wg >= co_ns) & ~co_help):
        i = int(np.nonzero((co_wg >= co_ns) & ~co_help)[0][0])
        bad.append(f"copy task {i} run by workgroup {int(co_wg[i])} while the copy target was {int(co_ns[i])}")
    if np.any(po_wg < po_ns):
        i = int(np.nonzero(po_wg < po_ns)[0][0])
        bad.append(f"tile {i} computed by workgroup {int(po_wg[i])} while the copy target was {int(po_ns[i])}")
    if mode in ("static", "deterministic"):
        if np.any(co_ns != n_copy) or np.any(po_ns != n_copy):
            bad.append("static partition changed during the launch")
    return bad


# ---------------------------------------------------------------------------
# Ring Attention, one rank's share
# ---------------------------------------------------------------------------
#
# Ring Attention row of the MarkTechPost page's five-kernel table: attention
# over a sequence split across ranks; at each step every rank passes the KV
# chunk it holds to the next rank while its local FlashAttention consumes the
# chunk it received before, both inside one persistent kernel.
# "【学习】mKernel 分析" section 2.6, Table 3: sequence parallelism, the
# step's compute and transfer are independent, KV moves in 128-row tiles.
#
# The readings used (the pages fix neither masking nor layout):
# - R ranks hold S consecutive tokens each; this is rank 0.  Q, K and V are
#   [S, H, D] (token, head, head dimension), bfloat16.  The ring brings the
#   other ranks' K and V one step at a time; peers[s - 1] is the KV chunk
#   that arrives at step s (s = 1 .. R - 1).  Step 0 uses the local K, V.
# - Attention is not causal: every query attends to all R S keys, so the
#   result does not depend on the ring order.  Scale 1 / sqrt(D).
# - Outputs: O [S, H, D] and the log-sum-exp LSE [H, S] (natural log) of
#   each query's scaled scores, the quantity a ring step passes on to merge
#   partial results.
# - A KV tile is 128 tokens of one step's K and V, all heads; its arrival
#   flag gates every read of it.  A copy task moves at most 64 KiB of one
#   tile (K and V together); the task whose count completes the tile sets
#   its flag.  A compute task is 128 queries of one head over every key.


def _scores_scale(D: int) -> float:
    return 1.0 / np.sqrt(float(D))


def ring_attention(q_bits: np.ndarray, k_local_bits: np.ndarray, v_local_bits: np.ndarray,
                   k_peers_bits: np.ndarray, v_peers_bits: np.ndarray,
                   row_block: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """Rank 0's share of Ring Attention, in float64 on the exact bfloat16
    values.  q, k_local, v_local [S, H, D]; k_peers, v_peers [R-1, S, H, D]
    (arrival order).  Returns (O [S, H, D], LSE [H, S]):
        s_ij = (q_i . k_j) / sqrt(D) over all R S keys j,
        O_i = sum_j exp(s_ij) v_j / sum_j exp(s_ij),   LSE_i = log sum_j exp(s_ij)."""
    q = np.asarray(q_bits, dtype=np.uint16)
    kl = np.asarray(k_local_bits, dtype=np.uint16)
    vl = np.asarray(v_local_bits, dtype=np.uint16)
    kp = np.asarray(k_peers_bits, dtype=np.uint16)
    vp = np.asarray(v_peers_bits, dtype=np.uint16)
    if q.ndim != 3 or kl.shape != q.shape or vl.shape != q.shape:
        raise ValueError("q, k_local, v_local must all be [S, H, D]")
    if kp.ndim != 4 or kp.shape != vp.shape or kp.shape[1:] != q.shape:
        raise ValueError("k_peers, v_peers must be [R-1, S, H, D]")
    S, H, D = q.shape
    K = bf16_bits_to_f64(np.concatenate([kl[None], kp], axis=0).reshape(-1, H, D))
    V = bf16_bits_to_f64(np.concatenate([vl[None], vp], axis=0).reshape(-1, H, D))
    Q = bf16_bits_to_f64(q)
    O = np.zeros((S, H, D), dtype=np.float64)
    L = np.zeros((H, S), dtype=np.float64)
    sc = _scores_scale(D)
    for h in range(H):
        Kh, Vh = K[:, h, :], V[:, h, :]
        for i0 in range(0, S, row_block):
            s_ = (Q[i0:i0 + row_block, h, :] @ Kh.T) * sc
            m = s_.max(axis=1, keepdims=True)
            w = np.exp(s_ - m)
            l = w.sum(axis=1, keepdims=True)
            O[i0:i0 + row_block, h, :] = (w @ Vh) / l
            L[h, i0:i0 + row_block] = (m + np.log(l))[:, 0]
    return O, L


def ring_attention_at(q_bits, k_local_bits, v_local_bits, k_peers_bits, v_peers_bits,
                      rows: Sequence[int], heads: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """The same definition for the sampled queries (rows[n], heads[n]) only:
    returns (O [n, D], LSE [n]).  For full-size checks."""
    q = np.asarray(q_bits, dtype=np.uint16)
    S, H, D = q.shape
    kl, vl = np.asarray(k_local_bits), np.asarray(v_local_bits)
    kp, vp = np.asarray(k_peers_bits), np.asarray(v_peers_bits)
    rows = np.asarray(rows, dtype=np.int64)
    heads = np.asarray(heads, dtype=np.int64)
    O = np.zeros((rows.size, D), dtype=np.float64)
    L = np.zeros(rows.size, dtype=np.float64)
    sc = _scores_scale(D)
    for h in np.unique(heads):
        Kh = bf16_bits_to_f64(np.concatenate([kl[None, :, h, :], kp[:, :, h, :]], axis=0).reshape(-1, D))
        Vh = bf16_bits_to_f64(np.concatenate([vl[None, :, h, :], vp[:, :, h, :]], axis=0).reshape(-1, D))
        sel = np.nonzero(heads == h)[0]
        s_ = (bf16_bits_to_f64(q[rows[sel], h, :]) @ Kh.T) * sc
        m = s_.max(axis=1, keepdims=True)
        w = np.exp(s_ - m)
        l = w.sum(axis=1, keepdims=True)
        O[sel] = (w @ Vh) / l
        L[sel] = (m + np.log(l))[:, 0]
    return O, L


def ra_kv_tiles(S: int, kv_rows: int = 128) -> int:
    """KV tiles of one step: ceil(S / 128) (the last one ragged)."""
    return -(-S // kv_rows)


def ra_parts_per_tile(H: int, D: int, kv_rows: int = 128) -> int:
    """Copy tasks one KV tile is split into: ceil(2 (K and V) x 128 H D x 2
    bytes / 64 KiB), at least 1 and at most 64."""
    parts = -(-(2 * kv_rows * H * D * 2) // 65536)
    return int(max(1, min(parts, 64)))


def ra_expected_state(n_tiles: int, n_tasks: int, epoch: int, calls: int,
                      parts: int = 1) -> Dict[str, np.ndarray]:
    """Integer state after `calls` complete launches of one shape: every
    arriving KV tile's flag holds the last epoch, each of its `parts` copy
    tasks ran and every compute task ran exactly once per call."""
    return {
        "tile_flag": np.full(n_tiles, epoch, dtype=np.int64),
        "tile_copy_cnt": np.full(n_tiles, parts * calls, dtype=np.int64),
        "task_compute_cnt": np.full(n_tasks, calls, dtype=np.int64),
    }


def ra_deterministic_owners(n_tiles: int, n_tasks: int, B: int, n_copy: int,
                            parts: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Owner maps of the deterministic static schedule: copy task i (tiles in
    arrival order, step by step, the parts of each in order; index
    tile * parts + part) goes to workgroup i mod n_copy, compute task j
    (head-major: j = head * query blocks + block) to n_copy + j mod
    (B - n_copy)."""
    i = np.arange(n_tiles * parts, dtype=np.int64)
    j = np.arange(n_tasks, dtype=np.int64)
    return i % n_copy, n_copy + j % (B - n_copy)


def ra_check_state(maps: Dict[str, np.ndarray], n_tiles: int, n_tasks: int, epoch: int, calls: int,
                   B: int, mode: str, n_copy: int, parts: int = 1) -> List[str]:
    """Compare a Ring Attention launch's protocol state with its closed form.
    Owner words are (mark << 31) | (copy target seen << 16) | workgroup; a
    copy task run by a workgroup at or above the copy target is legal only
    with the mark (a compute workgroup waiting for a tile helped), only in
    adaptive mode; a compute task never carries the mark and needs an index
    at or above the target."""
    bad: List[str] = []
    for key, want in ra_expected_state(n_tiles, n_tasks, epoch, calls, parts).items():
        got = np.asarray(maps[key], dtype=np.int64)
        if got.shape != want.shape:
            bad.append(f"{key}: shape {got.shape} != {want.shape}")
            continue
        idx = np.nonzero(got != want)[0]
        if idx.size:
            i = int(idx[0])
            bad.append(f"{key}[{i}] = {int(got[i])}, expected {int(want[i])} ({idx.size} mismatches)")
    co = np.asarray(maps["copy_owner"], dtype=np.int64)
    po = np.asarray(maps["compute_owner"], dtype=np.int64)
    if co.shape != (n_tiles * parts,) or po.shape != (n_tasks,):
        return bad + [f"owner maps: shapes {co.shape}, {po.shape}"]
    co_wg, co_ns, co_help = co & OWNER_WG_MASK, (co >> 16) & OWNER_NS_MASK, (co & OWNER_HELP) != 0
    po_wg, po_ns, po_mark = po & OWNER_WG_MASK, (po >> 16) & OWNER_NS_MASK, (po & OWNER_HELP) != 0
    if np.any(co_wg >= B) or np.any(po_wg >= B):
        bad.append("owner outside [0, B)")
    if mode == "deterministic":
        dc, dp = ra_deterministic_owners(n_tiles, n_tasks, B, n_copy, parts)
        if not np.array_equal(co_wg, dc):
            i = int(np.nonzero(co_wg != dc)[0][0])
            bad.append(f"copy_owner[{i}] = {int(co_wg[i])}, expected {int(dc[i])}")
        if not np.array_equal(po_wg, dp):
            i = int(np.nonzero(po_wg != dp)[0][0])
            bad.append(f"compute_owner[{i}] = {int(po_wg[i])}, expected {int(dp[i])}")
    if np.any(po_mark):
        bad.append(f"task {int(np.nonzero(po_mark)[0][0])}: compute owner carries the help mark")
    if mode != "adaptive" and np.any(co_help):
        bad.append(f"copy task {int(np.nonzero(co_help)[0][0])}: help copy outside adaptive mode")
    if np.any((co_wg >= co_ns) & ~co_help):
        i = int(np.nonzero((co_wg >= co_ns) & ~co_help)[0][0])
        bad.append(f"copy task {i} run by workgroup {int(co_wg[i])} while the copy target was {int(co_ns[i])}")
    if np.any(po_wg < po_ns):
        i = int(np.nonzero(po_wg < po_ns)[0][0])
        bad.append(f"task {i} computed by workgroup {int(po_wg[i])} while the copy target was {int(po_ns[i])}")
    if mode in ("static", "deterministic"):
        if np.any(co_ns != n_copy) or np.any(po_ns != n_copy):
            bad.append("static partition changed during the launch")
    return bad
