"""Seeded synthetic inputs for the fused GEMM + tile-reduce path.

This module is the only code shared by the HIP path's callers (tests, bench)
and the CPU oracle.  It holds no arithmetic of the method itself: it only
draws the operands, rounds A and B to bfloat16 (the input dtype), and
describes the workload shapes.

Workload shapes follow the problem statement of the GEMM+AllReduce fused
kernel ("mKernel: Fast Multi-GPU, Multi-Node Fused Kernels", abstract; the
five-kernel tables on the MarkTechPost and chathome pages): one rank's share
of a row-parallel projection computes a partial C_r = A_r . B_r over its
K-slice, and the partials of the R ranks are summed.  On one GPU the R-1 other
ranks' partials are synthetic fp32 buffers resident in HBM ("peers").

Recipe (fixed, documented):
  * generator: numpy PCG64 seeded by SeedSequence(entropy=seed,
    spawn_key=(workload_id, buffer_id)); buffer_id 0 = A, 1 = B, 2+p = peer p.
  * U(a, b)   = a + (b - a) * Generator.random(dtype=float32)
    N(0, s^2) = s * Generator.standard_normal(dtype=float32)
  * A and B are rounded to bfloat16 with round-to-nearest-even on the
    float32 bit pattern and returned as uint16 bit patterns.
  * peers stay float32, shape [P, M, N], contiguous.
  * the skewed-cost workload zeroes the first floor(frac * M) rows of A
    (after rounding; +0.0 in bfloat16 is the bit pattern 0).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "custom",
    "make_inputs",
    "round_to_bf16_bits",
    "DEFAULT_SEED",
]

DEFAULT_SEED = 0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, distributions, tiling and partition mode."""

    name: str
    wid: int                      # workload id, first element of the spawn key
    M: int
    N: int
    K: int
    peers: int                    # P = R - 1 peer-partial buffers
    dist_ab: Tuple                # ("uniform", a, b) or ("normal", sigma)
    dist_peer: Tuple
    tile_m: int
    tile_n: int
    tiles_per_chunk: int = 4
    mode: str = "adaptive"        # "adaptive" | "static" | "deterministic"
    n_reduce: int = 2             # static count, or initial count for adaptive
    zero_rows_frac: float = 0.0   # leading fraction of A rows set to zero
    description: str = ""

    @property
    def tiles(self) -> int:
        return -(-self.M // self.tile_m) * -(-self.N // self.tile_n)

    @property
    def chunks(self) -> int:
        return -(-self.tiles // self.tiles_per_chunk)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """A + B read once, peers read once, C written once."""
        return (2 * self.M * self.K + 2 * self.K * self.N
                + 4 * self.peers * self.M * self.N + 4 * self.M * self.N)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 0, 256, 256, 512, 1, ("uniform", -1.0, 1.0), ("normal", 1.0),
                 64, 64, 4, "static", 2,
                 description="256x256x512, 1 peer, 64x64 tiles, fixed 2 reduce workgroups"),
        Workload("tp_share", 1, 4096, 4096, 1792, 7, ("normal", 0.02), ("normal", 0.5),
                 128, 128, 4, "adaptive", 2,
                 description="row-parallel projection share: 4096 tokens x 4096, K_local 1792, 7 peers"),
        Workload("reduce_heavy", 2, 8192, 8192, 1024, 7, ("uniform", -0.5, 0.5), ("normal", 1.0),
                 128, 128, 4, "adaptive", 2,
                 description="8192x8192x1024, 7 peers: reduce traffic dominates"),
        Workload("compute_heavy", 3, 16384, 8192, 8192, 7, ("normal", 0.01), ("normal", 0.1),
                 256, 128, 4, "adaptive", 2,
                 description="16384x8192x8192, 7 peers, 256x128 tiles: MFMA work dominates"),
        Workload("wide_many_peer", 4, 2048, 12288, 4096, 15, ("uniform", -1.0, 1.0), ("normal", 1.0),
                 128, 128, 4, "adaptive", 2, zero_rows_frac=0.10,
                 description="2048x12288x4096, 15 peers, first 10% of A rows zero (skewed tile cost)"),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def custom(M, N, K, peers, tile_m=64, tile_n=64, tiles_per_chunk=4, wid=100,
           dist_ab=("uniform", -1.0, 1.0), dist_peer=("normal", 1.0), mode="static",
           n_reduce=2, zero_rows_frac=0.0, name=None) -> Workload:
    """A workload of arbitrary shape (tests: ragged tails, degenerate cases)."""
    return Workload(name or f"custom_{M}x{N}x{K}_p{peers}", wid, M, N, K, peers, dist_ab,
                    dist_peer, tile_m, tile_n, tiles_per_chunk, mode, n_reduce, zero_rows_frac)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Only finite inputs are produced by this module, so the add cannot carry
    out of 32 bits.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _rng(seed: int, wid: int, buf: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(wid, buf))
    return np.random.Generator(np.random.PCG64(ss))


def _draw(rng: np.random.Generator, shape, dist) -> np.ndarray:
    kind = dist[0]
    if kind == "uniform":
        a, b = float(dist[1]), float(dist[2])
        out = rng.random(shape, dtype=np.float32)
        out *= np.float32(b - a)
        out += np.float32(a)
        return out
    if kind == "normal":
        out = rng.standard_normal(shape, dtype=np.float32)
        out *= np.float32(dist[1])
        return out
    if kind == "zeros":
        return np.zeros(shape, dtype=np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def make_inputs(w: Workload, seed: int = DEFAULT_SEED, threads: Optional[int] = None):
    """Draw (A_bits [M,K] uint16, B_bits [K,N] uint16, peers [P,M,N] float32).

    Deterministic in (seed, w.wid, shapes, distributions); independent of
    `threads`, because every buffer has its own generator stream.
    """
    M, N, K, P = w.M, w.N, w.K, w.peers
    a = round_to_bf16_bits(_draw(_rng(seed, w.wid, 0), (M, K), w.dist_ab))
    nz = int(np.floor(w.zero_rows_frac * M))
    if nz:
        a[:nz, :] = 0
    b = round_to_bf16_bits(_draw(_rng(seed, w.wid, 1), (K, N), w.dist_ab))
    peers = np.empty((P, M, N), dtype=np.float32)

    def fill(p):
        peers[p] = _draw(_rng(seed, w.wid, 2 + p), (M, N), w.dist_peer)

    if P:
        nthreads = threads or min(P, max(1, min(16, os.cpu_count() or 1)))
        if nthreads > 1 and M * N >= (1 << 20):
            with _cf.ThreadPoolExecutor(nthreads) as ex:
                list(ex.map(fill, range(P)))
        else:
            for p in range(P):
                fill(p)
    return a, b, peers


def make_remote(w: Workload, seed: int = DEFAULT_SEED) -> np.ndarray:
    """Draw the initial contents [M,N] float32 of the buffer that stands in
    for the other ranks' outputs in GEMM+ReduceScatter (the peers'
    distribution, a stream of its own after every peer's)."""
    return _draw(_rng(seed, w.wid, 2 + w.peers), (w.M, w.N), w.dist_peer)


# ---------------------------------------------------------------------------
# AllGather+GEMM, one rank's share
# ---------------------------------------------------------------------------
# Each of R = peers + 1 ranks holds a shard of Ms = M rows of A ([Ms, K]); this
# rank's own shard is buffer 0, B [K, N] is buffer 1, the other ranks' shards
# are buffers 2 + p (all from dist_ab, rounded to bfloat16).  The pages give
# no shapes for this kernel; the workloads below take the GEMM+AllReduce
# workloads' token and hidden sizes as a sequence-sharded input gathered for a
# column-parallel layer (M tokens in total, R Ms = M).

AG_WORKLOADS = {
    w.name: w
    for w in [
        Workload("ag_tiny", 10, 64, 256, 256, 3, ("uniform", -1.0, 1.0), ("zeros",),
                 64, 64, 1, "static", 2,
                 description="4 ranks x 64 rows, K 256, N 256, 64x64 tiles (64-row chunks)"),
        Workload("ag_tp_share", 11, 512, 1792, 4096, 7, ("normal", 0.02), ("zeros",),
                 128, 128, 1, "adaptive", 0,
                 description="8 ranks x 512 tokens (4096), hidden 4096, N_local 1792, 128-row chunks"),
        Workload("ag_compute_heavy", 12, 2048, 8192, 8192, 7, ("normal", 0.01), ("zeros",),
                 256, 128, 1, "adaptive", 0,
                 description="8 ranks x 2048 tokens (16384), K 8192, N 8192, 256-row chunks"),
    ]
}


def ag_workload(name: str) -> Workload:
    return AG_WORKLOADS[name]


def make_ag_inputs(w: Workload, seed: int = DEFAULT_SEED):
    """Draw (A_local [Ms,K] uint16, A_peers [P,Ms,K] uint16, B [K,N] uint16)
    for one rank's share of AllGather+GEMM (w.M is the shard's rows)."""
    Ms, N, K, P = w.M, w.N, w.K, w.peers
    a_local = round_to_bf16_bits(_draw(_rng(seed, w.wid, 0), (Ms, K), w.dist_ab))
    b = round_to_bf16_bits(_draw(_rng(seed, w.wid, 1), (K, N), w.dist_ab))
    a_peers = np.empty((P, Ms, K), dtype=np.uint16)
    for p in range(P):
        a_peers[p] = round_to_bf16_bits(_draw(_rng(seed, w.wid, 2 + p), (Ms, K), w.dist_ab))
    return a_local, a_peers, b


# ---------------------------------------------------------------------------
# Ring Attention, one rank's share
# ---------------------------------------------------------------------------
# R ranks hold S consecutive tokens each; this rank's Q, K and V [S, H, D]
# are buffers 0, 1 and 2, the K and V that arrive at ring step s (s = 1 ..
# R - 1) are buffers 1 + 2s and 2 + 2s.  All from `dist`, rounded to
# bfloat16.  The pages give no shapes for this kernel; the workloads take a
# 4096-token share of a 32-head, 128-dimension attention layer (a 32k-token
# sequence over 8 ranks) and a long-context share (64k tokens over 4 ranks,
# 8 heads); with N(0, 1) inputs the scaled scores are N(0, 1).


@dataclasses.dataclass(frozen=True)
class RaWorkload:
    name: str
    wid: int
    ranks: int            # R: this rank plus the R - 1 whose KV arrives around the ring
    S: int                # tokens per rank
    H: int                # heads
    D: int                # head dimension
    dist: Tuple = ("normal", 1.0)
    mode: str = "adaptive"
    n_copy: int = 0
    description: str = ""

    @property
    def flops(self) -> int:
        """Q.K^T and P.V over every (query, key, head): 4 S (R S) D H."""
        return 4 * self.S * self.ranks * self.S * self.D * self.H

    @property
    def tasks(self) -> int:
        return self.H * -(-self.S // 128)

    @property
    def kv_tiles(self) -> int:
        """KV tiles that arrive (steps 1 .. R - 1)."""
        return (self.ranks - 1) * -(-self.S // 128)


RA_WORKLOADS = {
    w.name: w
    for w in [
        RaWorkload("ra_tiny", 20, 2, 256, 2, 128, mode="static", n_copy=2,
                   description="2 ranks x 256 tokens, 2 heads of 128"),
        RaWorkload("ra_sp_share", 21, 8, 4096, 32, 128,
                   description="8 ranks x 4096 tokens (32k), 32 heads of 128"),
        RaWorkload("ra_long", 22, 4, 16384, 8, 128,
                   description="4 ranks x 16384 tokens (64k), 8 heads of 128"),
    ]
}


def ra_workload(name: str) -> RaWorkload:
    return RA_WORKLOADS[name]


def ra_custom(ranks, S, H, D=128, wid=200, mode="static", n_copy=2) -> RaWorkload:
    return RaWorkload(f"ra_custom_{ranks}x{S}x{H}x{D}", wid, ranks, S, H, D, mode=mode, n_copy=n_copy)


def make_ra_inputs(w: RaWorkload, seed: int = DEFAULT_SEED):
    """Draw (q, k_local, v_local [S,H,D], k_peers, v_peers [R-1,S,H,D]), all
    uint16 bfloat16 patterns; peers in ring arrival order."""
    shape = (w.S, w.H, w.D)
    q = round_to_bf16_bits(_draw(_rng(seed, w.wid, 0), shape, w.dist))
    kl = round_to_bf16_bits(_draw(_rng(seed, w.wid, 1), shape, w.dist))
    vl = round_to_bf16_bits(_draw(_rng(seed, w.wid, 2), shape, w.dist))
    P = w.ranks - 1
    kp = np.empty((P,) + shape, dtype=np.uint16)
    vp = np.empty((P,) + shape, dtype=np.uint16)

    def fill(s):
        kp[s - 1] = round_to_bf16_bits(_draw(_rng(seed, w.wid, 1 + 2 * s), shape, w.dist))
        vp[s - 1] = round_to_bf16_bits(_draw(_rng(seed, w.wid, 2 + 2 * s), shape, w.dist))

    if P:
        with _cf.ThreadPoolExecutor(min(P, 8)) as ex:
            list(ex.map(fill, range(1, P + 1)))
    return q, kl, vl, kp, vp
