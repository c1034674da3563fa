// Kernels of the fused GEMM + tile-reduce library for MI355X (gfx950).
//
// One persistent kernel per call ("mKernel: Fast Multi-GPU, Multi-Node Fused
// Kernels", abstract): each workgroup owns one compute unit and, at every task
// boundary, takes the compute role (one output tile of the local partial
// C_r = A.B on MFMA) or the reduce role (one finished tile: C = C_r + sum of
// the peer partials).  A compute tile publishes a readiness flag after its
// payload ("【学习】mKernel 分析" section 2.2, Figure 2; section 2.5: the
// signal must name a completed payload).  Reduced tiles count into per-chunk
// counters and the last tile of a chunk releases it (section 2.3).  The
// reduce-role size follows the on-GPU controller of section 2.4.
//
// Design for CDNA4 rather than the pages' Hopper kernels:
//  - one 256-thread workgroup per CU (LDS use > 80 KiB forces it), so "reduce
//    CUs" and "reduce workgroups" are the same number;
//  - GEMM on v_mfma_f32_32x32x16_bf16 with A and B slabs staged through LDS,
//    double buffered, XOR-swizzled rows so MFMA operand reads are free of
//    bank conflicts; B is transposed in registers on its way into LDS;
//  - the MFMA is fed (B, A) so each lane ends with four consecutive columns
//    of one row: the tile leaves as 16-byte stores;
//  - the reduce role streams the partial and every peer with 16-byte buffer
//    loads, (P+1)*U of them in flight per lane, peers and the result
//    non-temporal;
//  - claims and flags are device-scope atomics; the tile hand-off between
//    XCDs uses device-coherent stores and loads of the tile data itself plus
//    a drain of outstanding stores before the flag, instead of whole-L2
//    release/acquire fences (see "buffer access" in mk_device.hpp).
#include "mk_device.hpp"

namespace mk {

// ---------------------------------------------------------------------------
// the persistent fused kernel
// ---------------------------------------------------------------------------

enum Role : int { kRoleCompute = 0, kRoleReduce = 1, kRoleExit = 2, kRoleNone = -1 };

struct Decision {
    int role;
    uint32_t tile;      // compute: block index; reduce: tile index
    uint32_t ns_seen;   // reduce target the claim was made under (logged in owner maps),
                        // | kHelp for a compute task taken while a reduce ticket waits
};

// Compute tasks are blocks of tpb adjacent tiles of one tile row (a ragged
// last block holds fewer): a wider block needs fewer operand bytes per flop.
// A reduce task is one tile, the unit the pages reduce; the shorter task
// lets every workgroup share the last of the reduce work.
constexpr int kMaxTpb = 2;   // largest tiles-per-block of any tile configuration
constexpr uint32_t kNoTile = 0xFFFFFFFFu;

struct Blocks {
    uint32_t tpb;       // tiles per block
    uint32_t bn;        // blocks per tile row
    uint32_t TB;        // blocks
    uint32_t tiles_n;
    __device__ __forceinline__ uint32_t first_tile(uint32_t b) const {
        return (b / bn) * tiles_n + (b % bn) * tpb;
    }
    __device__ __forceinline__ uint32_t count(uint32_t b) const {
        const uint32_t c0 = (b % bn) * tpb;
        return tiles_n - c0 < tpb ? tiles_n - c0 : tpb;
    }
};

__device__ __forceinline__ Blocks make_blocks(uint32_t tpb, uint32_t tiles_m, uint32_t tiles_n) {
    Blocks k;
    k.tpb = tpb;
    k.bn = (tiles_n + tpb - 1) / tpb;
    k.TB = tiles_m * k.bn;
    k.tiles_n = tiles_n;
    return k;
}

// Reduce tickets follow the blocks' claim order tile by tile: ticket q is tile
// q mod tpb of the (q / tpb)-th block (of the workgroup's partition when tiles
// stay on their XCD, else of the global order).  A ticket past a ragged
// block's last tile is empty (kNoTile).
__device__ __forceinline__ uint32_t ticket_count(bool local, const Parts &pt, const Blocks &bk,
                                                 uint32_t home) {
    return (local ? pt.size(home) : bk.TB) * bk.tpb;
}
__device__ __forceinline__ uint32_t ticket_tile(bool local, const Parts &pt, const Blocks &bk,
                                                uint32_t home, uint32_t q) {
    const uint32_t qb = q / bk.tpb, j = q % bk.tpb;
    const uint32_t b = local ? pt.tile(home, qb) : pt.ticket(qb);
    return j < bk.count(b) ? bk.first_tile(b) + j : kNoTile;
}

// chunk size in blocks for the claim order (1 when blocks do not divide chunks)
__device__ __forceinline__ uint32_t chunk_blocks(uint32_t tpc, uint32_t tpb) {
    return (tpc % tpb) == 0 ? tpc / tpb : 1u;
}


// Scheduling state kept by thread 0 of each workgroup.
struct Sched {
    uint64_t wait_start;      // start of the current wait (timeout reference)
    uint32_t det_i;           // deterministic mode: position in this workgroup's list
    uint32_t target;          // last reduce target read
    int last_role;
    bool compute_exhausted;   // every partition's compute claims came back exhausted
    uint32_t parts_done;      // bit x: partition x has no compute tiles left
    bool reduce_exhausted;    // a reduce ticket came back >= T
    int pending_role;         // a claim already taken for the next task, or kRoleNone
    uint32_t pending_q;
    uint32_t pending_ns;
    uint64_t decide_t0, decide_t1;   // constant-clock span of the last next_task call
    // taken at the end of the previous task, while its stores drained:
    bool early_claim;          // a compute claim on partition early_x returned early_i
    uint32_t early_x, early_i, early_ns;
    bool early_flag;           // the readiness flag of the pending ticket's tile
    uint32_t early_flag_value; // its value
    uint32_t trace_n;          // workgroup 0: target changes it has recorded
};

// Exactly-once and chunk counters of a reduced tile (a reduce task is one
// tile).  Thread 0 issues them as soon as the task's stores have drained at
// device scope (a released chunk must be complete), and reads what they
// return once its next task is under way: inside the next reduce task right
// after that task's first loads are issued, before the next compute task, or
// before any wait for a tile's flag.  The release therefore follows the
// chunk's last tile by one atomic round trip, which overlaps other work.
struct CntRead {
    uint32_t c;        // chunk of the tile; kNoChunk: nothing pending
    uint32_t want;     // the chunk's count once this call has reduced all its tiles
    uint32_t old_t, old_c;
};
constexpr uint32_t kNoChunk = 0xFFFFFFFFu;

__device__ __forceinline__ CntRead cnt_issue(const FusedArgs &a, uint32_t t) {
    CntRead k;
    k.c = t / a.tpc;
    const uint32_t first = k.c * a.tpc;
    const uint32_t size = (a.T - first) < a.tpc ? (a.T - first) : a.tpc;
    k.want = size * a.calls;
    k.old_t = add_relaxed(&a.ws.tile_cnt[t], 1u);
    k.old_c = add_relaxed(&a.ws.chunk_cnt[k.c], 1u);
    return k;
}

// Thread 0: exactly-once check, and release of a chunk whose last tile this
// was ("【学习】mKernel 分析" section 2.3: the last locally reduced tile of a
// chunk lets it go, without waiting for the rest of the GEMM).  Clears k.
__device__ __forceinline__ void cnt_finish(const FusedArgs &a, Live *L, CntRead &k) {
    if (k.c == kNoChunk) return;
    const uint32_t c = k.c, want = k.want;
    k.c = kNoChunk;
    if (k.old_t != a.calls - 1) note_violation(L);
    if (k.old_c + 1 == want) {
        // where a network send of the chunk would be posted: every tile of it
        // was stored write-through and drained before its count was taken
        a.ws.chunk_release[c] = (uint32_t)ticks_now();
        st_relaxed(&a.ws.chunk_flag[c], a.epoch);
        add_relaxed(&L->chunks_released.v, 1u);
    } else if (k.old_c + 1 > want) {
        note_violation(L);
    }
}

__device__ __forceinline__ bool timed_out(const FusedArgs &a, Live *L, uint64_t since) {
    if (ticks_now() - since <= a.timeout_ticks) return false;
    __hip_atomic_fetch_max(&L->error, (uint32_t)kErrTimeout, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(&L->sticky, kStickyTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// Wait (bounded) until tile t carries this launch's epoch.  False on timeout or
// on an error raised by another workgroup.  Counters still in flight are read
// (and a chunk released) before the first poll, so no release waits on it.
__device__ __forceinline__ bool wait_ready(const FusedArgs &a, Live *L, uint32_t t, CntRead &pend) {
    if (ld_relaxed(&a.ws.tile_flag[t]) == a.epoch) return true;
    cnt_finish(a, L, pend);
    const uint64_t since = ticks_now();
    for (;;) {
        if (ld_relaxed(&a.ws.tile_flag[t]) == a.epoch) return true;
        if (ld_relaxed(&L->error) != kErrNone) return false;
        if (timed_out(a, L, since)) return false;
        __builtin_amdgcn_s_sleep(1);
    }
}


// Thread 0: claim a compute block, from the workgroup's own partition first,
// then (unless tiles stay on their XCD) the others.  False once every
// partition it may claim from is exhausted.
__device__ __forceinline__ bool claim_compute(const FusedArgs &a, const Parts &pt, Live *L,
                                              uint32_t wg, Sched &s, uint32_t &block) {
    if (s.compute_exhausted) return false;
    const uint32_t home = wg % pt.nx;
    const uint32_t parts = a.local ? 1u : pt.nx;
    for (uint32_t k = 0; k < parts; ++k) {
        const uint32_t x = home + k < pt.nx ? home + k : home + k - pt.nx;
        if (s.parts_done & (1u << x)) continue;
        const uint32_t i = add_relaxed(&L->compute_claim[x].v, 1u);
        if (i < pt.size(x)) {
            block = pt.tile(x, i);
            return true;
        }
        s.parts_done |= 1u << x;
    }
    s.compute_exhausted = true;
    return false;
}

// Tile t carries this launch's epoch (one read, no wait).
__device__ __forceinline__ bool tile_ready(const FusedArgs &a, uint32_t t) {
    return ld_relaxed(&a.ws.tile_flag[t]) == a.epoch;
}

// Thread 0 only: the next task.  Roles follow the workgroup index against the
// current target and are re-read here, at every task boundary ("【学习】mKernel
// 分析" sections 2.4 and 4.1).  Claims are tickets from device-scope counters
// in one common order, so compute and reduce walk the tiles in step.  A claim
// taken ahead of time (prefetched during the previous task) is a commitment
// and is honoured first, so a role change takes effect one task later.
// Under the adaptive controller a workgroup whose reduce ticket is not ready
// yet computes a block meanwhile and keeps the ticket: a block waiting for its
// input helps the other role ("【学习】mKernel 分析" section 2.4, read in the
// direction data flows here, from compute to reduce).
__device__ __forceinline__ Decision next_task(const FusedArgs &a, const Parts &pt, const Blocks &bk, Live *L, uint32_t wg,
                             Sched &s, CntRead &pend) {
    const uint32_t B = (uint32_t)a.nwg;
    if (a.mode == kDeterministic) {
        const uint32_t ns = (uint32_t)a.ns_init;
        if (wg < ns) {
            const uint32_t t = wg + s.det_i * ns;
            if (t >= a.T) return {kRoleExit, 0, ns};
            if (!wait_ready(a, L, t, pend)) return {kRoleExit, 0, ns};
            ++s.det_i;
            return {kRoleReduce, t, ns};
        }
        const uint32_t b = (wg - ns) + s.det_i * (B - ns);
        if (b >= bk.TB) return {kRoleExit, 0, ns};
        ++s.det_i;
        return {kRoleCompute, b, ns};
    }
    if (s.early_claim) {
        // a compute claim taken while the previous task's stores drained
        s.early_claim = false;
        if (s.early_i < pt.size(s.early_x)) return {kRoleCompute, pt.tile(s.early_x, s.early_i), s.early_ns};
        s.parts_done |= 1u << s.early_x;
    }
    for (;;) {
        if (s.pending_role != kRoleNone) {
            // a reduce ticket taken ahead of time
            const uint32_t q = s.pending_q, ns_seen = s.pending_ns;
            s.pending_role = kRoleNone;
            const bool seen = s.early_flag && s.early_flag_value == a.epoch;
            s.early_flag = false;
            const uint32_t home = wg % pt.nx;
            if (q < ticket_count(a.local, pt, bk, home)) {
                const uint32_t t = ticket_tile(a.local, pt, bk, home, q);
                if (t == kNoTile) continue;     // empty ticket: take another
                if (!seen) {
                    uint32_t cb;
                    if (a.mode == kAdaptive && a.help && !s.compute_exhausted && !tile_ready(a, t) &&
                        claim_compute(a, pt, L, wg, s, cb)) {
                        s.pending_role = kRoleReduce;
                        s.pending_q = q;
                        s.pending_ns = ns_seen;
                        return {kRoleCompute, cb, s.target | kHelp};
                    }
                    if (!wait_ready(a, L, t, pend)) return {kRoleExit, 0, ns_seen};
                }
                return {kRoleReduce, t, ns_seen};
            }
            s.reduce_exhausted = true;
            continue;
        }
        const uint32_t ns = s.target;
        const bool compute_role = wg >= ns;
        if (compute_role && !s.compute_exhausted) {
            uint32_t cb;
            if (claim_compute(a, pt, L, wg, s, cb)) return {kRoleCompute, cb, ns};
            continue;
        }
        // static partition: compute workgroups leave once compute is all claimed
        if (compute_role && a.mode == kStatic) return {kRoleExit, 0, ns};
        if (s.reduce_exhausted) return {kRoleExit, 0, ns};
        // adaptive: a compute-role workgroup with no compute left reduces, as
        // every workgroup does once the controller's target reaches B
        s.pending_role = kRoleReduce;
        s.pending_q = add_relaxed(&L->reduce_claim[a.local ? wg % pt.nx : 0u].v, 1u);
        s.pending_ns = compute_role ? B : ns;
    }
}

// Thread 0, right after choosing reduce task d: take the ticket for the task
// after it now, so its round trip overlaps this task (the result is read at
// the next boundary), while the target still gives this workgroup the reduce
// role.
__device__ __forceinline__ void prefetch_claim(const FusedArgs &a, const Parts &pt, Live *L,
                                               uint32_t wg, Sched &s, const Decision &d) {
    if (a.mode == kDeterministic || s.pending_role != kRoleNone) return;
    const uint32_t ns = s.target;
    const bool compute_role = wg >= ns;
    // Compute claims are not taken ahead: a compute task is long against the
    // claim's round trip, and an early claim would delay a switch to the
    // reduce role by a whole task.
    if (d.role == kRoleReduce && !s.reduce_exhausted &&
               (!compute_role || (a.mode == kAdaptive && s.compute_exhausted))) {
        s.pending_role = kRoleReduce;
        s.pending_q = add_relaxed(&L->reduce_claim[a.local ? wg % pt.nx : 0u].v, 1u);
        s.pending_ns = compute_role ? (uint32_t)a.nwg : ns;
    }
}

// Round trips started as a task's work completes and read back after its
// stores are issued (kept in registers meanwhile, not in the LDS-resident
// scheduling state, so issuing them does not wait for their return).
struct Early {
    int kind;           // 0: none, 1: compute claim on partition x, 2: readiness flag
    uint32_t x, ns;
    uint32_t v0;
};

// Thread 0: start the round trips the next boundary needs.  A compute
// workgroup still in the compute role (under the target of its previous
// controller step) claims its next block; a workgroup holding a reduce
// ticket reads that tile's readiness flag.
__device__ __forceinline__ Early early_issue(const FusedArgs &a, const Parts &pt, const Blocks &bk,
                                             Live *L, uint32_t wg, const Sched &s) {
    Early e;
    e.kind = 0;
    e.x = e.ns = e.v0 = 0;
    if (a.mode == kDeterministic) return e;
    const uint32_t home = wg % pt.nx;
    if (s.pending_role == kRoleReduce) {
        if (s.pending_q < ticket_count(a.local, pt, bk, home)) {
            const uint32_t t = ticket_tile(a.local, pt, bk, home, s.pending_q);
            if (t != kNoTile) {
                e.kind = 2;
                e.v0 = ld_relaxed(&a.ws.tile_flag[t]);
            }
        }
        return e;
    }
    const uint32_t ns = s.target;
    if (wg >= ns && !s.compute_exhausted) {
        const uint32_t parts = a.local ? 1u : pt.nx;
        for (uint32_t k = 0; k < parts; ++k) {
            const uint32_t x = home + k < pt.nx ? home + k : home + k - pt.nx;
            if (s.parts_done & (1u << x)) continue;
            e.kind = 1;
            e.x = x;
            e.ns = ns;
            e.v0 = add_relaxed(&L->compute_claim[x].v, 1u);
            return e;
        }
    }
    return e;
}

// Thread 0: record what early_issue brought back.
__device__ __forceinline__ void early_finish(Sched &s, const Early &e) {
    if (e.kind == 1) {
        s.early_claim = true;
        s.early_x = e.x;
        s.early_ns = e.ns;
        s.early_i = e.v0;
    } else if (e.kind == 2) {
        s.early_flag = true;
        s.early_flag_value = e.v0;
    }
}

// Thread 0, after a task: one controller step from the two role words
// (adaptive mode only); returns the target to use next.  Workgroup 0 records
// the changes its own steps make in the trace, a sample of the target's path
// that costs no shared counter.
__device__ uint32_t controller_step(const FusedArgs &a, Live *L, uint32_t wg, Sched &s,
                                    uint64_t compute_word, uint64_t reduce_word,
                                    uint32_t raw_target) {
    const uint32_t cur = raw_target ? raw_target : (uint32_t)a.ns_init;
    const uint32_t n = controller_update(
        (uint32_t)a.nwg, a.T, (uint32_t)(compute_word & kCountMask),
        (uint32_t)(reduce_word & kCountMask), compute_word >> kCountBits,
        reduce_word >> kCountBits, cur, (uint32_t)a.ns_floor, (uint32_t)a.keep, (uint32_t)a.ns_cap);
    if (n != cur || raw_target == 0) {
        st_relaxed(&L->target_ns.v, n);
        min_relaxed(&L->ns_min, n);
        max_relaxed(&L->ns_max, n);
        if (wg == 0 && n != cur) {
            const uint32_t i = s.trace_n++;
            if (i < (uint32_t)kTraceCap) {
                a.ws.trace[2 * i] = (uint32_t)ticks_now();
                a.ws.trace[2 * i + 1] = n;
            }
        }
    }
    return n;
}

// Controller inputs read as a task's work completes: this role's progress
// word with the task added, the other role's word, the published target.
struct CtlRead {
    uint64_t mine, other;
    uint32_t raw_target;
};

// Thread 0, when a task's products are complete (its stores may still be in
// flight): record the task in its role word ((cycles << kCountBits) | tiles)
// and read what the controller needs.  The returns are consumed by ctl_finish
// after the tile's stores have been issued, so the round trip overlaps them.
__device__ __forceinline__ CtlRead ctl_issue(const FusedArgs &a, Live *L, int role, uint32_t units,
                                             uint64_t dt, uint64_t r0, uint64_t r1) {
    CtlRead c;
    const uint64_t inc = (dt << kCountBits) | units;
    if (role == kRoleCompute) {
        c.mine = add_relaxed(&L->role_compute.v, inc) + inc;
        c.other = ld_relaxed(&L->role_reduce.v);
    } else {
        c.mine = add_relaxed(&L->role_reduce.v, inc) + inc;
        c.other = ld_relaxed(&L->role_compute.v);
        min_relaxed(&L->r_start, r0);
        max_relaxed(&L->r_end, r1);
    }
    c.raw_target = a.mode == kAdaptive ? ld_relaxed(&L->target_ns.v) : 0u;
    return c;
}

// Thread 0: one controller step ("【学习】mKernel 分析" section 2.4) from the
// words ctl_issue read; the role of the next task follows from its result.
__device__ __forceinline__ void ctl_finish(const FusedArgs &a, Live *L, uint32_t wg, int role,
                                           const CtlRead &c, Sched &s) {
    if (a.mode != kAdaptive) return;
    const uint64_t cw = role == kRoleCompute ? c.mine : c.other;
    const uint64_t rw = role == kRoleCompute ? c.other : c.mine;
    s.target = controller_step(a, L, wg, s, cw, rw, c.raw_target);
}

// Cache policies of the tile hand-off.  When every tile is computed and
// reduced on one XCD (LOCAL), producer and consumer share that XCD's L2: the
// partial is stored write-back and read past the reader's L1 (sc0).  Across
// XCDs, whose L2s are not coherent with each other, the partial is written
// through (sc1) and read at device scope (sc1).  The reduced tile is what a
// released chunk hands on (to a sender, in the multi-GPU kernel), so in both
// modes it is streamed out write-through (nt sc1): once its stores have
// drained it is visible at device scope, and the chunk's release needs no
// L2 writeback.
template <bool LOCAL> struct HandOff {
    static constexpr int kPartialStore = LOCAL ? kPolicyDefault : kPolicyCoherentStore;
    static constexpr int kPartialLoad = LOCAL ? 1 : kPolicyCoherentLoad;
    static constexpr int kResultStore = kPolicyCoherentStream;
};

// RS selects the reduce-scatter share: the protocol covers this rank's shard
// (M, tiles_m), and once a workgroup has no task left in it, it computes the
// other ranks' tile rows as plain GEMM blocks into their inbox slots.  A
// separate instance keeps the AllReduce kernels free of that path and of the
// registers it takes.
template <int TM, int TN, bool LOCAL, bool RS>
__global__ __launch_bounds__((GemmFor<TM, TN, kPolicyDefault>::NT),
                             (TileCfg<TM, TN>::WPC * GemmFor<TM, TN, kPolicyDefault>::NWAVES / 4))
void fused_gemm_reduce_kernel(
    FusedArgs a) {
    using H = HandOff<LOCAL>;
    using G = GemmFor<TM, TN, H::kPartialStore>;
    __shared__ __attribute__((aligned(1024))) char lds_raw[fused_lds_bytes<TM, TN>()];
    __shared__ Decision sh_dec;
    // thread 0's scheduling state lives in LDS, not in registers every lane
    // would have to reserve next to the GEMM's
    __shared__ Sched sh_sched;
    __shared__ uint64_t sh_c0, sh_r0;
    lchar *lds = (lchar *)lds_raw;

    const int tid = threadIdx.x;
    const uint32_t wg = blockIdx.x;
    // the host launches this instance exactly when a.local is LOCAL: as a
    // constant it removes the other mode's claim paths from the scheduler
    a.local = LOCAL ? 1 : 0;
    Live *L = a.ws.live;
    typename G::Lane ln;
    G::init_lane(ln, a.N, a.K);

    constexpr int TPB = TileCfg<TM, TN>::TPB;
    static_assert(TPB <= kMaxTpb, "tiles per block");
    const Blocks bk = make_blocks(TPB, (uint32_t)a.tiles_m, (uint32_t)a.tiles_n);
    // the partitions serve thread 0's claims only: kept in LDS beside the
    // scheduling state
    __shared__ Parts sh_parts;
    const Parts &pt = sh_parts;
    if (tid == 0)
        sh_parts = make_parts((uint32_t)a.nxcd, a.local ? (uint32_t)a.xcd_cols : 1u, (uint32_t)a.tiles_m,
                              bk.bn, chunk_blocks(a.tpc, TPB), (uint32_t)a.group_m);
    Sched &s = sh_sched;
    if (LOCAL && tid == 0) {
        // tiles stay on their XCD only if this workgroup runs where its index
        // says (workgroup w on XCD w mod 8); otherwise stop everything
        uint32_t xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        if ((xcc & 0xFu) != wg % (uint32_t)a.nxcd) {
            __hip_atomic_fetch_max(&L->error, (uint32_t)kErrXcd, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_or(&L->sticky, kStickyXcd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (tid == 0) {
        s.det_i = 0;
        s.last_role = kRoleNone;
        s.compute_exhausted = false;
        s.parts_done = 0;
        s.reduce_exhausted = false;
        s.pending_role = kRoleNone;
        s.pending_q = 0;
        s.pending_ns = 0;
        s.wait_start = 0;
        s.target = (uint32_t)a.ns_init;   // the launch starts with the target unset
        s.early_claim = false;
        s.early_x = s.early_i = s.early_ns = 0;
        s.early_flag = false;
        s.early_flag_value = 0;
        s.decide_t0 = s.decide_t1 = 0;
        s.trace_n = 0;
        min_relaxed(&L->t_start, ticks_now());
    }

    // As every task's work completes, thread 0 records it in its role word,
    // reads the controller inputs and claims its next task (under the target
    // of its previous controller step), all at once; the round trips overlap
    // the task's stores, and the controller step that follows sets the role
    // for the task after.  The counters of a reduced tile are issued right
    // after its stores drain and read during the next task (see CntRead).
    CntRead pend;   // thread 0 only
    pend.c = kNoChunk;
    pend.want = pend.old_t = pend.old_c = 0;
    // reduce-scatter: the other ranks' tile rows, plain GEMM blocks each
    // stored straight into this rank's inbox slot at its owner.  Partition x
    // of the nx column bands of those rows has its own queue, taken row by
    // row, so an XCD keeps its band of B in its L2; a workgroup takes its own
    // XCD's band first and the others' once it is empty.
    const uint32_t extra_row0 = (uint32_t)a.tiles_m;
    __shared__ uint32_t sh_extra, sh_extra_done;
    if (tid == 0) sh_extra_done = 0;
    auto extra_block = [&]() -> bool {
        if (tid == 0) {
            const uint32_t nx = a.nxcd > 1 ? (uint32_t)a.nxcd : 1u;
            const uint32_t rows = (uint32_t)a.tiles_m_all - extra_row0;
            uint32_t blk = kNoTile;
            for (uint32_t k = 0; k < nx && blk == kNoTile; ++k) {
                const uint32_t x = (wg + k) % nx;
                if (sh_extra_done & (1u << x)) continue;
                const uint32_t c0 = bk.bn * x / nx, width = bk.bn * (x + 1) / nx - c0;
                const uint32_t i = add_relaxed(&L->extra_claim[x].v, 1u);
                if (i < rows * width)
                    blk = (i / width) * bk.bn + c0 + i % width;
                else
                    sh_extra_done |= 1u << x;
            }
            sh_extra = blk;
        }
        __syncthreads();
        const uint32_t q = __builtin_amdgcn_readfirstlane(sh_extra);
        // sh_extra is rewritten only after every thread has read it
        __syncthreads();
        if (q == kNoTile) return false;
        const int64_t Mp = opaque(a.M_all), Np = opaque(a.N), Kp = opaque(a.K);
        G::block(ln, a.A, a.B, a.remote, Mp, Np, Kp, (int64_t)(extra_row0 + q / bk.bn) * TM,
                 (int64_t)(q % bk.bn) * (TPB * TN), lds, [] {});
        return true;
    };
    // Before one block's compute time no shard tile is ready to reduce, and
    // the shard's blocks keep only its first compute workgroups busy (claims
    // go out in workgroup order): every other workgroup, reducers included,
    // computes one block outside the shard first
    if constexpr (RS)
        if (a.mode != kDeterministic && (wg < (uint32_t)a.ns_init || wg >= (uint32_t)a.ns_init + bk.TB))
            extra_block();
    for (;;) {
        if (tid == 0) {
            s.decide_t0 = ticks_now();
            const Decision d = next_task(a, pt, bk, L, wg, s, pend);
            s.decide_t1 = ticks_now();
            if (d.role == kRoleReduce) prefetch_claim(a, pt, L, wg, s, d);
            sh_dec = d;
            sh_c0 = cycles_now();
            sh_r0 = ticks_now();
        }
        __syncthreads();
        // the decision is workgroup-uniform: keep it in scalar registers, so
        // tile bases and buffer resources derived from it are scalar too
        Decision d;
        d.role = __builtin_amdgcn_readfirstlane(sh_dec.role);
        d.tile = __builtin_amdgcn_readfirstlane(sh_dec.tile);
        d.ns_seen = __builtin_amdgcn_readfirstlane(sh_dec.ns_seen);
        if (d.role == kRoleExit) break;
        const int64_t Mp = opaque(a.M), Np = opaque(a.N), Kp = opaque(a.K);
        // tiles [t0, t0 + nt): block d.tile (compute) or tile d.tile (reduce)
        const bool computing = d.role == kRoleCompute;
        const uint32_t t0 = computing ? bk.first_tile(d.tile) : d.tile;
        const uint32_t nt = computing ? bk.count(d.tile) : 1u;
        const int ti = (int)(t0 / (uint32_t)a.tiles_n);
        const int tj = (int)(t0 % (uint32_t)a.tiles_n);

        CtlRead ctl;
        Early early;
        // progress is counted in tiles for both roles, so the controller's
        // R_p C_p is the same remaining time whatever the block size
        auto work_done = [&](int role) {
            if (tid == 0) {
                ctl = ctl_issue(a, L, role, nt, cycles_now() - sh_c0, sh_r0, ticks_now());
                early = early_issue(a, pt, bk, L, wg, s);
            }
        };
        // the previous reduce task's counters: read once this task's first
        // loads are in flight (reduce), or before the K loop (compute)
        auto counters_back = [&]() {
            if (tid == 0) cnt_finish(a, L, pend);
        };
        if (d.role == kRoleCompute) {
            counters_back();
            G::block(ln, a.A, a.B, a.C, Mp, Np, Kp, (int64_t)ti * TM, (int64_t)tj * TN, lds,
                     [&] { work_done(kRoleCompute); });
        } else {
            // thread 0 saw the flag before the barrier; the partial is read
            // with device-coherent loads, after it
            if (a.P > 0) {
                // the peers are [P, M_all, N]: the shard's rows come first
                if constexpr (RS)
                    reduce_tile<TM, TN, G::NT, H::kPartialLoad, H::kResultStore, 64>(
                        a.peers, a.C, Mp, Np, a.peer_mn, a.P, (int64_t)ti * TM, (int64_t)tj * TN,
                        counters_back);
                else
                    reduce_tile<TM, TN, G::NT, H::kPartialLoad, H::kResultStore, LOCAL ? 128 : 64>(
                        a.peers, a.C, Mp, Np, Mp * Np, a.P, (int64_t)ti * TM, (int64_t)tj * TN,
                        counters_back);
            } else {
                counters_back();
            }
            work_done(kRoleReduce);
        }
        if (tid == 0) {
            ctl_finish(a, L, wg, d.role, ctl, s);
            early_finish(s, early);
        }
        // payload before flag ("【学习】mKernel 分析" section 2.5): every wave's
        // device-coherent tile stores have completed before thread 0
        // publishes the tile (compute) or counts it toward its chunk (reduce)
        drain_vmem();
        __syncthreads();
        if (tid == 0) {
            const uint32_t t_end = (uint32_t)ticks_now();
            // a reduced tile is complete at device scope: count it now.  (The
            // whole record is rewritten either way, so none of it stays live
            // across a compute task.)
            if (d.role == kRoleReduce) {
                pend = cnt_issue(a, t0);
            } else {
                pend.c = kNoChunk;
                pend.want = pend.old_t = pend.old_c = 0;
            }
            for (uint32_t k = 0; k < nt; ++k) {
                const uint32_t t = t0 + k;
                if (d.role == kRoleCompute) {
                    if ((int64_t)t != a.skip_publish) st_relaxed(&a.ws.tile_flag[t], a.epoch);
                    a.ws.cowner[t] = (d.ns_seen << 16) | wg;
                } else {
                    a.ws.rowner[t] = (d.ns_seen << 16) | wg;
                }
                // per-tile timeline (low 32 bits of the constant clock)
                uint32_t *tl = a.ws.timeline + (d.role == kRoleCompute ? 0u : 2u * a.Tcap);
                tl[t] = (uint32_t)sh_r0;
                tl[a.Tcap + t] = t_end;
                // how long choosing this task took (claim, readiness wait)
                a.ws.timeline[(d.role == kRoleCompute ? 4u : 5u) * a.Tcap + t] =
                    (uint32_t)(s.decide_t1 - s.decide_t0);
            }
            if (s.last_role != kRoleNone && s.last_role != d.role) add_relaxed(&L->role_switches, 1u);
            s.last_role = d.role;
        }
        // sh_dec is rewritten only after every thread has read it
        __syncthreads();
    }
    if (tid == 0) {
        // counters of the last reduced tile
        cnt_finish(a, L, pend);
    }
    // then whatever is left outside the shard
    if constexpr (RS)
        while (extra_block()) {
        }
    if (tid == 0) {
        max_relaxed(&L->t_end, ticks_now());
        if (wg == 0) st_relaxed(&L->trace_len, s.trace_n);
        // Every write this workgroup made to the control block is a
        // device-scope atomic, complete once the drain returns, so a relaxed
        // count suffices for the last workgroup to read them all.  A release
        // here would write back (and the acquire invalidate) the XCD's L2
        // under the workgroups still reducing.
        drain_vmem();
        const uint32_t old = add_relaxed(&L->exit_count, 1u);
        if (old == (uint32_t)a.nwg - 1) finish_launch(a, L);
    }
}

// ---------------------------------------------------------------------------
// unfused baseline: a GEMM kernel writes C_r, then a reduce kernel adds peers
// ---------------------------------------------------------------------------

// persistent GEMM over all blocks in the same claim order, same MFMA core
template <int TM, int TN>
__global__ __launch_bounds__((GemmFor<TM, TN, kPolicyDefault>::NT),
                             (TileCfg<TM, TN>::WPC * GemmFor<TM, TN, kPolicyDefault>::NWAVES / 4))
void gemm_kernel(GemmArgs a) {
    using G = GemmFor<TM, TN, kPolicyDefault>;
    constexpr int TPB = TileCfg<TM, TN>::TPB;
    __shared__ __attribute__((aligned(1024))) char lds_raw[G::LDS_BYTES];
    lchar *lds = (lchar *)lds_raw;
    typename G::Lane ln;
    G::init_lane(ln, a.N, a.K);
    const Blocks bk = make_blocks(TPB, (uint32_t)a.tiles_m, (uint32_t)a.tiles_n);
    const Parts pt = make_parts((uint32_t)a.nxcd, (uint32_t)a.xcd_cols, (uint32_t)a.tiles_m, bk.bn,
                                chunk_blocks((uint32_t)a.tpc, TPB), (uint32_t)a.group_m);
    for (uint32_t q = blockIdx.x; q < bk.TB; q += gridDim.x) {
        const uint32_t t0 = bk.first_tile(pt.ticket(q));
        const int64_t Mp = opaque(a.M), Np = opaque(a.N), Kp = opaque(a.K);
        const uint32_t ti = t0 / (uint32_t)a.tiles_n;
        // reduce-scatter: other ranks' tile rows go straight to their inboxes
        float *dst = ti < (uint32_t)a.own_tile_rows ? a.C : a.remote;
        G::block(ln, a.A, a.B, dst, Mp, Np, Kp, (int64_t)ti * TM, (int64_t)(t0 % (uint32_t)a.tiles_n) * TN,
                 lds, [] {});
    }
}

constexpr int kReduceThreads = 256;

__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(ReduceArgs a) {
    constexpr int U = 4;
    const int64_t stride = (int64_t)gridDim.x * kReduceThreads;
    int64_t i = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x;
    f32x4 *C = (f32x4 *)a.C;
    const f32x4 *Pp = (const f32x4 *)a.peers;
    const int64_t MN4 = a.MN / 4;
    for (; i + (U - 1) * stride < a.own4; i += U * stride) {
        f32x4 acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = C[i + u * stride];
        int p = 0;
        for (; p + 4 <= a.P; p += 4) {
            f32x4 v[4][U];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int u = 0; u < U; ++u)
                    v[q][u] = __builtin_nontemporal_load(Pp + (int64_t)(p + q) * MN4 + i + u * stride);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int u = 0; u < U; ++u) acc[u] += v[q][u];
        }
        for (; p < a.P; ++p)
#pragma unroll
            for (int u = 0; u < U; ++u)
                acc[u] += __builtin_nontemporal_load(Pp + (int64_t)p * MN4 + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_nontemporal_store(acc[u], C + i + u * stride);
    }
    for (; i < a.own4; i += stride) {
        f32x4 acc = C[i];
        for (int p = 0; p < a.P; ++p) acc += __builtin_nontemporal_load(Pp + (int64_t)p * MN4 + i);
        __builtin_nontemporal_store(acc, C + i);
    }
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ void live_init(Live *L) {
    for (int x = 0; x < kMaxXcd; ++x) L->compute_claim[x].v = 0;
    for (int x = 0; x < kMaxXcd; ++x) L->reduce_claim[x].v = 0;
    for (int x = 0; x < kMaxXcd; ++x) L->extra_claim[x].v = 0;
    L->exit_count = 0;
    L->target_ns.v = 0;
    L->role_switches = 0;
    L->chunks_released.v = 0;
    L->violations = 0;
    L->error = 0;
    L->ns_min = 0xFFFFFFFFu;
    L->ns_max = 0;
    L->trace_len = 0;
    L->ns_final = 0;
    L->sticky = 0;
    L->role_compute.v = 0;
    L->role_reduce.v = 0;
    L->t_start = ~(uint64_t)0;
    L->t_end = 0;
    L->r_start = ~(uint64_t)0;
    L->r_end = 0;
}

__global__ void ws_init_kernel(Live *live, Live *snap) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        live_init(live);
        live_init(snap);
    }
}

__global__ void fill_u32_kernel(uint32_t *p, uint32_t v, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// XCD of every workgroup of a one-per-CU grid (the launch asks for more
// than half a CU's LDS, which forces one per CU, as in the fused kernel)
__global__ __launch_bounds__(64) void xcc_probe_kernel(uint32_t *out) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if (threadIdx.x == 0) out[blockIdx.x] = xcc & 0xFu;
}

__global__ void controller_eval_kernel(const uint64_t *in, uint32_t *out, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint64_t *r = in + 10 * (int64_t)i;
    out[i] = controller_update((uint32_t)r[0], (uint32_t)r[1], (uint32_t)r[2], (uint32_t)r[3], r[4],
                               r[5], (uint32_t)r[6], (uint32_t)r[7], (uint32_t)r[8], (uint32_t)r[9]);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// Workgroups of the fused kernel that stay resident on one CU: the tile
// configuration's target, bounded by what the runtime reports for the
// compiled kernel (registers, LDS).  0 on error.
template <int TM, int TN>
static int fused_residency() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks, reinterpret_cast<const void *>(&fused_gemm_reduce_kernel<TM, TN, true, false>),
            GemmFor<TM, TN, kPolicyDefault>::NT, 0) != hipSuccess)
        return 0;
    return blocks < TileCfg<TM, TN>::WPC ? blocks : TileCfg<TM, TN>::WPC;
}

int workgroups_per_cu(int tm, int tn) {
    if (tm == 64 && tn == 64) return fused_residency<64, 64>();
    if (tm == 128 && tn == 128) return fused_residency<128, 128>();
    if (tm == 256 && tn == 128) return fused_residency<256, 128>();
    return 0;
}

int tiles_per_block(int tm, int tn) {
    if (tm == 64 && tn == 64) return TileCfg<64, 64>::TPB;
    if (tm == 128 && tn == 128) return TileCfg<128, 128>::TPB;
    if (tm == 256 && tn == 128) return TileCfg<256, 128>::TPB;
    return 0;
}

bool tile_supported(int tm, int tn) {
    return (tm == 64 && tn == 64) || (tm == 128 && tn == 128) || (tm == 256 && tn == 128);
}

template <int TM, int TN, bool RS>
static void launch_fused_rs(const FusedArgs &a, hipStream_t s) {
    if (a.local)
        hipLaunchKernelGGL((fused_gemm_reduce_kernel<TM, TN, true, RS>), dim3(a.nwg),
                           dim3(GemmFor<TM, TN, kPolicyDefault>::NT), 0, s, a);
    else
        hipLaunchKernelGGL((fused_gemm_reduce_kernel<TM, TN, false, RS>), dim3(a.nwg),
                           dim3(GemmFor<TM, TN, kPolicyDefault>::NT), 0, s, a);
}

template <int TM, int TN>
static hipError_t launch_fused_t(const FusedArgs &a, hipStream_t s) {
    if (a.remote)
        launch_fused_rs<TM, TN, true>(a, s);
    else
        launch_fused_rs<TM, TN, false>(a, s);
    return hipGetLastError();
}

hipError_t launch_fused(int tm, int tn, const FusedArgs &a, hipStream_t s) {
    if (tm == 64 && tn == 64) return launch_fused_t<64, 64>(a, s);
    if (tm == 128 && tn == 128) return launch_fused_t<128, 128>(a, s);
    if (tm == 256 && tn == 128) return launch_fused_t<256, 128>(a, s);
    return hipErrorInvalidValue;
}

template <int TM, int TN>
static hipError_t launch_gemm_t(const GemmArgs &a, int num_cu, hipStream_t s) {
    using G = GemmFor<TM, TN, kPolicyDefault>;
    constexpr int TPB = TileCfg<TM, TN>::TPB;
    const int per_cu = TileCfg<TM, TN>::WPC;
    const int64_t TB = (int64_t)a.tiles_m * ((a.tiles_n + TPB - 1) / TPB);
    const int64_t grid = TB < (int64_t)num_cu * per_cu ? TB : (int64_t)num_cu * per_cu;
    hipLaunchKernelGGL((gemm_kernel<TM, TN>), dim3((unsigned)grid), dim3(G::NT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm(int tm, int tn, const GemmArgs &a, int num_cu, hipStream_t s) {
    if (tm == 64 && tn == 64) return launch_gemm_t<64, 64>(a, num_cu, s);
    if (tm == 128 && tn == 128) return launch_gemm_t<128, 128>(a, num_cu, s);
    if (tm == 256 && tn == 128) return launch_gemm_t<256, 128>(a, num_cu, s);
    return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceArgs &a, int num_cu, hipStream_t s) {
    int64_t blocks = (a.count4 + kReduceThreads - 1) / kReduceThreads;
    const int64_t cap = (int64_t)num_cu * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)blocks), dim3(kReduceThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_ws_init(Live *live, Live *snap, hipStream_t s) {
    hipLaunchKernelGGL(ws_init_kernel, dim3(1), dim3(64), 0, s, live, snap);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t *p, uint32_t v, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, v, n);
    return hipGetLastError();
}

hipError_t launch_xcc_probe(uint32_t *out, int nwg, hipStream_t s) {
    hipLaunchKernelGGL(xcc_probe_kernel, dim3(nwg), dim3(64), 96 * 1024, s, out);
    return hipGetLastError();
}

hipError_t launch_controller_eval(const uint64_t *in, uint32_t *out, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(controller_eval_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, out, n);
    return hipGetLastError();
}

}  // namespace mk
