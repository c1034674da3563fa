// Kernels of the AllGather+GEMM share (communication feeds compute) and its
// unfused baseline's gather, on the GEMM core of the fused library.
#include "mk_device.hpp"
#include "mk_allgather.hpp"

namespace mk {

// ---------------------------------------------------------------------------
// AllGather+GEMM, one rank's share (communication feeds compute)
//
// AllGather + GEMM row of the MarkTechPost page's five-kernel table: every
// rank holds a shard of A, and the local GEMM consumes the gathered tiles as
// they arrive.  "【学习】mKernel 分析" section 2.6 (Table 3): 128-row chunks,
// shards submitted at launch, compute tiles taken in order of input
// availability (local first); section 2.4: the same on-GPU controller sets
// the communication-role size, and a compute block waiting for its input
// helps communication.
//
// On one GPU the other ranks' shards are buffers in local HBM and the copy
// role stands in for their transfer: a copy task moves one part of a chunk
// (one tile row of A: TM rows x K) into the gathered A and stores it
// write-through; once its stores have drained it counts the part into the
// chunk's counter, and the task whose count completes the chunk publishes
// the chunk's arrival flag.  One copy task moves at most 64 KiB: a single
// workgroup keeps only so many bytes in flight, and a chunk shared by many
// copiers arrives sooner (and a waiting compute workgroup helps in short
// steps).  A compute
// task is one block of TPB adjacent tiles of one tile row; tiles of this
// rank's own rows read the local shard at once, the others read the gathered
// A once their chunk's flag carries the launch's epoch.  Claims: copy tasks
// take the other ranks' chunks first (rank, then row), this rank's own last,
// the parts of a chunk one after another;
// compute blocks go in row order, so this rank's rows come first and the
// others follow in the order they are copied.  With column bands (one per
// XCD, workgroup w on XCD w mod 8) each band is its own row-order queue:
// the workgroups of one XCD share its band's B columns in their L2 and the
// chip reads B about once per band row group instead of once per XCD per
// row; a workgroup whose band is exhausted takes blocks from the next bands.
// Roles follow the
// workgroup index against the target (copy iff w < target), re-read at
// every task boundary.
// ---------------------------------------------------------------------------

enum AgRole : int { kAgCompute = 0, kAgCopy = 1, kAgExit = 2 };

struct AgDecision {
    int role;
    uint32_t unit;      // compute: block; copy: copy task (chunk * parts + part)
    uint32_t ns_seen;   // copy target the task was taken under | kHelp (copy by a waiting compute workgroup)
};

struct AgSched {
    uint32_t target;
    uint32_t det_i;
    bool copy_exhausted, compute_exhausted;
    bool have_block;        // a claimed compute block waiting for its input
    uint32_t block, block_ns;
    uint32_t bands_done;    // bit x: band x has no compute block left
    int last_role;
};

// copy task of the q-th copy claim: chunks in copy order (the other ranks'
// first), the parts of each in order
__device__ __forceinline__ uint32_t ag_copy_task(const AgArgs &a, uint32_t q) {
    const uint32_t k = q / a.parts, part = q % a.parts;
    const uint32_t peer_chunks = a.Ch - a.cps;
    const uint32_t c = k < peer_chunks ? a.cps + k : k - peer_chunks;
    return c * a.parts + part;
}

// the input rows of tile row `row` are there: this rank's own from the start,
// the others once their chunk has arrived (one read, no wait)
__device__ __forceinline__ bool ag_ready(const AgArgs &a, uint32_t row) {
    return row < a.cps || ld_relaxed(&a.ws.chunk_flag[row]) == a.epoch;
}

__device__ __forceinline__ bool ag_timed_out(const AgArgs &a, Live *L, uint64_t since) {
    if (ticks_now() - since <= a.timeout_ticks) return false;
    __hip_atomic_fetch_max(&L->error, (uint32_t)kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(&L->sticky, kStickyTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// wait (bounded) for tile row `row`'s input; false on timeout or another
// workgroup's error
__device__ bool ag_wait(const AgArgs &a, Live *L, uint32_t row) {
    const uint64_t since = ticks_now();
    for (;;) {
        if (ag_ready(a, row)) return true;
        if (ld_relaxed(&L->error) != kErrNone) return false;
        if (ag_timed_out(a, L, since)) return false;
        __builtin_amdgcn_s_sleep(1);
    }
}

// Thread 0: claim a compute block.  One band: the row-major queue.  Bands:
// block columns split as evenly as possible (the first bn mod bands bands
// one wider), band x's i-th claim is row i / cols, column col0 + i mod cols;
// the home band (the workgroup's XCD) first, then the others in turn.
__device__ __forceinline__ bool ag_claim_block(const AgArgs &a, Live *L, uint32_t wg, AgSched &s,
                                               uint32_t &j) {
    const uint32_t nb = a.bands;
    if (nb <= 1) {
        j = add_relaxed(&L->compute_claim[0].v, 1u);
        return j < a.TB;
    }
    const uint32_t cmin = a.bn / nb, crem = a.bn % nb;
    for (uint32_t k = 0; k < nb; ++k) {
        const uint32_t x = (wg + k) % nb;
        if ((s.bands_done >> x) & 1u) continue;
        const uint32_t cols = cmin + (x < crem ? 1u : 0u);
        const uint32_t col0 = x * cmin + (x < crem ? x : crem);
        const uint32_t i = add_relaxed(&L->extra_claim[x].v, 1u);
        if (i < a.Ch * cols) {
            j = (i / cols) * a.bn + col0 + i % cols;
            return true;
        }
        s.bands_done |= 1u << x;
    }
    return false;
}

// Thread 0: the next task.
__device__ AgDecision ag_next(const AgArgs &a, Live *L, uint32_t wg, AgSched &s) {
    const uint32_t B = (uint32_t)a.nwg;
    if (a.mode == kDeterministic) {
        const uint32_t ns = (uint32_t)a.ns_init;
        if (wg < ns) {
            const uint32_t q = wg + s.det_i * ns;
            if (q >= a.Q) return {kAgExit, 0, ns};
            ++s.det_i;
            return {kAgCopy, ag_copy_task(a, q), ns};
        }
        const uint32_t j = (wg - ns) + s.det_i * (B - ns);
        if (j >= a.TB) return {kAgExit, 0, ns};
        ++s.det_i;
        if (!ag_wait(a, L, j / a.bn)) return {kAgExit, 0, ns};
        return {kAgCompute, j, ns};
    }
    for (;;) {
        const uint32_t ns = s.target;
        if (s.have_block) {
            const uint32_t row = s.block / a.bn;
            if (ag_ready(a, row)) {
                s.have_block = false;
                return {kAgCompute, s.block, s.block_ns};
            }
            // waiting for its input: help the copy role meanwhile
            if (a.mode == kAdaptive && a.help && !s.copy_exhausted) {
                const uint32_t q = add_relaxed(&L->compute_claim[1].v, 1u);
                if (q < a.Q) return {kAgCopy, ag_copy_task(a, q), ns | kHelp};
                s.copy_exhausted = true;
            }
            if (!ag_wait(a, L, row)) return {kAgExit, 0, ns};
            s.have_block = false;
            return {kAgCompute, s.block, s.block_ns};
        }
        const bool copy_role = wg < ns;
        if (copy_role && !s.copy_exhausted) {
            const uint32_t q = add_relaxed(&L->compute_claim[1].v, 1u);
            if (q < a.Q) return {kAgCopy, ag_copy_task(a, q), ns};
            s.copy_exhausted = true;
        }
        // static copiers leave once every chunk is claimed
        if (copy_role && a.mode != kAdaptive) return {kAgExit, 0, ns};
        if (!s.compute_exhausted) {
            uint32_t j;
            if (ag_claim_block(a, L, wg, s, j)) {
                s.have_block = true;
                s.block = j;
                // a copy-role workgroup computes only once no chunk is left
                // to claim: no copy role remains (logged as target 0)
                s.block_ns = copy_role ? 0u : ns;
                continue;
            }
            s.compute_exhausted = true;
        }
        // adaptive: no compute left to claim, every workgroup copies (the
        // controller's target is B once no compute remains; logged as such)
        if (a.mode == kAdaptive && !s.copy_exhausted) {
            const uint32_t q = add_relaxed(&L->compute_claim[1].v, 1u);
            if (q < a.Q) return {kAgCopy, ag_copy_task(a, q), copy_role ? ns : B};
            s.copy_exhausted = true;
        }
        return {kAgExit, 0, ns};
    }
}

// one copy task: part `u mod parts` of chunk `u / parts` (TM rows x K of a
// shard) into the gathered A.  Source read once (nt); destination written
// through (nt sc1), visible at device scope once the stores have drained.
template <int NT, int TM>
__device__ __forceinline__ void ag_copy(const AgArgs &a, uint32_t u) {
    const uint32_t c = u / a.parts, part = u % a.parts;
    const uint32_t r = c / a.cps, lr = c % a.cps;
    const uint16_t *src = r == 0 ? a.A_local + (int64_t)lr * TM * a.K
                                 : a.A_peers + ((int64_t)(r - 1) * a.Ms + (int64_t)lr * TM) * a.K;
    uint16_t *dst = a.A_gath + (int64_t)c * TM * a.K;
    const uint64_t n16c = (uint64_t)TM * (uint64_t)a.K / 8;   // 16-byte pieces of the chunk
    const uint32_t i0 = (uint32_t)(n16c * part / a.parts);
    const uint32_t n16 = (uint32_t)(n16c * (part + 1) / a.parts) - i0;
    const auto rs = scalar_rsrc(src + (int64_t)i0 * 8);
    const auto rd = scalar_rsrc(dst + (int64_t)i0 * 8);
    // Every load of a pass is issued before its first store, and a pass
    // covers up to 80 KiB: a part of up to that size (64 KiB, or a little
    // more where the part count is capped) is one load round trip and one
    // store drain.  Pieces past the part read zero and drop their stores.
    constexpr int U = NT >= 512 ? 10 : 20;
    for (uint32_t b = 0; b < n16; b += U * NT) {
        uint32_t off[U];
        f32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t i = b + k * NT + threadIdx.x;
            off[k] = i < n16 ? i * 16u : kOOB;
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[k], 0, kPolicyStream);
        }
#pragma unroll
        for (int k = 0; k < U; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(v[k], rd, off[k], 0, kPolicyCoherentStream);
    }
}

template <int TM, int TN>
__global__ __launch_bounds__((GemmFor<TM, TN, kPolicyDefault>::NT),
                             (TileCfg<TM, TN>::WPC * GemmFor<TM, TN, kPolicyDefault>::NWAVES / 4))
void allgather_gemm_kernel(AgArgs a) {
    using G = GemmFor<TM, TN, kPolicyDefault>;
    constexpr int TPB = TileCfg<TM, TN>::TPB;
    __shared__ __attribute__((aligned(1024))) char lds_raw[fused_lds_bytes<TM, TN>()];
    __shared__ AgDecision sh_dec;
    __shared__ AgSched sh_sched;
    __shared__ uint64_t sh_c0, sh_r0;
    lchar *lds = (lchar *)lds_raw;
    const int tid = threadIdx.x;
    const uint32_t wg = blockIdx.x;
    Live *L = a.ws.live;
    typename G::Lane ln;
    G::init_lane(ln, a.N, a.K);
    AgSched &s = sh_sched;
    if (tid == 0) {
        s.target = (uint32_t)a.ns_init;
        s.det_i = 0;
        s.copy_exhausted = s.compute_exhausted = false;
        s.have_block = false;
        s.block = s.block_ns = 0;
        s.bands_done = 0;
        s.last_role = -1;
        min_relaxed(&L->t_start, ticks_now());
    }
    for (;;) {
        if (tid == 0) {
            sh_dec = ag_next(a, L, wg, s);
            sh_c0 = cycles_now();
            sh_r0 = ticks_now();
        }
        __syncthreads();
        AgDecision d;
        d.role = __builtin_amdgcn_readfirstlane(sh_dec.role);
        d.unit = __builtin_amdgcn_readfirstlane(sh_dec.unit);
        d.ns_seen = __builtin_amdgcn_readfirstlane(sh_dec.ns_seen);
        if (d.role == kAgExit) break;
        const int64_t Kp = opaque(a.K), Np = opaque(a.N), Mp = opaque(a.M);
        uint32_t t0 = 0, nt = 1;
        if (d.role == kAgCopy) {
            ag_copy<G::NT, TM>(a, d.unit);
        } else {
            const uint32_t row = d.unit / a.bn, bc = d.unit % a.bn;
            t0 = row * a.tiles_n + bc * TPB;
            nt = a.tiles_n - bc * TPB < (uint32_t)TPB ? a.tiles_n - bc * TPB : (uint32_t)TPB;
            // this rank's own rows straight from its shard, the others from
            // the gathered A (the chunk's flag was seen before the barrier)
            const uint16_t *Asrc = row < a.cps ? a.A_local : a.A_gath;
            G::block(ln, Asrc, a.B, a.C, Mp, Np, Kp, (int64_t)row * TM, (int64_t)bc * (TPB * TN), lds, [] {});
        }
        // payload before flag ("【学习】mKernel 分析" section 2.5)
        drain_vmem();
        __syncthreads();
        if (tid == 0) {
            const uint32_t t_end = (uint32_t)ticks_now();
            const uint64_t dt = cycles_now() - sh_c0;
            // every returning atomic and load of the task's bookkeeping is
            // issued before the first result is used: one round trip
            const bool copying = d.role == kAgCopy;
            const uint32_t u = d.unit, c = copying ? u / a.parts : 0u;
            uint32_t old0 = 0, old1 = 0;
            if (copying) {
                old0 = add_relaxed(&a.ws.chunk_cnt[c], 1u);
            } else {
                old0 = add_relaxed(&a.ws.tile_cnt[t0], 1u);
                if (nt > 1) old1 = add_relaxed(&a.ws.tile_cnt[t0 + 1], 1u);
            }
            // progress words, and one controller step: the copy role is the
            // communication role s (copy tasks), compute is p (tiles)
            const uint64_t inc = (dt << kCountBits) | (copying ? 1u : nt);
            const uint64_t mine = add_relaxed(copying ? &L->role_reduce.v : &L->role_compute.v, inc) + inc;
            const uint64_t other = ld_relaxed(copying ? &L->role_compute.v : &L->role_reduce.v);
            const uint32_t raw = a.mode == kAdaptive ? ld_relaxed(&L->target_ns.v) : 0u;
            if (copying) {
                // this part's stores drained before its count: the task
                // whose count completes the chunk sees every part landed
                const uint32_t base = (a.calls - 1) * a.parts;
                if (old0 < base || old0 >= base + a.parts) note_violation(L);
                if (old0 + 1 == base + a.parts) {
                    a.ws.chunk_release[c] = (uint32_t)ticks_now();
                    if ((int64_t)c != a.skip_publish) st_relaxed(&a.ws.chunk_flag[c], a.epoch);
                    add_relaxed(&L->chunks_released.v, 1u);
                }
                a.ws.rowner[u] = (d.ns_seen << 16) | wg;
                a.ws.timeline[2u * a.Tcap + u] = (uint32_t)sh_r0;
                a.ws.timeline[3u * a.Tcap + u] = t_end;
                min_relaxed(&L->r_start, (uint64_t)sh_r0);
                max_relaxed(&L->r_end, ticks_now());
            } else {
                static_assert(TPB <= 2, "bookkeeping issues at most two tile counts");
                if (old0 != a.calls - 1 || (nt > 1 && old1 != a.calls - 1)) note_violation(L);
                for (uint32_t k = 0; k < nt; ++k) {
                    const uint32_t t = t0 + k;
                    a.ws.cowner[t] = (d.ns_seen << 16) | wg;
                    a.ws.timeline[t] = (uint32_t)sh_r0;
                    a.ws.timeline[a.Tcap + t] = t_end;
                }
            }
            if (a.mode == kAdaptive) {
                const uint64_t cw = copying ? other : mine, sw = copying ? mine : other;
                const uint32_t cur = raw ? raw : (uint32_t)a.ns_init;
                const uint32_t n = controller_update_totals(
                    (uint32_t)a.nwg, a.T, a.Q, (uint32_t)(cw & kCountMask), (uint32_t)(sw & kCountMask),
                    cw >> kCountBits, sw >> kCountBits, cur, (uint32_t)a.ns_floor, 1u, (uint32_t)a.ns_cap);
                if (n != cur || raw == 0) {
                    st_relaxed(&L->target_ns.v, n);
                    min_relaxed(&L->ns_min, n);
                    max_relaxed(&L->ns_max, n);
                }
                s.target = n;
            }
            if (s.last_role >= 0 && s.last_role != d.role) add_relaxed(&L->role_switches, 1u);
            s.last_role = d.role;
        }
        __syncthreads();
    }
    if (tid == 0) {
        max_relaxed(&L->t_end, ticks_now());
        drain_vmem();
        const uint32_t old = add_relaxed(&L->exit_count, 1u);
        if (old == (uint32_t)a.nwg - 1) {
            FusedArgs f;
            f.mode = a.mode;
            f.ns_init = a.ns_init;
            f.ws = a.ws;
            finish_launch(f, L);
        }
    }
}

// the unfused baseline's first kernel: every shard into the gathered A
__global__ __launch_bounds__(256) void gather_kernel(AgArgs a) {
    const int64_t row16 = a.K / 8;                     // 16-byte pieces per row
    const int64_t shard16 = a.Ms * row16;
    const int64_t total = shard16 * (a.P + 1);
    const int64_t stride = (int64_t)gridDim.x * 256;
    u32x4 *dst = (u32x4 *)a.A_gath;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / shard16, o = i - r * shard16;
        const u32x4 *src = (const u32x4 *)(r == 0 ? a.A_local : a.A_peers + (r - 1) * a.Ms * a.K);
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + o), dst + i);
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <int TM, int TN>
static int ag_residency() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks, reinterpret_cast<const void *>(&allgather_gemm_kernel<TM, TN>),
            GemmFor<TM, TN, kPolicyDefault>::NT, 0) != hipSuccess)
        return 0;
    return blocks < TileCfg<TM, TN>::WPC ? blocks : TileCfg<TM, TN>::WPC;
}

int allgather_workgroups_per_cu(int tm, int tn) {
    if (tm == 64 && tn == 64) return ag_residency<64, 64>();
    if (tm == 128 && tn == 128) return ag_residency<128, 128>();
    if (tm == 256 && tn == 128) return ag_residency<256, 128>();
    return 0;
}

template <int TM, int TN>
static hipError_t launch_ag_t(const AgArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((allgather_gemm_kernel<TM, TN>), dim3(a.nwg), dim3(GemmFor<TM, TN, kPolicyDefault>::NT),
                       0, s, a);
    return hipGetLastError();
}

hipError_t launch_allgather_gemm(int tm, int tn, const AgArgs &a, hipStream_t s) {
    if (tm == 64 && tn == 64) return launch_ag_t<64, 64>(a, s);
    if (tm == 128 && tn == 128) return launch_ag_t<128, 128>(a, s);
    if (tm == 256 && tn == 128) return launch_ag_t<256, 128>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gather(const AgArgs &a, int num_cu, hipStream_t s) {
    const int64_t total = a.Ms * (a.K / 8) * (a.P + 1);
    int64_t blocks = (total + 255) / 256;
    const int64_t cap = (int64_t)num_cu * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace mk
