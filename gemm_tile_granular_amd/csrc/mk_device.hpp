// Device code shared by the kernels of the library (gfx950): vector types,
// buffer access with explicit cache policy, relaxed device-scope atomics and
// clocks, the on-GPU controller's closed form, the tile/claim maps, the MFMA
// GEMM core, the tile reduce, and the end-of-launch bookkeeping.  Included by
// every kernel source; everything here is inline or a template.
#pragma once
#include "mk_internal.hpp"

namespace mk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// buffer access with explicit cache policy
//
// Tile data crosses XCDs (a tile computed on one XCD is reduced on another),
// but only the tile hand-off needs device-scope coherence: A, B and the peers
// are read-only during a launch.  So the partial tile is stored with sc1
// (coherent at device scope) and read back with sc1 loads (device scope: not
// served from a stale line of the reader's caches); the writer drains its stores (vmcnt) before
// the flag is set.  This replaces agent-scope release/acquire fences, whose
// whole-L2 writeback and invalidate per tile cost 2-3x in reduce bandwidth.
// Buffer resources also give branch-free edge masking: an offset at or past
// kOOB reads zero and drops the store.
// ---------------------------------------------------------------------------

constexpr int kPolicyDefault = 0;
constexpr int kPolicyStream = 2;            // nt: read-once / write-once data
constexpr int kPolicyCoherentStore = 16;    // sc1: visible at device scope
constexpr int kPolicyCoherentLoad = 16;     // sc1: coherent at device (agent) scope
constexpr int kPolicyCoherentStream = 18;   // nt sc1
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint32_t kNumRecords = 0x7FFFFFFFu;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, kNumRecords, 0x00020000);
}

// Buffer resource of a workgroup-uniform address, built in scalar registers
// at the point of use.  The empty asm pins the address there, so the compiler
// neither hoists many resources out of a loop (crowding the scalar register
// file) nor moves them to vector registers (which would need a waterfall
// loop around every access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t scalar_rsrc(const void *p) {
    const uint64_t p64 = (uint64_t)p;
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p64);
    uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p64 >> 32));
    asm volatile("" : "+s"(lo), "+s"(hi));
    return make_rsrc((const void *)(((uint64_t)hi << 32) | lo));
}

// Wait until every vector memory operation of this wave has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left unconstrained).
__device__ __forceinline__ void drain_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A uniform value made opaque to the optimiser where it is taken: address
// arithmetic on it is redone per task instead of being hoisted out of a
// persistent loop, where its results would occupy registers across every task
// of both roles (in the fused kernel that pushed VGPRs into scratch, and each
// scratch reload inside the reduce pipeline drained all loads in flight).
__device__ __forceinline__ int64_t opaque(int64_t v) {
    asm volatile("" : "+s"(v));
    return v;
}

// ---------------------------------------------------------------------------
// clocks and atomics
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t cycles_now() { return __builtin_amdgcn_s_memtime(); }
__device__ __forceinline__ uint64_t ticks_now() { return __builtin_amdgcn_s_memrealtime(); }

template <class T> __device__ __forceinline__ T ld_relaxed(T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T> __device__ __forceinline__ void st_relaxed(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T> __device__ __forceinline__ T add_relaxed(T *p, T v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T> __device__ __forceinline__ void min_relaxed(T *p, T v) {
    __hip_atomic_fetch_min(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T> __device__ __forceinline__ void max_relaxed(T *p, T v) {
    __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// adaptive partition controller ("【学习】mKernel 分析" section 2.4)
//
// n_s* = B R_s C_s / (R_p C_p + R_s C_s): the reduce-workgroup count at which
// the predicted finish times R_s C_s / n_s and R_p C_p / (B - n_s) are equal.
// R_x = tasks of role x not finished, C_x = cumulative mean shader cycles per
// finished task.  Unsigned 64-bit arithmetic, nearest rounding with ties up;
// clamp to [min(floor, B-keep), B-keep] while compute remains (keep compute
// workgroups stay: 1, or one per XCD when every XCD works on its own tiles);
// B once it is done.
// Limits B <= 1024, T < 2^22 and C_x <= 2^26-1 keep every product exact.
// ---------------------------------------------------------------------------
// The step with each role's total given separately (T_p compute units, T_s
// communication units); controller_update is the case T_p = T_s = T.
__device__ inline uint32_t controller_update_totals(uint32_t B, uint32_t T_p, uint32_t T_s, uint32_t compute_done,
                                             uint32_t reduce_done, uint64_t sum_p, uint64_t sum_s,
                                             uint32_t current, uint32_t floor, uint32_t keep,
                                             uint32_t cap) {
    const uint32_t R_p = T_p - compute_done;
    const uint32_t R_s = T_s - reduce_done;
    if (R_p == 0) return B;
    const uint32_t hi = B - keep < cap ? B - keep : cap;
    const uint32_t lo = floor < hi ? floor : hi;
    uint64_t n;
    if (compute_done == 0 || reduce_done == 0) {
        n = current;
    } else {
        uint64_t C_p = sum_p / compute_done;
        uint64_t C_s = sum_s / reduce_done;
        if (C_p > kCostCap) C_p = kCostCap;
        if (C_s > kCostCap) C_s = kCostCap;
        const uint64_t num = (uint64_t)B * R_s * C_s;
        const uint64_t den = (uint64_t)R_p * C_p + (uint64_t)R_s * C_s;
        n = den ? (2 * num + den) / (2 * den) : current;
    }
    if (n < lo) n = lo;
    if (n > hi) n = hi;
    return (uint32_t)n;
}

__device__ inline uint32_t controller_update(uint32_t B, uint32_t T, uint32_t compute_done,
                                      uint32_t reduce_done, uint64_t sum_p, uint64_t sum_s,
                                      uint32_t current, uint32_t floor, uint32_t keep,
                                      uint32_t cap) {
    return controller_update_totals(B, T, T, compute_done, reduce_done, sum_p, sum_s, current, floor,
                                    keep, cap);
}

// ---------------------------------------------------------------------------
// claim order: chunk by chunk, chunks taken column-major inside bands of
// `group_m` tile rows, so the tiles in flight at once share A rows and B
// columns.  A chunk's tiles are consecutive claims.  Identity when chunks do
// not tile the rows evenly.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t tile_of_claim(uint32_t q, uint32_t tiles_m, uint32_t tiles_n,
                                                  uint32_t tpc, uint32_t group_m) {
    if (group_m <= 1 || tpc == 0 || (tiles_n % tpc) != 0) return q;
    const uint32_t ccols = tiles_n / tpc;
    const uint32_t cq = q / tpc, j = q % tpc;
    const uint32_t per_band = group_m * ccols;
    const uint32_t band = cq / per_band, r = cq % per_band;
    const uint32_t rows_left = tiles_m - band * group_m;
    const uint32_t rows = rows_left < group_m ? rows_left : group_m;
    const uint32_t col = r / rows, row = band * group_m + r % rows;
    return (row * ccols + col) * tpc + j;
}

// ---------------------------------------------------------------------------
// XCD-aware tile partitions
//
// MI355X has 8 XCDs, each with its own L2, and dispatches workgroup w to XCD
// w mod 8.  The blocks are cut into nx = px * py partitions: px row groups
// (tile row r -> group r mod px) times py column bands (contiguous runs of
// whole chunks).  Partition x is row group x / py, band x % py.  An XCD then
// fetches only its row groups' A panels and its band's B panels: operand
// traffic py*|A| + px*|B| against |A| + 8*|B| for whole rows (py = 1).
// Workgroups claim compute blocks from their own XCD's partition first, in
// the banded order above, so the blocks one L2 serves at once share A rows
// and B columns, and (unless tiles stay on their XCD) steal from the other
// partitions when theirs is done.  Without that restriction reduce tickets
// walk the partitions round-robin, which is the order in which tiles
// complete when the partitions progress together (whole rows only).
// ---------------------------------------------------------------------------
struct Parts {
    uint32_t nx;          // partitions (1 or the XCD count)
    uint32_t lpy;         // log2 of the column bands py (0: whole block rows)
    uint32_t px;          // row groups, nx / py
    uint32_t rows_min;    // block rows in the smaller row groups
    uint32_t rem;         // row groups [0, rem) hold one more block row
    uint32_t cch_min;     // chunk columns in the narrower bands (py > 1)
    uint32_t crem;        // bands [0, crem) hold one more chunk column
    uint32_t tiles_n, tpc, group_m;   // in blocks: per block row, per chunk

    __device__ __forceinline__ uint32_t rows(uint32_t x) const {
        return rows_min + ((x >> lpy) < rem ? 1u : 0u);
    }
    __device__ __forceinline__ uint32_t cols(uint32_t x) const {
        if (lpy == 0) return tiles_n;
        const uint32_t xc = x & ((1u << lpy) - 1u);
        return (cch_min + (xc < crem ? 1u : 0u)) * tpc;
    }
    __device__ __forceinline__ uint32_t col0(uint32_t x) const {
        if (lpy == 0) return 0;
        const uint32_t xc = x & ((1u << lpy) - 1u);
        return (xc * cch_min + (xc < crem ? xc : crem)) * tpc;
    }
    __device__ __forceinline__ uint32_t size(uint32_t x) const { return rows(x) * cols(x); }
    // block of the i-th claim of partition x
    __device__ __forceinline__ uint32_t tile(uint32_t x, uint32_t i) const {
        const uint32_t c = cols(x);
        const uint32_t local = tile_of_claim(i, rows(x), c, tpc, group_m);
        const uint32_t lr = local / c, lc = local % c;
        return (lr * px + (x >> lpy)) * tiles_n + col0(x) + lc;
    }
    // block of global ticket q: partitions interleaved claim by claim.  With
    // column bands every partition is the same size (the host checks); with
    // whole rows all but the last rem are.
    __device__ __forceinline__ uint32_t ticket(uint32_t q) const {
        if (lpy != 0) return tile(q % nx, q / nx);
        const uint32_t base = nx * rows_min * tiles_n;
        if (q < base) return tile(q % nx, q / nx);
        const uint32_t q2 = q - base;
        return tile(q2 % rem, rows_min * tiles_n + q2 / rem);
    }
};

// py (a power of two) must divide nx, and for py > 1 the chunk columns
// (tiles_n / tpc, whole) must number at least py; the host checks both.
__device__ __forceinline__ Parts make_parts(uint32_t nx, uint32_t py, uint32_t tiles_m, uint32_t tiles_n,
                                            uint32_t tpc, uint32_t group_m) {
    Parts p;
    p.nx = nx;
    p.lpy = py > 1 ? 31u - (uint32_t)__builtin_clz(py) : 0u;
    p.px = nx >> p.lpy;
    p.rows_min = tiles_m / p.px;
    p.rem = tiles_m % p.px;
    const uint32_t cch = py > 1 ? tiles_n / tpc : 0;
    p.cch_min = cch >> p.lpy;
    p.crem = cch & (py - 1u);
    p.tiles_n = tiles_n;
    p.tpc = tpc;
    p.group_m = group_m;
    return p;
}

// ---------------------------------------------------------------------------
// GEMM tile on MFMA
//
// A [M,K] and B [K,N] (both row-major bf16) reach LDS by direct buffer-to-LDS
// loads (no register staging) into a ring of NS K-slabs (KB deep), so later
// slabs stream in while slab s is multiplied (see slab() for the schedule).
// The load instruction is issued from inline assembly: the compiler cannot
// yet tell which ring slot a direct-to-LDS load writes and would otherwise
// wait for every outstanding load before any LDS read; the ring's waits are
// explicit (wait_vmcnt) and each is followed by a workgroup barrier.
//
// LDS layout per slab, chosen for the 64-bank LDS of gfx950:
//   A: row m = 128 bytes (64 k), 16-byte chunk c stored at c ^ ((m >> 1) & 7);
//      a 32x16 MFMA operand is one ds_read_b128 per lane, 16 lanes of a
//      read touch 16 distinct bank groups.
//   B: row k = TN*2 bytes (n contiguous, as in memory), chunk c stored at
//      c ^ swz_b(k).  The MFMA wants 8 consecutive k of one column per lane;
//      two ds_read_b64_tr_b16 give that: in each 16-lane group, lane j points
//      at row kbase + j/4, columns nbase + 4(j%4) .. +3, and lane i receives
//      rows kbase .. kbase+3 of column nbase + i.
// The MFMA is fed (B, A), so lane l ends with row (l & 31) and columns
// 8g + 4(l >> 5) + 0..3 of every 32x32 block: the tile leaves as 16-byte
// stores.  The per-lane LDS and buffer offsets of the K loop are computed once
// per kernel; those of the edge checks and the epilogue, once per block.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) char lchar;
typedef __attribute__((address_space(3))) bf16x8 lbf16x8;
typedef __attribute__((address_space(3))) bf16x4 lbf16x4;

// buffer resource as four scalar words, for the inline-assembly load
__device__ __forceinline__ u32x4 make_desc(const void *base) {
    const uint64_t p = (uint64_t)base;
    return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p),
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xFFFFu),
                 kNumRecords, 0x00020000u};
}

// 16 bytes per lane from the buffer (byte offset voff) into LDS at
// lds_base + 16 * lane; an offset at or past kOOB writes zeros.
__device__ __forceinline__ void dma16(u32x4 desc, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(desc)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Instruction schedule of one K slab: the wave issues its NMF MFMAs one at a
// time and slips the NDS LDS reads of the next slab's operands in between,
// spread over the first three quarters of the MFMAs, so the reads complete
// under the matrix work instead of in front of it.
template <int I, int NMF, int NDS>
struct Interleave {
    static constexpr int kSpan = NMF * 3 / 4 > 0 ? NMF * 3 / 4 : NMF;
    static constexpr int kDs = I < kSpan ? ((I + 1) * NDS / kSpan - I * NDS / kSpan) : 0;
    static __device__ __forceinline__ void run() {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        if constexpr (kDs > 0) __builtin_amdgcn_sched_group_barrier(0x100, kDs, 0);   // LDS reads
        if constexpr (I + 1 < NMF) Interleave<I + 1, NMF, NDS>::run();
    }
};

template <int BM, int BN, int KB, int NS, int WGM, int WGN, int kStorePolicy>
struct Gemm {
    static constexpr int NWAVES = WGM * WGN;
    static constexpr int NT = 64 * NWAVES;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;   // wave tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;     // 32x32 blocks per wave
    static constexpr int KK = KB / 16;                     // MFMA k-steps per slab
    static constexpr int A_ROW = KB * 2;                   // bytes of one A row in LDS
    static constexpr int A_CHUNKS = KB / 8;                // 16-byte chunks per A row
    static constexpr int A_ROWS = 1024 / A_ROW;            // A rows per 1 KiB load
    static constexpr int LDS_A = BM * A_ROW, LDS_B = KB * BN * 2;
    static constexpr int STAGE = LDS_A + LDS_B;
    static constexpr int LDS_BYTES = NS * STAGE;
    static constexpr int A_INST = BM / A_ROWS / NWAVES;    // 1 KiB loads per wave per slab
    static constexpr int B_ROWS = 1024 / (BN * 2);         // B rows per 1 KiB load
    static constexpr int B_CHUNKS = BN / 8;                // 16-byte chunks per B row
    static constexpr int B_INST = KB / B_ROWS / NWAVES;
    static constexpr int L = A_INST + B_INST;              // loads per wave per slab
    static_assert(KB == 32 || KB == 64, "K slab");
    static_assert(BN >= 64 && BN <= 512 && B_ROWS >= 1, "block width");
    static_assert(FM >= 1 && FN >= 1 && A_INST >= 1 && B_INST >= 1, "block/wave shape");
    static_assert(BM % (A_ROWS * NWAVES) == 0 && KB % (B_ROWS * NWAVES) == 0, "load split");
    static_assert(STAGE < 65536, "in-slab offsets must fit the LDS immediate");
    static_assert(NS >= 2 && NS <= 4, "ring depth");
    static_assert(NS >= 3, "a fill needs a ring slot beside the two being read");

    // XOR swizzles of 16-byte chunks (conflict-free operand reads, see above)
    static __device__ __forceinline__ int swz_a(int row) {
        return A_CHUNKS == 8 ? (row >> 1) & 7 : (row >> 2) & 3;
    }
    static __device__ __forceinline__ int swz_b(int k) {
        return B_CHUNKS >= 16 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
    }

    // per-lane constants, computed once per kernel
    struct Lane {
        uint32_t a_dma[A_INST];     // (row*K + c*8)*2 inside the A slab
        uint32_t b_dma[B_INST];     // (row*N + c*8)*2 inside the B slab
        uint32_t a_frag[KK];        // LDS offset of this lane's A operand (fm = 0) per k-step
        uint32_t b_frag[FN];        // LDS offset of this lane's first B piece per fn
    };

    // row and column (in elements) of the piece load i of thread t carries
    static __device__ __forceinline__ int a_row(int i, int t = threadIdx.x) {
        return ((t >> 6) * A_INST + i) * A_ROWS + (t & 63) / A_CHUNKS;
    }
    static __device__ __forceinline__ int a_col(int i, int t = threadIdx.x) {
        return (((t & 63) % A_CHUNKS) ^ swz_a(a_row(i, t))) * 8;
    }
    static __device__ __forceinline__ int b_row(int i, int t = threadIdx.x) {
        return ((t >> 6) * B_INST + i) * B_ROWS + (t & 63) / B_CHUNKS;
    }
    static __device__ __forceinline__ int b_col(int i, int t = threadIdx.x) {
        return (((t & 63) % B_CHUNKS) ^ swz_b(b_row(i, t))) * 8;
    }

    static __device__ __forceinline__ void init_lane(Lane &ln, int64_t N, int64_t K) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int i = 0; i < A_INST; ++i) ln.a_dma[i] = (uint32_t)((a_row(i) * K + a_col(i)) * 2);
#pragma unroll
        for (int i = 0; i < B_INST; ++i) ln.b_dma[i] = (uint32_t)((b_row(i) * N + b_col(i)) * 2);
        const int wm = wave / WGN, wn = wave % WGN;
        const int m = wm * WTM + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int c = kk * 2 + (lane >> 5);
            ln.a_frag[kk] = m * A_ROW + ((c ^ swz_a(m)) << 4);
        }
        const int i = lane & 15;
        const int kl = 8 * (lane >> 5) + (i >> 2);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = wn * WTN + fn * 32 + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
            ln.b_frag[fn] = LDS_A + kl * (BN * 2) + (((n >> 3) ^ swz_b(kl)) << 4) + (n & 7) * 2;
        }
    }

    // loads of one K slab into the ring slot at LDS byte address `slot`
    static __device__ __forceinline__ void issue(const Lane &ln, uint32_t slot, const uint16_t *A,
                                                 const uint16_t *B, int64_t M, int64_t N, int64_t K,
                                                 int64_t m0, int64_t n0, int64_t k0, bool a_full,
                                                 bool b_full) {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const uint32_t s0 = __builtin_amdgcn_readfirstlane(slot);
        const uint32_t sa = s0 + wave * A_INST * 1024, sb = s0 + LDS_A + wave * B_INST * 1024;
        const u32x4 da = make_desc(A + m0 * K + k0), db = make_desc(B + k0 * N + n0);
        if (__builtin_amdgcn_readfirstlane((int)(a_full && b_full && k0 + KB <= K))) {
#pragma unroll
            for (int i = 0; i < A_INST; ++i) dma16(da, ln.a_dma[i], sa + i * 1024);
#pragma unroll
            for (int i = 0; i < B_INST; ++i) dma16(db, ln.b_dma[i], sb + i * 1024);
        } else {
            // edge block or last K slab: out-of-range pieces read as zeros.
            // The extents left are compared in 32 bits with the piece
            // coordinates, recomputed here from a thread index the compiler
            // cannot hoist: kept live across the task loop they would take
            // registers the GEMM needs.
            int t = threadIdx.x;
            asm volatile("" : "+v"(t));
            const int mr = (int)(M - m0 < BM ? M - m0 : BM), nr = (int)(N - n0 < BN ? N - n0 : BN);
            const int kr = (int)(K - k0 < KB ? K - k0 : KB);
#pragma unroll
            for (int i = 0; i < A_INST; ++i) {
                const bool ok = a_row(i, t) < mr && a_col(i, t) < kr;
                dma16(da, ok ? ln.a_dma[i] : kOOB, sa + i * 1024);
            }
#pragma unroll
            for (int i = 0; i < B_INST; ++i) {
                const bool ok = b_row(i, t) < kr && b_col(i, t) < nr;
                dma16(db, ok ? ln.b_dma[i] : kOOB, sb + i * 1024);
            }
        }
    }

    // Loads [j0, j1) (the A pieces, then the B pieces) of a K slab that lies
    // wholly inside A and B; j0 and j1 are constants once the caller's k-step
    // loop is unrolled, so the loads sit between that k-step's MFMAs.
    static __device__ __forceinline__ void issue_part(const Lane &ln, uint32_t slot, const uint16_t *A,
                                                      const uint16_t *B, int64_t N, int64_t K,
                                                      int64_t m0, int64_t n0, int64_t k0, int j0,
                                                      int j1) {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const uint32_t s0 = __builtin_amdgcn_readfirstlane(slot);
        const uint32_t sa = s0 + wave * A_INST * 1024, sb = s0 + LDS_A + wave * B_INST * 1024;
#pragma unroll
        for (int i = 0; i < A_INST; ++i)
            if (i >= j0 && i < j1) dma16(make_desc(A + m0 * K + k0), ln.a_dma[i], sa + i * 1024);
#pragma unroll
        for (int i = 0; i < B_INST; ++i)
            if (A_INST + i >= j0 && A_INST + i < j1)
                dma16(make_desc(B + k0 * N + n0), ln.b_dma[i], sb + i * 1024);
    }

    // this lane's MFMA operands for one 16-deep k-step
    struct KFrag {
        bf16x8 a[FM];
        bf16x8 b[FN];
    };

    static __device__ __forceinline__ void kfrags(KFrag &f, const Lane &ln, const lchar *st, int kk) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            f.a[fm] = *(const lbf16x8 *)(st + ln.a_frag[kk] + fm * 32 * A_ROW);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const lchar *p = st + ln.b_frag[fn] + kk * 16 * (BN * 2);
            const bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4 *)p);
            const bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4 *)(p + 4 * (BN * 2)));
            f.b[fn] = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }

    static __device__ __forceinline__ void kmfma(f32x16 (&acc)[FM][FN], const KFrag &f) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[fn], f.a[fm], acc[fm][fn], 0, 0, 0);
    }

    // wait until at most n slabs of this wave's loads are still in flight
    static __device__ __forceinline__ void wait_slabs(int n) {
        static_assert((NS - 1) * L < 64, "vmcnt range");
        if (n <= 0) wait_vmcnt<0>();
        else if (n == 1) wait_vmcnt<L>();
        else if (n == 2) wait_vmcnt<(NS >= 3 ? 2 * L : 0)>();
        else wait_vmcnt<(NS >= 4 ? 3 * L : 0)>();
    }

    static constexpr int NMF = FM * FN;         // MFMAs per k-step per wave
    static constexpr int NDS = FM + 2 * FN;     // LDS reads per k-step per wave

    // One K slab s whose k-step-0 operands are in f0.  Each k-step multiplies
    // from registers while the next k-step's operands come out of LDS.  Before
    // the last k-step (when slab s+1 exists, kNext) the workgroup waits for
    // slab s+1 to land; after that barrier no wave reads slab s any more.  The
    // last k-step overlaps the reads of slab s+1's first operands, which end
    // in f0.
    //
    // Blocks wholly inside A and B with K a multiple of KB (kFast) keep NS-1
    // slabs ahead: the loads of slab s+NS-1 go into the slot slab s-1 left
    // free, a share of them in each k-step of slab s but the last (kFill,
    // while that slab exists), between the MFMAs.  One CU moves about 64
    // bytes a clock from L2 into LDS, so a slab's loads take most of a slab's
    // MFMA time; issued in one burst they would hold every wave at the load
    // issue while the matrix cores idle.  Other blocks (edges, ragged K) keep
    // NS slabs ahead: slab s+NS goes into slab s's slot in one burst right
    // after the barrier, with range checks.
    template <bool kNext, bool kFill, bool kFast>
    static __device__ __forceinline__ void slab(const Lane &ln, int s, int S, KFrag &f0, KFrag &f1,
                                                f32x16 (&acc)[FM][FN], const uint16_t *A,
                                                const uint16_t *B, int64_t M, int64_t N, int64_t K,
                                                int64_t m0, int64_t n0, bool a_full, bool b_full,
                                                lchar *lds, uint32_t base) {
        static_assert(!kFill || (kFast && kNext), "fills belong to the steady state of fast blocks");
        const lchar *st = lds + (s % NS) * STAGE;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            KFrag &cur = (kk & 1) ? f1 : f0;
            KFrag &nxt = (kk & 1) ? f0 : f1;
            if (kk + 1 < KK) {
                kfrags(nxt, ln, st, kk + 1);
                if constexpr (kFill)
                    issue_part(ln, base + ((s + NS - 1) % NS) * STAGE, A, B, N, K, m0, n0,
                               (int64_t)(s + NS - 1) * KB, kk * L / (KK - 1), (kk + 1) * L / (KK - 1));
            } else if (kNext) {
                if constexpr (kFill) {
                    wait_vmcnt<(NS - 2) * L>();   // slab s+1 has landed, s+2 .. s+NS-1 may not
                } else {
                    // slabs issued past s+1: NS-2, fewer near the end of K
                    const int later = (S - 2 - s) < (NS - 2) ? (S - 2 - s) : (NS - 2);
                    wait_slabs(later);
                }
                __syncthreads();   // every wave's part of slab s+1 has landed; slab s is free
                if (!kFast && s + NS < S)
                    issue(ln, base + (s % NS) * STAGE, A, B, M, N, K, m0, n0, (int64_t)(s + NS) * KB,
                          a_full, b_full);
                kfrags(nxt, ln, lds + ((s + 1) % NS) * STAGE, 0);
            }
            kmfma(acc, cur);
            if (kk + 1 < KK || kNext) Interleave<0, NMF, NDS>::run();
        }
    }

    // the K loop of one block (see slab())
    template <bool kFast>
    static __device__ __forceinline__ void kloop(const Lane &ln, f32x16 (&acc)[FM][FN], const uint16_t *A,
                                                 const uint16_t *B, int64_t M, int64_t N, int64_t K,
                                                 int64_t m0, int64_t n0, bool a_full, bool b_full,
                                                 lchar *lds, uint32_t base) {
        const int S = (int)((K + KB - 1) / KB);
        const int ahead = NS - (int)kFast;   // slabs the prologue issues
        const int pre = S < ahead ? S : ahead;
        for (int s = 0; s < pre; ++s)
            issue(ln, base + s * STAGE, A, B, M, N, K, m0, n0, (int64_t)s * KB, a_full, b_full);
        if (S <= 0) return;
        wait_slabs(pre - 1);
        __syncthreads();
        KFrag f0, f1;
        kfrags(f0, ln, lds, 0);
        int s = 0;
        if constexpr (kFast)
            for (; s + NS - 1 < S; ++s)
                slab<true, true, true>(ln, s, S, f0, f1, acc, A, B, M, N, K, m0, n0, a_full, b_full, lds, base);
        for (; s + 1 < S; ++s)
            slab<true, false, kFast>(ln, s, S, f0, f1, acc, A, B, M, N, K, m0, n0, a_full, b_full, lds, base);
        slab<false, false, kFast>(ln, S - 1, S, f0, f1, acc, A, B, M, N, K, m0, n0, a_full, b_full, lds, base);
    }

    // Whole block at rows m0.., columns n0..: C = A[rows, :] . B[:, cols] in
    // fp32.  `hook()` runs once the block's stores are issued (not drained).
    template <class Hook>
    static __device__ __forceinline__ void block(const Lane &ln, const uint16_t *A, const uint16_t *B,
                                                 float *C, int64_t M, int64_t N, int64_t K, int64_t m0,
                                                 int64_t n0, lchar *lds, Hook &&hook) {
        const bool a_full = m0 + BM <= M, b_full = n0 + BN <= N;
        const uint32_t base = (uint32_t)(uintptr_t)lds;
        f32x16 acc[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[fm][fn][i] = 0.0f;

        // Nothing of the caller's may still be in flight here: a returned
        // value the compiler has not yet waited for would make it wait for
        // every outstanding load (vmcnt(0)) inside the slab loop, draining
        // the operand ring each slab.
        drain_vmem();
        if (__builtin_amdgcn_readfirstlane((int)(a_full && b_full && K % KB == 0)))
            kloop<true>(ln, acc, A, B, M, N, K, m0, n0, a_full, b_full, lds, base);
        else
            kloop<false>(ln, acc, A, B, M, N, K, m0, n0, a_full, b_full, lds, base);
        // the ring is refilled by the next block only after every wave is done with it
        __syncthreads();

        // epilogue: 16-byte stores; rows >= M and columns >= N masked by an
        // out-of-range offset.  Offsets and the extents left are 32-bit (a
        // block lies within the buffer's 32-bit range), from a thread index
        // the compiler cannot hoist: kept live across the task loop, the
        // per-lane columns would take registers the K loop needs.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wave = tid >> 6;
        const int wm = wave / WGN, wn = wave % WGN;
        const int mr = (int)(M - m0 < BM ? M - m0 : BM), nr = (int)(N - n0 < BN ? N - n0 : BN);
        const uint32_t pitch = (uint32_t)N;
        const auto rc = scalar_rsrc(C + m0 * N + n0);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int r = wm * WTM + fm * 32 + (lane & 31);
            const bool row_ok = r < mr;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int cc = wn * WTN + fn * 32 + 8 * g + 4 * (lane >> 5);
                    const bool ok = row_ok && cc < nr;
                    const uint32_t off = ok ? ((uint32_t)r * pitch + (uint32_t)cc) * 4u : kOOB;
                    f32x4 v{acc[fm][fn][4 * g + 0], acc[fm][fn][4 * g + 1], acc[fm][fn][4 * g + 2],
                            acc[fm][fn][4 * g + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, kStorePolicy);
                }
            }
        }
        hook();
    }
};

// Compute blocks per tile shape.  One MI355X CU fetches operands at a bounded
// rate, so a compute task covers TPB output tiles side by side (one block of
// BM x (TPB*TN)) when that lowers the operand bytes per flop: two 128-wide
// tiles share their A rows.  WPC workgroups share one CU (LDS and registers
// sized for it); one per CU measured best for every shape here (a second
// workgroup per CU slowed both the GEMM and the fused schedule).
template <int TM, int TN> struct TileCfg;
template <> struct TileCfg<64, 64> {
    static constexpr int TPB = 1, KB = 64, NS = 4, WGM = 2, WGN = 2, WPC = 1;
};
template <> struct TileCfg<128, 128> {
    static constexpr int TPB = 2, KB = 64, NS = 3, WGM = 2, WGN = 2, WPC = 1;
};
template <> struct TileCfg<256, 128> {
    static constexpr int TPB = 2, KB = 32, NS = 4, WGM = 4, WGN = 2, WPC = 1;
};

template <int TM, int TN, int kStorePolicy>
using GemmFor = Gemm<TM, TN * TileCfg<TM, TN>::TPB, TileCfg<TM, TN>::KB, TileCfg<TM, TN>::NS,
                     TileCfg<TM, TN>::WGM, TileCfg<TM, TN>::WGN, kStorePolicy>;

// ---------------------------------------------------------------------------
// tile reduce: C[tile] = C[tile] (the local partial) + sum_p peers[p][tile]
//
// Each lane owns one float4 column of a strip of rows.  The tile is walked in
// groups of U row passes; a group's loads (the partial and every peer) are
// all issued before its first add, and the loads of group g+1 are issued
// before group g is summed, so two groups stay in flight.  Per-tile uniform buffer bases keep lane offsets in 32
// bits; ragged tiles use out-of-range offsets.
// ---------------------------------------------------------------------------
// Loads of one group per lane: KIB KiB per workgroup, and two groups are in
// flight.  Sharing the fabric with the GEMM and the other reducers, a
// reducer streams at a rate that follows its bytes in flight: the XCD-local
// fused kernel takes 128 KiB groups (256 KiB in flight), the other 64 KiB
// groups, as many as its registers hold without spilling.
template <int PP, int NT, int KIB>
struct ReducePlan {
    static constexpr int kLoads = KIB * 64 / NT;   // float4 per lane
    static constexpr int U = (kLoads / (PP + 1)) >= 16 ? 16
                           : (kLoads / (PP + 1)) >= 8 ? 8
                           : (kLoads / (PP + 1)) >= 4 ? 4
                           : (kLoads / (PP + 1)) >= 2 ? 2 : 1;
};

template <int TM, int BW, int NT>
struct ReduceGeom {
    static constexpr int C4 = BW / 4;              // float4 per row of the region
    static constexpr int RP = NT / C4;             // rows per pass
    static constexpr int PASSES = TM / RP;
    static_assert(NT % C4 == 0 && TM % RP == 0, "reduce layout");
};

// one group of U row passes: the partial and PP peers per pass, in registers
template <int PP, int U>
struct ReduceGroup {
    f32x4 v[PP + 1][U];
    uint32_t off[U];
};

// Region of TM rows x BW columns at (m0, n0): the tiles of one compute block.
// Rows past M are masked; peer p's partial starts p*MN elements into peers.
// `issued()` runs once the first group's loads are in flight (before them
// for the tallest tiles).
template <int TM, int BW, int NT, int PP, int kLoadPol, int kStorePol, int KIB, class Issued>
__device__ __forceinline__ void reduce_tile_pp(const float *__restrict__ peers, float *__restrict__ C,
                                               int64_t M, int64_t N, int64_t MN, int P, int64_t m0,
                                               int64_t n0, Issued &&issued) {
    using RG = ReduceGeom<TM, BW, NT>;
    constexpr int PB = 8;                   // peer block when PP is the generic 0
    constexpr int UP = ReducePlan<(PP > 0 ? PP : PB), NT, KIB>::U;
    constexpr int U = UP < RG::PASSES ? UP : RG::PASSES;
    constexpr int G = RG::PASSES / U;
    static_assert(RG::PASSES % U == 0, "reduce layout");
    const int tid = threadIdx.x;
    const int64_t base = m0 * N + n0;
    const int cc = (tid % RG::C4) * 4;
    const int r0 = tid / RG::C4;
    // rows and columns of the region inside the output, compared in 32 bits
    // (uniform per task; 64-bit per-lane bounds would hold register pairs
    // across the whole load pipeline)
    const int mr = (int)(M - m0 < TM ? M - m0 : TM);
    const int nr = (int)(N - n0 < BW ? N - n0 : BW);
    const bool col_ok = cc < nr;

    if constexpr (PP > 0) {
        // one peer's buffer resource at a time: a resource per peer held
        // across the tile would crowd out the scalar registers
        auto load = [&](ReduceGroup<PP, U> &g, int gi) {
            const auto rc = scalar_rsrc(C + base);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = (gi * U + u) * RG::RP + r0;
                g.off[u] = ((int)col_ok & (int)(r < mr)) ? (uint32_t)((r * N + cc) * 4) : kOOB;
                g.v[0][u] = __builtin_amdgcn_raw_buffer_load_b128(rc, g.off[u], 0, kLoadPol);
            }
#pragma unroll
            for (int q = 0; q < PP; ++q) {
                const auto rq = scalar_rsrc(peers + q * MN + base);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    g.v[q + 1][u] = __builtin_amdgcn_raw_buffer_load_b128(rq, g.off[u], 0, kPolicyStream);
            }
        };
        auto sum_store = [&](const ReduceGroup<PP, U> &g) {
            const auto rc = scalar_rsrc(C + base);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                f32x4 acc = g.v[0][u];
#pragma unroll
                for (int q = 0; q < PP; ++q) acc += g.v[q + 1][u];
                __builtin_amdgcn_raw_buffer_store_b128(acc, rc, g.off[u], 0, kStorePol);
            }
        };
        ReduceGroup<PP, U> g0, g1;
        // Tall tiles (eight waves, every register taken by the GEMM) read the
        // caller's returns before the first loads: held across them, the
        // compiler spilled to scratch inside the load pipeline.
        constexpr bool kFirst = TM >= 256;
        if constexpr (kFirst) issued();
        load(g0, 0);
        if constexpr (!kFirst) issued();
#pragma unroll
        for (int gi = 0; gi < G; gi += 2) {
            if (gi + 1 < G) load(g1, gi + 1);
            sum_store(g0);
            if (gi + 1 < G) {
                if (gi + 2 < G) load(g0, gi + 2);
                sum_store(g1);
            }
        }
    } else {
        // generic peer count: one group at a time, peers in blocks of PB
        bool first = true;
        for (int gi = 0; gi < G; ++gi) {
            const auto rc = scalar_rsrc(C + base);
            f32x4 acc[U];
            uint32_t off[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = (gi * U + u) * RG::RP + r0;
                off[u] = ((int)col_ok & (int)(r < mr)) ? (uint32_t)((r * N + cc) * 4) : kOOB;
                acc[u] = __builtin_amdgcn_raw_buffer_load_b128(rc, off[u], 0, kLoadPol);
            }
            if (first) {
                issued();
                first = false;
            }
            int p = 0;
            for (; p + PB <= P; p += PB) {
                f32x4 v[PB][U];
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    const auto rq = scalar_rsrc(peers + (p + q) * MN + base);
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[q][u] = __builtin_amdgcn_raw_buffer_load_b128(rq, off[u], 0, kPolicyStream);
                }
#pragma unroll
                for (int q = 0; q < PB; ++q)
#pragma unroll
                    for (int u = 0; u < U; ++u) acc[u] += v[q][u];
            }
            for (; p < P; ++p) {
                const auto rq = scalar_rsrc(peers + p * MN + base);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    acc[u] += __builtin_amdgcn_raw_buffer_load_b128(rq, off[u], 0, kPolicyStream);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                __builtin_amdgcn_raw_buffer_store_b128(acc[u], rc, off[u], 0, kStorePol);
        }
    }
}

// Dispatch on the peer count: the R-1 of 2, 4, 8 and 16 ranks get straight-line
// pipelined code; other counts take the blocked loop.
template <int TM, int BW, int NT, int kLoadPol, int kStorePol, int KIB, class Issued>
__device__ __forceinline__ void reduce_tile(const float *__restrict__ peers, float *__restrict__ C,
                                            int64_t M, int64_t N, int64_t MN, int P, int64_t m0, int64_t n0,
                                            Issued &&issued) {
    switch (P) {
#define MK_REDUCE_CASE(k) \
    case k: reduce_tile_pp<TM, BW, NT, k, kLoadPol, kStorePol, KIB>(peers, C, M, N, MN, P, m0, n0, issued); break;
        MK_REDUCE_CASE(1) MK_REDUCE_CASE(3) MK_REDUCE_CASE(7) MK_REDUCE_CASE(15)
#undef MK_REDUCE_CASE
        default: reduce_tile_pp<TM, BW, NT, 0, kLoadPol, kStorePol, KIB>(peers, C, M, N, MN, P, m0, n0, issued); break;
    }
}

// the owner-map mark of a task taken by a workgroup of the other role
constexpr uint32_t kHelp = 1u << 15;   // bit 31 of the owner word

__device__ __forceinline__ void note_violation(Live *L) {
    add_relaxed(&L->violations, 1u);
    __hip_atomic_fetch_or(&L->sticky, kStickyProtocol, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The last workgroup out: copy the control block to the snapshot and restore
// the initial values for the next launch.  Every field is loaded before the
// first store, so the device-scope loads are in flight together; the snapshot
// may alias nothing here, but the compiler cannot know that, and interleaved
// load/store pairs serialised into one round trip per field (about 10 us).
__device__ inline void finish_launch(const FusedArgs &a, Live *L) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    uint32_t cc[kMaxXcd], rc[kMaxXcd];
#pragma unroll
    for (int x = 0; x < kMaxXcd; ++x) {
        cc[x] = ld_relaxed(&L->compute_claim[x].v);
        rc[x] = ld_relaxed(&L->reduce_claim[x].v);
    }
    const uint32_t raw = ld_relaxed(&L->target_ns.v);
    const uint32_t exits = ld_relaxed(&L->exit_count);
    const uint32_t switches = ld_relaxed(&L->role_switches);
    const uint32_t released = ld_relaxed(&L->chunks_released.v);
    const uint32_t violations = ld_relaxed(&L->violations);
    const uint32_t error = ld_relaxed(&L->error);
    const uint32_t sticky = ld_relaxed(&L->sticky);
    const uint32_t ns_min = ld_relaxed(&L->ns_min);
    const uint32_t ns_max = ld_relaxed(&L->ns_max);
    const uint32_t trace_len = ld_relaxed(&L->trace_len);
    const uint64_t role_c = ld_relaxed(&L->role_compute.v);
    const uint64_t role_r = ld_relaxed(&L->role_reduce.v);
    const uint64_t t_start = ld_relaxed(&L->t_start);
    const uint64_t t_end = ld_relaxed(&L->t_end);
    const uint64_t r_start = ld_relaxed(&L->r_start);
    const uint64_t r_end = ld_relaxed(&L->r_end);

    Live *S = a.ws.snap;
#pragma unroll
    for (int x = 0; x < kMaxXcd; ++x) {
        S->compute_claim[x].v = cc[x];
        S->reduce_claim[x].v = rc[x];
    }
    S->exit_count = exits;
    S->target_ns.v = raw;
    S->role_switches = switches;
    S->chunks_released.v = released;
    S->violations = violations;
    S->error = error;
    S->sticky = sticky;   // L->sticky itself stays: errors of every launch are kept
    S->ns_min = ns_min;
    S->ns_max = ns_max;
    S->trace_len = trace_len;
    S->ns_final = a.mode == kAdaptive ? (raw ? raw : (uint32_t)a.ns_init) : (uint32_t)a.ns_init;
    S->role_compute.v = role_c;
    S->role_reduce.v = role_r;
    S->t_start = t_start;
    S->t_end = t_end;
    S->r_start = r_start;
    S->r_end = r_end;

#pragma unroll
    for (int x = 0; x < kMaxXcd; ++x) {
        st_relaxed(&L->compute_claim[x].v, 0u);
        st_relaxed(&L->reduce_claim[x].v, 0u);
    }
#pragma unroll
    for (int x = 0; x < kMaxXcd; ++x) st_relaxed(&L->extra_claim[x].v, 0u);
    st_relaxed(&L->target_ns.v, 0u);
    st_relaxed(&L->role_switches, 0u);
    st_relaxed(&L->chunks_released.v, 0u);
    st_relaxed(&L->violations, 0u);
    st_relaxed(&L->error, 0u);
    st_relaxed(&L->ns_min, 0xFFFFFFFFu);
    st_relaxed(&L->ns_max, 0u);
    st_relaxed(&L->trace_len, 0u);
    st_relaxed(&L->role_compute.v, (uint64_t)0);
    st_relaxed(&L->role_reduce.v, (uint64_t)0);
    st_relaxed(&L->t_start, ~(uint64_t)0);
    st_relaxed(&L->t_end, (uint64_t)0);
    st_relaxed(&L->r_start, ~(uint64_t)0);
    st_relaxed(&L->r_end, (uint64_t)0);
    // exit_count last: nothing touches the block after this
    st_relaxed(&L->exit_count, 0u);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

// static LDS of the fused kernel: at least the GEMM ring, and more than
// 160 KiB / (WPC + 1), so exactly WPC workgroups fit on a CU
template <int TM, int TN>
constexpr int fused_lds_bytes() {
    using G = GemmFor<TM, TN, kPolicyDefault>;
    constexpr int floor_bytes = (160 * 1024) / (TileCfg<TM, TN>::WPC + 1) + 1024;
    return G::LDS_BYTES > floor_bytes ? G::LDS_BYTES : floor_bytes;
}

}  // namespace mk
