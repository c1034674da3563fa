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
//    release/acquire fences (see "buffer access" below).
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
__device__ uint32_t controller_update_totals(uint32_t B, uint32_t T_p, uint32_t T_s, uint32_t compute_done,
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

__device__ uint32_t controller_update(uint32_t B, uint32_t T, uint32_t compute_done,
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
constexpr uint32_t kHelp = 1u << 15;   // bit 31 of the owner word

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

__device__ __forceinline__ void note_violation(Live *L) {
    add_relaxed(&L->violations, 1u);
    __hip_atomic_fetch_or(&L->sticky, kStickyProtocol, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// The last workgroup out: copy the control block to the snapshot and restore
// the initial values for the next launch.  Every field is loaded before the
// first store, so the device-scope loads are in flight together; the snapshot
// may alias nothing here, but the compiler cannot know that, and interleaved
// load/store pairs serialised into one round trip per field (about 10 us).
__device__ void finish_launch(const FusedArgs &a, Live *L) {
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

// static LDS of the fused kernel: at least the GEMM ring, and more than
// 160 KiB / (WPC + 1), so exactly WPC workgroups fit on a CU
template <int TM, int TN>
constexpr int fused_lds_bytes() {
    using G = GemmFor<TM, TN, kPolicyDefault>;
    constexpr int floor_bytes = (160 * 1024) / (TileCfg<TM, TN>::WPC + 1) + 1024;
    return G::LDS_BYTES > floor_bytes ? G::LDS_BYTES : floor_bytes;
}

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
// role stands in for their transfer: a copy task moves one chunk (one tile
// row of A: TM rows x K) into the gathered A, stores it write-through, and
// publishes the chunk's arrival flag once the stores have drained.  A compute
// task is one block of TPB adjacent tiles of one tile row; tiles of this
// rank's own rows read the local shard at once, the others read the gathered
// A once their chunk's flag carries the launch's epoch.  Claims: copy tasks
// take the other ranks' chunks first (rank, then row), this rank's own last;
// compute blocks go in row-major order, so this rank's rows come first and
// the others follow in the order they are copied.  Roles follow the
// workgroup index against the target (copy iff w < target), re-read at
// every task boundary.
// ---------------------------------------------------------------------------

enum AgRole : int { kAgCompute = 0, kAgCopy = 1, kAgExit = 2 };

struct AgDecision {
    int role;
    uint32_t unit;      // compute: block; copy: chunk
    uint32_t ns_seen;   // copy target the task was taken under | kHelp (copy by a waiting compute workgroup)
};

struct AgSched {
    uint32_t target;
    uint32_t det_i;
    bool copy_exhausted, compute_exhausted;
    bool have_block;        // a claimed compute block waiting for its input
    uint32_t block, block_ns;
    int last_role;
};

__device__ __forceinline__ uint32_t ag_copy_chunk(const AgArgs &a, uint32_t q) {
    const uint32_t peer_chunks = a.Ch - a.cps;
    return q < peer_chunks ? a.cps + q : q - peer_chunks;
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

// Thread 0: the next task.
__device__ AgDecision ag_next(const AgArgs &a, Live *L, uint32_t wg, AgSched &s) {
    const uint32_t B = (uint32_t)a.nwg;
    if (a.mode == kDeterministic) {
        const uint32_t ns = (uint32_t)a.ns_init;
        if (wg < ns) {
            const uint32_t q = wg + s.det_i * ns;
            if (q >= a.Ch) return {kAgExit, 0, ns};
            ++s.det_i;
            return {kAgCopy, ag_copy_chunk(a, q), ns};
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
                if (q < a.Ch) return {kAgCopy, ag_copy_chunk(a, q), ns | kHelp};
                s.copy_exhausted = true;
            }
            if (!ag_wait(a, L, row)) return {kAgExit, 0, ns};
            s.have_block = false;
            return {kAgCompute, s.block, s.block_ns};
        }
        const bool copy_role = wg < ns;
        if (copy_role && !s.copy_exhausted) {
            const uint32_t q = add_relaxed(&L->compute_claim[1].v, 1u);
            if (q < a.Ch) return {kAgCopy, ag_copy_chunk(a, q), ns};
            s.copy_exhausted = true;
        }
        // static copiers leave once every chunk is claimed
        if (copy_role && a.mode != kAdaptive) return {kAgExit, 0, ns};
        if (!s.compute_exhausted) {
            const uint32_t j = add_relaxed(&L->compute_claim[0].v, 1u);
            if (j < a.TB) {
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
            if (q < a.Ch) return {kAgCopy, ag_copy_chunk(a, q), copy_role ? ns : B};
            s.copy_exhausted = true;
        }
        return {kAgExit, 0, ns};
    }
}

// one chunk: TM rows x K of a shard into the gathered A.  Source read once
// (nt); destination written through (nt sc1), visible at device scope once
// the stores have drained.
template <int NT, int TM>
__device__ __forceinline__ void ag_copy(const AgArgs &a, uint32_t c) {
    const uint32_t r = c / a.cps, lr = c % a.cps;
    const uint16_t *src = r == 0 ? a.A_local + (int64_t)lr * TM * a.K
                                 : a.A_peers + ((int64_t)(r - 1) * a.Ms + (int64_t)lr * TM) * a.K;
    uint16_t *dst = a.A_gath + (int64_t)c * TM * a.K;
    const auto rs = scalar_rsrc(src);
    const auto rd = scalar_rsrc(dst);
    const uint32_t n16 = (uint32_t)(TM * a.K / 8);   // 16-byte pieces of the chunk
    constexpr int U = 8;
    uint32_t i = threadIdx.x;
    for (; i + (U - 1) * NT < n16; i += U * NT) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (i + u * NT) * 16u, 0,
                                                                                   kPolicyStream));
#pragma unroll
        for (int u = 0; u < U; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(f32x4, v[u]), rd, (i + u * NT) * 16u, 0,
                                                   kPolicyCoherentStream);
    }
    for (; i < n16; i += NT) {
        const f32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, i * 16u, 0, kPolicyStream);
        __builtin_amdgcn_raw_buffer_store_b128(v, rd, i * 16u, 0, kPolicyCoherentStream);
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
            if (d.role == kAgCopy) {
                const uint32_t c = d.unit;
                if ((int64_t)c != a.skip_publish) st_relaxed(&a.ws.chunk_flag[c], a.epoch);
                const uint32_t old = add_relaxed(&a.ws.chunk_cnt[c], 1u);
                if (old != a.calls - 1) note_violation(L);
                a.ws.rowner[c] = (d.ns_seen << 16) | wg;
                a.ws.timeline[2u * a.Tcap + c] = (uint32_t)sh_r0;
                a.ws.timeline[3u * a.Tcap + c] = t_end;
                add_relaxed(&L->chunks_released.v, 1u);
            } else {
                for (uint32_t k = 0; k < nt; ++k) {
                    const uint32_t t = t0 + k;
                    const uint32_t old = add_relaxed(&a.ws.tile_cnt[t], 1u);
                    if (old != a.calls - 1) note_violation(L);
                    a.ws.cowner[t] = (d.ns_seen << 16) | wg;
                    a.ws.timeline[t] = (uint32_t)sh_r0;
                    a.ws.timeline[a.Tcap + t] = t_end;
                }
            }
            // progress words, and one controller step: the copy role is the
            // communication role s (chunks), compute is p (tiles)
            const bool copying = d.role == kAgCopy;
            const uint64_t inc = (dt << kCountBits) | (copying ? 1u : nt);
            const uint64_t mine = add_relaxed(copying ? &L->role_reduce.v : &L->role_compute.v, inc) + inc;
            const uint64_t other = ld_relaxed(copying ? &L->role_compute.v : &L->role_reduce.v);
            if (copying) {
                min_relaxed(&L->r_start, (uint64_t)sh_r0);
                max_relaxed(&L->r_end, ticks_now());
            }
            if (a.mode == kAdaptive) {
                const uint64_t cw = copying ? other : mine, sw = copying ? mine : other;
                const uint32_t raw = ld_relaxed(&L->target_ns.v);
                const uint32_t cur = raw ? raw : (uint32_t)a.ns_init;
                const uint32_t n = controller_update_totals(
                    (uint32_t)a.nwg, a.T, a.Ch, (uint32_t)(cw & kCountMask), (uint32_t)(sw & kCountMask),
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
