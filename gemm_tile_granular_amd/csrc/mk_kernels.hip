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
// (coherent at device scope) and read back with sc0|sc1 (bypassing the CU's
// L1, coherent at device scope); the writer drains its stores (vmcnt) before
// the flag is set.  This replaces agent-scope release/acquire fences, whose
// whole-L2 writeback and invalidate per tile cost 2-3x in reduce bandwidth.
// Buffer resources also give branch-free edge masking: an offset at or past
// kOOB reads zero and drops the store.
// ---------------------------------------------------------------------------

constexpr int kPolicyDefault = 0;
constexpr int kPolicyStream = 2;            // nt: read-once / write-once data
constexpr int kPolicyCoherentStore = 16;    // sc1: visible at device scope
constexpr int kPolicyCoherentLoad = 17;     // sc0 sc1: bypass L1, device-coherent
constexpr int kPolicyCoherentStream = 18;   // nt sc1
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint32_t kNumRecords = 0x7FFFFFFFu;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, kNumRecords, 0x00020000);
}

// Wait until every vector memory operation of this wave has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left unconstrained).
__device__ __forceinline__ void drain_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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
template <class T> __device__ __forceinline__ T add_acq_rel(T *p, T v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
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
// clamp to [min(floor, B-1), B-1] while compute remains; B once it is done.
// Limits B <= 1024, T < 2^22 and C_x <= 2^26-1 keep every product exact.
// ---------------------------------------------------------------------------
__device__ uint32_t controller_update(uint32_t B, uint32_t T, uint32_t compute_done,
                                      uint32_t reduce_done, uint64_t sum_p, uint64_t sum_s,
                                      uint32_t current, uint32_t floor) {
    const uint32_t R_p = T - compute_done;
    const uint32_t R_s = T - reduce_done;
    if (R_p == 0) return B;
    const uint32_t hi = B - 1;
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
// w mod 8.  Tile rows are dealt to nx partitions (row r -> partition r mod nx,
// so chunks stay whole); workgroups claim compute tiles from their own XCD's
// partition first, in the banded order above, so the tiles one L2 serves at
// once share A rows and B columns, and steal from the other partitions when
// theirs is done.  Reduce tickets walk the partitions round-robin, which is
// the order in which tiles complete when the partitions progress together.
// ---------------------------------------------------------------------------
struct Parts {
    uint32_t nx;        // partitions (1 or the XCD count)
    uint32_t rows_min;  // tile rows in the smaller partitions
    uint32_t rem;       // partitions [0, rem) hold one more tile row
    uint32_t tiles_n, tiles_m, tpc, group_m;

    __device__ __forceinline__ uint32_t rows(uint32_t x) const { return rows_min + (x < rem ? 1u : 0u); }
    __device__ __forceinline__ uint32_t size(uint32_t x) const { return rows(x) * tiles_n; }
    // tile of the i-th claim of partition x
    __device__ __forceinline__ uint32_t tile(uint32_t x, uint32_t i) const {
        const uint32_t local = tile_of_claim(i, rows(x), tiles_n, tpc, group_m);
        const uint32_t lr = local / tiles_n, col = local % tiles_n;
        return (lr * nx + x) * tiles_n + col;
    }
    // tile of global ticket q: partitions interleaved claim by claim
    __device__ __forceinline__ uint32_t ticket(uint32_t q) const {
        const uint32_t base = nx * rows_min * tiles_n;
        if (q < base) return tile(q % nx, q / nx);
        const uint32_t q2 = q - base;
        return tile(q2 % rem, rows_min * tiles_n + q2 / rem);
    }
};

__device__ __forceinline__ Parts make_parts(uint32_t nx, uint32_t tiles_m, uint32_t tiles_n,
                                            uint32_t tpc, uint32_t group_m) {
    Parts p;
    p.nx = nx;
    p.rows_min = tiles_m / nx;
    p.rem = tiles_m % nx;
    p.tiles_n = tiles_n;
    p.tiles_m = tiles_m;
    p.tpc = tpc;
    p.group_m = group_m;
    return p;
}

// ---------------------------------------------------------------------------
// GEMM tile on MFMA
//
// A [M,K] and B [K,N] (both row-major bf16) reach LDS by direct buffer-to-LDS
// loads (no register staging) into a ring of NS K-slabs of 64, so the loads
// for slab s+NS-1 are in flight while slab s is multiplied.  The load
// instruction is issued from inline assembly: the compiler cannot yet tell
// which ring slot a direct-to-LDS load writes and would otherwise wait for
// every outstanding load before any LDS read; the ring's waits are explicit
// (wait_vmcnt) and each is followed by a workgroup barrier.
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
// stores.  All per-lane LDS and buffer offsets are computed once per kernel.
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

template <int TM, int TN, int NS, int WGM, int WGN, int kStorePolicy>
struct Gemm {
    static constexpr int NWAVES = WGM * WGN;
    static constexpr int NT = 64 * NWAVES;
    static constexpr int WTM = TM / WGM, WTN = TN / WGN;   // wave tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;     // 32x32 blocks per wave
    static constexpr int LDS_A = TM * kBK * 2, LDS_B = kBK * TN * 2;
    static constexpr int STAGE = LDS_A + LDS_B;
    static constexpr int LDS_BYTES = NS * STAGE;
    static constexpr int A_INST = TM / 8 / NWAVES;          // 1 KiB loads per wave per slab
    static constexpr int B_ROWS = 1024 / (TN * 2);          // B rows per 1 KiB load
    static constexpr int B_CHUNKS = TN / 8;                 // 16-byte chunks per B row
    static constexpr int B_INST = kBK / B_ROWS / NWAVES;
    static constexpr int L = A_INST + B_INST;               // loads per wave per slab
    static_assert(FM >= 1 && FN >= 1 && A_INST >= 1 && B_INST >= 1, "tile/wave shape");
    static_assert(STAGE < 65536, "in-slab offsets must fit the LDS immediate");
    static_assert(NS >= 2 && NS <= 4, "ring depth");

    static __device__ __forceinline__ int swz_a(int row) { return (row >> 1) & 7; }
    static __device__ __forceinline__ int swz_b(int k) {
        return B_CHUNKS == 16 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
    }

    // per-lane constants, computed once per kernel
    struct Lane {
        uint32_t a_dma[A_INST];     // (row*K + c*8)*2 inside the A slab
        int a_row[A_INST];
        int a_col[A_INST];
        uint32_t b_dma[B_INST];     // (row*N + c*8)*2 inside the B slab
        int b_row[B_INST];
        int b_col[B_INST];
        uint32_t a_frag[kBK / 16];  // LDS offset of this lane's A operand (fm = 0) per k-step
        uint32_t b_frag[FN];        // LDS offset of this lane's first B piece per fn
    };

    static __device__ __forceinline__ void init_lane(Lane &ln, int64_t N, int64_t K) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int i = 0; i < A_INST; ++i) {
            const int row = (wave * A_INST + i) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swz_a(row);
            ln.a_row[i] = row;
            ln.a_col[i] = c * 8;
            ln.a_dma[i] = (uint32_t)((row * K + c * 8) * 2);
        }
#pragma unroll
        for (int i = 0; i < B_INST; ++i) {
            const int row = (wave * B_INST + i) * B_ROWS + lane / B_CHUNKS;
            const int c = (lane % B_CHUNKS) ^ swz_b(row);
            ln.b_row[i] = row;
            ln.b_col[i] = c * 8;
            ln.b_dma[i] = (uint32_t)((row * N + c * 8) * 2);
        }
        const int wm = wave / WGN, wn = wave % WGN;
        const int m = wm * WTM + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int c = kk * 2 + (lane >> 5);
            ln.a_frag[kk] = m * 128 + ((c ^ swz_a(m)) << 4);
        }
        const int i = lane & 15;
        const int kl = 8 * (lane >> 5) + (i >> 2);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = wn * WTN + fn * 32 + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
            ln.b_frag[fn] = LDS_A + kl * (TN * 2) + (((n >> 3) ^ swz_b(kl)) << 4) + (n & 7) * 2;
        }
    }

    // loads of one K slab into the ring slot at LDS byte address `slot`
    static __device__ __forceinline__ void issue(const Lane &ln, uint32_t slot, const uint16_t *A,
                                                 const uint16_t *B, int64_t M, int64_t N, int64_t K,
                                                 int64_t m0, int64_t n0, int64_t k0, bool a_full,
                                                 bool b_full) {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const uint32_t sa = __builtin_amdgcn_readfirstlane(slot), sb = sa + LDS_A;
        const u32x4 da = make_desc(A + m0 * K + k0), db = make_desc(B + k0 * N + n0);
        const bool k_full = k0 + kBK <= K;
#pragma unroll
        for (int i = 0; i < A_INST; ++i) {
            uint32_t off = ln.a_dma[i];
            if (!(a_full && k_full)) off = (m0 + ln.a_row[i] < M && k0 + ln.a_col[i] < K) ? off : kOOB;
            dma16(da, off, sa + (wave * A_INST + i) * 1024);
        }
#pragma unroll
        for (int i = 0; i < B_INST; ++i) {
            uint32_t off = ln.b_dma[i];
            if (!(b_full && k_full)) off = (k0 + ln.b_row[i] < K && n0 + ln.b_col[i] < N) ? off : kOOB;
            dma16(db, off, sb + (wave * B_INST + i) * 1024);
        }
    }

    struct Frag {
        bf16x8 a[FM];
        bf16x8 b[FN];
    };

    static __device__ __forceinline__ void frags(Frag &f, const Lane &ln, const lchar *st, int kk) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) f.a[fm] = *(const lbf16x8 *)(st + ln.a_frag[kk] + fm * 32 * 128);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const lchar *p = st + ln.b_frag[fn] + kk * 16 * (TN * 2);
            const bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4 *)p);
            const bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4 *)(p + 4 * (TN * 2)));
            f.b[fn] = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }

    static __device__ __forceinline__ void mfma(f32x16 (&acc)[FM][FN], const Frag &f) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[fn], f.a[fm], acc[fm][fn], 0, 0, 0);
    }

    // Whole output tile (ti, tj): C[tile] = A[rows, :] . B[:, cols] in fp32.
    static __device__ __forceinline__ void tile(const Lane &ln, const uint16_t *A, const uint16_t *B,
                                                float *C, int64_t M, int64_t N, int64_t K, int ti,
                                                int tj, lchar *lds) {
        const int64_t m0 = (int64_t)ti * TM, n0 = (int64_t)tj * TN;
        const bool a_full = m0 + TM <= M, b_full = n0 + TN <= N;
        const uint32_t base = (uint32_t)(uintptr_t)lds;
        f32x16 acc[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[fm][fn][i] = 0.0f;

        const int S = (int)((K + kBK - 1) / kBK);
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (s < S) issue(ln, base + s * STAGE, A, B, M, N, K, m0, n0, (int64_t)s * kBK, a_full, b_full);
        if (S > 0) {
            // slab 0 landed: up to NS-2 later slabs may still be loading
            if (NS >= 4 && S - 1 >= 2) wait_vmcnt<(NS >= 4 ? 2 * L : 0)>();
            else if (NS >= 3 && S - 1 >= 1) wait_vmcnt<(NS >= 3 ? L : 0)>();
            else wait_vmcnt<0>();
            __syncthreads();
            Frag cur, nxt;
            frags(cur, ln, lds, 0);
            int slot = 0;
            for (int s = 0; s < S; ++s) {
                const lchar *st = lds + slot * STAGE;
                const int nslot = slot + 1 == NS ? 0 : slot + 1;
#pragma unroll
                for (int kk = 0; kk < kBK / 16; ++kk) {
                    if (kk < kBK / 16 - 1) {
                        // operands of the next k-step load while this one multiplies
                        frags(nxt, ln, st, kk + 1);
                        mfma(acc, cur);
                    } else {
                        mfma(acc, cur);
                        if (s + 1 < S) {
                            // slab s+1 landed (NS-3 later slabs may still load) and every
                            // wave is past slab s-1, whose slot is refilled now
                            const int later = (S - 2 - s) < (NS - 3) ? (S - 2 - s) : (NS - 3);
                            if (NS >= 4 && later >= 1) wait_vmcnt<(NS >= 4 ? L : 0)>();
                            else wait_vmcnt<0>();
                            __syncthreads();
                            if (s + NS - 1 < S) {
                                const int fslot = slot == 0 ? NS - 1 : slot - 1;
                                issue(ln, base + fslot * STAGE, A, B, M, N, K, m0, n0,
                                      (int64_t)(s + NS - 1) * kBK, a_full, b_full);
                            }
                            frags(nxt, ln, lds + nslot * STAGE, 0);
                        }
                    }
                    cur = nxt;
                }
                slot = nslot;
            }
        }
        // the ring is refilled by the next tile only after every wave is done with it
        __syncthreads();

        // epilogue: 16-byte stores; rows >= M and columns >= N masked by an
        // out-of-range offset
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave / WGN, wn = wave % WGN;
        const auto rc = make_rsrc(C + m0 * N + n0);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int r = wm * WTM + fm * 32 + (lane & 31);
            const bool row_ok = m0 + r < M;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int cc = wn * WTN + fn * 32 + 8 * g + 4 * (lane >> 5);
                    const bool ok = row_ok && n0 + cc < N;
                    const uint32_t off = ok ? (uint32_t)((r * N + cc) * 4) : kOOB;
                    f32x4 v{acc[fm][fn][4 * g + 0], acc[fm][fn][4 * g + 1], acc[fm][fn][4 * g + 2],
                            acc[fm][fn][4 * g + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, kStorePolicy);
                }
            }
        }
    }
};

// Tile configurations: ring depth and wave grid per output tile.
template <int TM, int TN> struct TileCfg;
template <> struct TileCfg<64, 64> { static constexpr int NS = 4, WGM = 2, WGN = 2; };
template <> struct TileCfg<128, 128> { static constexpr int NS = 4, WGM = 2, WGN = 4; };
template <> struct TileCfg<256, 128> { static constexpr int NS = 3, WGM = 4, WGN = 2; };

template <int TM, int TN, int kStorePolicy>
using GemmFor = Gemm<TM, TN, TileCfg<TM, TN>::NS, TileCfg<TM, TN>::WGM, TileCfg<TM, TN>::WGN, kStorePolicy>;

// ---------------------------------------------------------------------------
// tile reduce: C[tile] = C[tile] (the local partial) + sum_p peers[p][tile]
//
// Each lane owns one float4 column of a strip of rows; U row passes are in
// flight together and every load of a pass group (the partial and all PP
// peers) is issued before the first add, so a 4-wave workgroup keeps
// (PP+1)*U 16-byte loads per lane outstanding.  Per-tile uniform buffer bases
// keep lane offsets in 32 bits.  Ragged tiles use out-of-range offsets.
// ---------------------------------------------------------------------------
// about 128 KiB of loads in flight per workgroup: 32 per lane with 4 waves,
// 16 per lane with 8
template <int PP, int NT>
struct ReducePlan {
    static constexpr int kLoads = 8192 / NT;   // target loads in flight per lane
    static constexpr int U = (kLoads / (PP + 1)) >= 16 ? 16
                           : (kLoads / (PP + 1)) >= 8 ? 8
                           : (kLoads / (PP + 1)) >= 4 ? 4
                           : (kLoads / (PP + 1)) >= 2 ? 2 : 1;
};

// PP > 0 peers starting at peers0 (compile-time count); accumulate into acc
template <int TM, int TN, int PP, int U>
__device__ __forceinline__ void add_peers(f32x4 (&acc)[U], const float *peers0, int64_t MN,
                                          int64_t base, const uint32_t (&off)[U]) {
    f32x4 v[PP][U];
#pragma unroll
    for (int q = 0; q < PP; ++q) {
        const auto rp = make_rsrc(peers0 + q * MN + base);
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[q][u] = __builtin_amdgcn_raw_buffer_load_b128(rp, off[u], 0, kPolicyStream);
    }
#pragma unroll
    for (int q = 0; q < PP; ++q)
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] += v[q][u];
}

template <int TM, int TN, int NT, int PP>
__device__ void reduce_tile_pp(const float *__restrict__ peers, float *__restrict__ C, int64_t M,
                               int64_t N, int P, int ti, int tj) {
    constexpr int C4 = TN / 4;              // float4 per tile row
    constexpr int RP = NT / C4;             // rows per pass
    constexpr int PASSES = TM / RP;
    constexpr int PB = 8;                   // peer block when PP is the generic 0
    constexpr int UP = ReducePlan<(PP > 0 ? PP : PB), NT>::U;
    constexpr int U = UP < PASSES ? UP : PASSES;
    static_assert(NT % C4 == 0 && TM % RP == 0 && PASSES % U == 0, "reduce layout");
    const int tid = threadIdx.x;
    const int64_t m0 = (int64_t)ti * TM, n0 = (int64_t)tj * TN;
    const int64_t base = m0 * N + n0;
    const int64_t MN = M * N;
    const int cc = (tid % C4) * 4;
    const int r0 = tid / C4;
    const bool col_ok = n0 + cc < N;
    const auto rc = make_rsrc(C + base);
    for (int ps = 0; ps < PASSES; ps += U) {
        f32x4 acc[U];
        uint32_t off[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = (ps + u) * RP + r0;
            off[u] = (col_ok && m0 + r < M) ? (uint32_t)((r * N + cc) * 4) : kOOB;
            acc[u] = __builtin_amdgcn_raw_buffer_load_b128(rc, off[u], 0, kPolicyCoherentLoad);
        }
        if constexpr (PP > 0) {
            add_peers<TM, TN, PP, U>(acc, peers, MN, base, off);
        } else {
            // generic peer count: blocks of PB, then one at a time
            int p = 0;
            for (; p + PB <= P; p += PB) add_peers<TM, TN, PB, U>(acc, peers + p * MN, MN, base, off);
            for (; p < P; ++p) add_peers<TM, TN, 1, U>(acc, peers + p * MN, MN, base, off);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(acc[u], rc, off[u], 0, kPolicyCoherentStream);
    }
}

// Dispatch on the peer count so that every load of a pass group is a
// straight-line instruction (counts above 16 take the blocked loop).
template <int TM, int TN, int NT>
__device__ void reduce_tile(const float *__restrict__ peers, float *__restrict__ C, int64_t M,
                            int64_t N, int P, int ti, int tj) {
    switch (P) {
#define MK_REDUCE_CASE(k) \
    case k: reduce_tile_pp<TM, TN, NT, k>(peers, C, M, N, P, ti, tj); break;
        MK_REDUCE_CASE(1) MK_REDUCE_CASE(2) MK_REDUCE_CASE(3) MK_REDUCE_CASE(4)
        MK_REDUCE_CASE(5) MK_REDUCE_CASE(6) MK_REDUCE_CASE(7) MK_REDUCE_CASE(8)
        MK_REDUCE_CASE(9) MK_REDUCE_CASE(10) MK_REDUCE_CASE(11) MK_REDUCE_CASE(12)
        MK_REDUCE_CASE(13) MK_REDUCE_CASE(14) MK_REDUCE_CASE(15) MK_REDUCE_CASE(16)
#undef MK_REDUCE_CASE
        default: reduce_tile_pp<TM, TN, NT, 0>(peers, C, M, N, P, ti, tj); break;
    }
}

// ---------------------------------------------------------------------------
// the persistent fused kernel
// ---------------------------------------------------------------------------

enum Role : int { kRoleCompute = 0, kRoleReduce = 1, kRoleExit = 2, kRoleNone = -1 };

struct Decision {
    int role;
    uint32_t tile;
    uint32_t ns_seen;   // reduce target the claim was made under (logged in owner maps)
};

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
    uint32_t early_flag_value;
};

__device__ __forceinline__ bool timed_out(const FusedArgs &a, Live *L, uint64_t since) {
    if (ticks_now() - since <= a.timeout_ticks) return false;
    __hip_atomic_fetch_max(&L->error, (uint32_t)kErrTimeout, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// Wait (bounded) until tile t carries this launch's epoch.  False on timeout or
// on an error raised by another workgroup.
__device__ bool wait_ready(const FusedArgs &a, Live *L, uint32_t t) {
    const uint64_t since = ticks_now();
    for (;;) {
        if (ld_relaxed(&a.ws.tile_flag[t]) == a.epoch) return true;
        if (ld_relaxed(&L->error) != kErrNone) return false;
        if (timed_out(a, L, since)) return false;
        __builtin_amdgcn_s_sleep(1);
    }
}

// Thread 0 only: the next task.  Roles follow the workgroup index against the
// current target and are re-read here, at every task boundary ("【学习】mKernel
// 分析" sections 2.4 and 4.1).  Claims are tickets from device-scope counters
// in one common order, so compute and reduce walk the tiles in step.  A claim
// taken ahead of time (prefetched during the previous task) is a commitment
// and is honoured first, so a role change takes effect one task later.
__device__ Decision next_task(const FusedArgs &a, const Parts &pt, Live *L, uint32_t wg, Sched &s) {
    const uint32_t B = (uint32_t)a.nwg, T = a.T;
    if (a.mode == kDeterministic) {
        const uint32_t ns = (uint32_t)a.ns_init;
        if (wg < ns) {
            const uint32_t t = wg + s.det_i * ns;
            if (t >= T) return {kRoleExit, 0, ns};
            if (!wait_ready(a, L, t)) return {kRoleExit, 0, ns};
            ++s.det_i;
            return {kRoleReduce, t, ns};
        }
        const uint32_t t = (wg - ns) + s.det_i * (B - ns);
        if (t >= T) return {kRoleExit, 0, ns};
        ++s.det_i;
        return {kRoleCompute, t, ns};
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
            if (q < T) {
                const uint32_t t = pt.ticket(q);
                if (!seen && !wait_ready(a, L, t)) return {kRoleExit, 0, ns_seen};
                return {kRoleReduce, t, ns_seen};
            }
            s.reduce_exhausted = true;
            continue;
        }
        const uint32_t ns = s.target;
        const bool compute_role = wg >= ns;
        if (compute_role && !s.compute_exhausted) {
            // own XCD's partition first, then the others
            const uint32_t home = wg % pt.nx;
            for (uint32_t k = 0; k < pt.nx; ++k) {
                const uint32_t x = home + k < pt.nx ? home + k : home + k - pt.nx;
                if (s.parts_done & (1u << x)) continue;
                const uint32_t i = add_relaxed(&L->compute_claim[x], 1u);
                if (i < pt.size(x)) return {kRoleCompute, pt.tile(x, i), ns};
                s.parts_done |= 1u << x;
            }
            s.compute_exhausted = true;
            continue;
        }
        // static partition: compute workgroups leave once compute is all claimed
        if (compute_role && a.mode == kStatic) return {kRoleExit, 0, ns};
        if (s.reduce_exhausted) return {kRoleExit, 0, ns};
        // adaptive: a compute-role workgroup with no compute left reduces, as
        // every workgroup does once the controller's target reaches B
        s.pending_role = kRoleReduce;
        s.pending_q = add_relaxed(&L->reduce_claim, 1u);
        s.pending_ns = compute_role ? B : ns;
    }
}

// Thread 0, right after choosing reduce task d: take the ticket for the task
// after it now, so its round trip overlaps this task (the result is read at
// the next boundary), while the target still gives this workgroup the reduce
// role.
__device__ __forceinline__ void prefetch_claim(const FusedArgs &a, Live *L, uint32_t wg, Sched &s,
                                               const Decision &d) {
    if (a.mode == kDeterministic || s.pending_role != kRoleNone) return;
    const uint32_t ns = s.target;
    const bool compute_role = wg >= ns;
    // Compute claims are not taken ahead: a compute task is long against the
    // claim's round trip, and an early claim would delay a switch to the
    // reduce role by a whole task.
    if (d.role == kRoleReduce && !s.reduce_exhausted &&
               (!compute_role || (a.mode == kAdaptive && s.compute_exhausted))) {
        s.pending_role = kRoleReduce;
        s.pending_q = add_relaxed(&L->reduce_claim, 1u);
        s.pending_ns = compute_role ? (uint32_t)a.nwg : ns;
    }
}

// Thread 0, at the end of a task and before its stores drain: start the
// round trips the next boundary needs, so they overlap the drain.  A compute
// workgroup that is still in the compute role claims its next tile; a
// reducer holding a ticket reads that tile's readiness flag.
__device__ __forceinline__ void early_next(const FusedArgs &a, const Parts &pt, Live *L, uint32_t wg,
                                           Sched &s) {
    if (a.mode == kDeterministic) return;
    if (s.pending_role == kRoleReduce) {
        if (s.pending_q < a.T) {
            s.early_flag = true;
            s.early_flag_value = ld_relaxed(&a.ws.tile_flag[pt.ticket(s.pending_q)]);
        }
        return;
    }
    const uint32_t ns = s.target;
    if (wg >= ns && !s.compute_exhausted) {
        const uint32_t home = wg % pt.nx;
        for (uint32_t k = 0; k < pt.nx; ++k) {
            const uint32_t x = home + k < pt.nx ? home + k : home + k - pt.nx;
            if (s.parts_done & (1u << x)) continue;
            s.early_claim = true;
            s.early_x = x;
            s.early_ns = ns;
            s.early_i = add_relaxed(&L->compute_claim[x], 1u);
            return;
        }
    }
}

// Thread 0, after a task: one controller step from the two role words
// (adaptive mode only); returns the target to use next.
__device__ uint32_t controller_step(const FusedArgs &a, Live *L, uint64_t compute_word,
                                    uint64_t reduce_word, uint32_t raw_target) {
    const uint32_t cur = raw_target ? raw_target : (uint32_t)a.ns_init;
    const uint32_t n = controller_update(
        (uint32_t)a.nwg, a.T, (uint32_t)(compute_word & kCountMask),
        (uint32_t)(reduce_word & kCountMask), compute_word >> kCountBits,
        reduce_word >> kCountBits, cur, (uint32_t)a.ns_floor);
    if (n != cur || raw_target == 0) {
        st_relaxed(&L->target_ns, n);
        min_relaxed(&L->ns_min, n);
        max_relaxed(&L->ns_max, n);
        if (n != cur) {
            const uint32_t i = add_relaxed(&L->trace_len, 1u);
            if (i < (uint32_t)kTraceCap) {
                a.ws.trace[2 * i] = (uint32_t)ticks_now();
                a.ws.trace[2 * i + 1] = n;
            }
        }
    }
    return n;
}

// The last workgroup out: copy the control block to the snapshot and restore
// the initial values for the next launch.
__device__ void finish_launch(const FusedArgs &a, Live *L) {
    Live *S = a.ws.snap;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const uint32_t raw = ld_relaxed(&L->target_ns);
    for (int x = 0; x < kMaxXcd; ++x) S->compute_claim[x] = ld_relaxed(&L->compute_claim[x]);
    S->reduce_claim = ld_relaxed(&L->reduce_claim);
    S->exit_count = ld_relaxed(&L->exit_count);
    S->target_ns = raw;
    S->role_switches = ld_relaxed(&L->role_switches);
    S->chunks_released = ld_relaxed(&L->chunks_released);
    S->violations = ld_relaxed(&L->violations);
    S->error = ld_relaxed(&L->error);
    S->ns_min = ld_relaxed(&L->ns_min);
    S->ns_max = ld_relaxed(&L->ns_max);
    S->trace_len = ld_relaxed(&L->trace_len);
    S->ns_final = a.mode == kAdaptive ? (raw ? raw : (uint32_t)a.ns_init) : (uint32_t)a.ns_init;
    S->role_compute = ld_relaxed(&L->role_compute);
    S->role_reduce = ld_relaxed(&L->role_reduce);
    S->t_start = ld_relaxed(&L->t_start);
    S->t_end = ld_relaxed(&L->t_end);
    S->r_start = ld_relaxed(&L->r_start);
    S->r_end = ld_relaxed(&L->r_end);

    for (int x = 0; x < kMaxXcd; ++x) st_relaxed(&L->compute_claim[x], 0u);
    st_relaxed(&L->reduce_claim, 0u);
    st_relaxed(&L->target_ns, 0u);
    st_relaxed(&L->role_switches, 0u);
    st_relaxed(&L->chunks_released, 0u);
    st_relaxed(&L->violations, 0u);
    st_relaxed(&L->error, 0u);
    st_relaxed(&L->ns_min, 0xFFFFFFFFu);
    st_relaxed(&L->ns_max, 0u);
    st_relaxed(&L->trace_len, 0u);
    st_relaxed(&L->role_compute, (uint64_t)0);
    st_relaxed(&L->role_reduce, (uint64_t)0);
    st_relaxed(&L->t_start, ~(uint64_t)0);
    st_relaxed(&L->t_end, (uint64_t)0);
    st_relaxed(&L->r_start, ~(uint64_t)0);
    st_relaxed(&L->r_end, (uint64_t)0);
    // exit_count last: nothing touches the block after this
    st_relaxed(&L->exit_count, 0u);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

// A finished task whose bookkeeping is still to be done, and the values its
// atomics return.
struct Booked {
    bool valid;
    int role;
    uint32_t tile;
    uint64_t dt;       // shader cycles of the task
    uint64_t r0, r1;   // constant-clock start and end
};
struct BookResult {
    uint64_t mine, other;   // role words: this task's role before the add, the other role
    uint32_t old_t, old_c;  // tile and chunk counters before the add
    uint32_t raw_target;
};

// Thread 0: issue the bookkeeping atomics of task b (results are read later).
__device__ __forceinline__ BookResult book_issue(const FusedArgs &a, Live *L, const Booked &b) {
    BookResult r;
    const uint64_t inc = (b.dt << kCountBits) | 1ull;
    r.old_t = 0;
    r.old_c = 0;
    if (b.role == kRoleCompute) {
        r.mine = add_relaxed(&L->role_compute, inc);
        r.other = ld_relaxed(&L->role_reduce);
    } else {
        const uint32_t c = b.tile / a.tpc;
        r.old_t = add_relaxed(&a.ws.tile_cnt[b.tile], 1u);
        r.old_c = add_relaxed(&a.ws.chunk_cnt[c], 1u);
        r.mine = add_relaxed(&L->role_reduce, inc);
        r.other = ld_relaxed(&L->role_compute);
        min_relaxed(&L->r_start, b.r0);
        max_relaxed(&L->r_end, b.r1);
    }
    r.raw_target = a.mode == kAdaptive ? ld_relaxed(&L->target_ns) : 0u;
    return r;
}

// Thread 0: act on the returned values -- exactly-once check, release of a
// chunk whose last tile this was ("【学习】mKernel 分析" section 2.3), one
// controller step (section 2.4).
__device__ __forceinline__ void book_finish(const FusedArgs &a, Live *L, const Booked &b,
                                            const BookResult &r, Sched &s) {
    const uint64_t inc = (b.dt << kCountBits) | 1ull;
    if (b.role == kRoleReduce) {
        const uint32_t c = b.tile / a.tpc;
        const uint32_t first = c * a.tpc;
        const uint32_t size = (a.T - first) < a.tpc ? (a.T - first) : a.tpc;
        const uint32_t want = size * a.calls;
        if (r.old_t != a.calls - 1) add_relaxed(&L->violations, 1u);
        if (r.old_c + 1 == want) {
            // where a network send of the chunk would be posted
            st_relaxed(&a.ws.chunk_flag[c], a.epoch);
            add_relaxed(&L->chunks_released, 1u);
        } else if (r.old_c + 1 > want) {
            add_relaxed(&L->violations, 1u);
        }
    }
    if (a.mode == kAdaptive) {
        const uint64_t cw = b.role == kRoleCompute ? r.mine + inc : r.other;
        const uint64_t rw = b.role == kRoleCompute ? r.other : r.mine + inc;
        s.target = controller_step(a, L, cw, rw, r.raw_target);
    }
}

template <int TM, int TN>
constexpr int fused_lds_bytes() {
    using G = GemmFor<TM, TN, kPolicyCoherentStore>;
    return G::LDS_BYTES > kFusedLdsBytes ? G::LDS_BYTES : kFusedLdsBytes;
}

template <int TM, int TN>
__global__ __launch_bounds__((GemmFor<TM, TN, kPolicyCoherentStore>::NT)) void fused_gemm_reduce_kernel(
    FusedArgs a) {
    using G = GemmFor<TM, TN, kPolicyCoherentStore>;
    __shared__ __attribute__((aligned(1024))) char lds_raw[fused_lds_bytes<TM, TN>()];
    __shared__ Decision sh_dec;
    lchar *lds = (lchar *)lds_raw;

    const int tid = threadIdx.x;
    const uint32_t wg = blockIdx.x;
    Live *L = a.ws.live;
    typename G::Lane ln;
    G::init_lane(ln, a.N, a.K);

    Sched s;
    s.det_i = 0;
    s.last_role = kRoleNone;
    s.compute_exhausted = false;
    s.parts_done = 0;
    s.reduce_exhausted = false;
    const Parts pt = make_parts((uint32_t)a.nxcd, (uint32_t)a.tiles_m, (uint32_t)a.tiles_n, a.tpc,
                                (uint32_t)a.group_m);
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
    if (tid == 0) min_relaxed(&L->t_start, ticks_now());

    // Bookkeeping of a finished task (progress word, exactly-once counters,
    // chunk counter, controller inputs) is issued by thread 0 right after the
    // next task starts and read back when that task ends, so its device-scope
    // round trips overlap work instead of stalling the workgroup.  Readiness
    // flags are not deferred: they are stored as soon as the tile is complete.
    Booked bk;
    bk.valid = false;
    BookResult br;
    for (;;) {
        if (tid == 0) {
            s.decide_t0 = ticks_now();
            const Decision d = next_task(a, pt, L, wg, s);
            s.decide_t1 = ticks_now();
            if (d.role == kRoleReduce) prefetch_claim(a, L, wg, s, d);
            sh_dec = d;
        }
        __syncthreads();
        const Decision d = sh_dec;
        if (d.role == kRoleExit) break;
        if (tid == 0 && bk.valid) br = book_issue(a, L, bk);
        const uint64_t c0 = tid == 0 ? cycles_now() : 0;
        const uint64_t r0 = tid == 0 ? ticks_now() : 0;
        const int ti = (int)(d.tile / (uint32_t)a.tiles_n);
        const int tj = (int)(d.tile % (uint32_t)a.tiles_n);

        if (d.role == kRoleCompute) {
            G::tile(ln, a.A, a.B, a.C, a.M, a.N, a.K, ti, tj, lds);
            if (tid == 0) early_next(a, pt, L, wg, s);
            // payload before flag ("【学习】mKernel 分析" section 2.5): every wave's
            // device-coherent tile stores have completed before thread 0
            // publishes the tile
            drain_vmem();
            __syncthreads();
            if (tid == 0) {
                if ((int64_t)d.tile != a.skip_publish) st_relaxed(&a.ws.tile_flag[d.tile], a.epoch);
                a.ws.cowner[d.tile] = (d.ns_seen << 16) | wg;
            }
        } else {
            // thread 0 saw the flag before the barrier; the partial is read
            // with device-coherent loads, after it
            if (a.P > 0) reduce_tile<TM, TN, G::NT>(a.peers, a.C, a.M, a.N, a.P, ti, tj);
            if (tid == 0) early_next(a, pt, L, wg, s);
            // the reduced tile is complete before its chunk can be released
            drain_vmem();
            __syncthreads();
            if (tid == 0) a.ws.rowner[d.tile] = (d.ns_seen << 16) | wg;
        }
        if (tid == 0) {
            if (bk.valid) book_finish(a, L, bk, br, s);
            bk.valid = true;
            bk.role = d.role;
            bk.tile = d.tile;
            bk.dt = cycles_now() - c0;
            bk.r0 = r0;
            bk.r1 = ticks_now();
            // per-tile timeline (low 32 bits of the constant clock)
            uint32_t *tl = a.ws.timeline + (d.role == kRoleCompute ? 0u : 2u * a.Tcap);
            tl[d.tile] = (uint32_t)r0;
            tl[a.Tcap + d.tile] = (uint32_t)bk.r1;
            // how long choosing this task took (claim, readiness wait)
            a.ws.timeline[(d.role == kRoleCompute ? 4u : 5u) * a.Tcap + d.tile] =
                (uint32_t)(s.decide_t1 - s.decide_t0);
            if (s.last_role != kRoleNone && s.last_role != d.role) add_relaxed(&L->role_switches, 1u);
            s.last_role = d.role;
        }
        // sh_dec is rewritten only after every thread has read it
        __syncthreads();
    }
    if (tid == 0 && bk.valid) {
        br = book_issue(a, L, bk);
        book_finish(a, L, bk, br, s);
    }

    if (tid == 0) {
        max_relaxed(&L->t_end, ticks_now());
        const uint32_t old = add_acq_rel(&L->exit_count, 1u);
        if (old == (uint32_t)a.nwg - 1) finish_launch(a, L);
    }
}

// ---------------------------------------------------------------------------
// unfused baseline: a GEMM kernel writes C_r, then a reduce kernel adds peers
// ---------------------------------------------------------------------------

// persistent GEMM over all tiles in the same claim order, same MFMA core
template <int TM, int TN>
__global__ __launch_bounds__((GemmFor<TM, TN, kPolicyDefault>::NT)) void gemm_kernel(GemmArgs a) {
    using G = GemmFor<TM, TN, kPolicyDefault>;
    __shared__ __attribute__((aligned(1024))) char lds_raw[G::LDS_BYTES];
    lchar *lds = (lchar *)lds_raw;
    typename G::Lane ln;
    G::init_lane(ln, a.N, a.K);
    const uint32_t T = (uint32_t)a.tiles_m * (uint32_t)a.tiles_n;
    const Parts pt = make_parts((uint32_t)a.nxcd, (uint32_t)a.tiles_m, (uint32_t)a.tiles_n,
                                (uint32_t)a.tpc, (uint32_t)a.group_m);
    for (uint32_t q = blockIdx.x; q < T; q += gridDim.x) {
        const uint32_t t = pt.ticket(q);
        G::tile(ln, a.A, a.B, a.C, a.M, a.N, a.K, (int)(t / (uint32_t)a.tiles_n),
                (int)(t % (uint32_t)a.tiles_n), lds);
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
    for (; i + (U - 1) * stride < a.count4; i += U * stride) {
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
    for (; i < a.count4; i += stride) {
        f32x4 acc = C[i];
        for (int p = 0; p < a.P; ++p) acc += __builtin_nontemporal_load(Pp + (int64_t)p * MN4 + i);
        __builtin_nontemporal_store(acc, C + i);
    }
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ void live_init(Live *L) {
    for (int x = 0; x < kMaxXcd; ++x) L->compute_claim[x] = 0;
    L->reduce_claim = 0;
    L->exit_count = 0;
    L->target_ns = 0;
    L->role_switches = 0;
    L->chunks_released = 0;
    L->violations = 0;
    L->error = 0;
    L->ns_min = 0xFFFFFFFFu;
    L->ns_max = 0;
    L->trace_len = 0;
    L->ns_final = 0;
    L->role_compute = 0;
    L->role_reduce = 0;
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

__global__ void controller_eval_kernel(const uint64_t *in, uint32_t *out, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint64_t *r = in + 8 * (int64_t)i;
    out[i] = controller_update((uint32_t)r[0], (uint32_t)r[1], (uint32_t)r[2], (uint32_t)r[3], r[4],
                               r[5], (uint32_t)r[6], (uint32_t)r[7]);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

bool tile_supported(int tm, int tn) {
    return (tm == 64 && tn == 64) || (tm == 128 && tn == 128) || (tm == 256 && tn == 128);
}

template <int TM, int TN>
static hipError_t launch_fused_t(const FusedArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((fused_gemm_reduce_kernel<TM, TN>), dim3(a.nwg),
                       dim3(GemmFor<TM, TN, kPolicyCoherentStore>::NT), 0, s, a);
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
    const int per_cu = (160 * 1024) / G::LDS_BYTES >= 2 ? 2 : 1;
    const int64_t T = (int64_t)a.tiles_m * a.tiles_n;
    const int64_t grid = T < (int64_t)num_cu * per_cu ? T : (int64_t)num_cu * per_cu;
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

hipError_t launch_controller_eval(const uint64_t *in, uint32_t *out, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(controller_eval_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, out, n);
    return hipGetLastError();
}

}  // namespace mk
