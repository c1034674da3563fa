// Kernels of the Ring Attention share and its unfused baseline.
//
// Ring Attention row of the MarkTechPost page's five-kernel table: attention
// over a sequence split across ranks, where each step passes a KV chunk
// around the ring while the local FlashAttention consumes the chunk received
// before, compute and transfer inside one persistent kernel.  "【学习】mKernel
// 分析" section 2.6 (Table 3): sequence parallelism, KV moves in 128-row
// tiles; section 2.4: the same on-GPU controller sets the communication-role
// size; section 2.5: an arrival flag names a completed payload.
//
// On one GPU the other ranks' K and V are buffers in local HBM, in ring
// arrival order, and the copy role stands in for the ring transfer: a copy
// task moves one part (at most 64 KiB) of an arriving KV tile (128 tokens of
// one step, every head, K and V) into the ring buffers, written through; the
// task whose count completes the tile sets the tile's arrival flag.  Copy
// tasks go in arrival order (step by step), so tiles land in the order the
// ring would bring them.  A compute task is 128 queries of one head against
// every key: step 0 from the local K and V at once, then each arriving tile
// once its flag carries the launch's epoch, in arrival order.  Roles follow
// the workgroup index against the controller's target, re-read at every task
// boundary, as in the other kernels.
//
// FlashAttention on CDNA4 MFMA (v_mfma_f32_32x32x16_bf16), 4 waves, 32
// queries per wave:
//  - S^T = K Q^T: K (keys x d) is the first operand, read from LDS with
//    ds_read_b128 (row r's 16-byte chunk c stored at c ^ (r mod 16): the 16
//    lanes of a read hit 16 distinct chunks); Q^T is the second operand, held
//    in registers for the whole task.  Each lane then owns one query (column)
//    and 16 of every 32 keys, so the row maximum needs one exchange with the
//    lane 32 away and the running sum none until the end.
//  - O^T += V^T P^T: V^T comes from LDS through ds_read_b64_tr_b16 (row r's
//    chunk c at c ^ 4 (r mod 4)); P^T is the exponentiated S^T converted to
//    bf16 in place: the k slots of the MFMA are matched to the keys each lane
//    already holds (k slot order is free as long as both operands agree), so
//    no data moves between lanes.
//  - online softmax in base 2 with the 1/sqrt(D) scale folded in; the
//    accumulators are rescaled per 64-key stage.
//  - K and V reach LDS by direct buffer-to-LDS loads into a ring of four
//    64-key stages, three ahead.  An arriving tile's flag is fetched into LDS
//    by the same load queue two tiles ahead of its use, so the wait for a
//    stage's data also covers the flag, and the check costs an LDS read.
#include "mk_device.hpp"
#include "mk_ring.hpp"

namespace mk {

typedef float f32x8 __attribute__((ext_vector_type(8)));

struct Fa {
    static constexpr int D = kRaHeadDim;
    static constexpr int NWAVES = 4, NT = 64 * NWAVES;
    static constexpr int KVB = 64;                      // keys per LDS stage
    static constexpr int ROW = D * 2;                    // bytes of one K or V row in LDS
    static constexpr int KV_BYTES = KVB * ROW;           // 16 KiB
    static constexpr int SLOT = 2 * KV_BYTES;            // K, then V
    static constexpr int NSLOT = 4;
    static constexpr int AHEAD = NSLOT - 1;              // stages in flight
    static constexpr int FLAG_OFS = NSLOT * SLOT;        // arrival-flag words after the ring
    static constexpr int LDS_BYTES = FLAG_OFS + 64;
    static constexpr int PIECES = KV_BYTES / 16 / NT;    // 16-byte pieces of K (and V) per thread per stage
    static_assert(PIECES == 4, "one 1 KiB load per wave per piece");
    static_assert(kRaKvRows == 2 * KVB, "a KV tile is two stages");
    static_assert(kRaQRows == 32 * NWAVES, "32 queries per wave");
    static_assert(LDS_BYTES > 80 * 1024, "one workgroup per CU");

    struct Lane {
        uint32_t dk[PIECES], dv[PIECES];   // DMA offsets inside a stage's K and V rows
        uint32_t kofs[8];                  // LDS offset of the K operand per 16-deep d-step
        uint32_t vofs[4];                  // LDS offset of the V operand per 32-wide d block
    };

    // K/V row carried by piece i of thread t
    static __device__ __forceinline__ int prow(int i, int t) {
        return ((t >> 6) * PIECES + i) * 4 + ((t & 63) >> 4);
    }

    static __device__ __forceinline__ void init_lane(Lane &ln, uint32_t rowb) {
        const int t = threadIdx.x, l = t & 63, hl = l >> 5;
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
            const int r = prow(i, t), cp = l & 15;
            ln.dk[i] = (uint32_t)r * rowb + ((uint32_t)(cp ^ (r & 15)) << 4);
            ln.dv[i] = (uint32_t)r * rowb + ((uint32_t)(cp ^ (4 * (r & 3))) << 4);
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) ln.kofs[s] = (l & 31) * ROW + (((2 * s + hl) ^ (l & 15)) << 4);
        const int j = l & 15, g16 = (l >> 4) & 1;
#pragma unroll
        for (int fd = 0; fd < 4; ++fd)
            ln.vofs[fd] = ((j >> 2) + 4 * hl) * ROW +
                          (((4 * fd + 2 * g16 + ((j & 3) >> 1)) ^ (4 * (j >> 2))) << 4) + 8 * (j & 1);
    }

    // One stage (KVB keys of one head) of K and V into the slot at LDS byte
    // address `slot`; kp / vp point at the stage's first key.  Keys at or
    // past `rows` (the ragged end of a step) read as zeros.
    static __device__ __forceinline__ void issue(const Lane &ln, uint32_t slot, const uint16_t *kp,
                                                 const uint16_t *vp, int rows) {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const uint32_t s0 = __builtin_amdgcn_readfirstlane(slot) + wave * PIECES * 1024;
        const u32x4 dk = make_desc(kp), dv = make_desc(vp);
        if (__builtin_amdgcn_readfirstlane(rows) >= KVB) {
#pragma unroll
            for (int i = 0; i < PIECES; ++i) dma16(dk, ln.dk[i], s0 + i * 1024);
#pragma unroll
            for (int i = 0; i < PIECES; ++i) dma16(dv, ln.dv[i], s0 + KV_BYTES + i * 1024);
        } else {
            int t = threadIdx.x;
            asm volatile("" : "+v"(t));
#pragma unroll
            for (int i = 0; i < PIECES; ++i) dma16(dk, prow(i, t) < rows ? ln.dk[i] : kOOB, s0 + i * 1024);
#pragma unroll
            for (int i = 0; i < PIECES; ++i)
                dma16(dv, prow(i, t) < rows ? ln.dv[i] : kOOB, s0 + KV_BYTES + i * 1024);
        }
    }

    // S^T of one stage: s0 keys 0..31, s1 keys 32..63 (lane (j + 32 hl),
    // register v: key 8 (v / 4) + 4 hl + v % 4 of the block, query j)
    static __device__ __forceinline__ void qk(const Lane &ln, const lchar *sl, const bf16x8 (&qf)[8], f32x16 &s0,
                                              f32x16 &s1) {
        s0 = f32x16{};
        s1 = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bf16x8 k0 = *(const lbf16x8 *)(sl + ln.kofs[s]);
            const bf16x8 k1 = *(const lbf16x8 *)(sl + 32 * ROW + ln.kofs[s]);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], s1, 0, 0, 0);
        }
    }

    // Online softmax of one stage's scores and P.V.  `rows` keys are valid.
    // The running maximum m (log2 units) moves only when a stage's maximum
    // exceeds it by more than kLazy: then p <= 2^kLazy, which fp32 sums and
    // bf16 P hold without loss, and most stages skip rescaling O (the test is
    // per query, the skip per wave).
    static constexpr float kLazy = 8.f;

    // Keys at or past `rows` get score -inf (a stage at the ragged end of a
    // step).  Called under a uniform branch; the empty asm keeps it a branch
    // instead of selects executed in every stage.
    static __device__ __forceinline__ void mask(f32x16 &s0, f32x16 &s1, int rows) {
        asm volatile("" ::: "memory");
        const int hl = (threadIdx.x & 63) >> 5;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int key = 8 * (v >> 2) + 4 * hl + (v & 3);
            if (key >= rows) s0[v] = -__builtin_inff();
            if (key + 32 >= rows) s1[v] = -__builtin_inff();
        }
    }

    // Exponentiated scores of one stage as the bf16 P^T operands; returns the
    // new running maximum (m moves only when a stage's maximum exceeds it by
    // more than kLazy, so p <= 2^kLazy) and adds the stage's sum to ls.  No
    // branch inside: the caller's score MFMAs of the next stage can be
    // interleaved with this vector work.
    static __device__ __forceinline__ float softmax(const f32x16 &s0, const f32x16 &s1, float m, float c,
                                                    bf16x8 (&p)[2][2], float &ls) {
        float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(s0[v], s1[v]));
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;
        const float mn = mx > m + kLazy ? mx : m;
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x8 a0, a1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                a0[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[8 * t + e], c, -mn));
                a1[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[8 * t + e], c, -mn));
                acc += a0[e] + a1[e];
            }
            p[0][t] = __builtin_convertvector(a0, bf16x8);
            p[1][t] = __builtin_convertvector(a1, bf16x8);
        }
        ls = acc;
        return mn;
    }

    // O^T += V^T P^T for one stage
    static __device__ __forceinline__ void pv(const Lane &ln, const lchar *sl, const bf16x8 (&p)[2][2],
                                              f32x16 (&o)[4]) {
        const lchar *vb = sl + KV_BYTES;
#pragma unroll
        for (int fd = 0; fd < 4; ++fd)
#pragma unroll
            for (int fk = 0; fk < 2; ++fk)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const lchar *pp = vb + ln.vofs[fd] + (32 * fk + 16 * t) * ROW;
                    const bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4 *)pp);
                    const bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4 *)(pp + 8 * ROW));
                    o[fd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7), p[fk][t], o[fd], 0, 0, 0);
                }
    }
};

// wait (bounded) for arriving tile c's flag; false on timeout or another
// workgroup's error (the error is recorded)
// (arguments by value: a reference to the kernel's argument block would make
// the compiler copy the block to scratch to give it an address)
__device__ __noinline__ bool ra_wait_tile(uint32_t *flag, uint32_t epoch, uint64_t timeout_ticks, Live *L) {
    const uint64_t since = ticks_now();
    for (;;) {
        if (ld_relaxed(flag) == epoch) return true;
        if (ld_relaxed(&L->error) != kErrNone) return false;
        if (ticks_now() - since > timeout_ticks) {
            __hip_atomic_fetch_max(&L->error, (uint32_t)kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_or(&L->sticky, kStickyTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// One compute task: queries [128 qb, 128 qb + 128) of head h against every
// key.  GATED: arriving tiles are read only after their flag (the fused
// kernel); otherwise every tile is already in place (the unfused baseline).
// Returns false if a wait failed (the outputs are then not valid and the
// launch reports the error).
template <bool GATED>
__device__ __forceinline__ bool fa_task(const RaArgs &a, const Fa::Lane &ln, lchar *lds, Live *L, uint32_t h,
                                        uint32_t qb) {
    constexpr int D = Fa::D;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl = lane >> 5;
    // every field the task needs, read once into locals: the loads of the
    // K/V stream are inline assembly that clobbers memory, so fields read
    // inside the loop would be reloaded at every stage
    const int64_t S = a.S;
    const int64_t HD = (int64_t)a.H * D;
    const uint32_t nkv = a.nkv, epoch = a.epoch;
    const uint32_t U = (uint32_t)a.R * nkv;     // KV tiles in ring order, step 0 first
    const uint16_t *const k_loc = a.k_local + (int64_t)h * D, *const v_loc = a.v_local + (int64_t)h * D;
    const uint16_t *const k_rng = a.k_ring + (int64_t)h * D, *const v_rng = a.v_ring + (int64_t)h * D;
    uint32_t *const flags = a.ws.chunk_flag;
    const uint64_t timeout_ticks = a.timeout_ticks;
    const float c = a.scale_log2;
    float *const Oh = a.O + (int64_t)h * D;
    float *const lse_h = a.lse + (int64_t)h * S;
    const int64_t q0 = (int64_t)qb * kRaQRows;
    const int64_t row = q0 + 32 * wave + (lane & 31);
    const uint32_t base = (uint32_t)(uintptr_t)lds;

    // this lane's Q^T operand for the 8 d-steps (zero past the last query)
    bf16x8 qf[8];
    {
        const auto rq = scalar_rsrc(a.q + (int64_t)h * D);
        const uint32_t qoff = row < S ? (uint32_t)(row * HD) * 2u : kOOB;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            qf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rq, qoff == kOOB ? kOOB : qoff + (16 * s + 8 * hl) * 2, 0,
                                                   kPolicyDefault));
    }

    const uint32_t nst = 2 * U;
    // issue the next stage of the task's sequence (stages are issued in
    // order: tile u = (step, t), half j) into its ring slot; the position is
    // advanced here, without divisions
    uint32_t ix = 0, i_step = 0, i_t = 0;
    auto issue_stage = [&]() {
        const uint32_t x = ix++, u = x >> 1, j = x & 1;
        const uint32_t step = i_step, t = i_t;
        if (j == 1 && ++i_t == nkv) {
            i_t = 0;
            ++i_step;
        }
        if constexpr (GATED) {
            if (step > 0 && j == 0) {
                // the flag fetched two tiles ahead (a 32-bit word in LDS),
                // else a bounded wait; after a failed wait (the error is
                // recorded) the stage is read anyway and the launch's result
                // is reported invalid
                bool ok = false;
                if (u >= 2) ok = *(const volatile __attribute__((address_space(3))) uint32_t *)(
                                     lds + Fa::FLAG_OFS + 4 * (u & 3)) == epoch;
                if (!ok) ra_wait_tile(flags + (u - nkv), epoch, timeout_ticks, L);
            }
            // fetch the flag of tile u + 2 into LDS, behind this stage's loads
            // in wave 0's queue; it is read two tiles later
            if (j == 0 && wave == 0 && u + 2 < U && u + 2 >= nkv) {
                const uint32_t c2 = u + 2 - nkv;
                if (lane == 0) {
                    const u32x4 df = make_desc(flags);
                    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen sc1 lds"
                                 :
                                 : "s"(__builtin_amdgcn_readfirstlane(base + Fa::FLAG_OFS + 4 * ((u + 2) & 3))),
                                   "v"(c2 * 4u), "s"(df)
                                 : "memory", "m0");
                }
            }
        }
        const int64_t kv0 = (int64_t)t * kRaKvRows + (int64_t)j * Fa::KVB;
        const int rows = (int)(S - kv0 < Fa::KVB ? S - kv0 : Fa::KVB);
        const int64_t off = kv0 * HD;
        const uint16_t *kp = step == 0 ? k_loc + off : k_rng + (int64_t)(step - 1) * S * HD + off;
        const uint16_t *vp = step == 0 ? v_loc + off : v_rng + (int64_t)(step - 1) * S * HD + off;
        Fa::issue(ln, base + (x % Fa::NSLOT) * Fa::SLOT, kp, vp, rows);
    };

    const uint32_t pre = nst < (uint32_t)Fa::AHEAD ? nst : (uint32_t)Fa::AHEAD;
    for (uint32_t x = 0; x < pre; ++x) issue_stage();

    f32x16 o[4] = {};
    float m = -__builtin_inff(), l = 0.f;
    // valid keys of the stages consumed in order, tracked without divisions
    uint32_t c_t = 0, c_j = 0;
    auto rows_next = [&]() {
        const int64_t kv0 = (int64_t)c_t * kRaKvRows + (int64_t)c_j * Fa::KVB;
        if (c_j == 1 && ++c_t == nkv) c_t = 0;
        c_j ^= 1;
        return (int)(S - kv0 < Fa::KVB ? S - kv0 : Fa::KVB);
    };
    // Stage b's scores are computed one step ahead: the MFMAs of S(b + 1) run
    // while the vector units exponentiate S(b).  Two score sets alternate
    // (the loop body covers two stages), so no registers are copied.
    f32x16 sa0, sa1, sb0, sb1;
    // stages issued after stage 0: pre - 1
    if (pre >= 3) wait_vmcnt<2 * 2 * Fa::PIECES>();
    else if (pre == 2) wait_vmcnt<2 * Fa::PIECES>();
    else wait_vmcnt<0>();
    __syncthreads();   // stage 0 has landed
    Fa::qk(ln, lds, qf, sa0, sa1);
    // one step of the pipeline: wait for stage b + 1, refill, then S(b + 1)
    // on the matrix cores while the vector units exponentiate S(b), then
    // P.V of stage b.  The score MFMAs run even past the last stage (on a
    // stale slot, result unused) so that block has no branch to split it.
    auto step = [&](uint32_t b, f32x16 &c0, f32x16 &c1, f32x16 &n0, f32x16 &n1) {
        if (b + 1 < nst) {
            if (b + 2 < nst) wait_vmcnt<2 * Fa::PIECES>();
            else wait_vmcnt<0>();
        }
        __syncthreads();   // stage b + 1 has landed for every wave; slot (b - 1) is free
        if (b + Fa::AHEAD < nst) issue_stage();
        const int rows = rows_next();
        if (__builtin_amdgcn_readfirstlane(rows) < Fa::KVB) Fa::mask(c0, c1, rows);
        Fa::qk(ln, lds + ((b + 1) % Fa::NSLOT) * Fa::SLOT, qf, n0, n1);
        bf16x8 p[2][2];
        float ls;
        const float mn = Fa::softmax(c0, c1, m, c, p, ls);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one score MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // vector work of the softmax
        }
        if (__ballot(mn != m)) {
            const float alpha = __builtin_amdgcn_exp2f(m - mn);
            l *= alpha;
#pragma unroll
            for (int fd = 0; fd < 4; ++fd) o[fd] = o[fd] * alpha;
        }
        m = mn;
        l += ls;
        Fa::pv(ln, lds + (b % Fa::NSLOT) * Fa::SLOT, p, o);
    };
    for (uint32_t b = 0; b < nst; b += 2) {
        step(b, sa0, sa1, sb0, sb1);
        if (b + 1 < nst) step(b + 1, sb0, sb1, sa0, sa1);
    }
    __syncthreads();   // every wave is done with the ring before the next task refills it

    // normalise and store: lane (j + 32 hl) holds O^T rows 32 fd + 8 g + 4 hl + 0..3
    const float lt = l + __shfl_xor(l, 32);
    const float inv = 1.f / lt;
    const auto ro = scalar_rsrc(Oh);
    const bool ok = row < S;
#pragma unroll
    for (int fd = 0; fd < 4; ++fd)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int dv = 32 * fd + 8 * g + 4 * hl;
            const uint32_t off = ok ? ((uint32_t)(row * HD) + (uint32_t)dv) * 4u : kOOB;
            f32x4 v{o[fd][4 * g] * inv, o[fd][4 * g + 1] * inv, o[fd][4 * g + 2] * inv, o[fd][4 * g + 3] * inv};
            __builtin_amdgcn_raw_buffer_store_b128(v, ro, off, 0, kPolicyStream);
        }
    if (hl == 0 && ok) lse_h[row] = (m + __log2f(lt)) * 0.69314718055994531f;
    return true;
}

// ---------------------------------------------------------------------------
// copy role
// ---------------------------------------------------------------------------

// copy task u: part u mod parts of arriving tile u / parts (tile c = (s-1)
// nkv + t holds tokens [128 t, 128 t + 128) of step s), K then V.  Source
// read once (nt); destination written through (nt sc1), visible at device
// scope once the stores have drained.
template <int NT>
__device__ __forceinline__ void ra_copy(const RaArgs &a, uint32_t u) {
    const uint32_t c = u / a.parts, part = u % a.parts;
    const uint32_t s1 = c / a.nkv, t = c % a.nkv;
    const int64_t t0 = (int64_t)t * kRaKvRows;
    const int64_t rows = a.S - t0 < kRaKvRows ? a.S - t0 : kRaKvRows;
    const int64_t HD = (int64_t)a.H * kRaHeadDim;
    const uint64_t n16t = (uint64_t)(rows * HD / 8);   // 16-byte pieces of the tile's K (and of its V)
    const uint32_t i0 = (uint32_t)(n16t * part / a.parts);
    const uint32_t n16 = (uint32_t)(n16t * (part + 1) / a.parts) - i0;
    const int64_t eoff = ((int64_t)s1 * a.S + t0) * HD + (int64_t)i0 * 8;
    const auto rsk = scalar_rsrc(a.k_peers + eoff), rsv = scalar_rsrc(a.v_peers + eoff);
    const auto rdk = scalar_rsrc(a.k_ring + eoff), rdv = scalar_rsrc(a.v_ring + eoff);
    // The part's K and V loads of a pass are all issued before its first
    // store (up to 2 x 32 KiB per pass): a 64 KiB part is one load round trip
    // and one store drain.  Pieces past the part read zero and drop their
    // stores.
    constexpr int U = 8;
    for (uint32_t b = 0; b < n16; b += U * NT) {
        uint32_t off[U];
        f32x4 vk[U], vv[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t i = b + k * NT + threadIdx.x;
            off[k] = i < n16 ? i * 16u : kOOB;
            vk[k] = __builtin_amdgcn_raw_buffer_load_b128(rsk, off[k], 0, kPolicyStream);
        }
#pragma unroll
        for (int k = 0; k < U; ++k)
            vv[k] = __builtin_amdgcn_raw_buffer_load_b128(rsv, off[k], 0, kPolicyStream);
#pragma unroll
        for (int k = 0; k < U; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(vk[k], rdk, off[k], 0, kPolicyCoherentStream);
#pragma unroll
        for (int k = 0; k < U; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(vv[k], rdv, off[k], 0, kPolicyCoherentStream);
    }
}

// ---------------------------------------------------------------------------
// the persistent fused kernel
// ---------------------------------------------------------------------------

enum RaRole : int { kRaCompute = 0, kRaCopy = 1, kRaExit = 2 };

struct RaDecision {
    int role;
    uint32_t unit;      // compute: task (head * nqb + block); copy: copy task
    uint32_t ns_seen;   // copy target the task was taken under
};

struct RaSched {
    uint32_t target;
    uint32_t det_i;
    uint32_t bands_done;
    bool copy_exhausted, compute_exhausted;
    int last_role;
};

// Thread 0: claim a compute task.  One band: one head-major queue.  Bands:
// band x holds the heads h = x mod bands (the workgroups of one XCD share
// their heads' K and V in L2), its i-th claim is head x + bands (i / nqb),
// block i mod nqb; the home band first, then the others in turn.
__device__ __forceinline__ bool ra_claim_task(const RaArgs &a, Live *L, uint32_t wg, RaSched &s, uint32_t &j) {
    const uint32_t nb = a.bands;
    if (nb <= 1) {
        j = add_relaxed(&L->compute_claim[0].v, 1u);
        return j < a.NTk;
    }
    for (uint32_t k = 0; k < nb; ++k) {
        const uint32_t x = (wg + k) % nb;
        if ((s.bands_done >> x) & 1u) continue;
        const uint32_t heads = ((uint32_t)a.H - x + nb - 1) / nb;
        const uint32_t i = add_relaxed(&L->extra_claim[x].v, 1u);
        if (i < heads * a.nqb) {
            j = (x + nb * (i / a.nqb)) * a.nqb + i % a.nqb;
            return true;
        }
        s.bands_done |= 1u << x;
    }
    return false;
}

// Thread 0: the next task.
__device__ RaDecision ra_next(const RaArgs &a, Live *L, uint32_t wg, RaSched &s) {
    const uint32_t B = (uint32_t)a.nwg;
    const uint32_t ns = s.target;
    if (a.mode == kDeterministic) {
        if (wg < ns) {
            const uint32_t q = wg + s.det_i * ns;
            if (q >= a.Qc) return {kRaExit, 0, ns};
            ++s.det_i;
            return {kRaCopy, q, ns};
        }
        const uint32_t j = (wg - ns) + s.det_i * (B - ns);
        if (j >= a.NTk) return {kRaExit, 0, ns};
        ++s.det_i;
        return {kRaCompute, j, ns};
    }
    const bool copy_role = wg < ns;
    if (copy_role && !s.copy_exhausted) {
        const uint32_t q = add_relaxed(&L->compute_claim[1].v, 1u);
        if (q < a.Qc) return {kRaCopy, q, ns};
        s.copy_exhausted = true;
    }
    // static copiers leave once every copy task is claimed
    if (copy_role && a.mode != kAdaptive) return {kRaExit, 0, ns};
    if (!s.compute_exhausted) {
        uint32_t j;
        // a copy-role workgroup computes only once no copy task is left: no
        // copy role remains (logged as target 0)
        if (ra_claim_task(a, L, wg, s, j)) return {kRaCompute, j, copy_role ? 0u : ns};
        s.compute_exhausted = true;
    }
    // adaptive: no compute left to claim, every workgroup copies (the
    // controller's target is B once no compute remains; logged as such)
    if (a.mode == kAdaptive && !s.copy_exhausted) {
        const uint32_t q = add_relaxed(&L->compute_claim[1].v, 1u);
        if (q < a.Qc) return {kRaCopy, q, copy_role ? ns : B};
        s.copy_exhausted = true;
    }
    return {kRaExit, 0, ns};
}

// The argument block is read through a pointer to the kernel-argument
// segment that is laundered at the top of every task: each task reloads the
// fields it needs (scalar loads) instead of keeping all of them in scalar
// registers across the persistent loop, which spilled dozens of them into
// vector lanes read back inside the attention loop.
__device__ __forceinline__ const RaArgs *ra_args() {
    const RaArgs *p = (const RaArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return p;
}

__global__ __launch_bounds__(Fa::NT, 1) void ring_attention_kernel(RaArgs a_arg) {
    __shared__ __attribute__((aligned(1024))) char lds_raw[Fa::LDS_BYTES];
    __shared__ RaDecision sh_dec;
    __shared__ RaSched sh_sched;
    __shared__ uint64_t sh_c0, sh_r0;
    (void)a_arg;
    lchar *lds = (lchar *)lds_raw;
    const int tid = threadIdx.x;
    const uint32_t wg = blockIdx.x;
    Fa::Lane ln;
    Fa::init_lane(ln, (uint32_t)ra_args()->H * Fa::D * 2u);
    RaSched &s = sh_sched;
    if (tid == 0) {
        const RaArgs &a = *ra_args();
        Live *L = a.ws.live;
        s.target = (uint32_t)a.ns_init;
        s.det_i = 0;
        s.bands_done = 0;
        s.copy_exhausted = s.compute_exhausted = false;
        s.last_role = -1;
        min_relaxed(&L->t_start, ticks_now());
    }
    for (;;) {
        const RaArgs &a = *ra_args();
        Live *L = a.ws.live;
        if (tid == 0) {
            sh_dec = ld_relaxed(&L->error) != kErrNone ? RaDecision{kRaExit, 0, 0} : ra_next(a, L, wg, s);
            sh_c0 = cycles_now();
            sh_r0 = ticks_now();
        }
        __syncthreads();
        RaDecision d;
        d.role = __builtin_amdgcn_readfirstlane(sh_dec.role);
        d.unit = __builtin_amdgcn_readfirstlane(sh_dec.unit);
        d.ns_seen = __builtin_amdgcn_readfirstlane(sh_dec.ns_seen);
        if (d.role == kRaExit) break;
        if (d.role == kRaCopy) {
            ra_copy<Fa::NT>(a, d.unit);
        } else {
            const uint32_t h = d.unit / a.nqb, qb = d.unit % a.nqb;
            fa_task<true>(a, ln, lds, L, h, qb);
        }
        // payload before flag ("【学习】mKernel 分析" section 2.5)
        drain_vmem();
        __syncthreads();
        if (tid == 0) {
            const uint32_t t_end = (uint32_t)ticks_now();
            const uint64_t dt = cycles_now() - sh_c0;
            const bool copying = d.role == kRaCopy;
            const uint32_t u = d.unit;
            const uint32_t c = copying ? u / a.parts : 0u;
            // every returning atomic and load is issued before the first use
            const uint32_t old = add_relaxed(copying ? &a.ws.chunk_cnt[c] : &a.ws.tile_cnt[u], 1u);
            const uint64_t inc = (dt << kCountBits) | 1u;
            const uint64_t mine = add_relaxed(copying ? &L->role_reduce.v : &L->role_compute.v, inc) + inc;
            const uint64_t other = ld_relaxed(copying ? &L->role_compute.v : &L->role_reduce.v);
            const uint32_t raw = a.mode == kAdaptive ? ld_relaxed(&L->target_ns.v) : 0u;
            if (copying) {
                // this part's stores drained before its count: the task whose
                // count completes the tile sees every part landed
                const uint32_t base = (a.calls - 1) * a.parts;
                if (old < base || old >= base + a.parts) note_violation(L);
                if (old + 1 == base + a.parts) {
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
                if (old != a.calls - 1) note_violation(L);
                a.ws.cowner[u] = (d.ns_seen << 16) | wg;
                a.ws.timeline[u] = (uint32_t)sh_r0;
                a.ws.timeline[a.Tcap + u] = t_end;
            }
            // one controller step: the copy role is the communication role s
            // (copy tasks), compute is p (tasks)
            if (a.mode == kAdaptive) {
                const uint64_t cw = copying ? other : mine, sw = copying ? mine : other;
                const uint32_t cur = raw ? raw : (uint32_t)a.ns_init;
                const uint32_t n = controller_update_totals(
                    (uint32_t)a.nwg, a.NTk, a.Qc, (uint32_t)(cw & kCountMask), (uint32_t)(sw & kCountMask),
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
        const RaArgs &a = *ra_args();
        Live *L = a.ws.live;
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

// ---------------------------------------------------------------------------
// unfused baseline
// ---------------------------------------------------------------------------

// every arriving tile into the ring buffers
__global__ __launch_bounds__(256) void ring_gather_kernel(RaArgs a) {
    const int64_t n16 = (int64_t)(a.R - 1) * a.S * a.H * kRaHeadDim / 8;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int kv = 0; kv < 2; ++kv) {
        const u32x4 *src = (const u32x4 *)(kv ? a.v_peers : a.k_peers);
        u32x4 *dst = (u32x4 *)(kv ? a.v_ring : a.k_ring);
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
            __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
    }
}

// the same attention core over every tile, no flags; workgroup b takes the
// tasks of band b mod bands round-robin (the fused kernel's claim order,
// fixed)
__global__ __launch_bounds__(Fa::NT, 1) void ring_fa_kernel(RaArgs a_arg) {
    __shared__ __attribute__((aligned(1024))) char lds_raw[Fa::LDS_BYTES];
    (void)a_arg;
    lchar *lds = (lchar *)lds_raw;
    Fa::Lane ln;
    Fa::init_lane(ln, (uint32_t)ra_args()->H * Fa::D * 2u);
    const uint32_t b = blockIdx.x;
    for (uint32_t i = 0;; ++i) {
        const RaArgs &a = *ra_args();
        const uint32_t nb = a.bands, x = b % nb;
        const uint32_t per = (gridDim.x - x + nb - 1) / nb;   // workgroups of band x
        const uint32_t heads = ((uint32_t)a.H - x + nb - 1) / nb;
        const uint32_t k = b / nb + i * per;                  // this workgroup's i-th task of the band
        if (k >= heads * a.nqb) break;
        fa_task<false>(a, ln, lds, nullptr, x + nb * (k / a.nqb), k % a.nqb);
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

int ring_workgroups_per_cu() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void *>(&ring_attention_kernel),
                                                     Fa::NT, 0) != hipSuccess)
        return 0;
    return blocks < 1 ? blocks : 1;
}

hipError_t launch_ring_attention(const RaArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(ring_attention_kernel, dim3(a.nwg), dim3(Fa::NT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_ring_unfused(const RaArgs &a, int num_cu, bool xcd_bands, hipStream_t s) {
    if (a.R > 1) {
        const int64_t n16 = (int64_t)(a.R - 1) * a.S * a.H * kRaHeadDim / 8;
        int64_t blocks = (n16 + 255) / 256;
        const int64_t cap = (int64_t)num_cu * 8;
        if (blocks > cap) blocks = cap;
        if (blocks < 1) blocks = 1;
        hipLaunchKernelGGL(ring_gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    RaArgs f = a;
    f.bands = xcd_bands ? a.bands : 1u;
    const int64_t grid = (int64_t)a.NTk < num_cu ? (int64_t)a.NTk : num_cu;
    hipLaunchKernelGGL(ring_fa_kernel, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(Fa::NT), 0, s, f);
    return hipGetLastError();
}

}  // namespace mk
