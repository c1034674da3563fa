/*
 * mk.h -- C ABI of the fused GEMM + tile-reduce library for AMD Instinct
 * MI355X (gfx950).
 *
 * The library computes one GPU's share of a GEMM+AllReduce in a single
 * persistent kernel: the local partial C_r = A.B (bfloat16 operands, fp32
 * accumulation on MFMA) and, as soon as each output tile of C_r exists, the
 * sum of that tile with the R-1 other ranks' partial tiles.  On one GPU the
 * other ranks' partials are fp32 buffers in local HBM ("peers").
 *
 * Sources (the method's pages; no code was published with them):
 *  - "mKernel: Fast Multi-GPU, Multi-Node Fused Kernels", abstract: one
 *    persistent kernel whose workgroups are split into compute and
 *    communication roles, with an on-GPU controller that tunes the split at
 *    run time; tiles are forwarded as soon as they are produced.
 *  - MarkTechPost / chathome pages, five-kernel table, GEMM + AllReduce row:
 *    C = A @ B with the partial outputs reduced across all ranks in one launch.
 *  - "【学习】mKernel 分析": section 2.2 (Figure 2: compute blocks write a tile
 *    and its readiness flag), section 2.3 (4 locally reduced tiles form a
 *    chunk; a per-chunk counter lets the last tile release the chunk),
 *    section 2.4 (static sweep of 2-64 communication SMs; adaptive controller
 *    n_s* = B (R_s C_s) / (R_p C_p + R_s C_s); blocks re-check the target at
 *    task boundaries), section 2.5 (a ready signal must name a completed
 *    payload), section 4.1 (role by block index, ready flags, chunks).
 *
 * Conventions for every call:
 *  - Returns an int status (mk_status).  No call aborts or throws.
 *  - Argument checks run before any HIP call, so a bad argument is reported
 *    without touching the GPU.
 *  - Device pointers are plain HIP device addresses owned by the caller.
 *    `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - Launches are asynchronous and stream ordered.  The library keeps one
 *    workspace per device (flags, counters, owner maps, controller block);
 *    calls on one device must not overlap in time (the library is not
 *    reentrant across concurrent streams of one device).
 *  - Timer ticks are from the GPU's constant-rate clock (s_memrealtime,
 *    100 MHz on MI355X); cycle sums are from the shader clock (s_memtime).
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_ABI_VERSION 2

typedef enum {
    MK_OK = 0,
    MK_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad tile, bad mode     */
    MK_ERR_SHAPE = -2,       /* N or K not a multiple of 8, or too many tiles   */
    MK_ERR_HIP = -3,         /* a HIP runtime call failed (see mk_last_error)   */
    MK_ERR_TIMEOUT = -4,     /* a bounded wait in the kernel expired            */
    MK_ERR_NO_DEVICE = -5,   /* no HIP device is visible                        */
    MK_ERR_PROTOCOL = -6     /* the kernel counted a flag/counter violation     */
} mk_status;

typedef enum {
    /* On-GPU controller sets the reduce-workgroup count from measured
     * per-task cycle costs ("【学习】mKernel 分析" section 2.4), bounded
     * by mk_set_controller_floor and mk_set_controller_cap while compute
     * remains.  A reduce-role workgroup whose next block is not published
     * yet computes a block meanwhile (the same section: a block waiting
     * for input helps the other role) and keeps its reduce ticket.       */
    MK_PART_ADAPTIVE = 0,
    /* Fixed count of reduce workgroups; tasks are claimed dynamically.     */
    MK_PART_STATIC = 1,
    /* Fixed count; workgroup w < n reduces tiles t = w (mod n), workgroup
     * w >= n computes blocks b = w - n (mod B - n), each in increasing
     * order (a block is mk_stats.tiles_per_task adjacent tiles of one tile
     * row; blocks and tiles are numbered row by row).                     */
    MK_PART_STATIC_DETERMINISTIC = 2
} mk_part_mode;

/*
 * mk_gemm_reduce_local -- one persistent launch computing
 *     C[i][j] = sum_k A[i][k] * B[k][j]  +  sum_{p < num_peers} peers[p][i][j]
 * (GEMM + AllReduce row of the five-kernel table; fusion and tile-granular
 * overlap per the abstract and the analysis page's Figure 2).
 *
 *   A          bfloat16 [M, K], row-major, 16-byte aligned (device).
 *   B          bfloat16 [K, N], row-major, 16-byte aligned (device).
 *   peers      fp32 [num_peers, M, N], contiguous, 16-byte aligned (device);
 *              may be NULL only when num_peers == 0.  Read only.
 *   num_peers  R - 1 >= 0.
 *   C          fp32 [M, N], row-major, 16-byte aligned (device).  Receives the
 *              local partial of each tile first, then the reduced tile.  Must
 *              not overlap A, B or peers.
 *   M, N, K    >= 0; N and K must be multiples of 8 (16-byte rows).  M, N
 *              need not be multiples of the tile: edge tiles are masked.
 *              K == 0 gives C = sum of peers; M == 0 or N == 0 returns MK_OK
 *              without a launch.
 *   tile_m, tile_n   output tile (the unit of readiness flags and chunks):
 *              one of 64x64, 128x128, 256x128.  A compute task produces a
 *              block of adjacent tiles of one tile row (two for 128x128 and
 *              256x128, one for 64x64; see mk_stats.tiles_per_task) and
 *              publishes each tile's flag; a reduce task takes one tile once
 *              it is published.
 *   tiles_per_chunk  tiles per chunk (1..64; 4 in the method's
 *              GEMM+AllReduce).  Chunk c holds tiles [c*tpc, (c+1)*tpc) in
 *              row-major tile order; the last chunk may be short.
 *   stream     hipStream_t or NULL.
 *
 * Uses the partition set by mk_set_partition.  Errors: MK_ERR_INVALID_ARG
 * (also when C's bytes overlap A's, B's or the peers'), MK_ERR_SHAPE
 * (nothing launched), MK_ERR_NO_DEVICE, MK_ERR_HIP.  Kernel-side
 * timeouts and protocol violations are reported by mk_get_stats.
 */
int mk_gemm_reduce_local(const void *A, const void *B, const float *peers, int num_peers,
                         float *C, int64_t M, int64_t N, int64_t K,
                         int tile_m, int tile_n, int tiles_per_chunk, void *stream);

/*
 * mk_gemm_reduce_local_noalloc -- mk_gemm_reduce_local for callers that
 * cannot allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, result,
 * kernels, partition settings and statistics (mk_get_stats reports whichever
 * of the two entry points launched last).  The call allocates nothing (no
 * hipMalloc, hipFree, or allocating library routine): its flags, counters,
 * maps and control block live in a static device array of about 0.4 MiB,
 * one copy per device, held until the process ends and shared by every call
 * of this entry point on that device (it keeps the last call's contents; per
 * call state starts from epoch-valued flags and counters the call itself
 * clears when the tile grid changes).  Calls that overlap in time on one
 * device race on that array: serialize them (one stream, or events).
 * Limits: at most 8192 output tiles and 8192 chunks; larger grids fail with
 * MK_ERR_SHAPE before any launch (use mk_gemm_reduce_local).
 */
int mk_gemm_reduce_local_noalloc(const void *A, const void *B, const float *peers, int num_peers,
                                 float *C, int64_t M, int64_t N, int64_t K,
                                 int tile_m, int tile_n, int tiles_per_chunk, void *stream);

/*
 * mk_gemm_reduce_unfused -- the unfused two-kernel baseline with the same
 * arguments and result: a GEMM kernel writes the fp32 partial into C, then a
 * separate reduce kernel adds the peers (the host-driven, kernel-granular
 * overlap the abstract contrasts with fused kernels).  tiles_per_chunk is
 * checked but unused.  Touches no workspace state.
 */
int mk_gemm_reduce_unfused(const void *A, const void *B, const float *peers, int num_peers,
                           float *C, int64_t M, int64_t N, int64_t K,
                           int tile_m, int tile_n, int tiles_per_chunk, void *stream);

/*
 * mk_gemm_reduce_scatter_local -- one rank's share of GEMM+ReduceScatter in
 * one persistent launch (GEMM + ReduceScatter row of the MarkTechPost page's
 * five-kernel table; "【学习】mKernel 分析" section 2.6 and Table 3 for tiles
 * reaching their owner as they finish).  This rank is rank 0 of
 * R = num_peers + 1; rank o owns tile rows [floor(o*T_m/R), floor((o+1)*T_m/R))
 * of the T_m = ceil(M/tile_m) tile rows.  Each owner has an inbox with one
 * slot per other rank: a tile that rank 0 does not own is stored, as the
 * GEMM finishes it, into rank 0's slot at its owner, and rank 0 sums its own
 * tiles and its inbox (peers).  After the call, with own = min(M,
 * floor(T_m/R)*tile_m):
 *     C[i][j]      = (A.B)[i][j] + sum_p peers[p][i][j]   for i < own;
 *     remote[i][j] = (A.B)[i][j]                          for i >= own;
 * rows i >= own of C and rows i < own of remote are left untouched.  Only
 * peers' rows i < own are read.
 *
 *   remote     fp32 [M, N], row-major, 16-byte aligned (device): stands in
 *              for rank 0's inbox slots at the other owners (row i of it in
 *              the slot of row i's owner).  Overwritten on the other ranks'
 *              rows; may be NULL only when rank 0 owns every tile row
 *              (num_peers == 0, M == 0 or N == 0).  Must not overlap A, B,
 *              peers or C (MK_ERR_INVALID_ARG).
 *   Other arguments, layouts and errors as for mk_gemm_reduce_local; the
 *   same partition settings and statistics apply.
 */
int mk_gemm_reduce_scatter_local(const void *A, const void *B, const float *peers, int num_peers,
                                 float *C, float *remote, int64_t M, int64_t N, int64_t K,
                                 int tile_m, int tile_n, int tiles_per_chunk, void *stream);

/*
 * mk_gemm_reduce_scatter_unfused -- the same result from two launches: the
 * GEMM kernel writes rank 0's rows into C and the other rows into `remote`,
 * then one elementwise kernel reduces rank 0's rows.  Arguments as above.
 */
int mk_gemm_reduce_scatter_unfused(const void *A, const void *B, const float *peers, int num_peers,
                                   float *C, float *remote, int64_t M, int64_t N, int64_t K,
                                   int tile_m, int tile_n, int tiles_per_chunk, void *stream);

/*
 * mk_allgather_gemm_local -- one rank's share of AllGather+GEMM in one
 * persistent launch (AllGather + GEMM row of the MarkTechPost page's
 * five-kernel table: every rank holds a shard of A; while the shards are
 * gathered, the local GEMM consumes tiles as they arrive.  "【学习】mKernel
 * 分析" section 2.6, Table 3: communication feeds compute, 128-row chunks,
 * shards submitted at launch, tiles in order of input availability, local
 * first; section 2.4: the same controller sets the communication-role size,
 * and a compute block waiting for its input helps communication).  This
 * rank is rank 0 of R = num_peers + 1; after the call
 *     A_gathered[r*Ms + i][k] = (r == 0 ? A_local[i][k] : A_peers[r-1][i][k])
 *     C[i][j] = sum_k A_gathered[i][k] * B[k][j]        for i < R*Ms.
 * Workgroups take a copy role or a compute role.  A chunk (tile_m rows of a
 * shard) is moved by P_c = min(ceil(2 tile_m K / 64 KiB), tiles per row, 64)
 * copy tasks, each a run of its bytes written through into A_gathered; the
 * task that completes the chunk's count sets its arrival flag.  A compute
 * task is one block of adjacent tiles of one tile row, taken once its chunk
 * has arrived (this rank's own rows read A_local directly).  Copy claims take
 * the other ranks' chunks first (rank, then row), this rank's own last, the
 * parts of a chunk in order; compute claims go in row order, so local rows
 * come first, in one queue per XCD column band when the block columns allow
 * (mk_set_xcd_bands).
 *
 *   A_local    bfloat16 [Ms, K], row-major (device, read only).
 *   A_peers    bfloat16 [num_peers, Ms, K], contiguous, rank 1 first (device,
 *              read only; stands in for the other ranks' shards); NULL only
 *              when num_peers == 0.
 *   A_gathered bfloat16 [R*Ms, K] (device, written).
 *   B          bfloat16 [K, N] (device, read only).
 *   C          fp32 [R*Ms, N] (device, written).
 *   Ms         rows per shard; a multiple of tile_m (a chunk is one tile row).
 *   N, K       multiples of 8.
 *   tile_m, tile_n   64x64, 128x128 or 256x128.
 * Pointers 16-byte aligned; A_gathered and C must not overlap each other or
 * any input (MK_ERR_INVALID_ARG).  Partition (mk_set_partition): the count is
 * the copy role's; adaptive starts at 3B/4 (capped) unless set (0:
 * communication feeds compute, so the data dependency sets a copy-heavy
 * start, and this rank's own rows keep the rest busy), and the cap is B - 1
 * unless mk_set_controller_cap sets one; static copiers
 * leave once every chunk is claimed; the deterministic schedule deals copy
 * tasks (in copy order) round-robin to workgroups [0, n) and compute blocks
 * (row-major) to [n, B).  mk_set_adaptive_help(0) makes a waiting compute
 * workgroup wait instead of copying.  mk_get_stats reports kind 2, with
 * num_chunks = R*Ms/tile_m chunks, tiles_per_chunk = P_c (copy tasks per
 * chunk), compute_tasks = tiles computed, reduce_tasks = copy tasks run,
 * chunks_released = chunks arrived, xcd_bands = compute-claim bands, and in
 * the maps: chunk_flag = arrival flags, chunk_cnt = copy tasks per chunk
 * (P_c per call), tile_reduce_cnt = computations per tile, compute_owner per
 * tile, reduce_owner[c*P_c + p] = the owner of chunk c's copy task p (bit
 * 31: run by a compute workgroup waiting for input), reduce_start/end[same
 * index] = that task's span, chunk_release[c] = when chunk c arrived.
 * Errors as for mk_gemm_reduce_local; MK_ERR_SHAPE also when Ms is not a
 * multiple of tile_m.
 */
int mk_allgather_gemm_local(const void *A_local, const void *A_peers, int num_peers, void *A_gathered,
                            const void *B, float *C, int64_t Ms, int64_t N, int64_t K, int tile_m,
                            int tile_n, void *stream);

/*
 * mk_allgather_gemm_unfused -- the same result from two launches: a gather
 * kernel stacks every shard into A_gathered, then the GEMM kernel computes C
 * from it.  Arguments as above; touches no workspace state.
 */
int mk_allgather_gemm_unfused(const void *A_local, const void *A_peers, int num_peers, void *A_gathered,
                              const void *B, float *C, int64_t Ms, int64_t N, int64_t K, int tile_m,
                              int tile_n, void *stream);

/*
 * mk_ring_attention_local -- one rank's share of Ring Attention in one
 * persistent launch (Ring Attention row of the MarkTechPost page's
 * five-kernel table: sequence-parallel attention; each step passes a KV
 * chunk around the ring while the local FlashAttention consumes the chunk
 * received before, compute and transfer in one persistent kernel.
 * "【学习】mKernel 分析" section 2.6, Table 3: KV moves in 128-row tiles).
 * This rank is rank 0 of R = num_peers + 1; each rank holds S tokens.  After
 * the call, with keys j running over all R*S tokens (this rank's, then each
 * arriving step's) and scale 1/sqrt(D), no causal mask:
 *     O[i][h][:] = sum_j softmax_j(q_i . k_j * scale) v_j
 *     lse[h][i]  = log sum_j exp(q_i . k_j * scale)          (natural log)
 *     k_ring[s-1], v_ring[s-1] = k_peers[s-1], v_peers[s-1]  for every step s.
 * Workgroups take a copy role or a compute role.  A KV tile is 128 tokens of
 * one step's K and V, every head; P_t = min(ceil(2 * 128 * H * D * 2 / 64 KiB),
 * 64) copy tasks move a tile into the ring buffers, written through, and the
 * task that completes the tile's count sets its arrival flag.  Copy tasks go
 * in arrival order (step 1's tiles first).  A compute task is 128 queries of
 * one head against every key: the local K, V at once, then each arriving
 * tile once its flag carries the launch's epoch.
 *
 *   q, k_local, v_local  bfloat16 [S, H, D], row-major (device, read only).
 *   k_peers, v_peers     bfloat16 [num_peers, S, H, D], contiguous, in ring
 *                        arrival order: index s-1 arrives at step s (device,
 *                        read only; stands in for the other ranks' KV); NULL
 *                        only when num_peers == 0.
 *   k_ring, v_ring       bfloat16 [num_peers, S, H, D] (device, written: the
 *                        rank's receive buffers); NULL only when num_peers == 0.
 *   O                    fp32 [S, H, D] (device, written).
 *   lse                  fp32 [H, S] (device, written).
 *   S                    tokens per rank (any; the last tiles are ragged).
 *   H, D                 heads (>= 1) and head dimension (128 only).
 * Pointers 16-byte aligned; outputs must not overlap each other or any input
 * (MK_ERR_INVALID_ARG); S*H*D*4 must stay below 2^31 (MK_ERR_SHAPE).
 * Partition (mk_set_partition): the count is the copy role's; adaptive starts
 * at the cap unless set, and keeps at least one copy workgroup (the floor is
 * at least 1) while copy tasks remain; static copiers leave once every copy
 * task is claimed; the deterministic schedule deals copy tasks in arrival
 * order round-robin to workgroups [0, n) and compute tasks (head-major:
 * head * ceil(S/128) + block) to [n, B).  Compute claims go in one queue per
 * XCD band of heads (head h in band h mod 8) when H >= 8.  mk_get_stats
 * reports kind 3, with num_tiles = the length of the per-task maps
 * (max(compute tasks, copy tasks)), num_chunks = (R-1) ceil(S/128) arriving
 * tiles, tiles_per_chunk = P_t, tile_m = 128 (queries per compute task),
 * tile_n = 128 (tokens per KV tile), compute_tasks = H ceil(S/128),
 * reduce_tasks = copy tasks run, chunks_released = tiles arrived, and in the
 * maps: chunk_flag = arrival flags, chunk_cnt = copy tasks per tile (P_t per
 * call), tile_reduce_cnt[j] = runs of compute task j, compute_owner[j],
 * reduce_owner[t*P_t + p] = the owner of tile t's copy task p,
 * compute_start/end[j], reduce_start/end[t*P_t + p], chunk_release[t] = when
 * tile t arrived.  Errors as for mk_gemm_reduce_local.
 */
int mk_ring_attention_local(const void *q, const void *k_local, const void *v_local, const void *k_peers,
                            const void *v_peers, int num_peers, void *k_ring, void *v_ring, float *O,
                            float *lse, int64_t S, int H, int D, void *stream);

/*
 * mk_ring_attention_unfused -- the same results from two launches: a gather
 * kernel copies every arriving tile into the ring buffers, then the
 * attention kernel (the same core, no flags, one workgroup per CU, tasks
 * dealt round-robin within each head band) computes O and lse.  Arguments as
 * above; touches no workspace state.
 */
int mk_ring_attention_unfused(const void *q, const void *k_local, const void *v_local, const void *k_peers,
                              const void *v_peers, int num_peers, void *k_ring, void *v_ring, float *O,
                              float *lse, int64_t S, int H, int D, void *stream);

/*
 * mk_set_partition -- partition of the persistent workgroups into reduce and
 * compute roles for subsequent mk_gemm_reduce_local launches (process-wide).
 *   mode       mk_part_mode.
 *   n_reduce   STATIC*: reduce-workgroup count, must lie in [1, B-1] at launch
 *              time (B = workgroups of the launch).  ADAPTIVE: initial count,
 *              at most the controller cap (0 selects B/2; reducers with no
 *              tile ready compute meanwhile, so a high start leaves no
 *              workgroup idle).
 * Errors: MK_ERR_INVALID_ARG for an unknown mode or negative n_reduce.
 */
int mk_set_partition(int mode, int n_reduce);

/*
 * mk_set_controller_floor -- smallest reduce count the adaptive controller
 * may choose while compute remains (default 2; clamped to B-1 at run time).
 */
int mk_set_controller_floor(int floor);

/*
 * mk_set_controller_cap -- largest reduce count the adaptive controller may
 * choose while compute remains.  0 (default) = 5B/8: on MI355X the reduce
 * role saturates HBM with about half to five eighths of the CUs (one CU
 * streams 40-57 GB/s), and more reducers only lengthen every reduce task
 * while taking compute units from the tiles they wait for.  Valid: 0..1024; at run time it is
 * clamped to [1, B - keep_compute].  Also bounds the initial adaptive count.
 * Errors: MK_ERR_INVALID_ARG outside 0..1024.
 */
int mk_set_controller_cap(int cap);

/*
 * mk_set_xcd_bands -- column bands of the XCD-local tile partitions.  When
 * every tile stays on its XCD (mk_stats.xcd_local), the blocks are cut into
 * 8 partitions, one per XCD, as px row groups (tile row r in group r mod px)
 * times py = bands column bands of whole chunks, px * py = 8.  An XCD then
 * fetches only the A rows of its row group and the B columns of its band.
 * This assignment of tiles to an 8-L2 GPU is this library's own; the pages
 * fix none ("【学习】mKernel 分析" section 2.2 tiles the output, section 2.3
 * groups tiles into chunks).
 * 0 (default): the most bands the shape allows (eight on every benchmark
 * shape, where it measured fastest); 1, 2, 4 or 8: that split, when the
 * shape allows it (each row group needs a tile row and each band a chunk
 * column of blocks), else the default.  Results do not depend on the split;
 * mk_stats.xcd_bands reports the one used.
 * Errors: MK_ERR_INVALID_ARG for any other value.
 */
int mk_set_xcd_bands(int bands);

/*
 * mk_set_adaptive_help -- 1 (default): under MK_PART_ADAPTIVE, a reduce-role
 * workgroup whose next tile is not published computes a block meanwhile and
 * keeps its reduce ticket ("【学习】mKernel 分析" section 2.4: a block waiting
 * for its input helps the other role).  0: it waits, as in the plain rule.
 * Static partitions never help.  Errors: MK_ERR_INVALID_ARG unless 0 or 1.
 */
int mk_set_adaptive_help(int on);

/*
 * mk_set_num_workgroups -- persistent workgroups per launch (B).  0 (default)
 * = every workgroup that can be resident: the compute-unit count (256 on
 * MI355X) times the workgroups one CU holds for the tile configuration (1 for
 * every configuration, as the runtime's occupancy query confirms).
 * Valid: 0 or 2..1024; at launch time B must not exceed that resident count
 * (every workgroup of the persistent grid must run at once), else the launch
 * fails with MK_ERR_INVALID_ARG.
 */
int mk_set_num_workgroups(int num_wg);

/*
 * mk_set_timeout_us -- bound on every wait inside the fused kernel, in
 * microseconds of GPU constant-rate clock (default 2 000 000).  A workgroup
 * whose wait expires records MK_ERR_TIMEOUT and leaves the kernel; the others
 * see the error and leave too, so the kernel always ends.
 */
int mk_set_timeout_us(uint64_t timeout_us);

/*
 * mk_set_fault_skip_publish -- fault injection for tests: the compute task of
 * tile `tile` writes its partial but never sets its readiness flag, so the
 * launch must end with MK_ERR_TIMEOUT.  -1 (default) disables it.
 */
int mk_set_fault_skip_publish(int64_t tile);

/* Statistics of the most recent fused launch on the device (any kind). */
typedef struct mk_stats {
    uint32_t struct_size;         /* in: sizeof(mk_stats) as the caller knows it */
    int32_t status;               /* MK_OK, MK_ERR_TIMEOUT or MK_ERR_PROTOCOL    */
    uint32_t epoch;               /* epoch value the launch wrote into flags     */
    uint32_t calls_since_reset;   /* launches of this shape since counters reset */
    uint32_t num_wg;              /* B                                           */
    uint32_t num_tiles;           /* T                                           */
    uint32_t num_chunks;          /* ceil(T / tiles_per_chunk)                   */
    uint32_t tiles_per_chunk;
    uint32_t tile_m, tile_n;
    uint32_t mode;                /* mk_part_mode                                */
    uint32_t n_reduce_initial;
    uint32_t n_reduce_final;      /* target when the last workgroup left         */
    uint32_t n_reduce_min_seen;   /* over controller updates and the initial    */
    uint32_t n_reduce_max_seen;
    uint32_t role_switches;       /* workgroups changing role between tasks      */
    uint32_t compute_tasks;       /* tiles computed (== T)                       */
    uint32_t reduce_tasks;        /* tiles reduced (== T)                        */
    uint32_t chunks_released;     /* chunks whose last tile was reduced (== Ch)  */
    uint32_t invariant_violations;/* flag/counter mismatches seen on the device  */
    uint32_t ns_trace_len;        /* entries in the controller trace (the target
                                     changes made by workgroup 0's own steps)  */
    uint32_t tiles_per_task;      /* output tiles of one compute task (a reduce
                                     task is always one tile)                  */
    uint64_t sum_cycles_compute;  /* shader-clock cycles over compute tasks      */
    uint64_t sum_cycles_reduce;   /* shader-clock cycles over reduce tasks       */
    uint64_t kernel_ticks_start;  /* first workgroup start (constant clock)      */
    uint64_t kernel_ticks_end;    /* last workgroup end                          */
    uint64_t reduce_ticks_start;  /* first reduce task start                     */
    uint64_t reduce_ticks_end;    /* last reduce task end                        */
    uint64_t timer_hz;            /* constant clock frequency                    */
    uint32_t xcd_local;           /* 1: every tile stayed on its partition's XCD */
    uint32_t keep_compute;        /* compute workgroups the controller kept      */
    uint32_t controller_cap;      /* most reducers while compute remained        */
    uint32_t xcd_bands;           /* column bands of the XCD partitions (1: rows) */
    uint32_t adaptive_help;       /* 1: waiting reducers computed meanwhile        */
    uint32_t sticky_errors;       /* bit 0 timeout, 1 XCD mismatch, 2 protocol:
                                     every kind raised by any launch since the
                                     last mk_get_stats (see there)             */
    uint32_t kind;                /* 0 GEMM+AllReduce, 1 GEMM+ReduceScatter,
                                     2 AllGather+GEMM, 3 Ring Attention (see
                                     mk_allgather_gemm_local and
                                     mk_ring_attention_local for how their
                                     statistics map onto these)              */
} mk_stats;

/* Words per map in the optional `maps` output of mk_get_stats, in order:
 *   tile_flag[T] | tile_reduce_cnt[T] | chunk_cnt[Ch] | chunk_flag[Ch] |
 *   compute_owner[T] | reduce_owner[T] | ns_trace[2 * MK_TRACE_CAP] |
 *   compute_start[T] | compute_end[T] | reduce_start[T] | reduce_end[T] |
 *   compute_choice_ticks[T] | reduce_choice_ticks[T] | chunk_release[Ch]
 * Owner words are (help << 31) | (reduce target seen << 16) | workgroup, where
 * help marks a compute task taken by a workgroup waiting on a reduce ticket
 * (adaptive mode only).  Trace entries are
 * pairs (low 32 bits of the constant clock, new target), one for each step
 * of workgroup 0 that changed the target: a sample of the target's path.  The four timeline
 * maps hold the low 32 bits of the constant clock at each task's start and
 * end (compare with kernel_ticks_start modulo 2^32); the next two, the ticks
 * the workgroup spent choosing the task (claim and readiness wait).
 * chunk_release[c] is the constant clock (low 32 bits) at which chunk c was
 * released: its last tile's counters came back after that tile's stores had
 * drained, write-through, at device scope ("【学习】mKernel 分析" section 2.3:
 * the last reduced tile lets the chunk go at once). */
#define MK_TRACE_CAP 1024

/*
 * mk_get_stats -- waits for all work on the current device
 * (hipDeviceSynchronize), then fills *out with the statistics of the last
 * fused launch.  If maps is non-NULL it receives the maps above (maps_len is
 * its capacity in uint32 words; it must hold 10T + 3Ch + 2*MK_TRACE_CAP
 * words).  out->struct_size must be set.
 * Errors are sticky: out->status and the return value report every timeout,
 * XCD mismatch or flag/counter violation raised by ANY fused launch on this
 * device since the previous mk_get_stats (MK_ERR_PROTOCOL for an XCD
 * mismatch or violations, MK_ERR_TIMEOUT for a timeout), not only by the
 * last one; out->sticky_errors names the kinds.  Reporting an error marks the
 * workspace so that the next launch starts from a cleared control block and
 * cleared per-call counters.  Otherwise returns MK_OK, or an argument/HIP
 * error.
 */
int mk_get_stats(mk_stats *out, uint32_t *maps, size_t maps_len);

/*
 * mk_controller_eval -- evaluates the device's controller step on a table,
 * for parity tests against the host closed form.  `in` holds n rows of ten
 * uint64 (device memory): B, T, compute_done, reduce_done,
 * sum_cycles_compute, sum_cycles_reduce, current_target, floor, keep (compute
 * workgroups the clamp keeps while compute remains: 1, or one per XCD when
 * tiles stay on their XCD), cap (most reducers while compute remains).
 * `out` (device, n uint32) receives the new target for each row.  Limits:
 * B in [2, 1024], T < 2^22, 1 <= keep < B, cap >= 1.
 * Asynchronous on `stream`.
 */
int mk_controller_eval(const uint64_t *in, uint32_t *out, int n, void *stream);

/* Number of compute units of the current device, or a negative mk_status. */
int mk_device_cu_count(void);

/* Frees the current device's workspace (the next launch allocates anew). */
int mk_release_workspace(void);

/* Text of the last error on the calling thread ("" if none). */
const char *mk_last_error(void);

/* MK_ABI_VERSION of the built library. */
int mk_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MK_H */
