// Internal definitions shared by the kernels (mk_kernels.hip) and the C ABI
// (mk_api.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

constexpr int kBK = 64;               // K slab staged in LDS per pipeline step
constexpr int kMaxWG = 1024;
constexpr uint32_t kMaxTiles = 1u << 22;
constexpr uint64_t kCostCap = (1ull << 26) - 1;   // per-task mean cycles saturate here
constexpr int kTraceCap = 1024;
constexpr int kMaxXcd = 8;            // XCDs on MI355X (tile partitions)

enum Mode : int32_t { kAdaptive = 0, kStatic = 1, kDeterministic = 2 };
enum Err : uint32_t { kErrNone = 0, kErrTimeout = 1, kErrXcd = 2 };
// Bits of the sticky error word: every kind of error any launch raised since
// the word was last cleared (by mk_get_stats, through a workspace reinit).
constexpr uint32_t kStickyTimeout = 1u << 0;
constexpr uint32_t kStickyXcd = 1u << 1;
constexpr uint32_t kStickyProtocol = 1u << 2;

// Per-launch control block in device memory.  The last workgroup to leave a
// launch copies it into the snapshot and restores the initial values below,
// so every launch starts from the same state without a host-side clear.
// Each role's progress is one 64-bit word, (cycle sum << kCountBits) | tasks,
// so one atomic both records a finished task and returns what the controller
// needs.
constexpr int kCountBits = 22;
constexpr uint64_t kCountMask = (1ull << kCountBits) - 1;

// A counter on a 256-byte line of its own.  Every workgroup hits the claim
// counters, the role words and the target once per task; kept apart they do
// not serialise behind each other's atomics.
template <class T> struct alignas(256) Line {
    T v;
};

struct alignas(256) Live {
    Line<uint32_t> compute_claim[kMaxXcd];  // next compute claim per partition (init 0)
    Line<uint32_t> reduce_claim[kMaxXcd];   // next reduce ticket per partition (init 0)
    Line<uint32_t> extra_claim[kMaxXcd];  // reduce-scatter: next block outside the shard, per
                                          // column band of the outside rows (init 0)
    Line<uint64_t> role_compute;   // (cycles << kCountBits) | tasks      (init 0)
    Line<uint64_t> role_reduce;    //                                     (init 0)
    Line<uint32_t> target_ns;      // controller target, 0 = unset        (init 0)
    Line<uint32_t> chunks_released;//                                     (init 0)
    uint64_t r_start;          // min over reduce tasks              (init ~0)
    uint64_t r_end;            // max                                (init 0)
    alignas(256) uint32_t exit_count;  // workgroups that left       (init 0)
    uint32_t role_switches;    //                                    (init 0)
    uint32_t violations;       //                                    (init 0)
    uint32_t error;            // Err                                (init 0)
    uint32_t ns_min;           //                                    (init ~0)
    uint32_t ns_max;           //                                    (init 0)
    uint32_t trace_len;        // written by workgroup 0 at exit     (init 0)
    uint32_t ns_final;         // written at exit                    (init 0)
    uint32_t sticky;           // kSticky* bits; NOT restored at launch end (init 0)
    uint64_t t_start;          // min over workgroups                (init ~0)
    uint64_t t_end;            // max                                (init 0)
};

// Workspace: one device allocation per device.
//   [Live][Live snapshot][trace 2*kTraceCap u32]
//   [tile_flag Tcap][tile_cnt Tcap][chunk_cnt Chcap][chunk_flag Chcap]
//   [chunk_release Chcap][compute_owner Tcap][reduce_owner Tcap][timeline 6*Tcap]
struct WsView {
    Live *live;
    Live *snap;
    uint32_t *trace;
    uint32_t *tile_flag;
    uint32_t *tile_cnt;
    uint32_t *chunk_cnt;
    uint32_t *chunk_flag;
    uint32_t *chunk_release;   // constant-clock ticks (low 32 bits) of each chunk's release
    uint32_t *cowner;
    uint32_t *rowner;
    uint32_t *timeline;   // [6][Tcap]: compute start/end, reduce start/end, choice time compute/reduce
};

struct FusedArgs {
    const uint16_t *A;        // bf16 [M,K]
    const uint16_t *B;        // bf16 [K,N]
    const float *peers;       // fp32 [P,M,N]
    float *C;                 // fp32 [M,N]
    int64_t M, N, K;
    int32_t P;
    int32_t tiles_m, tiles_n;
    uint32_t T, tpc, Ch;
    uint32_t Tcap;            // workspace tile capacity (stride of the timeline rows)
    uint32_t epoch;           // value written into flags this launch
    uint32_t calls;           // launches of this shape since the counters were cleared
    int32_t mode;
    int32_t ns_init;          // static count, or initial adaptive target
    int32_t ns_floor;
    int32_t nwg;              // B
    int32_t group_m;          // tile-row band height of the claim order
    int32_t nxcd;             // tile partitions (XCDs) for the claim order
    int32_t local;            // 1: every tile is computed and reduced on its partition's XCD
    int32_t xcd_cols;         // local: column bands of the XCD partitions (1: whole tile rows)
    // reduce-scatter: M and tiles_m above are this rank's shard, the
    // protocol's whole extent; tile rows [tiles_m, tiles_m_all) of the
    // [M_all, N] product are plain GEMM blocks stored into `remote` (this
    // rank's inbox slots at the other owners).  GEMM+AllReduce: remote is
    // NULL and M_all == M.
    float *remote;
    int64_t M_all;
    int32_t tiles_m_all;
    int64_t peer_mn;          // elements between consecutive peers ([P, M_all, N])
    int32_t keep;             // compute workgroups the controller keeps while compute remains
    int32_t ns_cap;           // most reduce workgroups the controller sets while compute remains
    uint64_t timeout_ticks;   // bound on any wait, constant-clock ticks
    int64_t skip_publish;     // fault injection: tile whose flag is never set (-1 none)
    int32_t help;             // adaptive: a reducer whose ticket is not ready computes meanwhile
    WsView ws;
};

struct GemmArgs {
    const uint16_t *A;
    const uint16_t *B;
    float *C;
    int64_t M, N, K;
    int32_t tiles_m, tiles_n;
    int32_t tpc, group_m;
    int32_t nxcd;
    int32_t xcd_cols;         // column bands of the partitions (1: whole tile rows)
    int32_t own_tile_rows;    // tile rows [0, own) go to C, the rest to `remote` (reduce-scatter)
    float *remote;            // reduce-scatter: this rank's inbox slots at the other owners
};

struct ReduceArgs {
    const float *peers;
    float *C;
    int64_t count4;           // M*N/4 float4 elements
    int64_t own4;             // float4 elements reduced (the first own4; count4 for GEMM+AllReduce)
    int64_t MN;
    int32_t P;
};

// Host-side launchers (defined in mk_kernels.hip).  Return hipSuccess or the
// launch error.
hipError_t launch_fused(int tile_m, int tile_n, const FusedArgs &a, hipStream_t s);
hipError_t launch_gemm(int tile_m, int tile_n, const GemmArgs &a, int num_cu, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs &a, int num_cu, hipStream_t s);
hipError_t launch_ws_init(Live *live, Live *snap, hipStream_t s);
hipError_t launch_fill_u32(uint32_t *p, uint32_t value, int64_t n, hipStream_t s);
hipError_t launch_controller_eval(const uint64_t *in, uint32_t *out, int n, hipStream_t s);
hipError_t launch_xcc_probe(uint32_t *out, int nwg, hipStream_t s);   // XCD of each workgroup
bool tile_supported(int tile_m, int tile_n);
int tiles_per_block(int tile_m, int tile_n);   // output tiles per compute task
int workgroups_per_cu(int tile_m, int tile_n); // fused workgroups resident per CU

}  // namespace mk
