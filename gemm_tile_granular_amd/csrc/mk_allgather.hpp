// Host/device interface of the AllGather+GEMM share (mk_allgather.hip).
#pragma once
#include "mk_internal.hpp"

namespace mk {

// One rank's share of AllGather+GEMM: this rank's shard A_local [Ms, K], the
// other ranks' shards A_peers [P, Ms, K] (rank 1 first), the gathered A
// [R Ms, K] (output, shards stacked by rank) and C = gathered . B [R Ms, N].
// A chunk is one tile row of A (TM rows); chunk c holds rows [c TM, (c+1) TM).
// Its bytes are moved by `parts` copy tasks; task u = c parts + p moves the
// p-th of `parts` near-equal runs of the chunk's 16-byte pieces.
struct AgArgs {
    const uint16_t *A_local;
    const uint16_t *A_peers;
    uint16_t *A_gath;
    const uint16_t *B;
    float *C;
    int64_t Ms, M, N, K;      // M = R Ms
    int32_t P;
    uint32_t cps;             // chunks per shard (Ms / TM)
    uint32_t Ch;              // chunks: R cps
    uint32_t parts;           // copy tasks per chunk (consecutive pieces of its bytes)
    uint32_t Q;               // copy tasks: Ch parts
    uint32_t tiles_n, bn;     // tiles per tile row, compute blocks per tile row
    uint32_t bands;           // column bands of the compute claims (1: one row-major queue)
    uint32_t T, TB;           // tiles, compute blocks
    uint32_t Tcap;
    uint32_t epoch, calls;
    int32_t mode, ns_init, ns_floor, ns_cap, nwg, help;
    uint64_t timeout_ticks;
    int64_t skip_publish;     // fault injection: chunk whose arrival flag is never set (-1 none)
    WsView ws;
};

// Host-side launchers (defined in mk_allgather.hip).  Return hipSuccess or
// the launch error.
hipError_t launch_allgather_gemm(int tile_m, int tile_n, const AgArgs &a, hipStream_t s);
// gather every shard into A_gath (the unfused baseline's first kernel)
hipError_t launch_gather(const AgArgs &a, int num_cu, hipStream_t s);
int allgather_workgroups_per_cu(int tile_m, int tile_n);

}  // namespace mk
