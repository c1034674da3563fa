// Host/device interface of the Ring Attention share (mk_ring.hip).
#pragma once
#include "mk_internal.hpp"

namespace mk {

// One rank's share of Ring Attention: this rank's Q, K, V [S, H, D] and the
// K, V of the other ranks in ring arrival order [R-1, S, H, D] (peers[s-1]
// arrives at step s).  The copy role moves each arriving KV tile (128 tokens,
// every head, K and V) into k_ring / v_ring [R-1, S, H, D] and flags it; a
// compute task is 128 queries of one head against every key, reading step 0
// from k_local / v_local and step s from the ring buffers once each tile's
// flag carries the launch's epoch.  Outputs O [S, H, D] and LSE [H, S] fp32.
struct RaArgs {
    const uint16_t *q;
    const uint16_t *k_local;
    const uint16_t *v_local;
    const uint16_t *k_peers;
    const uint16_t *v_peers;
    uint16_t *k_ring;
    uint16_t *v_ring;
    float *O;
    float *lse;
    int64_t S;                // tokens per rank
    int32_t H, R;             // heads, ranks
    uint32_t nkv;             // KV tiles (128 tokens) per step
    uint32_t nqb;             // query blocks (128 queries) per head
    uint32_t Ch;              // arriving KV tiles: (R - 1) nkv
    uint32_t parts;           // copy tasks per KV tile
    uint32_t Qc;              // copy tasks: Ch parts
    uint32_t NTk;             // compute tasks: H nqb
    uint32_t bands;           // compute-claim bands (head h in band h mod bands)
    uint32_t Tcap;
    uint32_t epoch, calls;
    int32_t mode, ns_init, ns_floor, ns_cap, nwg;
    float scale_log2;         // log2(e) / sqrt(D)
    uint64_t timeout_ticks;
    int64_t skip_publish;     // fault injection: KV tile whose arrival flag is never set (-1 none)
    WsView ws;
};

constexpr int kRaHeadDim = 128;   // the head dimension the kernels are built for
constexpr int kRaKvRows = 128;    // tokens per KV tile (the transfer unit)
constexpr int kRaQRows = 128;     // queries per compute task

// Host-side launchers (defined in mk_ring.hip).  Return hipSuccess or the
// launch error.
hipError_t launch_ring_attention(const RaArgs &a, hipStream_t s);
// the unfused baseline: every arriving tile into the ring buffers, then the
// attention kernel over all of them (same core, no flags)
hipError_t launch_ring_unfused(const RaArgs &a, int num_cu, bool xcd_bands, hipStream_t s);
int ring_workgroups_per_cu();

}  // namespace mk
