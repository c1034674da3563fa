// C ABI of the fused GEMM + tile-reduce library (declarations and contracts
// in include/mk.h).  Host side only: argument checks, the per-device
// workspace (flags, counters, owner maps, control block), epochs, launches
// and statistics.  Every check that can fail on the caller's arguments runs
// before the first HIP call.
#include <algorithm>
#include <cstdarg>
#include <mutex>
#include <cstring>
#include <cstdio>
#include <cmath>

#include "mk.h"
#include "mk_internal.hpp"
#include "mk_allgather.hpp"
#include "mk_ring.hpp"

namespace {

using namespace mk;

// fixed buffer: recording an error allocates nothing
thread_local char g_last_error[512];
std::mutex g_mu;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    std::memcpy(g_last_error, buf, sizeof g_last_error);
    g_last_error[sizeof g_last_error - 1] = '\0';
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(MK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct Settings {
    int mode = MK_PART_ADAPTIVE;
    int n_reduce = 0;
    int floor = 2;
    int cap = 0;              // 0: five eighths of the workgroups
    int num_wg = 0;
    uint64_t timeout_us = 2000000;
    int64_t skip_publish = -1;
    int group_m = 8;
    int xcd_bands = 0;        // 0: the most column bands the shape allows
    int help = 1;             // adaptive: waiting reducers compute meanwhile
};
Settings g_set;

constexpr int kMaxDevices = 64;

struct Launch {
    bool valid = false;
    uint32_t kind = 0;   // 0 GEMM+AllReduce, 1 GEMM+ReduceScatter, 2 AllGather+GEMM, 3 Ring Attention
    uint32_t epoch = 0, calls = 0, nwg = 0, T = 0, Ch = 0, tpc = 0, tm = 0, tn = 0;
    uint32_t mode = 0, ns_init = 0;
    uint32_t local = 0, keep = 1, cap = 0, bands = 1, help = 1;
};

// Flags, counters, maps and control block of the fused launches, plus the
// host-side bookkeeping of the epochs and calls made on them.  Each device
// has two: one allocated (and grown) by the library, and one in the static
// device array below, used only by mk_gemm_reduce_local_noalloc.
struct Workspace {
    char *ws = nullptr;
    size_t ws_bytes = 0;
    uint32_t Tcap = 0, Chcap = 0;
    uint32_t epoch = 0;
    uint32_t calls = 0;
    uint32_t shape_T = 0, shape_tpc = 0;
    bool dirty = false;
    bool fixed = false;    // the static array: never freed, never grown
    Launch last;
};

struct DevState {
    bool init = false;
    int num_cu = 0;
    uint64_t timer_hz = 100000000ull;
    bool xcd_ok = false;   // workgroup w of a one-per-CU grid runs on XCD w mod 8
    char *fixed_base = nullptr;   // this device's copy of `scratch` (hipGetSymbolAddress)
    Workspace heap, fixed;
    Workspace *recent = nullptr;  // the workspace of the last fused launch
};
DevState g_dev[kMaxDevices];

constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
    size_t live, snap, trace, tile_flag, tile_cnt, chunk_cnt, chunk_flag, chunk_release, cowner, rowner,
        timeline, total;
};

constexpr Layout layout_for(uint32_t Tcap, uint32_t Chcap) {
    Layout L{};
    size_t o = 0;
    L.live = o; o += sizeof(Live);
    L.snap = o; o += sizeof(Live);
    L.trace = o; o = align_up(o + 2 * sizeof(uint32_t) * kTraceCap, 256);
    L.tile_flag = o; o = align_up(o + 4ull * Tcap, 256);
    L.tile_cnt = o; o = align_up(o + 4ull * Tcap, 256);
    L.chunk_cnt = o; o = align_up(o + 4ull * Chcap, 256);
    L.chunk_flag = o; o = align_up(o + 4ull * Chcap, 256);
    L.chunk_release = o; o = align_up(o + 4ull * Chcap, 256);
    L.cowner = o; o = align_up(o + 4ull * Tcap, 256);
    L.rowner = o; o = align_up(o + 4ull * Tcap, 256);
    L.timeline = o; o = align_up(o + 24ull * Tcap, 256);
    L.total = o;
    return L;
}

// The allocation-free entry point's workspace: a static device array, one
// copy per device, kept until the process ends.  Capacity: 8192 tiles and
// 8192 chunks (every workload here has at most 4096 tiles), about 0.4 MiB.
// Host code never passes the array's name to a kernel or a copy (on the host
// it is only a stand-in for the symbol): each device's copy is reached
// through the address hipGetSymbolAddress returns for it (DevState::fixed_base).
constexpr uint32_t kFixedTiles = 8192;
constexpr uint32_t kFixedChunks = 8192;
constexpr size_t kFixedBytes = layout_for(kFixedTiles, kFixedChunks).total;
static_assert(kFixedBytes >= sizeof(uint32_t) * kMaxWG, "the XCD probe writes one word per workgroup");
static __device__ __align__(256) char scratch[kFixedBytes];

WsView view_of(const Workspace &d) {
    const Layout L = layout_for(d.Tcap, d.Chcap);
    WsView v;
    v.live = (Live *)(d.ws + L.live);
    v.snap = (Live *)(d.ws + L.snap);
    v.trace = (uint32_t *)(d.ws + L.trace);
    v.tile_flag = (uint32_t *)(d.ws + L.tile_flag);
    v.tile_cnt = (uint32_t *)(d.ws + L.tile_cnt);
    v.chunk_cnt = (uint32_t *)(d.ws + L.chunk_cnt);
    v.chunk_flag = (uint32_t *)(d.ws + L.chunk_flag);
    v.chunk_release = (uint32_t *)(d.ws + L.chunk_release);
    v.cowner = (uint32_t *)(d.ws + L.cowner);
    v.rowner = (uint32_t *)(d.ws + L.rowner);
    v.timeline = (uint32_t *)(d.ws + L.timeline);
    return v;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Partitions of the claim order: one per XCD (workgroup w runs on XCD w mod 8
// on MI355X) when the grid spans whole XCDs, else a single partition.
int xcd_partitions(int nwg, int num_cu) {
    return (num_cu % kMaxXcd == 0 && nwg >= 2 * kMaxXcd && nwg % kMaxXcd == 0) ? kMaxXcd : 1;
}

// Column bands of the XCD-local partitions: nxcd = px * py, px row groups
// (each must hold a tile row) by py bands of whole chunks (each must hold a
// chunk column of blocks; py = 1 is whole rows).  An XCD fetches the A rows
// of its row group and the B columns of its band.  The default is the most
// bands the shape allows: on all four benchmark shapes the fused kernel ran
// fastest with eight bands (1-6% over whole rows), square shapes included,
// where the operand traffic py*M + px*N of each split is the same or larger.
// `want`, when that split is valid, overrides.  0: no valid split.
int xcd_bands(int nxcd, int tiles_m, int tiles_n, int tile_m, int tile_n, int tpc, int want) {
    const int tpb = tiles_per_block(tile_m, tile_n);
    const int bn = (tiles_n + tpb - 1) / tpb;            // blocks per block row
    const int cb = (tpc % tpb == 0) ? tpc / tpb : 1;      // blocks per chunk
    int best = 0, forced = 0;
    for (int py = 1; py <= nxcd; py *= 2) {
        if (nxcd % py != 0 || tiles_m < nxcd / py) continue;
        if (py > 1 && (bn % cb != 0 || bn / cb < py)) continue;
        best = py;
        if (py == want) forced = py;
    }
    return forced ? forced : best;
}

// The same for the persistent GEMM of the unfused baseline, whose blocks are
// taken in one interleaved order (partition w mod 8 for workgroup w): a split
// with py > 1 is used only when every partition is the same size.
int gemm_xcd_bands(int nxcd, int tiles_m, int tiles_n, int tile_m, int tile_n, int tpc, int want) {
    const int tpb = tiles_per_block(tile_m, tile_n);
    const int bn = (tiles_n + tpb - 1) / tpb;
    const int cb = (tpc % tpb == 0) ? tpc / tpb : 1;
    int py = xcd_bands(nxcd, tiles_m, tiles_n, tile_m, tile_n, tpc, want);
    while (py > 1 && (tiles_m % (nxcd / py) != 0 || (bn / cb) % py != 0)) py /= 2;
    return py > 0 ? py : 1;
}

// All argument checks that do not need the GPU.
// Byte ranges [p, p + pb) and [q, q + qb) share a byte (NULL or empty: never).
bool overlaps(const void *p, int64_t pb, const void *q, int64_t qb) {
    if (!p || !q || pb <= 0 || qb <= 0) return false;
    const uint64_t a = (uint64_t)(uintptr_t)p, b = (uint64_t)(uintptr_t)q;
    return a < b + (uint64_t)qb && b < a + (uint64_t)pb;
}

int check_args(const void *A, const void *B, const float *peers, int num_peers, const float *C,
               int64_t M, int64_t N, int64_t K, int tile_m, int tile_n, int tpc) {
    if (M < 0 || N < 0 || K < 0) return fail(MK_ERR_INVALID_ARG, "negative dimension");
    if (num_peers < 0) return fail(MK_ERR_INVALID_ARG, "num_peers < 0");
    if (!tile_supported(tile_m, tile_n))
        return fail(MK_ERR_INVALID_ARG, "tile %dx%d not supported (64x64, 128x128, 256x128)",
                    tile_m, tile_n);
    if (tpc < 1 || tpc > 64) return fail(MK_ERR_INVALID_ARG, "tiles_per_chunk must be in [1, 64]");
    if (N % 8 != 0 || K % 8 != 0)
        return fail(MK_ERR_SHAPE, "N (%lld) and K (%lld) must be multiples of 8", (long long)N,
                    (long long)K);
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return fail(MK_ERR_SHAPE, "dimension exceeds 2^31-1");
    if (M == 0 || N == 0) return MK_OK;
    // byte offsets inside one tile's row band (and one K slab) stay below 2^31
    // (32-bit buffer offsets)
    if ((int64_t)tile_m * N * 4 >= (int64_t)INT32_MAX || (int64_t)tile_m * K * 2 >= (int64_t)INT32_MAX ||
        (int64_t)64 * N * 2 >= (int64_t)INT32_MAX)
        return fail(MK_ERR_SHAPE, "N (%lld) or K (%lld) too large for 32-bit in-tile offsets",
                    (long long)N, (long long)K);
    const int64_t T = ((M + tile_m - 1) / tile_m) * ((N + tile_n - 1) / tile_n);
    if (T >= (int64_t)kMaxTiles) return fail(MK_ERR_SHAPE, "too many tiles (%lld)", (long long)T);
    if (!C) return fail(MK_ERR_INVALID_ARG, "C is NULL");
    if (K > 0 && (!A || !B)) return fail(MK_ERR_INVALID_ARG, "A or B is NULL");
    if (num_peers > 0 && !peers) return fail(MK_ERR_INVALID_ARG, "peers is NULL with num_peers > 0");
    if (num_peers == 0 && peers) return fail(MK_ERR_INVALID_ARG, "peers must be NULL when num_peers == 0");
    if (!aligned16(C) || (A && !aligned16(A)) || (B && !aligned16(B)) || (peers && !aligned16(peers)))
        return fail(MK_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    const int64_t cb = M * N * 4;
    if (overlaps(C, cb, A, M * K * 2) || overlaps(C, cb, B, K * N * 2) ||
        overlaps(C, cb, peers, (int64_t)num_peers * M * N * 4))
        return fail(MK_ERR_INVALID_ARG, "C overlaps A, B or peers");
    return MK_OK;
}

int current_device(int *dev) {
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count == 0) {
        (void)hipGetLastError();
        return fail(MK_ERR_NO_DEVICE, "no HIP device visible");
    }
    e = hipGetDevice(dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (*dev < 0 || *dev >= kMaxDevices) return fail(MK_ERR_NO_DEVICE, "device index out of range");
    return MK_OK;
}

// Whether workgroups are dealt to XCDs round-robin (workgroup w on XCD
// w mod 8), read from each workgroup's XCC id register once per device.
// Tiles are kept on one XCD only when this holds.  The probe writes into the
// device's static array (before any workspace lives there), so setting up a
// device allocates nothing.
int probe_xcd_mapping(DevState &d) {
    d.xcd_ok = false;
    if (d.num_cu <= 0 || d.num_cu % kMaxXcd != 0 || d.num_cu > kMaxWG) return MK_OK;
    uint32_t *buf = (uint32_t *)d.fixed_base;
    uint32_t host[kMaxWG];
    hipError_t e = launch_xcc_probe(buf, d.num_cu, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(host, buf, sizeof(uint32_t) * (size_t)d.num_cu, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "xcd probe");
    bool ok = true;
    for (int w = 0; w < d.num_cu; ++w) ok = ok && host[w] == (uint32_t)(w % kMaxXcd);
    d.xcd_ok = ok;
    return MK_OK;
}

int device_state(DevState **out) {
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    DevState &d = g_dev[dev];
    if (!d.init) {
        hipDeviceProp_t prop;
        hipError_t e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        d.num_cu = prop.multiProcessorCount;
        int khz = 0;
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0)
            d.timer_hz = (uint64_t)khz * 1000ull;
        // this device's copy of the static array: its address, not the
        // host-side symbol, is what kernels and copies are given
        void *base = nullptr;
        e = hipGetSymbolAddress(&base, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !base) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        d.fixed_base = (char *)base;
        rc = probe_xcd_mapping(d);
        if (rc) return rc;
        d.init = true;
    }
    *out = &d;
    return MK_OK;
}

// Zero a workspace (flags at 0 never equal an epoch, which starts at 1), set
// its control blocks and restart its bookkeeping.  Fill kernels, not
// hipMemsetAsync, so the sequence stays valid inside a captured graph.
int clear_workspace(Workspace &d, hipStream_t s) {
    const Layout L = layout_for(d.Tcap, d.Chcap);
    hipError_t e = launch_fill_u32((uint32_t *)d.ws, 0u, (int64_t)(L.total / 4), s);
    if (e != hipSuccess) return hip_fail(e, "workspace clear launch");
    WsView v = view_of(d);
    e = launch_ws_init(v.live, v.snap, s);
    if (e != hipSuccess) return hip_fail(e, "workspace init launch");
    d.epoch = 0;
    d.calls = 0;
    d.shape_T = 0;
    d.shape_tpc = 0;
    d.dirty = false;
    d.last.valid = false;
    return MK_OK;
}

// The static workspace: its capacity is fixed, it is set up on its first
// use, and a launch that needs more is refused.
int ensure_fixed_workspace(DevState &dev, uint32_t T, uint32_t Ch, hipStream_t s) {
    Workspace &d = dev.fixed;
    if (T > kFixedTiles || Ch > kFixedChunks)
        return fail(MK_ERR_SHAPE,
                    "%u tiles / %u chunks exceed the allocation-free workspace (at most %u tiles and "
                    "%u chunks); use mk_gemm_reduce_local", T, Ch, kFixedTiles, kFixedChunks);
    if (d.ws) return MK_OK;
    d.ws = dev.fixed_base;
    d.fixed = true;
    d.Tcap = kFixedTiles;
    d.Chcap = kFixedChunks;
    d.ws_bytes = layout_for(kFixedTiles, kFixedChunks).total;
    return clear_workspace(d, s);
}

// Make room for T tiles and Ch chunks in the library's own workspace; a new
// one is cleared.
int ensure_workspace(Workspace &d, uint32_t T, uint32_t Ch, hipStream_t s) {
    if (d.ws && T <= d.Tcap && Ch <= d.Chcap) return MK_OK;
    uint32_t Tcap = d.Tcap, Chcap = d.Chcap;
    while (Tcap < T) Tcap = Tcap ? 2 * Tcap : 4096;
    while (Chcap < Ch) Chcap = Chcap ? 2 * Chcap : 1024;
    if (d.ws) {
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
        e = hipFree(d.ws);
        d.ws = nullptr;
        if (e != hipSuccess) return hip_fail(e, "hipFree");
    }
    const Layout L = layout_for(Tcap, Chcap);
    hipError_t e = hipMalloc((void **)&d.ws, L.total);
    if (e != hipSuccess) {
        d.ws = nullptr;
        return hip_fail(e, "hipMalloc(workspace)");
    }
    d.ws_bytes = L.total;
    d.Tcap = Tcap;
    d.Chcap = Chcap;
    return clear_workspace(d, s);
}

// Per-launch bookkeeping of a workspace: a clean control block after an
// early-ended launch, per-call counters cleared when the shape changes (`key`
// tells the launch kinds and chunk sizes apart: counters of one kind mean
// nothing to another), flags cleared before the epoch wraps; then the
// launch's epoch and call number.
int prepare_launch(Workspace &d, uint32_t T, uint32_t key, hipStream_t s) {
    WsView v = view_of(d);
    hipError_t e;
    if (d.dirty) {
        // a launch ended early: control block and counters are not trustworthy
        e = launch_ws_init(v.live, v.snap, s);
        if (e != hipSuccess) return hip_fail(e, "workspace reinit launch");
        d.shape_T = 0;
        d.dirty = false;
    }
    if (T != d.shape_T || key != d.shape_tpc) {
        // new shape: per-call counters restart from zero (flags are epoch
        // valued and need no clearing)
        e = launch_fill_u32(v.tile_cnt, 0, d.Tcap, s);
        if (e == hipSuccess) e = launch_fill_u32(v.chunk_cnt, 0, d.Chcap, s);
        if (e != hipSuccess) return hip_fail(e, "counter clear launch");
        d.calls = 0;
        d.shape_T = T;
        d.shape_tpc = key;
    }
    if (d.epoch == 0xFFFFFFFFu) {
        e = launch_fill_u32(v.tile_flag, 0, d.Tcap, s);
        if (e == hipSuccess) e = launch_fill_u32(v.chunk_flag, 0, d.Chcap, s);
        if (e != hipSuccess) return hip_fail(e, "flag clear launch");
        d.epoch = 0;
    }
    d.epoch += 1;
    d.calls += 1;
    return MK_OK;
}

// `rs`: one rank's share of GEMM+ReduceScatter (rank 0 of num_peers + 1):
// tile rows [0, floor(tiles_m / R)) are computed into C and reduced there;
// the GEMM stores every other tile row straight into `remote` (this rank's
// inbox slots at the other owners) and leaves those rows of C untouched.
// Otherwise GEMM+AllReduce.
// `noalloc`: the fused launch uses the device's static workspace and the
// call allocates nothing.
int run(bool fused, bool rs, const void *A, const void *B, const float *peers, int num_peers, float *C,
        float *remote, int64_t M, int64_t N, int64_t K, int tile_m, int tile_n, int tpc, void *stream,
        bool noalloc = false) {
    int rc = check_args(A, B, peers, num_peers, C, M, N, K, tile_m, tile_n, tpc);
    if (rc) return rc;
    if (!rs && remote) return fail(MK_ERR_INVALID_ARG, "remote is for reduce-scatter only");
    if (rs && M > 0 && N > 0) {
        const int64_t tm = (M + tile_m - 1) / tile_m;
        const int64_t own = tm / (num_peers + 1);
        if (own < tm && num_peers > 0 && !remote)
            return fail(MK_ERR_INVALID_ARG, "remote is NULL while other ranks own tile rows");
        if (remote && !aligned16(remote))
            return fail(MK_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
        const int64_t rb = M * N * 4;
        if (overlaps(remote, rb, A, M * K * 2) || overlaps(remote, rb, B, K * N * 2) ||
            overlaps(remote, rb, peers, (int64_t)num_peers * M * N * 4) || overlaps(remote, rb, C, rb))
            return fail(MK_ERR_INVALID_ARG, "remote overlaps A, B, peers or C");
    }
    if (M == 0 || N == 0) return MK_OK;
    const Settings set = g_set;
    DevState *dp = nullptr;
    rc = device_state(&dp);
    if (rc) return rc;
    DevState &dev = *dp;
    hipStream_t s = (hipStream_t)stream;

    const int tiles_m_all = (int)((M + tile_m - 1) / tile_m);
    const int own_tile_rows = rs ? tiles_m_all / (num_peers + 1) : tiles_m_all;
    const int tiles_n = (int)((N + tile_n - 1) / tile_n);

    // A rank that owns no tile row has nothing to reduce: the GEMM alone
    // stores every tile into the other owners' inboxes.
    if (!fused || own_tile_rows == 0) {
        const int tiles_m = tiles_m_all;
        GemmArgs g;
        g.A = (const uint16_t *)A;
        g.B = (const uint16_t *)B;
        g.C = C;
        g.M = M;
        g.N = N;
        g.K = K;
        g.tiles_m = tiles_m;
        g.tiles_n = tiles_n;
        g.tpc = tpc;
        g.group_m = set.group_m;
        g.own_tile_rows = own_tile_rows;
        g.remote = own_tile_rows < tiles_m ? remote : nullptr;
        g.nxcd = xcd_partitions(dev.num_cu, dev.num_cu);
        g.xcd_cols = g.nxcd == kMaxXcd
                         ? gemm_xcd_bands(g.nxcd, tiles_m, tiles_n, tile_m, tile_n, tpc, set.xcd_bands)
                         : 1;
        hipError_t e = launch_gemm(tile_m, tile_n, g, dev.num_cu, s);
        if (e != hipSuccess) return hip_fail(e, "GEMM launch");
        if (num_peers > 0 && own_tile_rows > 0) {
            ReduceArgs r;
            r.peers = peers;
            r.C = C;
            r.MN = M * N;
            r.count4 = M * N / 4;
            r.own4 = std::min<int64_t>(M, (int64_t)own_tile_rows * tile_m) * N / 4;
            r.P = num_peers;
            e = launch_reduce(r, dev.num_cu, s);
            if (e != hipSuccess) return hip_fail(e, "reduce launch");
        }
        return MK_OK;
    }

    // The fused protocol (flags, chunks, reduce tasks, controller) covers the
    // rows this rank reduces: all of them for GEMM+AllReduce, its shard for
    // reduce-scatter, whose other rows are plain GEMM blocks.
    const int tiles_m = own_tile_rows;
    const int64_t Mf = std::min<int64_t>(M, (int64_t)tiles_m * tile_m);
    const uint32_t T = (uint32_t)tiles_m * (uint32_t)tiles_n;
    const uint32_t Ch = (T + tpc - 1) / tpc;

    // every workgroup of the persistent grid must be resident at once
    const int per_cu = workgroups_per_cu(tile_m, tile_n);
    if (per_cu < 1) return fail(MK_ERR_HIP, "occupancy query for the fused kernel failed");
    const int resident = dev.num_cu * per_cu;
    const int nwg = set.num_wg ? set.num_wg : (resident < kMaxWG ? resident : kMaxWG);
    if (nwg < 2 || nwg > resident)
        return fail(MK_ERR_INVALID_ARG, "workgroups %d outside [2, %d resident workgroups]", nwg,
                    resident);
    int ns_init = set.n_reduce;
    if (set.mode != MK_PART_ADAPTIVE && (ns_init < 1 || ns_init > nwg - 1))
        return fail(MK_ERR_INVALID_ARG, "static reduce count %d outside [1, %d]", ns_init, nwg - 1);
    // Keep every tile on the XCD of its partition (write-back hand-off in one
    // L2) when the grid spans whole XCDs dealt round-robin, every partition
    // holds tiles, and every XCD keeps both roles: the controller keeps one
    // compute workgroup per XCD, and a static partition must give each XCD a
    // reducer and a compute workgroup (8 <= n_reduce <= B - 8).  Otherwise
    // tiles cross XCDs with write-through hand-off.
    const int nxcd = xcd_partitions(nwg, dev.num_cu);
    const int bands = nxcd == kMaxXcd ? xcd_bands(nxcd, tiles_m, tiles_n, tile_m, tile_n, tpc, set.xcd_bands)
                                      : 0;
    const bool local = dev.xcd_ok && nxcd == kMaxXcd && bands > 0 &&
                       set.mode != MK_PART_STATIC_DETERMINISTIC &&
                       (set.mode == MK_PART_ADAPTIVE || (ns_init >= nxcd && ns_init <= nwg - nxcd));
    const int keep = local ? nxcd : 1;
    // most reducers while compute remains: five eighths of the workgroups by
    // default (the reduce role saturates HBM with about half to five eighths
    // of the CUs: one CU streams 40-57 GB/s)
    int cap = set.cap ? set.cap : (5 * nwg) / 8;
    if (cap > nwg - keep) cap = nwg - keep;
    if (cap < 1) cap = 1;
    if (set.mode == MK_PART_ADAPTIVE) {
        // default start: half the workgroups.  Reducers with nothing ready
        // yet compute, so a high start costs no idle workgroups, and the
        // reduce role is staffed the moment the first tiles are published.
        if (ns_init == 0) ns_init = nwg / 2;
        if (ns_init > cap) ns_init = cap;
        if (ns_init < 1) ns_init = 1;
    }

    rc = noalloc ? ensure_fixed_workspace(dev, T, Ch, s) : ensure_workspace(dev.heap, T, Ch, s);
    if (rc) return rc;
    Workspace &d = noalloc ? dev.fixed : dev.heap;
    rc = prepare_launch(d, T, (uint32_t)tpc, s);
    if (rc) return rc;
    WsView v = view_of(d);
    hipError_t e;

    FusedArgs a;
    std::memset(&a, 0, sizeof a);
    a.A = (const uint16_t *)A;
    a.B = (const uint16_t *)B;
    a.peers = peers;
    a.C = C;
    a.M = Mf;
    a.N = N;
    a.K = K;
    a.P = num_peers;
    a.tiles_m = tiles_m;
    a.tiles_n = tiles_n;
    a.T = T;
    a.tpc = (uint32_t)tpc;
    a.Ch = Ch;
    a.Tcap = d.Tcap;
    a.epoch = d.epoch;
    a.calls = d.calls;
    a.mode = set.mode;
    a.ns_init = ns_init;
    a.ns_floor = set.floor;
    a.nwg = nwg;
    a.group_m = set.group_m;
    a.nxcd = nxcd;
    a.local = local ? 1 : 0;
    a.keep = keep;
    a.ns_cap = cap;
    a.xcd_cols = local ? bands : 1;
    a.remote = own_tile_rows < tiles_m_all ? remote : nullptr;
    a.M_all = M;
    a.tiles_m_all = tiles_m_all;
    a.peer_mn = M * N;
    a.timeout_ticks = set.timeout_us * (dev.timer_hz / 1000000ull);
    a.skip_publish = set.skip_publish;
    a.help = set.help;
    a.ws = v;
    e = launch_fused(tile_m, tile_n, a, s);
    if (e != hipSuccess) {
        d.dirty = true;
        return hip_fail(e, "fused launch");
    }
    dev.recent = &d;
    d.last.valid = true;
    d.last.kind = rs ? 1u : 0u;
    d.last.epoch = d.epoch;
    d.last.calls = d.calls;
    d.last.nwg = (uint32_t)nwg;
    d.last.T = T;
    d.last.Ch = Ch;
    d.last.tpc = (uint32_t)tpc;
    d.last.tm = (uint32_t)tile_m;
    d.last.tn = (uint32_t)tile_n;
    d.last.mode = (uint32_t)set.mode;
    d.last.ns_init = (uint32_t)ns_init;
    d.last.local = local ? 1u : 0u;
    d.last.keep = (uint32_t)keep;
    d.last.cap = (uint32_t)cap;
    d.last.bands = local ? (uint32_t)bands : 1u;
    d.last.help = (uint32_t)set.help;
    return MK_OK;
}

// One rank's share of AllGather+GEMM (fused: one persistent launch; else the
// gather kernel, then the GEMM kernel on the gathered A).
int run_allgather(bool fused, const void *A_local, const void *A_peers, int num_peers, void *A_gath,
                  const void *B, float *C, int64_t Ms, int64_t N, int64_t K, int tile_m, int tile_n,
                  void *stream) {
    if (Ms < 0 || N < 0 || K < 0) return fail(MK_ERR_INVALID_ARG, "negative dimension");
    if (num_peers < 0) return fail(MK_ERR_INVALID_ARG, "num_peers < 0");
    if (!tile_supported(tile_m, tile_n))
        return fail(MK_ERR_INVALID_ARG, "tile %dx%d not supported (64x64, 128x128, 256x128)", tile_m, tile_n);
    if (N % 8 != 0 || K % 8 != 0)
        return fail(MK_ERR_SHAPE, "N (%lld) and K (%lld) must be multiples of 8", (long long)N, (long long)K);
    if (Ms % tile_m != 0)
        return fail(MK_ERR_SHAPE, "shard rows (%lld) must be a multiple of tile_m (%d): a chunk is one tile row",
                    (long long)Ms, tile_m);
    const int64_t R = (int64_t)num_peers + 1;
    const int64_t M = R * Ms;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(MK_ERR_SHAPE, "dimension exceeds 2^31-1");
    if (M == 0 || N == 0) return MK_OK;
    if ((int64_t)tile_m * N * 4 >= (int64_t)INT32_MAX || (int64_t)tile_m * K * 2 >= (int64_t)INT32_MAX ||
        (int64_t)64 * N * 2 >= (int64_t)INT32_MAX)
        return fail(MK_ERR_SHAPE, "N or K too large for 32-bit in-tile offsets");
    const int64_t tiles_n = (N + tile_n - 1) / tile_n;
    const int64_t T = (M / tile_m) * tiles_n;
    if (T >= (int64_t)kMaxTiles) return fail(MK_ERR_SHAPE, "too many tiles (%lld)", (long long)T);
    if (!C || !A_gath || !B || !A_local) return fail(MK_ERR_INVALID_ARG, "NULL pointer");
    if (num_peers > 0 && !A_peers) return fail(MK_ERR_INVALID_ARG, "A_peers is NULL with num_peers > 0");
    if (!aligned16(C) || !aligned16(A_gath) || !aligned16(B) || !aligned16(A_local) ||
        (A_peers && !aligned16(A_peers)))
        return fail(MK_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    const int64_t gb = M * K * 2, cb = M * N * 4, lb = Ms * K * 2, pb = (int64_t)num_peers * Ms * K * 2;
    if (overlaps(A_gath, gb, A_local, lb) || overlaps(A_gath, gb, A_peers, pb) || overlaps(A_gath, gb, B, K * N * 2) ||
        overlaps(A_gath, gb, C, cb) || overlaps(C, cb, A_local, lb) || overlaps(C, cb, A_peers, pb) ||
        overlaps(C, cb, B, K * N * 2))
        return fail(MK_ERR_INVALID_ARG, "outputs (gathered A, C) overlap each other or an input");
    const Settings set = g_set;
    DevState *dp = nullptr;
    int rc = device_state(&dp);
    if (rc) return rc;
    DevState &dev = *dp;
    hipStream_t s = (hipStream_t)stream;
    const int tpb = tiles_per_block(tile_m, tile_n);

    AgArgs a;
    std::memset(&a, 0, sizeof a);
    a.A_local = (const uint16_t *)A_local;
    a.A_peers = (const uint16_t *)A_peers;
    a.A_gath = (uint16_t *)A_gath;
    a.B = (const uint16_t *)B;
    a.C = C;
    a.Ms = Ms;
    a.M = M;
    a.N = N;
    a.K = K;
    a.P = num_peers;
    a.cps = (uint32_t)(Ms / tile_m);
    a.Ch = (uint32_t)(M / tile_m);
    a.tiles_n = (uint32_t)tiles_n;
    a.bn = (uint32_t)((tiles_n + tpb - 1) / tpb);
    a.T = (uint32_t)T;
    a.TB = a.Ch * a.bn;
    // a copy task moves at most 64 KiB of a chunk: ceil(chunk bytes / 64 KiB)
    // parts, at least 1, at most min(tiles_n, 64) (so copy tasks <= tiles)
    {
        int64_t parts = (2 * (int64_t)tile_m * K + 65535) / 65536;
        if (parts > tiles_n) parts = tiles_n;
        if (parts > 64) parts = 64;
        if (parts < 1) parts = 1;
        a.parts = (uint32_t)parts;
        a.Q = a.Ch * a.parts;
    }
    // compute claims in column bands, one per XCD, when workgroups map to
    // XCDs round-robin and every band gets a block column
    {
        const int want = set.xcd_bands ? set.xcd_bands : kMaxXcd;
        a.bands = (dev.xcd_ok && (int64_t)a.bn >= want) ? (uint32_t)want : 1u;
    }

    if (!fused) {
        hipError_t e = launch_gather(a, dev.num_cu, s);
        if (e != hipSuccess) return hip_fail(e, "gather launch");
        GemmArgs g;
        std::memset(&g, 0, sizeof g);
        g.A = (const uint16_t *)A_gath;
        g.B = (const uint16_t *)B;
        g.C = C;
        g.M = M;
        g.N = N;
        g.K = K;
        g.tiles_m = (int32_t)(M / tile_m);
        g.tiles_n = (int32_t)tiles_n;
        g.tpc = 4;
        g.group_m = set.group_m;
        g.own_tile_rows = g.tiles_m;
        g.remote = nullptr;
        g.nxcd = xcd_partitions(dev.num_cu, dev.num_cu);
        g.xcd_cols = g.nxcd == kMaxXcd
                         ? gemm_xcd_bands(g.nxcd, g.tiles_m, g.tiles_n, tile_m, tile_n, 4, set.xcd_bands)
                         : 1;
        e = launch_gemm(tile_m, tile_n, g, dev.num_cu, s);
        if (e != hipSuccess) return hip_fail(e, "GEMM launch");
        return MK_OK;
    }

    const int per_cu = allgather_workgroups_per_cu(tile_m, tile_n);
    if (per_cu < 1) return fail(MK_ERR_HIP, "occupancy query for the AllGather+GEMM kernel failed");
    const int resident = dev.num_cu * per_cu;
    const int nwg = set.num_wg ? set.num_wg : (resident < kMaxWG ? resident : kMaxWG);
    if (nwg < 2 || nwg > resident)
        return fail(MK_ERR_INVALID_ARG, "workgroups %d outside [2, %d resident workgroups]", nwg, resident);
    int ns_init = set.n_reduce;
    if (set.mode != MK_PART_ADAPTIVE && (ns_init < 1 || ns_init > nwg - 1))
        return fail(MK_ERR_INVALID_ARG, "static copy count %d outside [1, %d]", ns_init, nwg - 1);
    int cap = set.cap ? set.cap : nwg - 1;
    if (cap > nwg - 1) cap = nwg - 1;
    if (cap < 1) cap = 1;
    if (set.mode == MK_PART_ADAPTIVE) {
        // default start: three quarters of the workgroups.  Communication
        // feeds compute here, and the analysis page's section 2.4 lets the
        // data dependency decide the initial split: rows must arrive before
        // they are computed, so the copy role starts large and the controller
        // shrinks it once both roles have measured costs.  A quarter computes
        // from the start: this rank's own rows need no copy.
        if (ns_init == 0) ns_init = (3 * nwg) / 4;
        if (ns_init > cap) ns_init = cap;
        if (ns_init < 1) ns_init = 1;
    }
    rc = ensure_workspace(dev.heap, a.T, a.Ch, s);
    if (rc) return rc;
    Workspace &d = dev.heap;
    // counters restart when the tile grid, the chunk count or the copy
    // tasks per chunk change (chunk_cnt grows by `parts` per call)
    rc = prepare_launch(d, a.T, 0x80000000u | ((a.parts - 1u) << 24) | a.Ch, s);
    if (rc) return rc;
    a.Tcap = d.Tcap;
    a.epoch = d.epoch;
    a.calls = d.calls;
    a.mode = set.mode;
    a.ns_init = ns_init;
    a.ns_floor = set.floor;
    a.ns_cap = cap;
    a.nwg = nwg;
    a.help = set.help;
    a.timeout_ticks = set.timeout_us * (dev.timer_hz / 1000000ull);
    a.skip_publish = set.skip_publish;
    a.ws = view_of(d);
    hipError_t e = launch_allgather_gemm(tile_m, tile_n, a, s);
    if (e != hipSuccess) {
        d.dirty = true;
        return hip_fail(e, "AllGather+GEMM launch");
    }
    dev.recent = &d;
    d.last = Launch();
    d.last.valid = true;
    d.last.kind = 2;
    d.last.epoch = d.epoch;
    d.last.calls = d.calls;
    d.last.nwg = (uint32_t)nwg;
    d.last.T = a.T;
    d.last.Ch = a.Ch;
    d.last.tpc = a.parts;   // reported as copy tasks per chunk
    d.last.tm = (uint32_t)tile_m;
    d.last.tn = (uint32_t)tile_n;
    d.last.mode = (uint32_t)set.mode;
    d.last.ns_init = (uint32_t)ns_init;
    d.last.cap = (uint32_t)cap;
    d.last.help = (uint32_t)set.help;
    d.last.bands = a.bands;
    return MK_OK;
}


// One rank's share of Ring Attention (see mk_ring.hip).  fused: one
// persistent launch with copy and compute roles; otherwise a gather kernel
// then the attention kernel.
int run_ring(bool fused, const void *q, const void *k_local, const void *v_local, const void *k_peers,
             const void *v_peers, int num_peers, void *k_ring, void *v_ring, float *O, float *lse, int64_t S,
             int H, int D, void *stream) {
    if (S < 0 || H < 1) return fail(MK_ERR_INVALID_ARG, "S must be >= 0 and H >= 1");
    if (num_peers < 0) return fail(MK_ERR_INVALID_ARG, "num_peers < 0");
    if (D != kRaHeadDim) return fail(MK_ERR_SHAPE, "head dimension %d not supported (128)", D);
    if (S * (int64_t)H * D * 4 >= (int64_t)INT32_MAX)
        return fail(MK_ERR_SHAPE, "S x H x D too large for 32-bit in-buffer offsets");
    const int64_t R = (int64_t)num_peers + 1;
    if (S == 0) return MK_OK;
    if (!q || !k_local || !v_local || !O || !lse) return fail(MK_ERR_INVALID_ARG, "NULL pointer");
    if (num_peers > 0 && (!k_peers || !v_peers || !k_ring || !v_ring))
        return fail(MK_ERR_INVALID_ARG, "peer or ring buffers NULL with num_peers > 0");
    const void *ptrs[] = {q, k_local, v_local, k_peers, v_peers, k_ring, v_ring, O, lse};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(MK_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    const int64_t eb = S * H * D * 2, pb = (int64_t)num_peers * eb, ob = S * H * D * 4, lb = S * H * 4;
    const void *ins[] = {q, k_local, v_local, k_peers, v_peers};
    const int64_t inb[] = {eb, eb, eb, pb, pb};
    const void *outs[] = {k_ring, v_ring, O, lse};
    const int64_t outb[] = {pb, pb, ob, lb};
    for (int i = 0; i < 4; ++i) {
        if (!outs[i] || outb[i] == 0) continue;
        for (int j = 0; j < 5; ++j)
            if (ins[j] && inb[j] && overlaps(outs[i], outb[i], ins[j], inb[j]))
                return fail(MK_ERR_INVALID_ARG, "an output overlaps an input");
        for (int j = i + 1; j < 4; ++j)
            if (outs[j] && outb[j] && overlaps(outs[i], outb[i], outs[j], outb[j]))
                return fail(MK_ERR_INVALID_ARG, "outputs overlap each other");
    }
    const Settings set = g_set;
    DevState *dp = nullptr;
    int rc = device_state(&dp);
    if (rc) return rc;
    DevState &dev = *dp;
    hipStream_t s = (hipStream_t)stream;

    RaArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = (const uint16_t *)q;
    a.k_local = (const uint16_t *)k_local;
    a.v_local = (const uint16_t *)v_local;
    a.k_peers = (const uint16_t *)k_peers;
    a.v_peers = (const uint16_t *)v_peers;
    a.k_ring = (uint16_t *)k_ring;
    a.v_ring = (uint16_t *)v_ring;
    a.O = O;
    a.lse = lse;
    a.S = S;
    a.H = H;
    a.R = (int32_t)R;
    a.nkv = (uint32_t)((S + kRaKvRows - 1) / kRaKvRows);
    a.nqb = (uint32_t)((S + kRaQRows - 1) / kRaQRows);
    a.Ch = (uint32_t)(num_peers * (int64_t)a.nkv);
    {
        // a copy task moves at most 64 KiB of a tile (K and V together)
        int64_t parts = (2 * (int64_t)kRaKvRows * H * D * 2 + 65535) / 65536;
        if (parts > 64) parts = 64;
        if (parts < 1) parts = 1;
        a.parts = (uint32_t)parts;
    }
    a.Qc = a.Ch * a.parts;
    a.NTk = (uint32_t)H * a.nqb;
    {
        const int want = set.xcd_bands ? set.xcd_bands : kMaxXcd;
        a.bands = (dev.xcd_ok && H >= want) ? (uint32_t)want : 1u;
    }
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
    const uint64_t Tmap = a.NTk > a.Qc ? a.NTk : a.Qc;
    if (Tmap >= (uint64_t)kMaxTiles || a.Ch >= (1u << 22))
        return fail(MK_ERR_SHAPE, "too many tasks (%llu)", (unsigned long long)Tmap);

    if (!fused) {
        hipError_t e = launch_ring_unfused(a, dev.num_cu, dev.xcd_ok, s);
        if (e != hipSuccess) return hip_fail(e, "Ring Attention (unfused) launch");
        return MK_OK;
    }

    const int per_cu = ring_workgroups_per_cu();
    if (per_cu < 1) return fail(MK_ERR_HIP, "occupancy query for the Ring Attention kernel failed");
    const int resident = dev.num_cu * per_cu;
    const int nwg = set.num_wg ? set.num_wg : (resident < kMaxWG ? resident : kMaxWG);
    if (nwg < 2 || nwg > resident)
        return fail(MK_ERR_INVALID_ARG, "workgroups %d outside [2, %d resident workgroups]", nwg, resident);
    int ns_init = set.n_reduce;
    if (set.mode != MK_PART_ADAPTIVE && (ns_init < 1 || ns_init > nwg - 1))
        return fail(MK_ERR_INVALID_ARG, "static copy count %d outside [1, %d]", ns_init, nwg - 1);
    int cap = set.cap ? set.cap : nwg - 1;
    if (cap > nwg - 1) cap = nwg - 1;
    if (cap < 1) cap = 1;
    // at least one copy workgroup while copy tasks remain: compute tasks wait
    // for arriving tiles, so the copy role never empties
    const int floor = set.floor < 1 ? 1 : set.floor;
    if (set.mode == MK_PART_ADAPTIVE) {
        // default start: the cap (communication feeds compute; the data
        // dependency sets a copy-heavy start, as for AllGather+GEMM)
        if (ns_init == 0) ns_init = cap;
        if (ns_init > cap) ns_init = cap;
        if (ns_init < 1) ns_init = 1;
    }
    const uint32_t Ch_ws = a.Ch ? a.Ch : 1u;
    rc = ensure_workspace(dev.heap, (uint32_t)Tmap, Ch_ws, s);
    if (rc) return rc;
    Workspace &d = dev.heap;
    rc = prepare_launch(d, (uint32_t)Tmap, 0xC0000000u | ((a.parts - 1u) << 24) | a.Ch, s);
    if (rc) return rc;
    a.Tcap = d.Tcap;
    a.epoch = d.epoch;
    a.calls = d.calls;
    a.mode = set.mode;
    a.ns_init = ns_init;
    a.ns_floor = floor;
    a.ns_cap = cap;
    a.nwg = nwg;
    a.timeout_ticks = set.timeout_us * (dev.timer_hz / 1000000ull);
    a.skip_publish = set.skip_publish;
    a.ws = view_of(d);
    hipError_t e = launch_ring_attention(a, s);
    if (e != hipSuccess) {
        d.dirty = true;
        return hip_fail(e, "Ring Attention launch");
    }
    dev.recent = &d;
    d.last = Launch();
    d.last.valid = true;
    d.last.kind = 3;
    d.last.epoch = d.epoch;
    d.last.calls = d.calls;
    d.last.nwg = (uint32_t)nwg;
    d.last.T = (uint32_t)Tmap;   // length of the per-task maps
    d.last.Ch = a.Ch;
    d.last.tpc = a.parts;        // reported as copy tasks per KV tile
    d.last.tm = (uint32_t)kRaQRows;
    d.last.tn = (uint32_t)kRaKvRows;
    d.last.mode = (uint32_t)set.mode;
    d.last.ns_init = (uint32_t)ns_init;
    d.last.cap = (uint32_t)cap;
    d.last.bands = a.bands;
    d.last.help = 0;
    return MK_OK;
}

}  // namespace

extern "C" {

int mk_allgather_gemm_local(const void *A_local, const void *A_peers, int num_peers, void *A_gathered,
                            const void *B, float *C, int64_t Ms, int64_t N, int64_t K, int tile_m, int tile_n,
                            void *stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    return run_allgather(true, A_local, A_peers, num_peers, A_gathered, B, C, Ms, N, K, tile_m, tile_n, stream);
}

int mk_allgather_gemm_unfused(const void *A_local, const void *A_peers, int num_peers, void *A_gathered,
                              const void *B, float *C, int64_t Ms, int64_t N, int64_t K, int tile_m, int tile_n,
                              void *stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    return run_allgather(false, A_local, A_peers, num_peers, A_gathered, B, C, Ms, N, K, tile_m, tile_n, stream);
}


int mk_ring_attention_local(const void *q, const void *k_local, const void *v_local, const void *k_peers,
                            const void *v_peers, int num_peers, void *k_ring, void *v_ring, float *O, float *lse,
                            int64_t S, int H, int D, void *stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    return run_ring(true, q, k_local, v_local, k_peers, v_peers, num_peers, k_ring, v_ring, O, lse, S, H, D,
                    stream);
}

int mk_ring_attention_unfused(const void *q, const void *k_local, const void *v_local, const void *k_peers,
                              const void *v_peers, int num_peers, void *k_ring, void *v_ring, float *O, float *lse,
                              int64_t S, int H, int D, void *stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    return run_ring(false, q, k_local, v_local, k_peers, v_peers, num_peers, k_ring, v_ring, O, lse, S, H, D,
                    stream);
}

int mk_gemm_reduce_local(const void *A, const void *B, const float *peers, int num_peers, float *C,
                         int64_t M, int64_t N, int64_t K, int tile_m, int tile_n,
                         int tiles_per_chunk, void *stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    return run(true, false, A, B, peers, num_peers, C, nullptr, M, N, K, tile_m, tile_n, tiles_per_chunk,
               stream);
}

int mk_gemm_reduce_local_noalloc(const void *A, const void *B, const float *peers, int num_peers, float *C,
                                 int64_t M, int64_t N, int64_t K, int tile_m, int tile_n,
                                 int tiles_per_chunk, void *stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    return run(true, false, A, B, peers, num_peers, C, nullptr, M, N, K, tile_m, tile_n, tiles_per_chunk,
               stream, true);
}

int mk_gemm_reduce_unfused(const void *A, const void *B, const float *peers, int num_peers,
                           float *C, int64_t M, int64_t N, int64_t K, int tile_m, int tile_n,
                           int tiles_per_chunk, void *stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    return run(false, false, A, B, peers, num_peers, C, nullptr, M, N, K, tile_m, tile_n, tiles_per_chunk,
               stream);
}

int mk_gemm_reduce_scatter_local(const void *A, const void *B, const float *peers, int num_peers, float *C,
                                 float *remote, int64_t M, int64_t N, int64_t K, int tile_m, int tile_n,
                                 int tiles_per_chunk, void *stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    return run(true, true, A, B, peers, num_peers, C, remote, M, N, K, tile_m, tile_n, tiles_per_chunk,
               stream);
}

int mk_gemm_reduce_scatter_unfused(const void *A, const void *B, const float *peers, int num_peers,
                                   float *C, float *remote, int64_t M, int64_t N, int64_t K, int tile_m,
                                   int tile_n, int tiles_per_chunk, void *stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    return run(false, true, A, B, peers, num_peers, C, remote, M, N, K, tile_m, tile_n, tiles_per_chunk,
               stream);
}

int mk_set_partition(int mode, int n_reduce) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (mode != MK_PART_ADAPTIVE && mode != MK_PART_STATIC && mode != MK_PART_STATIC_DETERMINISTIC)
        return fail(MK_ERR_INVALID_ARG, "unknown partition mode %d", mode);
    if (n_reduce < 0 || n_reduce > kMaxWG) return fail(MK_ERR_INVALID_ARG, "n_reduce out of range");
    if (mode != MK_PART_ADAPTIVE && n_reduce == 0)
        return fail(MK_ERR_INVALID_ARG, "a static partition needs n_reduce >= 1");
    g_set.mode = mode;
    g_set.n_reduce = n_reduce;
    return MK_OK;
}

int mk_set_controller_floor(int floor) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (floor < 1 || floor > kMaxWG) return fail(MK_ERR_INVALID_ARG, "floor must be in [1, 1024]");
    g_set.floor = floor;
    return MK_OK;
}

int mk_set_controller_cap(int cap) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (cap < 0 || cap > kMaxWG) return fail(MK_ERR_INVALID_ARG, "cap must be in [0, 1024]");
    g_set.cap = cap;
    return MK_OK;
}

int mk_set_xcd_bands(int bands) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (bands != 0 && bands != 1 && bands != 2 && bands != 4 && bands != 8)
        return fail(MK_ERR_INVALID_ARG, "bands must be 0, 1, 2, 4 or 8");
    g_set.xcd_bands = bands;
    return MK_OK;
}

int mk_set_adaptive_help(int on) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (on != 0 && on != 1) return fail(MK_ERR_INVALID_ARG, "help must be 0 or 1");
    g_set.help = on;
    return MK_OK;
}

int mk_set_num_workgroups(int num_wg) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (num_wg != 0 && (num_wg < 2 || num_wg > kMaxWG))
        return fail(MK_ERR_INVALID_ARG, "num_wg must be 0 or in [2, 1024]");
    g_set.num_wg = num_wg;
    return MK_OK;
}

int mk_set_timeout_us(uint64_t timeout_us) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (timeout_us == 0 || timeout_us > 600000000ull)
        return fail(MK_ERR_INVALID_ARG, "timeout must be in (0, 600 s]");
    g_set.timeout_us = timeout_us;
    return MK_OK;
}

int mk_set_fault_skip_publish(int64_t tile) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (tile < -1) return fail(MK_ERR_INVALID_ARG, "tile must be >= -1");
    g_set.skip_publish = tile;
    return MK_OK;
}

int mk_get_stats(mk_stats *out, uint32_t *maps, size_t maps_len) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!out) return fail(MK_ERR_INVALID_ARG, "out is NULL");
    if (out->struct_size != sizeof(mk_stats))
        return fail(MK_ERR_INVALID_ARG, "struct_size %u != %zu", out->struct_size, sizeof(mk_stats));
    DevState *dp = nullptr;
    int rc = device_state(&dp);
    if (rc) return rc;
    DevState &dev = *dp;
    if (!dev.recent || !dev.recent->last.valid || !dev.recent->ws)
        return fail(MK_ERR_INVALID_ARG, "no fused launch on this device yet");
    Workspace &d = *dev.recent;
    const Launch &l = d.last;
    const size_t need = 10ull * l.T + 3ull * l.Ch + 2ull * kTraceCap;
    if (maps && maps_len < need)
        return fail(MK_ERR_INVALID_ARG, "maps_len %zu < %zu words", maps_len, need);
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        d.dirty = true;
        return hip_fail(e, "hipDeviceSynchronize");
    }
    const WsView v = view_of(d);
    Live snap;
    e = hipMemcpy(&snap, v.snap, sizeof snap, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(stats)");

    const uint32_t size = out->struct_size;
    std::memset(out, 0, sizeof *out);
    out->struct_size = size;
    out->epoch = l.epoch;
    out->calls_since_reset = l.calls;
    out->num_wg = l.nwg;
    out->num_tiles = l.T;
    out->num_chunks = l.Ch;
    out->tiles_per_chunk = l.tpc;
    out->tile_m = l.tm;
    out->tile_n = l.tn;
    out->tiles_per_task = (uint32_t)tiles_per_block((int)l.tm, (int)l.tn);
    out->mode = l.mode;
    out->n_reduce_initial = l.ns_init;
    out->n_reduce_final = snap.ns_final;
    out->n_reduce_min_seen = snap.ns_min < l.ns_init ? snap.ns_min : l.ns_init;
    out->n_reduce_max_seen = snap.ns_max > l.ns_init ? snap.ns_max : l.ns_init;
    out->role_switches = snap.role_switches;
    out->compute_tasks = (uint32_t)(snap.role_compute.v & kCountMask);
    out->reduce_tasks = (uint32_t)(snap.role_reduce.v & kCountMask);
    out->chunks_released = snap.chunks_released.v;
    out->invariant_violations = snap.violations;
    out->ns_trace_len = snap.trace_len < (uint32_t)kTraceCap ? snap.trace_len : (uint32_t)kTraceCap;
    out->sum_cycles_compute = snap.role_compute.v >> kCountBits;
    out->sum_cycles_reduce = snap.role_reduce.v >> kCountBits;
    out->kernel_ticks_start = snap.t_start;
    out->kernel_ticks_end = snap.t_end;
    out->reduce_ticks_start = snap.r_start;
    out->reduce_ticks_end = snap.r_end;
    out->timer_hz = dev.timer_hz;
    out->xcd_local = l.local;
    out->keep_compute = l.keep;
    out->controller_cap = l.cap;
    out->xcd_bands = l.bands;
    out->kind = l.kind;
    out->adaptive_help = l.help;
    out->sticky_errors = snap.sticky;

    if (maps) {
        uint32_t *p = maps;
        struct { const uint32_t *src; size_t n; } parts[] = {
            {v.tile_flag, l.T}, {v.tile_cnt, l.T}, {v.chunk_cnt, l.Ch}, {v.chunk_flag, l.Ch},
            {v.cowner, l.T}, {v.rowner, l.T}, {v.trace, 2ull * kTraceCap},
            {v.timeline, l.T}, {v.timeline + d.Tcap, l.T}, {v.timeline + 2ull * d.Tcap, l.T},
            {v.timeline + 3ull * d.Tcap, l.T}, {v.timeline + 4ull * d.Tcap, l.T},
            {v.timeline + 5ull * d.Tcap, l.T}, {v.chunk_release, l.Ch}};
        for (auto &pt : parts) {
            e = hipMemcpy(p, pt.src, 4 * pt.n, hipMemcpyDeviceToHost);
            if (e != hipSuccess) return hip_fail(e, "hipMemcpy(maps)");
            p += pt.n;
        }
    }
    // Errors are sticky across launches: the word gathers every kind any
    // launch since the last report raised, so a failed launch followed by
    // clean ones is still reported.  Reporting one marks the workspace for
    // a clean start (control block, sticky word and per-call counters).
    const uint32_t sticky = snap.sticky | (snap.error == kErrXcd ? kStickyXcd : 0u) |
                            (snap.error == kErrTimeout ? kStickyTimeout : 0u) |
                            (snap.violations ? kStickyProtocol : 0u);
    if (sticky) d.dirty = true;
    if (sticky & kStickyXcd) {
        // a workgroup ran on another XCD than its index implies: the launch's
        // hand-off assumption failed, so tiles no longer stay on one XCD
        dev.xcd_ok = false;
        out->status = MK_ERR_PROTOCOL;
        fail(MK_ERR_PROTOCOL, "a workgroup ran on an unexpected XCD; result not valid");
        return MK_ERR_PROTOCOL;
    }
    if (sticky & kStickyTimeout) {
        out->status = MK_ERR_TIMEOUT;
        fail(MK_ERR_TIMEOUT, "a bounded wait in the fused kernel expired (this launch or an earlier "
                             "one since the last report)");
        return MK_ERR_TIMEOUT;
    }
    if (sticky & kStickyProtocol) {
        out->status = MK_ERR_PROTOCOL;
        fail(MK_ERR_PROTOCOL, "flag/counter violations (%u in the last launch)", snap.violations);
        return MK_ERR_PROTOCOL;
    }
    out->status = MK_OK;
    return MK_OK;
}

int mk_controller_eval(const uint64_t *in, uint32_t *out, int n, void *stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (n < 0) return fail(MK_ERR_INVALID_ARG, "n < 0");
    if (n == 0) return MK_OK;
    if (!in || !out) return fail(MK_ERR_INVALID_ARG, "NULL table");
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    hipError_t e = launch_controller_eval(in, out, n, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "controller eval launch");
    return MK_OK;
}

int mk_device_cu_count(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    DevState *dp = nullptr;
    int rc = device_state(&dp);
    if (rc) return rc;
    return dp->num_cu;
}

int mk_release_workspace(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    Workspace &d = g_dev[dev].heap;
    if (d.ws) {
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
        e = hipFree(d.ws);
        if (e != hipSuccess) return hip_fail(e, "hipFree");
    }
    d.ws = nullptr;
    d.ws_bytes = 0;
    d.Tcap = d.Chcap = 0;
    d.last.valid = false;
    if (g_dev[dev].recent == &d) g_dev[dev].recent = nullptr;
    return MK_OK;
}

const char *mk_last_error(void) { return g_last_error; }

int mk_abi_version(void) { return MK_ABI_VERSION; }

}  // extern "C"
