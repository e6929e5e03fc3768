// fused_common.h -- the parts of the one-launch decode layer that do not
// depend on the weight format: the route built in LDS by every block, the
// one-writer epoch flags that blocks hand data over with, the bounded waits,
// and the resident launch.  Included by the E4M3 and NVFP4 GEMV sources,
// each of which supplies its gate/up and down items.
#pragma once

#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace {

constexpr int kFusedThreads = 256;

// Every block is resident at once (the grid is sized by the occupancy API).
// Each block first builds the route of the S <= kFusedMaxSlots slots in LDS
// (the same stable pack as route_pack_kernel; block 0 also writes the route
// tables, the status at once and the rest at the end).  Then it runs its share of the gate/up items (active expert x 16 h
// rows); each finished item stores the call's epoch into its own
// flag.  Then its share of the down items (32-row tile x active expert,
// tile-major): the first weight chunks go out, the block waits until all the
// gate/up flags of the expert hold the epoch, stages h and finishes the item,
// and stores its own flag.  The down item of the last active expert of a
// tile waits for the tile's other down flags and applies the top-k weights
// for every token of that tile, in slot order (multiply, then add).
//
// No read-modify-write anywhere: each flag has one writer, and flags hold an
// epoch no earlier call used, so a workspace needs no clearing and stale
// contents cannot satisfy a wait.  A block does all its gate/up items before
// it waits for anything and takes its down items in increasing index; the
// combining item has the largest index of its tile, so it only waits on items
// of smaller index.  With every block resident, each wait therefore ends; a
// wait also gives up after a bounded spin and flags the call in route status.
constexpr int kFusedMaxSlots = 256;
constexpr uint32_t kFusedTimeoutFlag = 1u << 30;    // added to route status on a timed-out wait

template <class GU, class DN>
struct FusedArgsT {
    GU gu;                           // offsets/sorted_token/active unused (route built in LDS)
    DN dn;                           // idem
    const int32_t *ids;              // [M][k]
    const float *w;                  // [M][k]
    int32_t M, k, E, A;              // A = min(M*k, E): active-expert capacity
    uint32_t epoch;
    uint32_t *flag_gu;               // [A][inter / 16] per gate/up item
    uint32_t *flag_dn;               // [hidden / 32][A] per down item
    float *out;                      // [M][H]
    MoeRouteDev r;                   // route tables written by block 0
};

struct FusedRoute {
    int32_t ids[kFusedMaxSlots];
    int32_t first[kFusedMaxSlots];   // 1: first slot of its (valid) expert
    int32_t tok[kFusedMaxSlots];     // packed row -> token
    int32_t t2p[kFusedMaxSlots];     // slot -> packed row, -1 if invalid
    int32_t ae[kFusedMaxSlots];      // active experts, ascending
    int32_t ap0[kFusedMaxSlots];     // their first packed row
    int32_t acnt[kFusedMaxSlots];    // their slot counts
    int32_t na, nvalid, ninvalid, flag;
};

// h and y move between blocks through device-coherent stores and loads
// (written through to memory, read past the L2 of the reader's XCD); a
// release or acquire at device scope would instead write back or invalidate
// a whole L2 per item.  Each wave waits for its stores before the caller's
// barrier; then one thread publishes the epoch in the item's flag.
__device__ __forceinline__ void publish(uint32_t *flag, uint32_t epoch)
{
    __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// wave 0 waits until flags[0..n) all hold epoch; false on timeout.  The other
// waves wait at the caller's barrier; the data behind the flags is then read
// with device-coherent loads.
__device__ __forceinline__ bool flags_wait(const uint32_t *flags, int n, uint32_t epoch)
{
    const int lane = threadIdx.x & 63;
    for (int it = 0; it < (1 << 21); ++it) {
        bool ok = true;
        for (int i = lane; i < n; i += 64)
            ok &= __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) return true;
        __builtin_amdgcn_s_sleep(16);
    }
    return false;
}

// wave 0 waits for an expert's gate/up flags (flagging a timeout), then the block goes on
struct FusedWait {
    const uint32_t *flags;
    int n;
    uint32_t epoch;
    int *flag;
    __device__ void operator()() const
    {
        if (threadIdx.x < 64 && !flags_wait(flags, n, epoch) && threadIdx.x == 0) *flag = 1;
        moe::lds_barrier();
    }
};

// The route of the S slots in LDS, for any block.  id_in is this thread's
// slot id (slot tid; -1 past S), loaded by the caller; the barriers inside are
// LDS-only, so global loads the caller has in flight stay in flight.
static_assert(kFusedMaxSlots == kFusedThreads, "one slot per thread");
template <class Args>
__device__ __forceinline__ void fused_route(const Args &a, FusedRoute &R, int id_in)
{
    const int tid = threadIdx.x, S = a.M * a.k, E = a.E;
    if (tid == 0) { R.na = 0; R.nvalid = 0; R.ninvalid = 0; R.flag = 0; }
    R.ids[tid] = id_in;
    moe::lds_barrier();
    const int id = tid < S ? R.ids[tid] : -1;
    const bool valid = tid < S && id >= 0 && id < E;
    int less = 0, before = 0, total = 0;
    for (int q = 0; q < S; ++q) {
        const int v = R.ids[q];
        if (v >= 0 && v < E) {
            less += v < id;
            if (v == id) { ++total; before += q < tid; }
        }
    }
    R.first[tid] = valid && before == 0;
    if (tid < S && !valid && id != -1) atomicAdd(&R.ninvalid, 1);
    if (valid) atomicAdd(&R.nvalid, 1);
    moe::lds_barrier();
    int rank = 0;                                    // distinct valid experts below id
    for (int q = 0; q < S; ++q) rank += R.first[q] && R.ids[q] < id;
    const int p = less + before;
    if (tid < S) R.t2p[tid] = valid ? p : -1;
    if (valid) R.tok[p] = tid / a.k;
    if (valid && before == 0) {
        R.ae[rank] = id; R.ap0[rank] = less; R.acnt[rank] = total;
        atomicAdd(&R.na, 1);
    }
    moe::lds_barrier();
}

// The active expert of index ai of a route of S <= 128 slots, worked out by
// each wave on its own from the ids (lane s holds slots s and s + 64; no LDS,
// no barrier), for a launch whose blocks each need only their own expert: e
// (-1 when ai is past the active experts), its first packed row p0 (the
// valid slots of smaller experts), its slot count ne and the masks of its
// slots (bit s of mask[h]: slot 64 h + s chose it), in slot order -- the
// stable pack.  Key comparisons come from one ballot per key bit and half,
// most significant bit first: for each of a lane's two keys, the lanes of
// each half holding a smaller key (lt) and an equal one (eq).
struct LightRoute {
    int e, p0, ne;
    uint64_t mask[2];
};

__device__ __forceinline__ LightRoute light_route_wide(const int32_t *ids, int S, int E, int ai)
{
    const int lane = threadIdx.x & 63;
    const int id0 = lane < S ? ids[lane] : -1;
    const int id1 = lane + 64 < S ? ids[lane + 64] : -1;
    // key: the expert, E for an invalid or missing slot (after every expert)
    const int k0 = id0 >= 0 && id0 < E ? id0 : E;
    const int k1 = id1 >= 0 && id1 < E ? id1 : E;
    uint64_t lt00 = 0, eq00 = ~0ull, lt01 = 0, eq01 = ~0ull;   // key k0 against halves 0, 1
    uint64_t lt10 = 0, eq10 = ~0ull, lt11 = 0, eq11 = ~0ull;   // key k1 against halves 0, 1
    for (int b = 9; b >= 0; --b) {                   // keys <= E <= 512
        const uint64_t b0 = __ballot((k0 >> b) & 1), b1 = __ballot((k1 >> b) & 1);
        if ((k0 >> b) & 1) {
            lt00 |= eq00 & ~b0; eq00 &= b0;
            lt01 |= eq01 & ~b1; eq01 &= b1;
        } else {
            eq00 &= ~b0; eq01 &= ~b1;
        }
        if ((k1 >> b) & 1) {
            lt10 |= eq10 & ~b0; eq10 &= b0;
            lt11 |= eq11 & ~b1; eq11 &= b1;
        } else {
            eq10 &= ~b0; eq11 &= ~b1;
        }
    }
    const uint64_t below = (1ull << lane) - 1;
    // the first slot of its expert: no earlier slot holds the same key
    const bool first0 = k0 < E && (eq00 & below) == 0;
    const bool first1 = k1 < E && eq10 == 0 && (eq11 & below) == 0;
    const uint64_t fm0 = __ballot(first0), fm1 = __ballot(first1);
    // distinct valid experts below the key
    const int rank0 = __popcll(lt00 & fm0) + __popcll(lt01 & fm1);
    const int rank1 = __popcll(lt10 & fm0) + __popcll(lt11 & fm1);
    const uint64_t sel0 = __ballot(first0 && rank0 == ai), sel1 = __ballot(first1 && rank1 == ai);
    LightRoute r{-1, 0, 0, {0, 0}};
    if (sel0 == 0 && sel1 == 0) return r;
    r.e = sel0 ? __builtin_amdgcn_readlane(k0, __ffsll((unsigned long long)sel0) - 1)
               : __builtin_amdgcn_readlane(k1, __ffsll((unsigned long long)sel1) - 1);
    r.p0 = __popcll(__ballot(k0 < r.e)) + __popcll(__ballot(k1 < r.e));
    r.mask[0] = __ballot(k0 == r.e);
    r.mask[1] = __ballot(k1 == r.e);
    r.ne = __popcll(r.mask[0]) + __popcll(r.mask[1]);
    return r;
}

// The same for S <= 16 slots (one token's top-k): lane s holds slot s, and
// the duplicates before it and the distinct experts below it are counted over
// the S slots one by one, which is shorter here than the 20 ballots above.
__device__ __forceinline__ LightRoute light_route_narrow(const int32_t *ids, int S, int E, int ai)
{
    const int lane = threadIdx.x & 63;
    const int id = lane < S ? ids[lane] : -1;
    const int key = id >= 0 && id < E ? id : 0x7FFFFFFF;
    int dup_before = 0;
    for (int j = 0; j < S; ++j) {
        const int kj = __builtin_amdgcn_readlane(key, j);
        dup_before += (j < lane) & (kj == key);
    }
    const bool first = key != 0x7FFFFFFF && dup_before == 0;
    const uint64_t fm = __ballot(first);
    int rank = 0;                                    // distinct valid experts below key
    for (int j = 0; j < S; ++j) {
        const int kj = __builtin_amdgcn_readlane(key, j);
        rank += (int)((fm >> j) & 1) & (kj < key);
    }
    const uint64_t sel = __ballot(first && rank == ai);
    LightRoute r{-1, 0, 0, {0, 0}};
    if (sel == 0) return r;
    r.e = __builtin_amdgcn_readlane(key, __ffsll((unsigned long long)sel) - 1);
    r.p0 = __popcll(__ballot(key < r.e));
    r.mask[0] = __ballot(key == r.e);
    r.ne = __popcll(r.mask[0]);
    return r;
}

__device__ __forceinline__ LightRoute light_route(const int32_t *ids, int S, int E, int ai)
{
    return S <= 16 ? light_route_narrow(ids, S, E, ai) : light_route_wide(ids, S, E, ai);
}

// Token of each slot of lr's expert, in slot order, into tok[0..ne): thread
// t < 128 looks at slot t.
__device__ __forceinline__ void light_route_tokens(const LightRoute &lr, int k, int32_t *tok)
{
    const int t = threadIdx.x;
    if (lr.e < 0 || t >= 128) return;
    const int s = t & 63;
    const uint64_t m = t < 64 ? lr.mask[0] : lr.mask[1];   // (a select: no indexed private array)
    if ((m >> s) & 1)
        tok[(t < 64 ? 0 : __popcll(lr.mask[0])) + __popcll(m & ((1ull << s) - 1))] = t / k;
}

// Block 0 writes the other route tables, as route_pack writes them.  Nothing
// in the launch reads them, so this runs at the end, off the critical path.
template <class Args>
__device__ __forceinline__ void fused_route_tables(const Args &a, const FusedRoute &R)
{
    if (blockIdx.x != 0) return;
    const int tid = threadIdx.x, S = a.M * a.k, E = a.E;
    for (int e = tid; e <= E; e += kFusedThreads) {
        int c = 0;
        for (int q = 0; q < S; ++q) {
            const int v = R.ids[q];
            c += v >= 0 && v < e;
        }
        a.r.offsets[e] = c;
    }
    if (tid < S) {
        const int p = R.t2p[tid];
        a.r.token_to_perm[tid] = p;
        if (p >= 0) { a.r.sorted_slot[p] = tid; a.r.sorted_token[p] = tid / a.k; }
    }
    const int A = S < E ? S : E;
    for (int i = tid; i < A; i += kFusedThreads) a.r.active[i] = i < R.na ? R.ae[i] : -1;
    if (tid == 0) *a.r.num_active = R.na;
}

// Block 0 sets the route status right after the route: a wait that times out
// later adds its flag to it.
template <class Args>
__device__ __forceinline__ void fused_route_status(const Args &a, const FusedRoute &R)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.r.status = R.ninvalid;
}

// ---------------------------------------------------------------------------
// fused decode layer launch
// ---------------------------------------------------------------------------
// One block per slot the occupancy allows: every block must be resident for
// the waits to end.  The occupancy and CU count are kept per kernel.
template <auto Kern, class Args>
hipError_t resident_launch(const Args &a, size_t lds, hipStream_t st)
{
    static int per_cu = -1;
    static size_t per_cu_lds = 0;
    static int n_cu = 0;
    if (per_cu < 0 || per_cu_lds != lds) {
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)Kern, kFusedThreads, lds);
        if (e != hipSuccess) return e;
        per_cu_lds = lds;
    }
    if (n_cu == 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(Kern, dim3((unsigned)(per_cu * n_cu)), dim3(kFusedThreads), lds, st, a);
    return hipGetLastError();
}


}  // namespace
