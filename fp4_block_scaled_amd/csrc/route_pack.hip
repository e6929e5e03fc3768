// route_pack.hip -- stable counting sort of routed slots by expert.
//
// Builds the expert-sorted route tables of "spark_model
// glm5next_mlp/forward.rs" (struct Glm5NextMlpWorkspace: per-expert prefix
// offsets, sorted row -> token, slot -> sorted row) on the device, so the
// layer never reads routing back to the host (the same page's fn forward_moe
// explains the cost of a stream sync + D2H per layer).  The active-expert
// list doubles as the union of the rows' experts that the multi-row GEMV
// sweeps once per expert.
//
// Routes of up to 64 slots and of 65 to 128 take one-wave kernels of their
// own (below); 8192 slots and more a split pack of three launches.  The
// general form is one workgroup of 1024 threads (16 wave64s); wave w owns a
// contiguous run of whole 64-slot groups, so ordering by (wave, group, lane)
// is slot order:
//   1. Each wave counts its slots per expert.  Inside a group, lanes holding
//      the same expert find each other by ballots over the id bits; the
//      lowest such lane adds the group's count to the wave's LDS counter (one
//      writer per expert and group: no atomics, exact).
//   2. Block scans give expert_offsets and the compacted active-expert list;
//      each wave's counter becomes the number of that expert's slots in
//      lower waves.
//   3. Each wave walks its groups again in order: a slot lands at expert
//      offset + lower waves' count + the wave's running count + its rank
//      among lower peer lanes.  The result is stable in slot order and
//      bit-identical on every run.
// A wave loads the ids of 32 groups at once, so each pass over up to 32K
// slots costs one memory round trip.
#include "moe.h"
#include "moe_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / moe::kWave;
constexpr int kSplitMin = 8192;                  // slots from which the pack is split
constexpr int kMaxRuns = 64;                     // runs of a split pack
constexpr size_t kCountLds = 64 * 1024;          // LDS of its per-run counters

__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

constexpr int kGroups = 32;                      // 64-slot groups per id load of a wave

// Lanes of this wave whose slot holds the same valid expert as this lane's
// (found with one ballot per id bit; invalid lanes get no peers).
__device__ __forceinline__ uint64_t expert_peers(bool valid, int e, int nbits)
{
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

// Whole 64-slot groups [g0, g1) of run w of R (R runs over S slots).
__device__ __forceinline__ void wave_run(int S, int R, int w, int &g0, int &g1)
{
    const int ngroups = (S - 1) / 64 + 1;          // (S >= 1; no overflow near 2^31)
    const int gpw = (ngroups + R - 1) / R;
    g0 = w * gpw;
    g1 = min(ngroups, g0 + gpw);
}

// Runs of a split pack: 2^lg groups each, so a slot's run is s >> (6 + lg).
__device__ __forceinline__ void split_run(int S, int lg, int w, int &g0, int &g1)
{
    const int ngroups = (S - 1) / 64 + 1;
    g0 = w << lg;
    g1 = min(ngroups, g0 + (1 << lg));
}

// ids of groups c0 .. c0 + kGroups - 1 (-1 past g1 or S): one load per group,
// all in flight together
__device__ __forceinline__ void load_ids(const int32_t *ids, int S, int c0, int g1, int lane,
                                         int (&idr)[kGroups])
{
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        const int64_t s = (int64_t)(c0 + g) * 64 + lane;
        idr[g] = (c0 + g < g1 && s < S) ? ids[s] : -1;
    }
}

// Stable placement of one wave's run: a slot lands at pos[e] (LDS: the
// expert's offset + the slots of lower runs, then the run's own running
// count) + its rank among lower peer lanes.  sorted_token may be null (it is
// then filled from sorted_slot afterwards).
__device__ __forceinline__ void place_run(const int32_t *ids, int S, int k, int E, int nbits,
                                          int g0, int g1, int lane, int32_t *pos,
                                          int32_t *sorted_slot, int32_t *sorted_token,
                                          int32_t *token_to_perm)
{
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = g0; c0 < g1; c0 += kGroups) {
        int idr[kGroups];
        load_ids(ids, S, c0, g1, lane, idr);
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            if (c0 + g >= g1) break;                 // (wave-uniform)
            const int64_t s64 = (int64_t)(c0 + g) * 64 + lane;
            const int s = (int)(s64 < S ? s64 : S);  // a slot index when s64 < S
            const int e = idr[g];
            const bool valid = e >= 0 && e < E;
            const uint64_t peers = expert_peers(valid, e, nbits);
            if (valid) {
                // every lane reads the expert's running position before the
                // group's lowest peer lane moves it on (one wave, in order)
                const int p = pos[e] + __popcll(peers & lower);
                sorted_slot[p] = s;
                if (sorted_token) sorted_token[p] = s / k;
                token_to_perm[s] = p;
                if ((peers & lower) == 0) pos[e] += __popcll(peers);
            } else if (s < S) {
                token_to_perm[s] = -1;
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void route_pack_kernel(
    const int32_t *__restrict__ ids, int32_t S, int32_t k, int32_t E, int32_t nbits,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot,
    int32_t *__restrict__ sorted_token, int32_t *__restrict__ token_to_perm,
    int32_t *__restrict__ active, int32_t *__restrict__ num_active,
    int32_t *__restrict__ status)
{
    extern __shared__ int32_t lds[];
    int32_t *ebase = lds;          // [E] expert offsets
    int32_t *cnt = ebase + E;      // [kWaves][E] per-run counts, then positions
    __shared__ int32_t wsum_c[kWaves], wsum_f[kWaves], s_invalid;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kWaves * E; i += kThreads) cnt[i] = 0;
    if (tid == 0) s_invalid = 0;
    __syncthreads();

    int g0, g1;
    wave_run(S, kWaves, wave, g0, g1);
    int32_t *mine = cnt + wave * E;
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // 1. per-run counts
    int bad = 0;
    for (int c0 = g0; c0 < g1; c0 += kGroups) {
        int idr[kGroups];
        load_ids(ids, S, c0, g1, lane, idr);
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            if (c0 + g >= g1) break;                 // (wave-uniform)
            const int e = idr[g];
            const bool valid = e >= 0 && e < E;
            bad += (!valid && e != -1) ? 1 : 0;
            const uint64_t peers = expert_peers(valid, e, nbits);
            if (valid && (peers & lower) == 0) mine[e] += __popcll(peers);
        }
    }
    for (int d = 32; d >= 1; d >>= 1) bad += __shfl_xor(bad, d, 64);
    if (lane == 0 && bad) atomicAdd(&s_invalid, bad);
    __syncthreads();

    // 2. per expert (E <= kThreads: one expert per thread): lower runs'
    // counts, then exclusive scans over experts of the totals and of the
    // active flags
    int c = 0;
    if (tid < E) {
        for (int w = 0; w < kWaves; ++w) {
            const int v = cnt[w * E + tid];
            cnt[w * E + tid] = c;
            c += v;
        }
    }
    const int f = c > 0 ? 1 : 0;
    const int ic = wave_incl_scan(c, lane), iff = wave_incl_scan(f, lane);
    if (lane == 63) { wsum_c[wave] = ic; wsum_f[wave] = iff; }
    __syncthreads();
    int pc = 0, pf = 0;
    for (int w = 0; w < wave; ++w) { pc += wsum_c[w]; pf += wsum_f[w]; }
    const int ex_c = pc + ic - c, ex_f = pf + iff - f;
    if (tid < E) {
        offsets[tid] = ex_c;
        for (int w = 0; w < kWaves; ++w) cnt[w * E + tid] += ex_c;
        if (f) active[ex_f] = tid;
        if (tid == E - 1) { offsets[E] = ex_c + c; *num_active = ex_f + f; }
    }
    // entries past num_active hold -1, so a consumer that reads active[i]
    // for i < min(E, S) can tell an unused entry without reading num_active
    {
        int na = 0;
        for (int w = 0; w < kWaves; ++w) na += wsum_f[w];
        const int A = S < E ? S : E;
        for (int i = na + tid; i < A; i += kThreads) active[i] = -1;
    }
    if (tid == 0) *status = s_invalid;
    __syncthreads();

    // 3. stable placement, each run in order
    place_run(ids, S, k, E, nbits, g0, g1, lane, mine, sorted_slot, sorted_token, token_to_perm);
}

// Large routes, in three more launches so that the work spreads over the
// chip (the ballots of one workgroup's placement kept a single CU busy for
// tens of microseconds).  R runs of whole 64-slot groups:
//   route_count_kernel  one workgroup: per-run expert counts with LDS
//                       atomics (order-free, exact), the expert offsets,
//                       the active list, and each run's starting positions
//                       ([R][E], in `stash`);
//   route_place_kernel  one wave per run: stable placement as above;
//   route_token_kernel  sorted_token from sorted_slot.
__global__ __launch_bounds__(kThreads) void route_count_kernel(
    const int32_t *__restrict__ ids, int32_t S, int32_t E, int32_t R, int32_t lg,
    int32_t *__restrict__ offsets,
    int32_t *__restrict__ active, int32_t *__restrict__ num_active, int32_t *__restrict__ status,
    int32_t *__restrict__ stash)
{
    extern __shared__ int32_t cnt[];                 // [R][E]
    __shared__ int32_t wsum_c[kWaves], wsum_f[kWaves], s_invalid;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < R * E; i += kThreads) cnt[i] = 0;
    if (tid == 0) s_invalid = 0;
    __syncthreads();

    const int sh = 6 + lg;                           // run of slot s: s >> sh
    int bad = 0;
    for (int64_t s0 = 0; s0 < S; s0 += kThreads * kGroups) {
        int idr[kGroups];                            // all loads of a pass in flight together
#pragma unroll
        for (int i = 0; i < kGroups; ++i) {
            const int64_t s = s0 + i * kThreads + tid;
            idr[i] = s < S ? ids[s] : -1;
        }
#pragma unroll
        for (int i = 0; i < kGroups; ++i) {
            const int64_t s = s0 + i * kThreads + tid;
            const int e = idr[i];
            if (e >= 0 && e < E) atomicAdd(&cnt[(s >> sh) * E + e], 1);
            else if (e != -1) ++bad;
        }
    }
    for (int d = 32; d >= 1; d >>= 1) bad += __shfl_xor(bad, d, 64);
    if (lane == 0 && bad) atomicAdd(&s_invalid, bad);
    __syncthreads();

    int c = 0;
    if (tid < E) {
        for (int w = 0; w < R; ++w) {
            const int v = cnt[w * E + tid];
            cnt[w * E + tid] = c;
            c += v;
        }
    }
    const int f = c > 0 ? 1 : 0;
    const int ic = wave_incl_scan(c, lane), iff = wave_incl_scan(f, lane);
    if (lane == 63) { wsum_c[wave] = ic; wsum_f[wave] = iff; }
    __syncthreads();
    int pc = 0, pf = 0;
    for (int w = 0; w < wave; ++w) { pc += wsum_c[w]; pf += wsum_f[w]; }
    const int ex_c = pc + ic - c, ex_f = pf + iff - f;
    if (tid < E) {
        offsets[tid] = ex_c;
        for (int w = 0; w < R; ++w) stash[w * E + tid] = cnt[w * E + tid] + ex_c;
        if (f) active[ex_f] = tid;
        if (tid == E - 1) { offsets[E] = ex_c + c; *num_active = ex_f + f; }
    }
    {
        int na = 0;
        for (int w = 0; w < kWaves; ++w) na += wsum_f[w];
        const int A = S < E ? S : E;
        for (int i = na + tid; i < A; i += kThreads) active[i] = -1;
    }
    if (tid == 0) *status = s_invalid;
}

__global__ __launch_bounds__(64) void route_place_kernel(
    const int32_t *__restrict__ ids, int32_t S, int32_t k, int32_t E, int32_t nbits, int32_t lg,
    const int32_t *__restrict__ stash, int32_t *__restrict__ sorted_slot,
    int32_t *__restrict__ token_to_perm)
{
    extern __shared__ int32_t pos[];                 // [E]
    const int lane = threadIdx.x, w = blockIdx.x;
    int sp[MOE_MAX_EXPERTS / 64];                    // every stash load in flight together
#pragma unroll
    for (int i = 0; i < MOE_MAX_EXPERTS / 64; ++i) {
        const int e = lane + 64 * i;
        sp[i] = e < E ? stash[w * E + e] : 0;
    }
#pragma unroll
    for (int i = 0; i < MOE_MAX_EXPERTS / 64; ++i)
        if (lane + 64 * i < E) pos[lane + 64 * i] = sp[i];
    int g0, g1;
    split_run(S, lg, w, g0, g1);
    place_run(ids, S, k, E, nbits, g0, g1, lane, pos, sorted_slot, nullptr, token_to_perm);
}

__global__ __launch_bounds__(256) void route_token_kernel(const int32_t *__restrict__ sorted_slot,
                                                          const int32_t *__restrict__ offsets,
                                                          int32_t E, int32_t k,
                                                          int32_t *__restrict__ sorted_token)
{
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p < offsets[E]) sorted_token[p] = sorted_slot[p] / k;
}

// Small routes (S <= 64: decode and speculative verify), one wave and no
// LDS: lane s holds slot s.  With key = id for a valid slot and INT_MAX
// otherwise, the packed position of a valid slot is
//   #{j : key_j < key_s} + #{j < s : key_j == key_s}
// (expert offset plus stable rank), and expert_offsets[e] = #{j : key_j < e};
// both are counted by broadcasting each slot's key in turn.  Same tables,
// bit for bit, as the general kernel.
__global__ __launch_bounds__(64) void route_pack_small_kernel(
    const int32_t *__restrict__ ids, int32_t S, int32_t k, int32_t E,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot,
    int32_t *__restrict__ sorted_token, int32_t *__restrict__ token_to_perm,
    int32_t *__restrict__ active, int32_t *__restrict__ num_active,
    int32_t *__restrict__ status)
{
    const int lane = threadIdx.x;
    const int id = lane < S ? ids[lane] : -1;
    const bool valid = id >= 0 && id < E;
    const int key = valid ? id : 0x7FFFFFFF;
    const uint64_t bad = __ballot(lane < S && !valid && id != -1);

    // packed position of this lane's slot
    int below = 0, before = 0;
    for (int j = 0; j < S; ++j) {
        const int kj = __builtin_amdgcn_readlane(key, j);
        below += kj < key;
        before += (j < lane) & (kj == key);
    }
    if (lane < S) {
        const int pos = below + before;
        token_to_perm[lane] = valid ? pos : -1;
        if (valid) {
            sorted_slot[pos] = lane;
            sorted_token[pos] = lane / k;
        }
    }

    // expert offsets and the ascending active list, 64 experts per pass
    const int A = S < E ? S : E;
    int na = 0;
    for (int e0 = 0; e0 <= E; e0 += 64) {
        const int e = e0 + lane;
        int lt = 0, le = 0;                       // slots with key < e, key <= e
        for (int j = 0; j < S; ++j) {
            const int kj = __builtin_amdgcn_readlane(key, j);
            lt += kj < e;
            le += kj <= e;
        }
        if (e <= E) offsets[e] = lt;
        const bool act = e < E && le > lt;
        const uint64_t m = __ballot(act);
        if (act) active[na + __popcll(m & ((1ull << lane) - 1))] = e;
        na += __popcll(m);
    }
    for (int i = na + lane; i < A; i += 64) active[i] = -1;
    if (lane == 0) {
        *num_active = na;
        *status = __popcll(bad);
    }
}

// Routes of 65 to 128 slots (verify and NVFP4 at 16 tokens): one wave, lane
// l holding slots l and l + 64.  The key is the expert of a valid slot and E
// for any other slot, so it sorts after every expert.  One ballot per key bit
// and half, most significant bit first, gives for each of a lane's two keys
// the slots of each half holding a smaller key (lt) and an equal one (eq).  A
// valid slot's packed position is then popcount(lt) plus the equal keys in
// earlier slots: the stable pack.  The first slot of each expert holds that
// expert's first packed row, and expert_offsets is the suffix minimum of
// those rows over the experts (an expert with no slot takes the next one's),
// with the valid-slot count past the last.  Same tables, bit for bit, as the
// general kernel.
__global__ __launch_bounds__(64) void route_pack_pair_kernel(
    const int32_t *__restrict__ ids, int32_t S, int32_t k, int32_t E,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot,
    int32_t *__restrict__ sorted_token, int32_t *__restrict__ token_to_perm,
    int32_t *__restrict__ active, int32_t *__restrict__ num_active,
    int32_t *__restrict__ status)
{
    __shared__ int32_t fp[MOE_MAX_EXPERTS + 1];      // first packed row per expert, else nvalid
    const int lane = threadIdx.x;
    const int id0 = lane < S ? ids[lane] : -1;
    const int id1 = lane + 64 < S ? ids[lane + 64] : -1;
    const bool v0 = id0 >= 0 && id0 < E, v1 = id1 >= 0 && id1 < E;
    const int k0 = v0 ? id0 : E, k1 = v1 ? id1 : E;
    const int nbad = __popcll(__ballot(lane < S && !v0 && id0 != -1)) +
                     __popcll(__ballot(lane + 64 < S && !v1 && id1 != -1));
    const int nvalid = __popcll(__ballot(v0)) + __popcll(__ballot(v1));
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
    // slot l has the earlier slots of half 0 below it; slot 64 + l all of
    // half 0 and the earlier slots of half 1
    const int pos0 = __popcll(lt00) + __popcll(lt01) + __popcll(eq00 & below);
    const int pos1 = __popcll(lt10) + __popcll(lt11) + __popcll(eq10) + __popcll(eq11 & below);
    const bool first0 = v0 && (eq00 & below) == 0;
    const bool first1 = v1 && eq10 == 0 && (eq11 & below) == 0;
    const uint64_t fm0 = __ballot(first0), fm1 = __ballot(first1);
    const int na = __popcll(fm0) + __popcll(fm1);
    if (lane < S) token_to_perm[lane] = v0 ? pos0 : -1;
    if (lane + 64 < S) token_to_perm[lane + 64] = v1 ? pos1 : -1;
    if (v0) {
        sorted_slot[pos0] = lane;
        sorted_token[pos0] = lane / k;
    }
    if (v1) {
        sorted_slot[pos1] = lane + 64;
        sorted_token[pos1] = (lane + 64) / k;
    }
    // the ascending active list: an expert's rank is the distinct experts below it
    if (first0) active[__popcll(lt00 & fm0) + __popcll(lt01 & fm1)] = k0;
    if (first1) active[__popcll(lt10 & fm0) + __popcll(lt11 & fm1)] = k1;
    const int A = S < E ? S : E;
    for (int i = na + lane; i < A; i += 64) active[i] = -1;
    // expert_offsets
    for (int e = lane; e <= E; e += 64) fp[e] = nvalid;
    moe::lds_barrier();
    if (first0) fp[k0] = pos0;
    if (first1) fp[k1] = pos1;
    moe::lds_barrier();
    int carry = nvalid;
    for (int c0 = E & ~63; c0 >= 0; c0 -= 64) {
        const int e = c0 + lane;
        int v = e <= E ? fp[e] : nvalid;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_down(v, d, 64);
            if (lane + d < 64) v = min(v, o);
        }
        v = min(v, carry);
        if (e <= E) offsets[e] = v;
        carry = __builtin_amdgcn_readfirstlane(v);
    }
    if (lane == 0) {
        *num_active = na;
        *status = nbad;
    }
}

}  // namespace

hipError_t launch_route_pack(const int32_t *ids, int32_t M, int32_t k, int32_t E,
                             const MoeRouteDev &r, hipStream_t st)
{
    const int32_t S = M * k;
    if (S <= 64) {
        hipLaunchKernelGGL(route_pack_small_kernel, dim3(1), dim3(64), 0, st, ids, S, k, E, r.offsets,
                           r.sorted_slot, r.sorted_token, r.token_to_perm, r.active, r.num_active,
                           r.status);
        return hipGetLastError();
    }
    if (S <= 128) {
        hipLaunchKernelGGL(route_pack_pair_kernel, dim3(1), dim3(64), 0, st, ids, S, k, E, r.offsets,
                           r.sorted_slot, r.sorted_token, r.token_to_perm, r.active, r.num_active,
                           r.status);
        return hipGetLastError();
    }
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const size_t lds = sizeof(int32_t) * (size_t)E * (1 + kWaves);
    // Large routes: R runs of 2^lg groups, as few groups per run as the LDS
    // counters ([R][E] ints in 64 KB) and the stash (sorted_token: R*E <= S)
    // allow, and at most 64 runs.
    if (S >= kSplitMin) {
        const int ngroups = (S - 1) / 64 + 1;
        auto runs = [&](int l) { return (ngroups + (1 << l) - 1) >> l; };
        auto fits = [&](int R) {
            return R <= kMaxRuns && (size_t)R * E * 4 <= kCountLds && (int64_t)R * E <= S;
        };
        int lg = 0;
        while (lg < 30 && !fits(runs(lg))) ++lg;
        const int R = runs(lg);
        if (fits(R) && R >= kWaves) {
            hipLaunchKernelGGL(route_count_kernel, dim3(1), dim3(kThreads),
                               sizeof(int32_t) * (size_t)R * E, st, ids, S, E, R, lg, r.offsets,
                               r.active, r.num_active, r.status, r.sorted_token);
            hipLaunchKernelGGL(route_place_kernel, dim3(R), dim3(64), sizeof(int32_t) * (size_t)E, st,
                               ids, S, k, E, nbits, lg, r.sorted_token, r.sorted_slot, r.token_to_perm);
            hipLaunchKernelGGL(route_token_kernel, dim3((unsigned)(((int64_t)S + 255) / 256)), dim3(256), 0, st,
                               r.sorted_slot, r.offsets, E, k, r.sorted_token);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL(route_pack_kernel, dim3(1), dim3(kThreads), lds, st, ids, S, k, E, nbits,
                       r.offsets, r.sorted_slot, r.sorted_token, r.token_to_perm, r.active,
                       r.num_active, r.status);
    return hipGetLastError();
}
