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
// One workgroup of 1024 threads (16 wave64s):
//   1. LDS histogram of ids (integer LDS atomics: order-free, exact).
//   2. Block exclusive scans give expert_offsets and the compacted
//      active-expert list.
//   3. Placement in chunks of 1024 slots.  Inside a wave, lanes holding the
//      same expert find each other by ballots over the id bits; a lane's rank
//      is the popcount of its lower peers.  Per-wave counts go to LDS so each
//      slot adds the counts of lower waves and of earlier chunks: the result
//      is stable in slot order and bit-identical on every run.
#include "moe_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / moe::kWave;

__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

__global__ __launch_bounds__(kThreads) void route_pack_kernel(
    const int32_t *__restrict__ ids, int32_t S, int32_t k, int32_t E, int32_t nbits,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot,
    int32_t *__restrict__ sorted_token, int32_t *__restrict__ token_to_perm,
    int32_t *__restrict__ active, int32_t *__restrict__ num_active,
    int32_t *__restrict__ status)
{
    extern __shared__ int32_t lds[];
    int32_t *base = lds;           // [E]  counts, then exclusive offsets
    int32_t *fill = base + E;      // [E]  slots already placed per expert
    int32_t *hist = fill + E;      // [kWaves][E] per-wave counts of one chunk
    __shared__ int32_t wsum_c[kWaves], wsum_f[kWaves], s_invalid;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int i = tid; i < E; i += kThreads) { base[i] = 0; fill[i] = 0; }
    for (int i = tid; i < kWaves * E; i += kThreads) hist[i] = 0;
    if (tid == 0) s_invalid = 0;
    __syncthreads();

    // 1. histogram
    int bad = 0;
    for (int s = tid; s < S; s += kThreads) {
        int e = ids[s];
        if (e >= 0 && e < E) atomicAdd(&base[e], 1);
        else if (e != -1) ++bad;
    }
    for (int d = 32; d >= 1; d >>= 1) bad += __shfl_xor(bad, d, 64);
    if (lane == 0 && bad) atomicAdd(&s_invalid, bad);
    __syncthreads();

    // 2. exclusive scans over experts (E <= kThreads: one expert per thread)
    int c = tid < E ? base[tid] : 0;
    int f = c > 0 ? 1 : 0;
    int ic = wave_incl_scan(c, lane), iff = wave_incl_scan(f, lane);
    if (lane == 63) { wsum_c[wave] = ic; wsum_f[wave] = iff; }
    __syncthreads();
    int pc = 0, pf = 0;
    for (int w = 0; w < wave; ++w) { pc += wsum_c[w]; pf += wsum_f[w]; }
    int ex_c = pc + ic - c, ex_f = pf + iff - f;
    if (tid < E) {
        offsets[tid] = ex_c;
        base[tid] = ex_c;
        if (f) active[ex_f] = tid;
        if (tid == E - 1) { offsets[E] = ex_c + c; *num_active = ex_f + f; }
    }
    __syncthreads();
    // entries past num_active hold -1, so a consumer that reads active[i]
    // for i < min(E, S) can tell an unused entry without reading num_active
    {
        int na = 0;
        for (int w = 0; w < kWaves; ++w) na += wsum_f[w];
        const int A = S < E ? S : E;
        for (int i = na + tid; i < A; i += kThreads) active[i] = -1;
    }

    // 3. stable placement, 1024 slots per chunk
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < S; c0 += kThreads) {
        const int s = c0 + tid;
        int e = (s < S) ? ids[s] : -1;
        const bool valid = (e >= 0 && e < E);
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const int rank = __popcll(peers & lower);
        if (valid && rank == 0) hist[wave * E + e] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int pos = base[e] + fill[e] + rank;
            for (int w = 0; w < wave; ++w) pos += hist[w * E + e];
            sorted_slot[pos] = s;
            sorted_token[pos] = s / k;
            token_to_perm[s] = pos;
        } else if (s < S) {
            token_to_perm[s] = -1;
        }
        __syncthreads();
        for (int i = tid; i < E; i += kThreads) {
            int add = 0;
            for (int w = 0; w < kWaves; ++w) { add += hist[w * E + i]; hist[w * E + i] = 0; }
            fill[i] += add;
        }
        __syncthreads();
    }
    if (tid == 0) *status = s_invalid;
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
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const size_t lds = sizeof(int32_t) * (size_t)E * (2 + kWaves);
    hipLaunchKernelGGL(route_pack_kernel, dim3(1), dim3(kThreads), lds, st, ids, S, k, E, nbits,
                       r.offsets, r.sorted_slot, r.sorted_token, r.token_to_perm, r.active,
                       r.num_active, r.status);
    return hipGetLastError();
}
