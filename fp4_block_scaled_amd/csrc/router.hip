// router.hip -- top-k experts and their weights for every token row, in one
// launch.
//
// The router step before the routed layer: "spark_model
// glm5next_mlp/forward.rs", fn forward_moe, runs one top-k launch for all
// rows (bias, routed_scale, renormalize, one expert group) instead of one per
// row; "memra-engine src/bin/ep_step_fp8_gate.rs" gates its full layer on a
// sigmoid top-k router with a router bias, a router scale and a route norm.
//
// One wave64 per token row; lane l holds experts l, l + 64, ... (up to 8 each,
// 512 experts).  The k-th largest key is found by a radix select on its
// order-preserving bits with wave ballots (no cross-lane shuffles); the keys
// above it, then the equal ones by ascending id, are the choice.  The chosen
// entries are ranked in LDS (larger key first, equal keys by id).  Everything a weight is
// made of is computed in double and rounded once to binary32; sums over the
// chosen experts run in rank order, the full softmax denominator over experts
// in ascending order, so the weights follow one fixed sequence of operations.
#include <cfloat>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace {

constexpr int kRouterThreads = 256;
constexpr int kRowsPerBlock = kRouterThreads / moe::kWave;
constexpr int kPerLane = MOE_MAX_EXPERTS / moe::kWave;

struct RouterArgs {
    const float *logits;     // [M][E]
    const float *bias;       // [E] or null (sigmoid only)
    int32_t *ids;            // [M][k]
    float *w;                // [M][k]
    int32_t M, E, k, kind, renorm;
    float scale;
};

// NaN counts as -FLT_MAX, +-inf as +-FLT_MAX: keys and weights stay finite
__device__ __forceinline__ float canon_logit(float v)
{
    if (v != v) return -FLT_MAX;
    return fminf(fmaxf(v, -FLT_MAX), FLT_MAX);
}

// binary32 -> unsigned key with the same order; -0 and +0 map to one key
__device__ __forceinline__ uint32_t order_bits(float f)
{
    if (f == 0.0f) f = 0.0f;
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float wave_max_f32(float v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
    return v;
}

// LDS written by some lanes of this wave is read by others after this point
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per wave in dynamic LDS, k entries each: the chosen experts in id order
// (key, id, value), then the ids and values in rank order; for the softmax
// without renormalization also exp(l - m) of every expert.
struct RouterLds {
    uint32_t *key;
    int32_t *id;
    double *val;
    int32_t *rid;
    double *rval;
    double *all;
};

__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(RouterArgs a)
{
    extern __shared__ double dyn[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * kRowsPerBlock + wave;
    if (row >= a.M) return;                          // whole wave
    const int E = a.E, k = a.k;
    const float *lr = a.logits + (size_t)row * E;
    RouterLds L;
    {
        double *base = dyn + (size_t)wave * 3 * k;   // 24 bytes per chosen entry
        L.val = base;
        L.rval = base + k;
        L.key = reinterpret_cast<uint32_t *>(base + 2 * k);
        L.id = reinterpret_cast<int32_t *>(L.key + k);
        L.rid = reinterpret_cast<int32_t *>(dyn + (size_t)kRowsPerBlock * 3 * k) + wave * k;
        L.all = dyn + (size_t)kRowsPerBlock * 3 * k + ((size_t)kRowsPerBlock * k + 1) / 2 + (size_t)wave * E;
    }
    const bool full_softmax = a.kind == 0 && !a.renorm;

    float l[kPerLane];                               // canonical logits
    double s[kPerLane];                              // sigmoid, or exp(l - m) for the softmax
    uint32_t key[kPerLane];                          // order-preserving key bits
    bool ok[kPerLane];                               // an expert (e < E)
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        const int e = lane + 64 * q;
        ok[q] = e < E;
        l[q] = ok[q] ? canon_logit(lr[e]) : -FLT_MAX;
    }
    float m = 0.0f;                                  // softmax: the largest logit
    if (a.kind == 0) {
        float mm = l[0];
#pragma unroll
        for (int q = 1; q < kPerLane; ++q) mm = fmaxf(mm, l[q]);
        m = wave_max_f32(mm);
    }
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        s[q] = 0.0;
        key[q] = 0;
        if (64 * q >= E) continue;                   // uniform: no expert in this slot
        const int e = lane + 64 * q;
        float kf;
        if (a.kind == 0) {
            if (full_softmax) s[q] = exp((double)l[q] - (double)m);
            kf = l[q];
        } else {
            s[q] = 1.0 / (1.0 + exp(-(double)l[q]));
            kf = __fadd_rn((float)s[q], a.bias ? a.bias[ok[q] ? e : 0] : 0.0f);
        }
        key[q] = order_bits(kf);
    }

    // T = the k-th largest key: the largest value with at least k keys >= it,
    // found bit by bit from the top with ballots.  Once exactly k keys are >= T
    // the choice is made (it is those k) and the remaining bits change nothing.
    uint32_t T = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = T | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int q = 0; q < kPerLane; ++q)
            if (64 * q < E) cnt += __popcll(__ballot(ok[q] && key[q] >= cand));
        if (cnt >= k) {
            T = cand;
            if (cnt == k) break;
        }
    }
    // chosen: every key above T, then keys equal to T by ascending id; each
    // chosen entry gets its place in id order
    int need = k, before = 0;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q)
        if (64 * q < E) need -= __popcll(__ballot(ok[q] && key[q] > T));
    const uint64_t below = (1ull << lane) - 1;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        if (64 * q >= E) continue;
        const uint64_t eq = __ballot(ok[q] && key[q] == T);
        const int take = min(__popcll(eq), need);
        need -= take;
        const bool pick_eq = key[q] == T && ok[q] && __popcll(eq & below) < take;
        const bool chosen = (ok[q] && key[q] > T) || pick_eq;
        const uint64_t ch = __ballot(chosen);
        if (chosen) {
            const int c = before + __popcll(ch & below);
            L.key[c] = key[q];
            L.id[c] = lane + 64 * q;
            L.val[c] = a.kind == 0 ? (double)l[q] : s[q];   // the softmax keeps the logit here
        }
        before += __popcll(ch);
    }
    wave_lds_sync();

    // rank of each chosen entry: larger keys first, equal keys by id
    for (int c = lane; c < k; c += 64) {
        const uint32_t kc = L.key[c];
        const int ic = L.id[c];
        int r = 0;
        for (int o = 0; o < k; ++o) {
            const uint32_t ko = L.key[o];
            r += ko > kc || (ko == kc && L.id[o] < ic);
        }
        L.rid[r] = ic;
        L.rval[r] = L.val[c];
    }
    wave_lds_sync();

    // softmax without renormalization: the denominator over every expert, e ascending
    double den = 1.0;
    if (full_softmax) {
#pragma unroll
        for (int q = 0; q < kPerLane; ++q)
            if (ok[q]) L.all[lane + 64 * q] = s[q];
        wave_lds_sync();
        den = 0.0;
        for (int e = 0; e < E; ++e) den += L.all[e];
    }
    // raw value per rank, then the chosen sum in rank order
    const double l0 = L.rval[0];
    for (int r = lane; r < k; r += 64) {
        const double x = L.rval[r];
        double v;
        if (a.kind == 0) v = a.renorm ? exp(x - l0) : exp(x - (double)m) / den;
        else v = x;
        L.val[r] = v;                                 // reuse: raw values in rank order
    }
    wave_lds_sync();
    double sum = 0.0;
    if (a.renorm)
        for (int r = 0; r < k; ++r) sum += L.val[r];
    for (int r = lane; r < k; r += 64) {
        // the sigmoid's chosen sum is 0 only if every chosen s underflows: weights 0
        const double v = a.renorm ? (sum > 0.0 ? L.val[r] / sum : 0.0) : L.val[r];
        a.ids[(size_t)row * k + r] = L.rid[r];
        a.w[(size_t)row * k + r] = (float)(v * (double)a.scale);
    }
}

}  // namespace

hipError_t launch_router_topk(const float *logits, int32_t M, int32_t E, int32_t k, int32_t kind,
                              const float *bias, float routed_scale, int32_t renormalize,
                              int32_t *ids, float *w, hipStream_t st)
{
    RouterArgs a{logits, bias, ids, w, M, E, k, kind, renormalize ? 1 : 0, routed_scale};
    const int grid = (M + kRowsPerBlock - 1) / kRowsPerBlock;
    // per wave: val, rval (double) and key, id (32-bit) for k entries, then rid
    // (rounded up to whole doubles), then E doubles for the full softmax
    size_t lds = (size_t)kRowsPerBlock * 3 * k * sizeof(double) +
                 (((size_t)kRowsPerBlock * k + 1) / 2) * sizeof(double);
    if (kind == 0 && !renormalize) lds += (size_t)kRowsPerBlock * E * sizeof(double);
    hipLaunchKernelGGL(router_topk_kernel, dim3(grid), dim3(kRouterThreads), lds, st, a);
    return hipGetLastError();
}
