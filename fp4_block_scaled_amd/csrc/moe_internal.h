// moe_internal.h -- launchers and device helpers shared by libmoe's kernels.
// gfx950 (CDNA4) only: 64-lane wavefronts, OCP FP8 conversions, MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// workspace layout (shared by the host entry points)
// ---------------------------------------------------------------------------
inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Bytes of the route region for S = M*k slots and E experts.
inline size_t route_region_bytes(int64_t S, int64_t E)
{
    int64_t A = S < E ? S : E;
    return align256(sizeof(int32_t) * (size_t)(E + 1)) +      // expert_offsets
           3 * align256(sizeof(int32_t) * (size_t)S) +         // sorted_slot, sorted_token, token_to_perm
           align256(sizeof(int32_t) * (size_t)(A > 0 ? A : 1)) + // active_experts
           align256(sizeof(int32_t) * 2);                      // num_active, status
}

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Sum over each aligned group of 8 lanes; every lane of the group ends with
// the group sum.  quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror.
__device__ __forceinline__ float sum8_lanes(float v)
{
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    return v;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace moe

// ---------------------------------------------------------------------------
// launchers (return hipError_t of the launch)
// ---------------------------------------------------------------------------
struct MoeRouteDev {
    int32_t *offsets, *sorted_slot, *sorted_token, *token_to_perm, *active, *num_active, *status;
};

hipError_t launch_route_pack(const int32_t *ids, int32_t M, int32_t k, int32_t E,
                             const MoeRouteDev &r, hipStream_t st);

// E4M3 dequant-GEMV tier.
struct GemvBankDev {
    const uint8_t *codes;
    const void *scales;
    const float *scale2;
};

// M bounds the slots one expert usually holds (one per token); it sizes the
// LDS slot tile.  Experts holding more slots are swept in several passes.
hipError_t launch_gemv_gateup_e4m3(const GemvBankDev &gate, const GemvBankDev &up,
                                   const uint16_t *x, const MoeRouteDev &r, int32_t M,
                                   int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                   float *partials, int32_t nks, hipStream_t st);
// Down projection; with more than one K slice the slices go to slice_scratch
// ([gemv_down_slices(fmt, inter)][S][hidden] floats) and are summed in order
// into y.
hipError_t launch_gemv_down_e4m3(const GemvBankDev &down, const float *h, const MoeRouteDev &r,
                                 int32_t M, int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                 float *y, float *slice_scratch, hipStream_t st);

hipError_t launch_gemv_gateup_nvfp4(const GemvBankDev &gate, const GemvBankDev &up,
                                    const uint16_t *x, const MoeRouteDev &r, int32_t M,
                                    int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                    float *partials, int32_t nks, hipStream_t st);
hipError_t launch_gemv_down_nvfp4(const GemvBankDev &down, const float *h, const MoeRouteDev &r,
                                  int32_t M, int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                  float *y, float *slice_scratch, hipStream_t st);

// h[p][n] = swiglu_clamp(sum_ks P[ks][p][n], sum_ks P[ks][p][I + n]) for p < offsets[E].
hipError_t launch_swiglu_partials(const float *partials, int32_t nks, int32_t S, int32_t inter,
                                  const int32_t *offsets, int32_t E, float limit, float *h,
                                  hipStream_t st);

// FP8 GEMM tier (E4M3 banks, wide M).
int gemm_max_tiles(int32_t S, int32_t E);
hipError_t launch_quant_act(const uint16_t *x, int32_t M, int32_t hidden, uint8_t *xq, float *xs,
                            hipStream_t st);
hipError_t launch_gemm_tiles(const int32_t *offsets, int32_t E, int32_t tmax, int4 *tiles,
                             int32_t *ntiles, hipStream_t st);
hipError_t launch_gemm_gateup(const uint8_t *xq, const float *xs, const int32_t *sorted_token,
                              const uint8_t *gcodes, const float *gscales, const uint8_t *ucodes,
                              const float *uscales, const int32_t *offsets, const int4 *tiles,
                              const int32_t *ntiles, int32_t tmax, int32_t hidden, int32_t inter,
                              float limit, uint8_t *hq, float *hs, hipStream_t st);
hipError_t launch_gemm_down(const uint8_t *hq, const float *hs, const uint8_t *dcodes,
                            const float *dscales, const int32_t *offsets, const int4 *tiles,
                            const int32_t *ntiles, int32_t tmax, int32_t hidden, int32_t inter,
                            float *y, hipStream_t st);

hipError_t launch_combine(const float *y, const int32_t *token_to_perm, const float *w,
                          int32_t M, int32_t k, int32_t hidden, float *out, hipStream_t st);

// K slicing of the GEMV tier.  A segment is the K span of one 128-byte row
// chunk (128 values for E4M3, 256 for NVFP4); a slice is SEGS segments with
// SEGS the largest divisor of the segment count not above the cap (8, or 16
// for the E4M3 down projection when it divides).  Host sizing and launches
// both use these.
constexpr int kFmtE4M3 = 1, kFmtNVFP4 = 2;
inline int gemv_seg_k(int fmt) { return fmt == kFmtNVFP4 ? 256 : 128; }
inline int gemv_pick_segs(int nsegs, int cap)
{
    for (int d = cap; d > 1; --d)
        if (nsegs % d == 0) return d;
    return 1;
}
inline int gemv_segs_gateup(int fmt, int hidden) { return gemv_pick_segs(hidden / gemv_seg_k(fmt), 8); }
inline int gemv_segs_down(int fmt, int inter)
{
    const int n = inter / gemv_seg_k(fmt);
    if (fmt == kFmtE4M3 && n % 16 == 0) return 16;
    return gemv_pick_segs(n, 8);
}
inline int gemv_gateup_slices(int fmt, int hidden)
{
    return hidden / gemv_seg_k(fmt) / gemv_segs_gateup(fmt, hidden);
}
inline int gemv_down_slices(int fmt, int inter)
{
    return inter / gemv_seg_k(fmt) / gemv_segs_down(fmt, inter);
}
