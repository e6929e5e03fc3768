// moe_internal.h -- workspace layout and launchers shared by libmoe's
// sources; the device helpers the kernels share are in moe_device.h.
// gfx950 (CDNA4) only: 64-lane wavefronts, OCP FP8 conversions, MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {

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

}  // namespace moe

// ---------------------------------------------------------------------------
// launchers (return hipError_t of the launch)
// ---------------------------------------------------------------------------
struct MoeRouteDev {
    int32_t *offsets, *sorted_slot, *sorted_token, *token_to_perm, *active, *num_active, *status;
};

// Router: one wave per token row (router.hip).
hipError_t launch_router_topk(const float *logits, int32_t M, int32_t E, int32_t k, int32_t kind,
                              const float *bias, float routed_scale, int32_t renormalize,
                              int32_t *ids, float *w, hipStream_t st);

hipError_t launch_route_pack(const int32_t *ids, int32_t M, int32_t k, int32_t E,
                             const MoeRouteDev &r, hipStream_t st);

// E4M3 dequant-GEMV tier.
struct GemvBankDev {
    const uint8_t *codes;
    const void *scales;
    const float *scale2;
};

// M bounds the slots one expert usually holds (one per token); it sizes the
// slot tile of a pass.  Experts holding more slots are swept in several
// passes.  Gate/up covers the whole of K per block and writes h =
// SwiGLU(gate x, up x) ([S][inter] floats) directly.
// With route_ids (S <= 128 slots of top_k each), the route is built inside
// the launch from the ids and block 0 writes the tables of r; otherwise the
// tables of r come from route_pack.
hipError_t launch_gemv_gateup_e4m3(const GemvBankDev &gate, const GemvBankDev &up,
                                   const uint16_t *x, const MoeRouteDev &r, int32_t M,
                                   int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                   float limit, float *h, hipStream_t st,
                                   const int32_t *route_ids = nullptr, int32_t top_k = 0);
// Down projection: a block covers 32 output rows over the whole of K and
// writes y ([S][hidden] floats) directly.
hipError_t launch_gemv_down_e4m3(const GemvBankDev &down, const float *h, const MoeRouteDev &r,
                                 int32_t M, int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                 float *y, hipStream_t st);

// Fused decode layer (E4M3): route pack, gate/up + SwiGLU, down and combine
// in one launch of resident blocks.  S = M*k <= fused_decode_max_slots();
// flags: min(S, E) x (inter/2 + hidden/32) 32-bit words, any contents;
// epoch: a value no earlier call on these flags used.
int fused_decode_max_slots();
hipError_t launch_fused_decode_e4m3(const GemvBankDev &gate, const GemvBankDev &up,
                                    const GemvBankDev &down, const uint16_t *x, const int32_t *ids,
                                    const float *w, int32_t M, int32_t k, int32_t E, int32_t hidden,
                                    int32_t inter, float limit, const MoeRouteDev &r, float *h,
                                    float *y, float *out, void *flags, uint32_t epoch,
                                    hipStream_t st);

// Fused decode layer for NVFP4 banks: one token (M == 1), hidden a multiple
// of 2048 up to 16384; flags and epoch as for launch_fused_decode_e4m3.
hipError_t launch_fused_decode_nvfp4(const GemvBankDev &gate, const GemvBankDev &up,
                                     const GemvBankDev &down, const uint16_t *x, const int32_t *ids,
                                     const float *w, int32_t M, int32_t k, int32_t E, int32_t hidden,
                                     int32_t inter, float limit, const MoeRouteDev &r, float *h,
                                     float *y, float *out, void *flags, uint32_t epoch,
                                     hipStream_t st);

hipError_t launch_gemv_gateup_nvfp4(const GemvBankDev &gate, const GemvBankDev &up,
                                    const uint16_t *x, const MoeRouteDev &r, int32_t M,
                                    int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                    float limit, float *h, hipStream_t st,
                                    const int32_t *route_ids = nullptr, int32_t top_k = 0);
hipError_t launch_gemv_down_nvfp4(const GemvBankDev &down, const float *h, const MoeRouteDev &r,
                                  int32_t M, int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                  float *y, hipStream_t st);

// FP8 GEMM tier (E4M3 banks, wide M).
int gemm_max_tiles(int32_t S, int32_t E);
hipError_t launch_quant_act(const uint16_t *x, int32_t M, int32_t hidden, uint8_t *xq, float *xs,
                            hipStream_t st);
// Row tiles per expert: balanced chunks of at most 128 rows (E4M3 tier),
// or runs of exactly 128 rows but the last (NVFP4 tier).
hipError_t launch_gemm_tiles(const int32_t *offsets, int32_t E, int32_t tmax, int4 *tiles,
                             int32_t *ntiles, hipStream_t st, bool balanced);
hipError_t launch_gemm_gateup(const uint8_t *xq, const float *xs, const int32_t *sorted_token,
                              const uint8_t *gcodes, const float *gscales, const uint8_t *ucodes,
                              const float *uscales, const int32_t *offsets, const int4 *tiles,
                              const int32_t *ntiles, int32_t tmax, int32_t hidden, int32_t inter,
                              float limit, uint8_t *hq, float *hs, hipStream_t st);
hipError_t launch_gemm_down(const uint8_t *hq, const float *hs, const uint8_t *dcodes,
                            const float *dscales, const int32_t *offsets, const int4 *tiles,
                            const int32_t *ntiles, int32_t tmax, int32_t hidden, int32_t inter,
                            float *y, hipStream_t st);

// 16-bit MFMA GEMM tier (NVFP4 banks, wide M): gate/up (bf16 x) with SwiGLU
// writes h as FP16 [S][inter], scaled by a power of two picked from the clamp
// limit; down (FP16 MFMA) reads it and takes the same limit to undo the scale.
hipError_t launch_gemm_gateup_nvfp4(const uint16_t *x, const int32_t *sorted_token,
                                    const GemvBankDev &gate, const GemvBankDev &up,
                                    const int32_t *offsets, const int4 *tiles,
                                    const int32_t *ntiles, int32_t tmax, int32_t hidden,
                                    int32_t inter, float limit, uint16_t *h16, hipStream_t st);
hipError_t launch_gemm_down_nvfp4(const uint16_t *h16, const GemvBankDev &down,
                                  const int32_t *offsets, const int4 *tiles, const int32_t *ntiles,
                                  int32_t tmax, int32_t hidden, int32_t inter, float limit, float *y,
                                  hipStream_t st);

// shared and residual ([M][hidden] FP32) may be null; each is added after
// the routed sum, in that order.
hipError_t launch_combine(const float *y, const int32_t *token_to_perm, const float *w,
                          int32_t M, int32_t k, int32_t hidden, const float *shared,
                          const float *residual, float *out, hipStream_t st);

// Shared expert (dense bf16 SwiGLU MLP of width W) for M <= 16 tokens:
// h [M][W] FP32 scratch, out [M][hidden] FP32.  hidden and W multiples of
// 512 up to 8192.
hipError_t launch_shared_expert(const uint16_t *gate, const uint16_t *up, const uint16_t *down,
                                const uint16_t *x, int32_t M, int32_t hidden, int32_t W,
                                float limit, float *h, float *out, hipStream_t st);

// K chunking of the GEMV tier.  A segment is the K span of one 128-byte row
// chunk (128 values for E4M3, 256 for NVFP4); both projections stream the
// whole of K per block, in chunks of a few segments.
constexpr int kFmtE4M3 = 1, kFmtNVFP4 = 2;
inline int gemv_seg_k(int fmt) { return fmt == kFmtNVFP4 ? 256 : 128; }
inline int gemv_pick_segs(int nsegs, int cap)
{
    for (int d = cap; d > 1; --d)
        if (nsegs % d == 0) return d;
    return 1;
}

// Slots per weight pass of the gate/up GEMV: their bf16 x rows sit in LDS
// for the whole of K, so the pass holds as many as fit in 32 KB (at least
// one), at most cap and at most M.
inline int gemv_gateup_pass_slots(int M, int hidden, int cap)
{
    int n = 32768 / (2 * hidden);
    if (n < 1) n = 1;
    if (n > cap) n = cap;
    return n < M ? n : M;
}

// Same for the down GEMV, whose FP32 h rows sit in LDS: as many as fit in
// 16 KB (at least one), at most cap and at most M.
inline int gemv_down_pass_slots(int M, int inter, int cap)
{
    int n = 16384 / (4 * inter);
    if (n < 1) n = 1;
    if (n > cap) n = cap;
    return n < M ? n : M;
}

// Segments per K chunk: the largest divisor of the segment count up to 8
// (E4M3 gate/up), 4 (NVFP4 gate/up, E4M3 down) or 2 (NVFP4 down), so a chunk
// spans at most 1024 K values for gate/up and 512 for down.
inline int gemv_chunk_segs(int fmt, int hidden)
{
    return gemv_pick_segs(hidden / gemv_seg_k(fmt), fmt == kFmtNVFP4 ? 4 : 8);
}
inline int gemv_down_chunk_segs(int fmt, int inter)
{
    return gemv_pick_segs(inter / gemv_seg_k(fmt), fmt == kFmtNVFP4 ? 2 : 4);
}

// Down projection and combine of one token in one launch (M == 1): y rows as
// launch_gemv_down_*, and out[hidden] = the slots' y rows weighted by w and
// added in slot order (the combine's arithmetic).  t2p [k]: the packed row
// of each slot, -1 for none; ids [k]: the slots' experts.  For the shapes
// gemv_down1_fits accepts (else hipErrorInvalidValue).
inline bool gemv_down1_fits(int fmt, int M, int k, int hidden, int inter)
{
    if (M != 1 || k < 1 || k > 8 || hidden % 16 != 0 || inter % 512 != 0) return false;
    return fmt == kFmtNVFP4 ? inter <= 2048 : inter <= 2560;
}
hipError_t launch_gemv_down1_e4m3(const GemvBankDev &down, const float *h, const int32_t *ids,
                                  const int32_t *t2p, const float *w, int32_t k, int32_t hidden,
                                  int32_t inter, float *y, float *out, hipStream_t st);
hipError_t launch_gemv_down1_nvfp4(const GemvBankDev &down, const float *h, const int32_t *ids,
                                   const int32_t *t2p, const float *w, int32_t k, int32_t hidden,
                                   int32_t inter, float *y, float *out, hipStream_t st);
