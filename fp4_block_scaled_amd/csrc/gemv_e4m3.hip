// gemv_e4m3.hip -- dequant-GEMV tier for block-scaled E4M3 expert banks.
//
// The small-M projections stream weights and do ~2 FLOP per weight byte, so
// they are bound by HBM bandwidth, not by matrix cores ("spark_model
// glm5next_mlp/forward.rs", doc of fn w4a16_gemv: the tile GEMM was far too
// slow on single-token expert projections, hence a GEMV).  Each block takes
// one ACTIVE expert (from the route pack) and applies every weight row it
// streams to all slots routed to that expert, so a union expert is read once
// however many rows chose it (the same page, fn w4a16_gemv_moe_batchm).
//
// Layout of the work on a 64-lane wave: lanes form 8 groups of 8; a group
// owns one weight row and each lane loads 16 consecutive code bytes, so one
// load instruction covers 8 rows x 128 bytes -- one full cache line per row,
// and exactly one 128-wide scale block along K.  Codes are converted on the
// fly (gfx950 OCP-FP8 converts), multiplied with the activation slice held in
// LDS, scaled by the block scale once per 16 products, accumulated in FP32,
// and reduced over the 8 lanes of a group with DPP.
//
//   gate+up: one launch covers both banks; K is cut into 1024-wide slices and
//            each slice writes an FP32 partial row; the SwiGLU kernel adds the
//            slices in a fixed order (deterministic, no atomics).
//   down:    K (= inter) in slices of 2048; with one slice the rows go
//            straight to y, otherwise slice partials are summed in order by a
//            small reduction kernel.
#include "moe_internal.h"

namespace {

using moe::bf16x2;
using moe::f32x2;

constexpr int kThreads = 256;                    // 4 waves

// Launch-shape constants (rows per wave = 8 * RG; slots per weight pass = ST).
#ifndef MOE_E4M3_GU_RG
#define MOE_E4M3_GU_RG 1
#endif
#ifndef MOE_E4M3_GU_ST
#define MOE_E4M3_GU_ST 8
#endif
#ifndef MOE_E4M3_DN_RG
#define MOE_E4M3_DN_RG 1
#endif
#ifndef MOE_E4M3_DN_ST
#define MOE_E4M3_DN_ST 4
#endif
// minimum waves per SIMD the register allocation must allow
#ifndef MOE_GEMV_MIN_WAVES
#define MOE_GEMV_MIN_WAVES 1
#endif

struct GateUpArgs {
    const uint8_t *gcodes, *ucodes;
    const float *gscales, *uscales;
    const uint16_t *x;
    const int32_t *offsets, *sorted_token, *active, *num_active;
    float *partials;
    int32_t S, H, I, nks, ntiles, st;   // st: slots per weight pass (<= ST)
};

struct DownArgs {
    const uint8_t *codes;
    const float *scales;
    const float *h;
    const int32_t *offsets, *active, *num_active;
    float *out;          // y [S][H] when nks == 1, else partials [nks][S][H]
    int32_t S, H, I, nks, ntiles, st;   // st: slots per weight pass (<= ST)
};

// Weights are streamed once per call: non-temporal loads keep them from
// displacing the activations and partial sums in the caches.
__device__ __forceinline__ uint4 load16(const uint8_t *p)
{
#ifndef MOE_GEMV_CACHED_LOADS
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    return *reinterpret_cast<const uint4 *>(p);
#endif
}

// 4 code bytes -> two bf16 pairs (bytes 0,1 and 2,3).  E4M3 values are exact
// in bf16 (3 mantissa bits, exponent range inside bf16's).
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t d, bf16x2 &lo, bf16x2 &hi)
{
    lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d, 1.0f, true);
}

__device__ __forceinline__ float dot2(bf16x2 a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b), c, false);
}

// ---------------------------------------------------------------------------
// gate + up
// ---------------------------------------------------------------------------
// SEGS: 128-wide K segments per slice (the slice width divides hidden);
// RG: 8-row groups per wave; ST: slots per pass over the weights.  A wave
// issues all RG*SEGS 16-byte loads of its rows before the first multiply, so
// up to RG*SEGS KB per wave are in flight.  The block's 128 rows share one
// 128-row scale block, so the SEGS scales are loaded once per block.
template <int SEGS, int RG, int ST>
__global__ __launch_bounds__(kThreads, MOE_GEMV_MIN_WAVES) void gemv_gateup_e4m3_kernel(GateUpArgs a)
{
    constexpr int RPW = RG * 8;
    constexpr int RPB = RPW * (kThreads / 64);
    static_assert(128 % RPB == 0, "block rows inside one 128-row scale block");
    extern __shared__ uint4 lds_x[];                 // bf16 x slice per slot: [a.st][SEGS*16]
    uint4 (*xs)[SEGS * 16] = reinterpret_cast<uint4 (*)[SEGS * 16]>(lds_x);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int grp = lane >> 3, sub = lane & 7;
    int bid = blockIdx.x;
    const int ks = bid % a.nks;
    bid /= a.nks;
    const int tile = bid % a.ntiles;
    const int ai = bid / a.ntiles;
    const int e = a.active[ai];              // -1 past the active experts
    if (e < 0) return;
    const int H = a.H, I = a.I;
    const int half = a.ntiles >> 1;
    const bool is_up = tile >= half;
    const uint8_t *codes = (is_up ? a.ucodes : a.gcodes) + (size_t)e * I * H;
    const int sc_cols = H >> 7;
    const int row_b0 = (is_up ? tile - half : tile) * RPB;
    const int col_b0 = (is_up ? I : 0) + row_b0;
    const int k0 = ks * SEGS * 128;
    const size_t pstride = (size_t)2 * I;

    // block scales of this slice: lane l holds scale (l % SEGS)
    const float *sc_blk = (is_up ? a.uscales : a.gscales) + (size_t)e * (I >> 7) * sc_cols +
                          (size_t)(row_b0 >> 7) * sc_cols + (k0 >> 7);
    const float sc_lane = sc_blk[lane % SEGS];

    const uint8_t *rp = codes + (size_t)(row_b0 + wave * RPW + grp) * H + k0 + sub * 16;
    // weight loads go out first; the slot range is read while they fly
    int p0 = 0, ne = 1;
    for (int st = 0; st < ne; st += a.st) {
        uint4 w[RG][SEGS];
#ifdef MOE_GEMV_X_FIRST
        if (st == 0) { p0 = a.offsets[e]; ne = a.offsets[e + 1] - p0; }
        const int nt = min(a.st, ne - st);
        for (int c = tid; c < nt * SEGS * 16; c += kThreads) {
            const int j = c / (SEGS * 16), r = c - j * (SEGS * 16);
            const int tok = a.sorted_token[p0 + st + j];
            xs[j][r] = *reinterpret_cast<const uint4 *>(a.x + (size_t)tok * H + k0 + r * 8);
        }
#endif
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) w[rg][sg] = load16(rp + (size_t)rg * 8 * H + sg * 128);
#ifndef MOE_GEMV_X_FIRST
        if (st == 0) { p0 = a.offsets[e]; ne = a.offsets[e + 1] - p0; }
        const int nt = min(a.st, ne - st);
        for (int c = tid; c < nt * SEGS * 16; c += kThreads) {
            const int j = c / (SEGS * 16), r = c - j * (SEGS * 16);
            const int tok = a.sorted_token[p0 + st + j];
            xs[j][r] = *reinterpret_cast<const uint4 *>(a.x + (size_t)tok * H + k0 + r * 8);
        }
#endif
        __syncthreads();

#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            float acc[ST];
#pragma unroll
            for (int j = 0; j < ST; ++j) acc[j] = 0.0f;
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                const float s = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_lane), sg));
                bf16x2 wb[8];
                e4m3x4_to_bf16(w[rg][sg].x, wb[0], wb[1]);
                e4m3x4_to_bf16(w[rg][sg].y, wb[2], wb[3]);
                e4m3x4_to_bf16(w[rg][sg].z, wb[4], wb[5]);
                e4m3x4_to_bf16(w[rg][sg].w, wb[6], wb[7]);
#pragma unroll
                for (int j = 0; j < ST; ++j) {
                    if (j < nt) {
                        const uint4 xa = xs[j][sg * 16 + sub * 2];
                        const uint4 xb = xs[j][sg * 16 + sub * 2 + 1];
                        float d = dot2(wb[0], xa.x, 0.0f);
                        d = dot2(wb[1], xa.y, d);
                        d = dot2(wb[2], xa.z, d);
                        d = dot2(wb[3], xa.w, d);
                        d = dot2(wb[4], xb.x, d);
                        d = dot2(wb[5], xb.y, d);
                        d = dot2(wb[6], xb.z, d);
                        d = dot2(wb[7], xb.w, d);
                        acc[j] = fmaf(d, s, acc[j]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                if (j < nt) {
                    const float v = moe::sum8_lanes(acc[j]);
                    if (sub == 0)
                        a.partials[((size_t)ks * a.S + p0 + st + j) * pstride + col_b0 + wave * RPW +
                                   rg * 8 + grp] = v;
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------
// h slice staged in LDS with the float4 of lane `sub`, part q of segment sg at
// index sg*32 + q*8 + sub, so the 8 lanes of a group read 128 contiguous
// bytes per LDS instruction (no bank conflicts).  The block's 64 rows lie in
// one 128-row scale block.
template <int SEGS, int RG, int ST>
__global__ __launch_bounds__(kThreads, MOE_GEMV_MIN_WAVES) void gemv_down_e4m3_kernel(DownArgs a)
{
    constexpr int RPW = RG * 8;
    constexpr int RPB = RPW * (kThreads / 64);
    static_assert(128 % RPB == 0, "block rows inside one 128-row scale block");
    extern __shared__ float4 lds_h[];                // FP32 h slice per slot: [a.st][SEGS*32]
    float4 (*hs)[SEGS * 32] = reinterpret_cast<float4 (*)[SEGS * 32]>(lds_h);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int grp = lane >> 3, sub = lane & 7;
    int bid = blockIdx.x;
    const int ks = bid % a.nks;
    bid /= a.nks;
    const int tile = bid % a.ntiles;
    const int ai = bid / a.ntiles;
    const int e = a.active[ai];              // -1 past the active experts
    if (e < 0) return;
    const int H = a.H, I = a.I;
    const uint8_t *codes = a.codes + (size_t)e * H * I;
    const int sc_cols = I >> 7;
    const int row_b0 = tile * RPB;
    const int k0 = ks * SEGS * 128;
    float *out = a.out + (size_t)ks * a.S * H;

    const float *sc_blk = a.scales + (size_t)e * (H >> 7) * sc_cols +
                          (size_t)(row_b0 >> 7) * sc_cols + (k0 >> 7);
    const float sc_lane = sc_blk[lane % SEGS];

    const uint8_t *rp = codes + (size_t)(row_b0 + wave * RPW + grp) * I + k0 + sub * 16;
    int p0 = 0, ne = 1;
    for (int st = 0; st < ne; st += a.st) {
        uint4 w[RG][SEGS];
#ifdef MOE_GEMV_X_FIRST
        if (st == 0) { p0 = a.offsets[e]; ne = a.offsets[e + 1] - p0; }
        const int nt = min(a.st, ne - st);
        for (int c = tid; c < nt * SEGS * 32; c += kThreads) {
            const int j = c / (SEGS * 32), f = c - j * (SEGS * 32);  // f = source float4 index
            const int sg = f >> 5, r = f & 31, sb = r >> 2, q = r & 3;
            hs[j][sg * 32 + q * 8 + sb] =
                *reinterpret_cast<const float4 *>(a.h + (size_t)(p0 + st + j) * I + k0 + f * 4);
        }
#endif
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) w[rg][sg] = load16(rp + (size_t)rg * 8 * I + sg * 128);
#ifndef MOE_GEMV_X_FIRST
        if (st == 0) { p0 = a.offsets[e]; ne = a.offsets[e + 1] - p0; }
        const int nt = min(a.st, ne - st);
        for (int c = tid; c < nt * SEGS * 32; c += kThreads) {
            const int j = c / (SEGS * 32), f = c - j * (SEGS * 32);  // f = source float4 index
            const int sg = f >> 5, r = f & 31, sb = r >> 2, q = r & 3;
            hs[j][sg * 32 + q * 8 + sb] =
                *reinterpret_cast<const float4 *>(a.h + (size_t)(p0 + st + j) * I + k0 + f * 4);
        }
#endif
        __syncthreads();

#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            float acc[ST];
#pragma unroll
            for (int j = 0; j < ST; ++j) acc[j] = 0.0f;
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                const float s = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_lane), sg));
                f32x2 wf[8];
                const uint32_t dw[4] = {w[rg][sg].x, w[rg][sg].y, w[rg][sg].z, w[rg][sg].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    wf[2 * q] = __builtin_amdgcn_cvt_pk_f32_fp8((int)dw[q], false);
                    wf[2 * q + 1] = __builtin_amdgcn_cvt_pk_f32_fp8((int)dw[q], true);
                }
#pragma unroll
                for (int j = 0; j < ST; ++j) {
                    if (j < nt) {
                        float d = 0.0f;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 hv = hs[j][sg * 32 + q * 8 + sub];
                            d = fmaf(wf[2 * q].x, hv.x, d);
                            d = fmaf(wf[2 * q].y, hv.y, d);
                            d = fmaf(wf[2 * q + 1].x, hv.z, d);
                            d = fmaf(wf[2 * q + 1].y, hv.w, d);
                        }
                        acc[j] = fmaf(d, s, acc[j]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                if (j < nt) {
                    const float v = moe::sum8_lanes(acc[j]);
                    if (sub == 0)
                        out[(size_t)(p0 + st + j) * H + row_b0 + wave * RPW + rg * 8 + grp] = v;
                }
            }
        }
        __syncthreads();
    }
}

// y[p][m] = sum over slices of partials, slice order; rows p < offsets[E].
__global__ __launch_bounds__(256) void sum_slices_kernel(const float *__restrict__ part, int32_t nks,
                                                         int32_t S, int32_t H,
                                                         const int32_t *__restrict__ offsets,
                                                         int32_t E, float *__restrict__ y)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;    // float4 index
    const size_t n4 = (size_t)offsets[E] * H / 4;
    if (i >= n4) return;
    float4 acc = reinterpret_cast<const float4 *>(part)[i];
    for (int ks = 1; ks < nks; ++ks) {
        const float4 v = reinterpret_cast<const float4 *>(part + (size_t)ks * S * H)[i];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    reinterpret_cast<float4 *>(y)[i] = acc;
}

}  // namespace

// Launch shapes.  Grid = (upper bound on active experts) x (row tiles) x
// (K slices); blocks whose active index is past num_active exit at once, so
// the host never needs the routing.
namespace {

template <int SEGS>
void gateup_launch(const GateUpArgs &a, int grid, hipStream_t st)
{
    const size_t lds = (size_t)a.st * SEGS * 16 * sizeof(uint4);
    hipLaunchKernelGGL((gemv_gateup_e4m3_kernel<SEGS, MOE_E4M3_GU_RG, MOE_E4M3_GU_ST>), dim3(grid),
                       dim3(kThreads), lds, st, a);
}

template <int SEGS>
void down_launch(const DownArgs &a, int grid, hipStream_t st)
{
    const size_t lds = (size_t)a.st * SEGS * 32 * sizeof(float4);
    hipLaunchKernelGGL((gemv_down_e4m3_kernel<SEGS, MOE_E4M3_DN_RG, MOE_E4M3_DN_ST>), dim3(grid),
                       dim3(kThreads), lds, st, a);
}

}  // namespace

hipError_t launch_gemv_gateup_e4m3(const GemvBankDev &gate, const GemvBankDev &up,
                                   const uint16_t *x, const MoeRouteDev &r, int32_t M, int32_t S,
                                   int32_t E, int32_t hidden, int32_t inter, float *partials,
                                   int32_t nks, hipStream_t st)
{
    GateUpArgs a;
    a.st = M < MOE_E4M3_GU_ST ? M : MOE_E4M3_GU_ST;
    a.gcodes = gate.codes; a.ucodes = up.codes;
    a.gscales = (const float *)gate.scales; a.uscales = (const float *)up.scales;
    a.x = x; a.offsets = r.offsets; a.sorted_token = r.sorted_token; a.active = r.active;
    a.num_active = r.num_active; a.partials = partials;
    a.S = S; a.H = hidden; a.I = inter;
    const int segs = gemv_segs_gateup(kFmtE4M3, hidden);
    a.nks = gemv_gateup_slices(kFmtE4M3, hidden);
    if (a.nks != nks) return hipErrorInvalidValue;
    a.ntiles = 2 * (inter / (MOE_E4M3_GU_RG * 32));
    const int grid = (S < E ? S : E) * a.ntiles * a.nks;
    switch (segs) {
    case 8: gateup_launch<8>(a, grid, st); break;
    case 7: gateup_launch<7>(a, grid, st); break;
    case 6: gateup_launch<6>(a, grid, st); break;
    case 5: gateup_launch<5>(a, grid, st); break;
    case 4: gateup_launch<4>(a, grid, st); break;
    case 3: gateup_launch<3>(a, grid, st); break;
    case 2: gateup_launch<2>(a, grid, st); break;
    default: gateup_launch<1>(a, grid, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_down_e4m3(const GemvBankDev &down, const float *h, const MoeRouteDev &r,
                                 int32_t M, int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                 float *y, float *slice_scratch, hipStream_t st)
{
    DownArgs a;
    a.st = M < MOE_E4M3_DN_ST ? M : MOE_E4M3_DN_ST;
    a.codes = down.codes; a.scales = (const float *)down.scales; a.h = h;
    a.offsets = r.offsets; a.active = r.active; a.num_active = r.num_active;
    a.S = S; a.H = hidden; a.I = inter;
    const int segs = gemv_segs_down(kFmtE4M3, inter);
    a.nks = gemv_down_slices(kFmtE4M3, inter);
    a.out = a.nks == 1 ? y : slice_scratch;
    a.ntiles = hidden / (MOE_E4M3_DN_RG * 32);
    const int grid = (S < E ? S : E) * a.ntiles * a.nks;
    switch (segs) {
    case 16: down_launch<16>(a, grid, st); break;
    case 8: down_launch<8>(a, grid, st); break;
    case 7: down_launch<7>(a, grid, st); break;
    case 6: down_launch<6>(a, grid, st); break;
    case 5: down_launch<5>(a, grid, st); break;
    case 4: down_launch<4>(a, grid, st); break;
    case 3: down_launch<3>(a, grid, st); break;
    case 2: down_launch<2>(a, grid, st); break;
    default: down_launch<1>(a, grid, st); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.nks == 1) return err;
    const size_t n4 = (size_t)S * hidden / 4;
    hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                       slice_scratch, a.nks, S, hidden, r.offsets, E, y);
    return hipGetLastError();
}
