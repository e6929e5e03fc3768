// gemv_nvfp4.hip -- dequant-GEMV tier for NVFP4 expert banks.
//
// NVFP4 weight = E2M1 code x E4M3 scale (one per 16 inputs) x FP32 scale_2
// (one per expert projection): "memra-engine src/dsv4_ep.rs", fn chain (code
// stride inter*hidden/2, scale stride inter*hidden/16, a scale_2 per expert)
// and "spark_model glm5next_mlp/forward.rs", fn w4a16_gemv (the NVFP4 operand
// triple, scale_2 by value).  Same work layout as the E4M3 GEMV: 8 lanes per
// weight row, 16 code bytes (32 weights) per lane per 128-byte segment, one
// pass over each active expert for all of its slots.
//
// Decode: gfx950 converts E2M1 pairs straight to bf16 (gate/up, against bf16
// activations with v_dot2) or to f32 (down, against FP32 h); the E2M1 values
// are exact in both.  The two E4M3 group scales of a lane's 32 weights are
// applied once per 16 products; scale_2 once per output.
#include "moe_internal.h"

namespace {

using moe::bf16x2;
using moe::f32x2;

constexpr int kThreads = 256;
constexpr int kSegK = 256;                          // K values per 128-byte segment

struct GateUpArgs {
    const uint8_t *gcodes, *ucodes, *gscales, *uscales;
    const float *gscale2, *uscale2;
    const uint16_t *x;
    const int32_t *offsets, *sorted_token, *active, *num_active;
    float *partials;
    int32_t S, H, I, nks, ntiles, st;   // st: slots per weight pass (<= ST)
};

struct DownArgs {
    const uint8_t *codes, *scales;
    const float *scale2;
    const float *h;
    const int32_t *offsets, *active, *num_active;
    float *out;
    int32_t S, H, I, nks, ntiles, st;   // st: slots per weight pass (<= ST)
};

// Codes and group scales are streamed once per call (non-temporal loads).
__device__ __forceinline__ uint4 load16(const uint8_t *p)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t load2(const uint8_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
}

__device__ __forceinline__ float dot2(bf16x2 a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b), c, false);
}

// 8 E2M1 codes of one dword against 8 bf16 activations (one uint4).
__device__ __forceinline__ float dot8_fp4_bf16(uint32_t c, uint4 x, float d)
{
    d = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)c, 1.0f, 0), x.x, d);
    d = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)c, 1.0f, 1), x.y, d);
    d = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)c, 1.0f, 2), x.z, d);
    d = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)c, 1.0f, 3), x.w, d);
    return d;
}

// 8 E2M1 codes of one dword against 8 FP32 activations (two float4).
__device__ __forceinline__ float dot8_fp4_f32(uint32_t c, float4 a, float4 b, float d)
{
    f32x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)c, 1.0f, 0);
    f32x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)c, 1.0f, 1);
    f32x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)c, 1.0f, 2);
    f32x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)c, 1.0f, 3);
    d = fmaf(w0.x, a.x, d); d = fmaf(w0.y, a.y, d);
    d = fmaf(w1.x, a.z, d); d = fmaf(w1.y, a.w, d);
    d = fmaf(w2.x, b.x, d); d = fmaf(w2.y, b.y, d);
    d = fmaf(w3.x, b.z, d); d = fmaf(w3.y, b.w, d);
    return d;
}

// SEGS: 256-wide K segments per slice; RG: 8-row groups per wave; ST: slots
// per pass.  All RG*SEGS code and scale loads of a wave are issued before the
// first multiply.
template <int SEGS, int RG, int ST>
__global__ __launch_bounds__(kThreads) void gemv_gateup_nvfp4_kernel(GateUpArgs a)
{
    constexpr int RPW = RG * 8;
    constexpr int RPB = RPW * (kThreads / 64);
    // bf16 x slice per slot; uint4 q of lane sub in segment sg at sg*32 + q*8 + sub.
    extern __shared__ uint4 lds_x[];                 // [a.st][SEGS*32]
    uint4 (*xs)[SEGS * 32] = reinterpret_cast<uint4 (*)[SEGS * 32]>(lds_x);

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
    const size_t rowb = (size_t)H / 2, rows = (size_t)H / 16;
    const int row_b0 = (is_up ? tile - half : tile) * RPB;
    const int col_b0 = (is_up ? I : 0) + row_b0;
    const int k0 = ks * SEGS * kSegK;
    const size_t pstride = (size_t)2 * I;
    const float s2 = (is_up ? a.uscale2 : a.gscale2)[e];
    const size_t row0 = (size_t)e * I + row_b0 + wave * RPW + grp;
    const uint8_t *rp = (is_up ? a.ucodes : a.gcodes) + row0 * rowb + k0 / 2 + sub * 16;
    const uint8_t *sp = (is_up ? a.uscales : a.gscales) + row0 * rows + k0 / 16 + sub * 2;

    // weight loads go out first; the slot range is read while they fly
    int p0 = 0, ne = 1;
    for (int st = 0; st < ne; st += a.st) {
        uint4 w[RG][SEGS];
        uint32_t sv[RG][SEGS];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                w[rg][sg] = load16(rp + (size_t)rg * 8 * rowb + sg * 128);
                sv[rg][sg] = load2(sp + (size_t)rg * 8 * rows + sg * 16);
            }
        if (st == 0) { p0 = a.offsets[e]; ne = a.offsets[e + 1] - p0; }
        const int nt = min(a.st, ne - st);

        for (int c = tid; c < nt * SEGS * 32; c += kThreads) {
            const int j = c / (SEGS * 32), f = c - j * (SEGS * 32);
            const int sg = f >> 5, r = f & 31, sb = r >> 2, q = r & 3;
            const int tok = a.sorted_token[p0 + st + j];
            xs[j][sg * 32 + q * 8 + sb] =
                *reinterpret_cast<const uint4 *>(a.x + (size_t)tok * H + k0 + f * 8);
        }
        __syncthreads();

#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            float acc[ST];
#pragma unroll
            for (int j = 0; j < ST; ++j) acc[j] = 0.0f;
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                const f32x2 sc = __builtin_amdgcn_cvt_pk_f32_fp8((int)sv[rg][sg], false);
#pragma unroll
                for (int j = 0; j < ST; ++j) {
                    if (j < nt) {
                        const uint4 *xv = &xs[j][sg * 32 + sub];
                        float d0 = dot8_fp4_bf16(w[rg][sg].x, xv[0], 0.0f);
                        d0 = dot8_fp4_bf16(w[rg][sg].y, xv[8], d0);
                        float d1 = dot8_fp4_bf16(w[rg][sg].z, xv[16], 0.0f);
                        d1 = dot8_fp4_bf16(w[rg][sg].w, xv[24], d1);
                        acc[j] = fmaf(d0, sc.x, acc[j]);
                        acc[j] = fmaf(d1, sc.y, acc[j]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                if (j < nt) {
                    const float v = moe::sum8_lanes(acc[j]) * s2;
                    if (sub == 0)
                        a.partials[((size_t)ks * a.S + p0 + st + j) * pstride + col_b0 + wave * RPW +
                                   rg * 8 + grp] = v;
                }
            }
        }
        __syncthreads();
    }
}

template <int SEGS, int RG, int ST>
__global__ __launch_bounds__(kThreads) void gemv_down_nvfp4_kernel(DownArgs a)
{
    constexpr int RPW = RG * 8;
    constexpr int RPB = RPW * (kThreads / 64);
    // FP32 h slice per slot; float4 q of lane sub in segment sg at sg*64 + q*8 + sub.
    extern __shared__ float4 lds_h[];                // [a.st][SEGS*64]
    float4 (*hs)[SEGS * 64] = reinterpret_cast<float4 (*)[SEGS * 64]>(lds_h);

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
    const size_t rowb = (size_t)I / 2, rows = (size_t)I / 16;
    const float s2 = a.scale2[e];
    const int row_b0 = tile * RPB;
    const int k0 = ks * SEGS * kSegK;
    float *out = a.out + (size_t)ks * a.S * H;
    const size_t row0 = (size_t)e * H + row_b0 + wave * RPW + grp;
    const uint8_t *rp = a.codes + row0 * rowb + k0 / 2 + sub * 16;
    const uint8_t *sp = a.scales + row0 * rows + k0 / 16 + sub * 2;

    // weight loads go out first; the slot range is read while they fly
    int p0 = 0, ne = 1;
    for (int st = 0; st < ne; st += a.st) {
        uint4 w[RG][SEGS];
        uint32_t sv[RG][SEGS];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                w[rg][sg] = load16(rp + (size_t)rg * 8 * rowb + sg * 128);
                sv[rg][sg] = load2(sp + (size_t)rg * 8 * rows + sg * 16);
            }
        if (st == 0) { p0 = a.offsets[e]; ne = a.offsets[e + 1] - p0; }
        const int nt = min(a.st, ne - st);

        for (int c = tid; c < nt * SEGS * 64; c += kThreads) {
            const int j = c / (SEGS * 64), f = c - j * (SEGS * 64);
            const int sg = f >> 6, r = f & 63, sb = r >> 3, q = r & 7;
            hs[j][sg * 64 + q * 8 + sb] =
                *reinterpret_cast<const float4 *>(a.h + (size_t)(p0 + st + j) * I + k0 + f * 4);
        }
        __syncthreads();

#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            float acc[ST];
#pragma unroll
            for (int j = 0; j < ST; ++j) acc[j] = 0.0f;
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                const f32x2 sc = __builtin_amdgcn_cvt_pk_f32_fp8((int)sv[rg][sg], false);
#pragma unroll
                for (int j = 0; j < ST; ++j) {
                    if (j < nt) {
                        const float4 *hv = &hs[j][sg * 64 + sub];
                        float d0 = dot8_fp4_f32(w[rg][sg].x, hv[0], hv[8], 0.0f);
                        d0 = dot8_fp4_f32(w[rg][sg].y, hv[16], hv[24], d0);
                        float d1 = dot8_fp4_f32(w[rg][sg].z, hv[32], hv[40], 0.0f);
                        d1 = dot8_fp4_f32(w[rg][sg].w, hv[48], hv[56], d1);
                        acc[j] = fmaf(d0, sc.x, acc[j]);
                        acc[j] = fmaf(d1, sc.y, acc[j]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                if (j < nt) {
                    const float v = moe::sum8_lanes(acc[j]) * s2;
                    if (sub == 0)
                        out[(size_t)(p0 + st + j) * H + row_b0 + wave * RPW + rg * 8 + grp] = v;
                }
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void sum_slices_kernel(const float *__restrict__ part, int32_t nks,
                                                         int32_t S, int32_t H,
                                                         const int32_t *__restrict__ offsets,
                                                         int32_t E, float *__restrict__ y)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
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

namespace {

constexpr int kGUST = 8, kDNST = 4;

template <int SEGS>
void gateup_launch(const GateUpArgs &a, int grid, hipStream_t st)
{
    const size_t lds = (size_t)a.st * SEGS * 32 * sizeof(uint4);
    hipLaunchKernelGGL((gemv_gateup_nvfp4_kernel<SEGS, 1, kGUST>), dim3(grid), dim3(kThreads), lds,
                       st, a);
}

template <int SEGS>
void down_launch(const DownArgs &a, int grid, hipStream_t st)
{
    const size_t lds = (size_t)a.st * SEGS * 64 * sizeof(float4);
    hipLaunchKernelGGL((gemv_down_nvfp4_kernel<SEGS, 1, kDNST>), dim3(grid), dim3(kThreads), lds,
                       st, a);
}

#define MOE_SEGS_SWITCH(segs, fn, ...)        \
    switch (segs) {                           \
    case 8: fn<8>(__VA_ARGS__); break;        \
    case 7: fn<7>(__VA_ARGS__); break;        \
    case 6: fn<6>(__VA_ARGS__); break;        \
    case 5: fn<5>(__VA_ARGS__); break;        \
    case 4: fn<4>(__VA_ARGS__); break;        \
    case 3: fn<3>(__VA_ARGS__); break;        \
    case 2: fn<2>(__VA_ARGS__); break;        \
    default: fn<1>(__VA_ARGS__); break;       \
    }

}  // namespace

hipError_t launch_gemv_gateup_nvfp4(const GemvBankDev &gate, const GemvBankDev &up,
                                    const uint16_t *x, const MoeRouteDev &r, int32_t M, int32_t S,
                                    int32_t E, int32_t hidden, int32_t inter, float *partials,
                                    int32_t nks, hipStream_t st)
{
    GateUpArgs a;
    a.st = M < kGUST ? M : kGUST;
    a.gcodes = gate.codes; a.ucodes = up.codes;
    a.gscales = (const uint8_t *)gate.scales; a.uscales = (const uint8_t *)up.scales;
    a.gscale2 = gate.scale2; a.uscale2 = up.scale2;
    a.x = x; a.offsets = r.offsets; a.sorted_token = r.sorted_token; a.active = r.active;
    a.num_active = r.num_active; a.partials = partials;
    a.S = S; a.H = hidden; a.I = inter;
    const int segs = gemv_segs_gateup(kFmtNVFP4, hidden);
    a.nks = gemv_gateup_slices(kFmtNVFP4, hidden);
    if (a.nks != nks) return hipErrorInvalidValue;
    a.ntiles = 2 * (inter / 32);
    const int grid = (S < E ? S : E) * a.ntiles * a.nks;
    MOE_SEGS_SWITCH(segs, gateup_launch, a, grid, st)
    return hipGetLastError();
}

hipError_t launch_gemv_down_nvfp4(const GemvBankDev &down, const float *h, const MoeRouteDev &r,
                                  int32_t M, int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                  float *y, float *slice_scratch, hipStream_t st)
{
    DownArgs a;
    a.st = M < kDNST ? M : kDNST;
    a.codes = down.codes; a.scales = (const uint8_t *)down.scales; a.scale2 = down.scale2;
    a.h = h; a.offsets = r.offsets; a.active = r.active; a.num_active = r.num_active;
    a.S = S; a.H = hidden; a.I = inter;
    const int segs = gemv_segs_down(kFmtNVFP4, inter);
    a.nks = gemv_down_slices(kFmtNVFP4, inter);
    a.out = a.nks == 1 ? y : slice_scratch;
    a.ntiles = hidden / 32;
    const int grid = (S < E ? S : E) * a.ntiles * a.nks;
    MOE_SEGS_SWITCH(segs, down_launch, a, grid, st)
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.nks == 1) return err;
    const size_t n4 = (size_t)S * hidden / 4;
    hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                       slice_scratch, a.nks, S, hidden, r.offsets, E, y);
    return hipGetLastError();
}
