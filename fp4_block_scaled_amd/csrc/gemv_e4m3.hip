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
constexpr int kGUSegs = kGemvSliceE4M3 / 128;    // 8 segments of 128 K per slice
constexpr int kDownSlice = 2048;
constexpr int kDownSegs = kDownSlice / 128;      // 16

struct GateUpArgs {
    const uint8_t *gcodes, *ucodes;
    const float *gscales, *uscales;
    const uint16_t *x;
    const int32_t *offsets, *sorted_token, *active, *num_active;
    float *partials;
    int32_t S, H, I, nks, ntiles;
};

struct DownArgs {
    const uint8_t *codes;
    const float *scales;
    const float *h;
    const int32_t *offsets, *active, *num_active;
    float *out;          // y [S][H] when nks == 1, else partials [nks][S][H]
    int32_t S, H, I, nks, ntiles;
};

__device__ __forceinline__ uint4 load16(const uint8_t *p)
{
    return *reinterpret_cast<const uint4 *>(p);
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
// RG: 8-row groups per wave; ST: slots per pass over the weights.
template <int RG, int ST>
__global__ __launch_bounds__(kThreads) void gemv_gateup_e4m3_kernel(GateUpArgs a)
{
    constexpr int RPW = RG * 8;
    constexpr int RPB = RPW * (kThreads / 64);
    __shared__ uint4 xs[ST][kGUSegs * 16];           // bf16 x slice per slot (1024 values)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int grp = lane >> 3, sub = lane & 7;
    int bid = blockIdx.x;
    const int ks = bid % a.nks;
    bid /= a.nks;
    const int tile = bid % a.ntiles;
    const int ai = bid / a.ntiles;
    if (ai >= *a.num_active) return;
    const int e = a.active[ai];
    const int p0 = a.offsets[e];
    const int ne = a.offsets[e + 1] - p0;
    const int H = a.H, I = a.I;
    const int half = a.ntiles >> 1;
    const bool is_up = tile >= half;
    const uint8_t *codes = (is_up ? a.ucodes : a.gcodes) + (size_t)e * I * H;
    const int sc_cols = H >> 7;
    const float *sc_e = (is_up ? a.uscales : a.gscales) + (size_t)e * (I >> 7) * sc_cols;
    const int row_b0 = (is_up ? tile - half : tile) * RPB;
    const int col_b0 = (is_up ? I : 0) + row_b0;
    const int k0 = ks * kGemvSliceE4M3;
    const int segs = min(kGUSegs, (H - k0) >> 7);
    const size_t pstride = (size_t)2 * I;

    for (int st = 0; st < ne; st += ST) {
        const int nt = min(ST, ne - st);
        const int cpr = segs * 16;                   // uint4 chunks per staged row
        for (int c = tid; c < nt * cpr; c += kThreads) {
            const int j = c / cpr, r = c - j * cpr;
            const int tok = a.sorted_token[p0 + st + j];
            xs[j][r] = *reinterpret_cast<const uint4 *>(a.x + (size_t)tok * H + k0 + r * 8);
        }
        __syncthreads();

        uint4 wn[kGUSegs];
        {
            const uint8_t *rp = codes + (size_t)(row_b0 + wave * RPW + grp) * H + k0 + sub * 16;
#pragma unroll
            for (int sg = 0; sg < kGUSegs; ++sg)
                if (sg < segs) wn[sg] = load16(rp + sg * 128);
        }
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            uint4 w[kGUSegs];
#pragma unroll
            for (int sg = 0; sg < kGUSegs; ++sg) w[sg] = wn[sg];
            const int wrow0 = row_b0 + wave * RPW + rg * 8;
            if (rg + 1 < RG) {
                const uint8_t *rp = codes + (size_t)(wrow0 + 8 + grp) * H + k0 + sub * 16;
#pragma unroll
                for (int sg = 0; sg < kGUSegs; ++sg)
                    if (sg < segs) wn[sg] = load16(rp + sg * 128);
            }
            const float *sp = sc_e + (size_t)(wrow0 >> 7) * sc_cols + (k0 >> 7);
            float acc[ST];
#pragma unroll
            for (int j = 0; j < ST; ++j) acc[j] = 0.0f;
#pragma unroll
            for (int sg = 0; sg < kGUSegs; ++sg) {
                if (sg < segs) {
                    const float s = sp[sg];
                    bf16x2 wb[8];
                    e4m3x4_to_bf16(w[sg].x, wb[0], wb[1]);
                    e4m3x4_to_bf16(w[sg].y, wb[2], wb[3]);
                    e4m3x4_to_bf16(w[sg].z, wb[4], wb[5]);
                    e4m3x4_to_bf16(w[sg].w, wb[6], wb[7]);
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
// bytes per LDS instruction (no bank conflicts).
template <int RG, int ST>
__global__ __launch_bounds__(kThreads) void gemv_down_e4m3_kernel(DownArgs a)
{
    constexpr int RPW = RG * 8;
    constexpr int RPB = RPW * (kThreads / 64);
    __shared__ float4 hs[ST][kDownSegs * 32];        // 2048 floats per slot

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int grp = lane >> 3, sub = lane & 7;
    int bid = blockIdx.x;
    const int ks = bid % a.nks;
    bid /= a.nks;
    const int tile = bid % a.ntiles;
    const int ai = bid / a.ntiles;
    if (ai >= *a.num_active) return;
    const int e = a.active[ai];
    const int p0 = a.offsets[e];
    const int ne = a.offsets[e + 1] - p0;
    const int H = a.H, I = a.I;
    const uint8_t *codes = a.codes + (size_t)e * H * I;
    const int sc_cols = I >> 7;
    const float *sc_e = a.scales + (size_t)e * (H >> 7) * sc_cols;
    const int row_b0 = tile * RPB;
    const int k0 = ks * kDownSlice;
    const int segs = min(kDownSegs, (I - k0) >> 7);
    float *out = a.out + (size_t)ks * a.S * H;

    for (int st = 0; st < ne; st += ST) {
        const int nt = min(ST, ne - st);
        const int cpr = segs * 32;                   // float4 per staged row
        for (int c = tid; c < nt * cpr; c += kThreads) {
            const int j = c / cpr, f = c - j * cpr;  // f = source float4 index
            const int sg = f >> 5, r = f & 31, sb = r >> 2, q = r & 3;
            hs[j][sg * 32 + q * 8 + sb] =
                *reinterpret_cast<const float4 *>(a.h + (size_t)(p0 + st + j) * I + k0 + f * 4);
        }
        __syncthreads();

        uint4 wn[kDownSegs];
        {
            const uint8_t *rp = codes + (size_t)(row_b0 + wave * RPW + grp) * I + k0 + sub * 16;
#pragma unroll
            for (int sg = 0; sg < kDownSegs; ++sg)
                if (sg < segs) wn[sg] = load16(rp + sg * 128);
        }
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            uint4 w[kDownSegs];
#pragma unroll
            for (int sg = 0; sg < kDownSegs; ++sg) w[sg] = wn[sg];
            const int wrow0 = row_b0 + wave * RPW + rg * 8;
            if (rg + 1 < RG) {
                const uint8_t *rp = codes + (size_t)(wrow0 + 8 + grp) * I + k0 + sub * 16;
#pragma unroll
                for (int sg = 0; sg < kDownSegs; ++sg)
                    if (sg < segs) wn[sg] = load16(rp + sg * 128);
            }
            const float *sp = sc_e + (size_t)(wrow0 >> 7) * sc_cols + (k0 >> 7);
            float acc[ST];
#pragma unroll
            for (int j = 0; j < ST; ++j) acc[j] = 0.0f;
#pragma unroll
            for (int sg = 0; sg < kDownSegs; ++sg) {
                if (sg < segs) {
                    const float s = sp[sg];
                    f32x2 wf[8];
                    const uint32_t dw[4] = {w[sg].x, w[sg].y, w[sg].z, w[sg].w};
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
            }
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                if (j < nt) {
                    const float v = moe::sum8_lanes(acc[j]);
                    if (sub == 0) out[(size_t)(p0 + st + j) * H + wrow0 + grp] = v;
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
// the host never needs the routing.  Row tiles (128 rows for gate/up, 64 for
// down) divide every legal size because n_out % 128 == 0.
hipError_t launch_gemv_gateup_e4m3(const GemvBankDev &gate, const GemvBankDev &up,
                                   const uint16_t *x, const MoeRouteDev &r, int32_t S,
                                   int32_t E, int32_t hidden, int32_t inter, float *partials,
                                   int32_t nks, hipStream_t st)
{
    constexpr int RG = 4, ST = 8;
    constexpr int RPB = RG * 8 * (kThreads / 64);
    static_assert(128 % RPB == 0 || RPB % 128 == 0, "row tile vs 128-row blocks");
    GateUpArgs a;
    a.gcodes = gate.codes; a.ucodes = up.codes;
    a.gscales = (const float *)gate.scales; a.uscales = (const float *)up.scales;
    a.x = x; a.offsets = r.offsets; a.sorted_token = r.sorted_token; a.active = r.active;
    a.num_active = r.num_active; a.partials = partials;
    a.S = S; a.H = hidden; a.I = inter; a.nks = nks;
    a.ntiles = 2 * (inter / RPB);
    const int amax = S < E ? S : E;
    hipLaunchKernelGGL((gemv_gateup_e4m3_kernel<RG, ST>), dim3(amax * a.ntiles * nks),
                       dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

int gemv_down_slices(int32_t inter) { return (inter + kDownSlice - 1) / kDownSlice; }

hipError_t launch_gemv_down_e4m3(const GemvBankDev &down, const float *h, const MoeRouteDev &r,
                                 int32_t S, int32_t E, int32_t hidden, int32_t inter, float *y,
                                 float *slice_scratch, hipStream_t st)
{
    constexpr int RG = 2, ST = 4;
    constexpr int RPB = RG * 8 * (kThreads / 64);
    DownArgs a;
    a.codes = down.codes; a.scales = (const float *)down.scales; a.h = h;
    a.offsets = r.offsets; a.active = r.active; a.num_active = r.num_active;
    a.S = S; a.H = hidden; a.I = inter;
    a.nks = gemv_down_slices(inter);
    a.out = a.nks == 1 ? y : slice_scratch;
    a.ntiles = hidden / RPB;
    const int amax = S < E ? S : E;
    hipLaunchKernelGGL((gemv_down_e4m3_kernel<RG, ST>), dim3(amax * a.ntiles * a.nks),
                       dim3(kThreads), 0, st, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.nks == 1) return err;
    const size_t n4 = (size_t)S * hidden / 4;
    hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                       slice_scratch, a.nks, S, hidden, r.offsets, E, y);
    return hipGetLastError();
}
