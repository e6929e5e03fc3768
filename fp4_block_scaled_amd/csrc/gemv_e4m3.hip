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
//   gate+up: one launch covers both banks and the whole of K; a block holds
//            the gate and the up rows of the same 16 h rows and applies the
//            clamped SwiGLU itself, so h leaves the kernel finished.
//   down:    a block covers 32 output rows over the whole of K (= inter)
//            and writes y rows directly.
#include "moe_internal.h"
#include "fused_common.h"

#include <type_traits>

namespace {

using moe::bf16x2;
using moe::f32x2;

constexpr int kThreads = 256;                    // 4 waves

// Most slots one weight pass serves (the pass size is also capped by the LDS
// that holds the slots' activation rows).
constexpr int MOE_E4M3_GU_ST = 8;
constexpr int MOE_E4M3_DN_ST = 8;

struct GateUpArgs {
    const uint8_t *gcodes, *ucodes;
    const float *gscales, *uscales;
    const uint16_t *x;
    const int32_t *offsets, *sorted_token, *active;
    float *h;                           // [S][I]
    int32_t H, I, ntiles, st;           // st: slots per weight pass (<= ST)
    float limit;
    // route built inside the launch (small routes): ids [M][k], and the
    // tables block 0 writes for the launches after it
    const int32_t *ids;
    int32_t M, k, E;
    MoeRouteDev r;
};

struct DownArgs {
    const uint8_t *codes;
    const float *scales;
    const float *h;                     // [S][I]
    const int32_t *offsets, *active;
    float *y;                           // [S][H]
    int32_t H, I, ntiles, st;           // st: slots per weight pass (<= ST)
};

// Down projection and combine of one token (gemv_down1_e4m3_kernel).
struct Down1Args {
    const uint8_t *codes;
    const float *scales;
    const float *h;                     // [S][I]
    const int32_t *ids, *t2p;           // [k]: the token's expert ids and packed rows (-1: none)
    const float *w;                     // [k]: its top-k weights
    float *y, *out;                     // y [S][H] packed rows, out [H]
    int32_t H, k;
};

// Weights are streamed once per call: non-temporal loads keep them from
// displacing the activations and partial sums in the caches.
__device__ __forceinline__ uint4 load16(const uint8_t *p)
{
#ifndef MOE_GEMV_CACHED_LOADS
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = moe::load_nt_global<u32x4>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    return *reinterpret_cast<const uint4 *>(p);
#endif
}

// The down kernels keep an FP32 h row in LDS permuted per 128-wide segment,
// so that the 8 lanes of a weight row read 128 contiguous bytes: LDS float4
// q*8 + sub of a segment holds the source float4 sub*4 + q (K values
// sub*16 + q*4 .. +3).  Staging walks the LDS positions in order (each
// 64-lane store is one contiguous 1 KB, free of bank conflicts) and loads the
// source float4 of each position.
__device__ __forceinline__ int h_src(int pos)
{
    return (pos & ~31) | ((pos & 7) << 2) | ((pos >> 3) & 3);
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

// silu(min(g, L)) * clamp(u, -L, L), silu(z) = z / (1 + e^-z)
__device__ __forceinline__ float swiglu_clamp(float g, float u, float L)
{
    const float gc = fminf(g, L);
    const float uc = fminf(fmaxf(u, -L), L);
    return gc / (1.0f + expf(-gc)) * uc;
}

// ---------------------------------------------------------------------------
// gate + up + SwiGLU
// ---------------------------------------------------------------------------
// One block = 16 h rows of one active expert over the whole of K: waves 0-1
// stream those 16 rows of the gate bank, waves 2-3 the same 16 rows of the up
// bank (8 rows per wave).  At the start of a pass the bf16 x rows of up to
// a.st slots are copied to LDS for the whole of K; the K loop then only
// streams weights, in chunks of CH segments, with the next two chunks' loads
// in flight while the current one is multiplied (three register buffers).
// With NCH > 0 (the chunk count known at compile time) the K loop is fully
// unrolled: straight-line code lets the compiler wait for exactly the chunk
// it multiplies; at most 128 VGPRs (4 waves per SIMD), so the 4 blocks of
// 16 rows that a CU holds all stay resident.  NCH == 0 is the generic looped form (one chunk in flight,
// an explicit wait at each step).  At the end the up sums go through LDS to
// the gate waves, which apply the clamped SwiGLU and write h: no partial sums
// leave the block.  The 16 rows lie in one 128-row scale block, so a wave
// keeps the block scales of all K segments in two registers (lane l:
// segments l and l + 64).
//
// XW (unrolled form, more slots than whole x rows fit): the x rows of the
// pass go to LDS one K chunk at a time into two buffers ([2][ST][CH * 16]
// uint4): chunk c+1's rows are loaded into VGPRs while chunk c is
// multiplied, stored after it, and a barrier ends the chunk.  Every slot of
// the expert (up to ST) is then served by one weight pass.
//
// gateup_e4m3_item does one (expert e, 16-row tile) item for the ne slots of
// e, whose packed rows start at p0 and whose tokens are tok[0..ne); xl is
// the LDS x tile ([a.st][H / 8] uint4), ush the LDS up-sum exchange.
template <int CH, int NCH, int ST, bool FUSED = false, bool XW = false>
__device__ __forceinline__ void gateup_e4m3_item(const GateUpArgs &a, int e, int tile, int p0, int ne,
                                                 const int32_t *tok, uint4 *xl, float (*ush)[16])
{
    static_assert(!XW || (NCH > 0 && !FUSED), "chunked x staging is an unrolled, standalone form");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int grp = lane >> 3, sub = lane & 7;
    const int H = a.H, I = a.I, H8 = H >> 3;
    const int nseg = H >> 7, nch = NCH > 0 ? NCH : nseg / CH;
    const bool is_up = wave >= 2;
    const int hrow0 = tile * 16;
    const int hrow = hrow0 + (wave & 1) * 8 + grp;
    // weight address = wave-uniform base (SGPRs) + fixed 32-bit lane offset
    const uint8_t *wb0 = (is_up ? a.ucodes : a.gcodes) + ((size_t)e * I + hrow0 + (wave & 1) * 8) * H;
    const uint32_t loff = (uint32_t)grp * H + sub * 16;
    const float *scb = (is_up ? a.uscales : a.gscales) + ((size_t)e * (I >> 7) + (hrow0 >> 7)) * nseg;
    const float sc_lo = lane < nseg ? scb[lane] : 0.0f;
    const float sc_hi = lane + 64 < nseg ? scb[lane + 64] : 0.0f;

    for (int s0 = 0; s0 < ne; s0 += a.st) {          // passes over the weights
        const int nt = min(a.st, ne - s0);
        // opaque copies: the per-chunk address arithmetic stays inside the
        // pass instead of being hoisted out of it into live registers
        const uint8_t *wbp = moe::uniform_ptr(wb0);
        uint32_t lo = loff;
        asm volatile("" : "+s"(wbp), "+v"(lo));
        auto load_w = [&](uint4 (&wb)[CH], int c) {
            const uint8_t *cb = wbp + c * CH * 128;
#pragma unroll
            for (int sg = 0; sg < CH; ++sg) wb[sg] = load16(cb + lo + sg * 128);
        };
        float acc[ST];
#pragma unroll
        for (int j = 0; j < ST; ++j) acc[j] = 0.0f;
        // x tile as mul_chunk reads it: base, row stride (uint4), first segment
        const uint4 *xcur = xl;
        int xstr = H8, xseg0 = 0;

        auto mul_chunk = [&](const uint4 (&wc)[CH], int c) {
#pragma unroll
            for (int sg = 0; sg < CH; ++sg) {
                const int seg = c * CH + sg;
                const float s = seg < 64 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                               __builtin_bit_cast(int, sc_lo), seg))
                                         : __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                               __builtin_bit_cast(int, sc_hi), seg - 64));
                const uint4 wv = wc[sg];
                bf16x2 wb[8];
                e4m3x4_to_bf16(wv.x, wb[0], wb[1]);
                e4m3x4_to_bf16(wv.y, wb[2], wb[3]);
                e4m3x4_to_bf16(wv.z, wb[4], wb[5]);
                e4m3x4_to_bf16(wv.w, wb[6], wb[7]);
#pragma unroll
                for (int j = 0; j < ST; ++j) {
                    if (j < nt) {
                        const uint4 xa = xcur[j * xstr + (seg - xseg0) * 16 + sub * 2];
                        const uint4 xb = xcur[j * xstr + (seg - xseg0) * 16 + sub * 2 + 1];
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
                if constexpr (NCH > 0) __builtin_amdgcn_sched_barrier(0);  // convert per segment
            }
        };

        if constexpr (XW) {
            constexpr int XC = CH * 16;              // uint4 of one slot's x per chunk
            constexpr int XB = ST * XC;              // uint4 per buffer
            constexpr int XR = (XB + kThreads - 1) / kThreads;
            moe::u32x4 xr[XR];                       // (native vectors stay in VGPRs)
            // each load's source in chunk 0, looked up once per pass (the
            // chunks of a load differ by XC uint4): no token read per chunk
            const moe::u32x4 *xsrc[XR];
#pragma unroll
            for (int i = 0; i < XR; ++i) {
                // past the pass's last uint4 a lane reloads that one (never stored)
                const int f = min(tid + i * kThreads, nt * XC - 1);
                const int j = f / XC, r = f - j * XC;
                xsrc[i] = reinterpret_cast<const moe::u32x4 *>(a.x + (size_t)tok[s0 + j] * H + (size_t)r * 8);
            }
            auto load_x = [&](int c) {
#pragma unroll
                for (int i = 0; i < XR; ++i) xr[i] = xsrc[i][c * XC];
            };
            auto store_x = [&](int c) {
                moe::u32x4 *buf = reinterpret_cast<moe::u32x4 *>(xl) + (c & 1) * XB;
#pragma unroll
                for (int i = 0; i < XR; ++i) {
                    const int f = tid + i * kThreads;
                    if (f < nt * XC) buf[f] = xr[i];
                }
            };
            uint4 w[3][CH];
            xstr = XC;
            load_x(0);
            load_w(w[0], 0);
            if (NCH > 1) load_w(w[1], 1);
            store_x(0);
            moe::lds_barrier();
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                // x of chunk c+1 before the weights of c+2, so the wait for the x
                // leaves those weight loads in flight
                if (c + 1 < NCH) load_x(c + 1);
                if (c + 2 < NCH) load_w(w[(c + 2) % 3], c + 2);
                __builtin_amdgcn_sched_barrier(0);
                xcur = xl + (c & 1) * XB;
                xseg0 = c * CH;
                mul_chunk(w[c % 3], c);
                __builtin_amdgcn_sched_barrier(0);
                if (c + 1 < NCH) {
                    store_x(c + 1);
                    moe::lds_barrier();
                }
            }
        } else if constexpr (NCH > 0) {
            constexpr int H8C = NCH * CH * 16;       // uint4 per x row (H8)
            constexpr int XV = (ST * H8C + kThreads - 1) / kThreads;
            uint4 w[3][CH];
            if constexpr (XV <= 4 && ST == 1 && !FUSED) {   // (within the register budget)
                // x rows to LDS: every x load goes out at once, then the first
                // weight chunk; the LDS stores wait for the x loads only, so
                // staging x costs one memory round trip, under the first chunk
                moe::u32x4 xr[XV];                   // (native vectors stay in VGPRs)
#pragma unroll
                for (int i = 0; i < XV; ++i) {
                    // past the pass's last uint4 a lane reloads that one (never stored)
                    const int f = min(tid + i * kThreads, nt * H8C - 1);
                    const int j = f / H8C, r = f - j * H8C;
                    xr[i] = *reinterpret_cast<const moe::u32x4 *>(a.x + (size_t)tok[s0 + j] * H + r * 8);
                }
                __builtin_amdgcn_sched_barrier(0);
                load_w(w[0], 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < XV; ++i) {
                    const int f = tid + i * kThreads;
                    if (f < nt * H8C) reinterpret_cast<moe::u32x4 *>(xl)[f] = xr[i];
                }
                __builtin_amdgcn_sched_barrier(0);
            } else {
                // larger passes: x rows to LDS in a loop, then the first chunk
                for (int f = tid; f < nt * H8; f += kThreads) {
                    const int j = f / H8, r = f - j * H8;
                    xl[f] = *reinterpret_cast<const uint4 *>(a.x + (size_t)tok[s0 + j] * H + r * 8);
                }
                load_w(w[0], 0);
            }
            if (NCH > 1) load_w(w[1], 1);
            moe::lds_barrier();
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                // the scheduling fences keep each chunk's loads where they are
                // issued (two chunks ahead), not hoisted into a register spill
                if (c + 2 < NCH) load_w(w[(c + 2) % 3], c + 2);
                __builtin_amdgcn_sched_barrier(0);
                mul_chunk(w[c % 3], c);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // x rows to LDS, with the first weight chunk in flight across the
            // barrier
            for (int f = tid; f < nt * H8; f += kThreads) {
                const int j = f / H8, r = f - j * H8;
                xl[f] = *reinterpret_cast<const uint4 *>(a.x + (size_t)tok[s0 + j] * H + r * 8);
            }
            uint4 w0[CH], w1[CH];
            load_w(w0, 0);
            moe::lds_barrier();
            // wait for chunk c (the only loads in flight), start chunk c + 1,
            // multiply chunk c; unrolled by two so both buffers stay static
            auto step = [&](int c, uint4 (&wc)[CH], uint4 (&wn)[CH]) {
                moe::wait_vm0();
                if (c + 1 < nch) load_w(wn, c + 1);
                mul_chunk(wc, c);
            };
            for (int c = 0; c < nch; c += 2) {
                step(c, w0, w1);
                if (c + 1 >= nch) break;
                step(c + 1, w1, w0);
            }
        }

        // up sums to LDS, then SwiGLU in the gate waves
        float v[ST];
#pragma unroll
        for (int j = 0; j < ST; ++j) v[j] = j < nt ? moe::sum8_lanes(acc[j]) : 0.0f;
        if (is_up && sub == 0) {
#pragma unroll
            for (int j = 0; j < ST; ++j)
                if (j < nt) ush[j][(wave & 1) * 8 + grp] = v[j];
        }
        moe::lds_barrier();
        if (!is_up && sub == 0) {
#pragma unroll
            for (int j = 0; j < ST; ++j)
                if (j < nt) {
                    float *hp = a.h + (size_t)(p0 + s0 + j) * I + hrow;
                    const float hv = swiglu_clamp(v[j], ush[j][(wave & 1) * 8 + grp], a.limit);
                    if constexpr (FUSED) moe::store_dev(hp, hv);
                    else *hp = hv;
                }
        }
        moe::lds_barrier();                           // x and ush are reused by the next pass
    }
}

// ROUTE: the route of the S <= 128 slots comes from the ids inside the launch
// (the same stable pack as route_pack) instead of from the tables of a route
// pack launched before: every block works out its own expert; block 0 also
// builds the whole route and writes the tables for the down and combine
// launches that follow.
template <int CH, int NCH, int ST, bool ROUTE, bool XW = false>
__global__ __launch_bounds__(kThreads, 4) void gemv_gateup_e4m3_kernel(GateUpArgs a)
{
    extern __shared__ uint4 xl[];                    // [a.st][H / 8] bf16 x rows, K order
    __shared__ float ush[ST][16];                    // up sums of the 16 rows per slot
    const int tile = blockIdx.x % a.ntiles;
    const int ai = blockIdx.x / a.ntiles;
    if constexpr (ROUTE) {
        // every wave finds this block's expert from the ids on its own; the
        // tokens of its slots go to LDS; block 0 builds and writes the whole
        // route tables after its item, off the critical path
        __shared__ int32_t tokl[128];
        const LightRoute lr = light_route(a.ids, a.M * a.k, a.E, ai);
        light_route_tokens(lr, a.k, tokl);
        moe::lds_barrier();
        if (lr.e >= 0)
            gateup_e4m3_item<CH, NCH, ST, false, XW>(a, moe::uniform(lr.e), tile, moe::uniform(lr.p0),
                                                     moe::uniform(lr.ne), tokl, xl, ush);
        if (blockIdx.x == 0) {
            // the route in the x tile's LDS, free once the item has ended (the
            // launch sizes it for both): no block holds static LDS for it
            FusedRoute &R = *reinterpret_cast<FusedRoute *>(xl);
            const int id_in = (int)threadIdx.x < a.M * a.k ? a.ids[threadIdx.x] : -1;
            fused_route(a, R, id_in);
            fused_route_status(a, R);
            fused_route_tables(a, R);
        }
    } else {
        const int e = moe::uniform(a.active[ai]);   // -1 past the active experts
        if (e < 0) return;
        const int p0 = moe::uniform(a.offsets[e]);
        const int ne = moe::uniform(a.offsets[e + 1]) - p0;
        gateup_e4m3_item<CH, NCH, ST, false, XW>(a, e, tile, p0, ne, a.sorted_token + p0, xl, ush);
    }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------
// One block = 32 output rows of one active expert over the whole of K (=
// inter), 8 rows per wave.  At the start of a pass the FP32 h rows of up to
// a.st slots go to LDS (float4 q of lane sub in segment sg at sg*32 + q*8 +
// sub, so the 8 lanes of a row read 128 contiguous bytes); the K loop then
// streams weights in chunks of CH segments.  With NCH > 0 the loop is fully
// unrolled with the next two chunks in flight; NCH == 0 is the looped form
// with one chunk in flight.  The 32 rows lie in one 128-row scale block, so
// a wave keeps the block scales of all K segments in two registers.  With
// one slot per pass the kernel fits 72 VGPRs (7 waves per SIMD): the decode
// grid of 8 experts x 224 row tiles is then one round of 7 blocks per CU.
//
// down_e4m3_item does one (expert e, 32-row tile) item for the ne slots of e
// (packed rows p0..p0+ne) with hl the LDS h tile ([a.st][I / 4] float4).
// wait_h() runs once the first weight chunks are in flight and before h is
// read (a no-op in the standalone kernel, the wait for the expert's h in the
// fused one).  FUSED (the fused layer's item): the first chunks go out before
// the wait and h and y move through device-coherent accesses; otherwise the
// h loads go out first (in the unrolled form all of them, followed by the
// first chunk's loads before h is written to LDS).
struct NoWait {
    __device__ void operator()() const {}
};

template <int CH, int NCH, int ST, bool FUSED, class WaitH>
__device__ __forceinline__ void down_e4m3_item(const DownArgs &a, int e, int tile, int p0, int ne,
                                               float4 *hl, const WaitH &wait_h)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int grp = lane >> 3, sub = lane & 7;
    const int H = a.H, I = a.I, I4 = I >> 2;
    const int nseg = I >> 7, nch = NCH > 0 ? NCH : nseg / CH;
    const int row0 = tile * 32;
    const int row = row0 + wave * 8 + grp;
    const uint8_t *wb0 = a.codes + ((size_t)e * H + row0 + wave * 8) * I;
    const uint32_t loff = (uint32_t)grp * I + sub * 16;
    const float *scb = a.scales + ((size_t)e * (H >> 7) + (row0 >> 7)) * nseg;
    const float sc_lo = lane < nseg ? scb[lane] : 0.0f;
    const float sc_hi = lane + 64 < nseg ? scb[lane + 64] : 0.0f;

    for (int s0 = 0; s0 < ne; s0 += a.st) {          // passes over the weights
        const int nt = min(a.st, ne - s0);
        const uint8_t *wbp = moe::uniform_ptr(wb0);
        uint32_t lo = loff;
        asm volatile("" : "+s"(wbp), "+v"(lo));      // keep per-chunk addresses inside the pass
        auto load_w = [&](uint4 (&wb)[CH], int c) {
            const uint8_t *cb = wbp + c * CH * 128;
#pragma unroll
            for (int sg = 0; sg < CH; ++sg) wb[sg] = load16(cb + lo + sg * 128);
        };
        float acc[ST];
#pragma unroll
        for (int j = 0; j < ST; ++j) acc[j] = 0.0f;
        auto mul_chunk = [&](const uint4 (&wc)[CH], int c) {
#pragma unroll
            for (int sg = 0; sg < CH; ++sg) {
                const int seg = c * CH + sg;
                const float s = seg < 64 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                               __builtin_bit_cast(int, sc_lo), seg))
                                         : __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                               __builtin_bit_cast(int, sc_hi), seg - 64));
                const uint32_t dw[4] = {wc[sg].x, wc[sg].y, wc[sg].z, wc[sg].w};
                float d[ST];
#pragma unroll
                for (int j = 0; j < ST; ++j) d[j] = 0.0f;
                // one dword (4 weights) at a time keeps few temporaries live
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x2 w01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)dw[q], false);
                    const f32x2 w23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)dw[q], true);
#pragma unroll
                    for (int j = 0; j < ST; ++j) {
                        if (j < nt) {
                            const float4 hv = hl[j * I4 + seg * 32 + q * 8 + sub];
                            d[j] = fmaf(w01.x, hv.x, d[j]);
                            d[j] = fmaf(w01.y, hv.y, d[j]);
                            d[j] = fmaf(w23.x, hv.z, d[j]);
                            d[j] = fmaf(w23.y, hv.w, d[j]);
                        }
                    }
                    if constexpr (NCH > 0 && ST == 1) __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int j = 0; j < ST; ++j)
                    if (j < nt) acc[j] = fmaf(d[j], s, acc[j]);
                if constexpr (NCH > 0 && ST > 1) __builtin_amdgcn_sched_barrier(0);
            }
        };

        auto stage_h = [&]() {
            for (int f = tid; f < nt * I4; f += kThreads) {
                const int j = f / I4, r = h_src(f - j * I4);   // r: source float4 (4 K values)
                const float *hp = a.h + (size_t)(p0 + s0 + j) * I + r * 4;
                float4 hv;
                if constexpr (FUSED) {
                    hv = make_float4(moe::load_dev(hp), moe::load_dev(hp + 1), moe::load_dev(hp + 2),
                                     moe::load_dev(hp + 3));
                } else {
                    hv = *reinterpret_cast<const float4 *>(hp);
                }
                hl[f] = hv;
            }
        };
        if constexpr (NCH > 0) {
            uint4 w[3][CH];
            constexpr int I4C = NCH * CH * 32;       // float4 per h row (I4)
            constexpr int HV = (ST * I4C + kThreads - 1) / kThreads;
            if constexpr (FUSED) {
                load_w(w[0], 0);
                if (NCH > 1) load_w(w[1], 1);
                wait_h();
                stage_h();
            } else if constexpr (HV <= 2) {
                // every h load goes out at once, then the first weight chunk;
                // the LDS stores wait for the h loads only
                moe::f32x4 hr[HV];                   // (native vectors stay in VGPRs)
#pragma unroll
                for (int i = 0; i < HV; ++i) {
                    // past the pass's last float4 a lane reloads that one (never stored)
                    const int f = min(tid + i * kThreads, nt * I4C - 1);
                    const int j = f / I4C, r = h_src(f - j * I4C);
                    hr[i] = *reinterpret_cast<const moe::f32x4 *>(a.h + (size_t)(p0 + s0 + j) * I + r * 4);
                }
                __builtin_amdgcn_sched_barrier(0);
                load_w(w[0], 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < HV; ++i) {
                    const int f = tid + i * kThreads;
                    if (f < nt * I4C) reinterpret_cast<moe::f32x4 *>(hl)[f] = hr[i];
                }
                __builtin_amdgcn_sched_barrier(0);
                if (NCH > 1) load_w(w[1], 1);
            } else {
                stage_h();
                load_w(w[0], 0);
                if (NCH > 1) load_w(w[1], 1);
            }
            moe::lds_barrier();
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                if (c + 2 < NCH) load_w(w[(c + 2) % 3], c + 2);
                __builtin_amdgcn_sched_barrier(0);
                mul_chunk(w[c % 3], c);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            if constexpr (!FUSED) stage_h();
            uint4 w0[CH], w1[CH];
            load_w(w0, 0);
            if constexpr (FUSED) {
                wait_h();
                stage_h();
            }
            moe::lds_barrier();
            auto step = [&](int c, uint4 (&wc)[CH], uint4 (&wn)[CH]) {
                moe::wait_vm0();
                if (c + 1 < nch) load_w(wn, c + 1);
                mul_chunk(wc, c);
            };
            for (int c = 0; c < nch; c += 2) {
                step(c, w0, w1);
                if (c + 1 >= nch) break;
                step(c + 1, w1, w0);
            }
        }
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            if (j < nt) {
                const float v = moe::sum8_lanes(acc[j]);
                float *yp = a.y + (size_t)(p0 + s0 + j) * H + row;
                if (sub == 0) {
                    if constexpr (FUSED) moe::store_dev(yp, v);
                    else *yp = v;
                }
            }
        }
        moe::lds_barrier();                           // h is reused by the next pass
    }
}

template <int CH, int NCH, int ST>
__global__ __launch_bounds__(kThreads, ST == 1 ? 7 : 4) void gemv_down_e4m3_kernel(DownArgs a)
{
    extern __shared__ float4 hl[];                   // [a.st][I / 4], permuted per segment
    const int tile = blockIdx.x % a.ntiles;
    const int ai = blockIdx.x / a.ntiles;
    const int e = moe::uniform(a.active[ai]);       // -1 past the active experts
    if (e < 0) return;
    const int p0 = moe::uniform(a.offsets[e]);
    const int ne = moe::uniform(a.offsets[e + 1]) - p0;
    down_e4m3_item<CH, NCH, ST, false>(a, e, tile, p0, ne, hl, NoWait{});
}

// ---------------------------------------------------------------------------
// down, several slots a pass
// ---------------------------------------------------------------------------
// With more slots per pass every weight value meets more h values, and the LDS
// reads of h (one float4 per slot for every 4 weights) become the limit.  So
// each wave here takes RG row groups 32 rows apart (a block: 32*RG output rows)
// and every h value it reads from LDS serves all of them: with RG = 2, four
// slots a pass cost the LDS reads per weight byte of two.  The products of a
// slot are those of the down item, in the same order (y is bit-identical).
// Unrolled only: K = NCH chunks of CH segments, the next two chunks in flight.
template <int CH, int NCH, int ST, int RG>
__global__ __launch_bounds__(kThreads, 4) void gemv_down_rg_e4m3_kernel(DownArgs a)
{
    extern __shared__ float4 hl[];                   // [a.st][I / 4], permuted per segment
    constexpr int I4 = NCH * CH * 32, I = I4 * 4;    // float4 per h row, K
    constexpr int NSEG = I / 128, HV = (ST * I4 + kThreads - 1) / kThreads;
    static_assert(NSEG <= 128, "K at most 16384");
    const int tile = blockIdx.x % a.ntiles;
    const int ai = blockIdx.x / a.ntiles;
    const int e = moe::uniform(a.active[ai]);       // -1 past the active experts
    if (e < 0) return;
    const int p0 = moe::uniform(a.offsets[e]);
    const int ne = moe::uniform(a.offsets[e + 1]) - p0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int grp = lane >> 3, sub = lane & 7;
    const int H = a.H, row0 = tile * 32 * RG;
    const float *scb = a.scales + ((size_t)e * (H >> 7) + (row0 >> 7)) * NSEG;
    const float sc_lo = lane < NSEG ? scb[lane] : 0.0f;
    const float sc_hi = lane + 64 < NSEG ? scb[lane + 64] : 0.0f;

    for (int s0 = 0; s0 < ne; s0 += a.st) {          // passes over the weights
        const int nt = min(a.st, ne - s0);
        const uint8_t *wb = moe::uniform_ptr(a.codes + ((size_t)e * H + row0 + wave * 8) * I);
        uint32_t lo = (uint32_t)grp * I + sub * 16;
        asm volatile("" : "+s"(wb), "+v"(lo));      // keep per-chunk addresses inside the pass
        auto load_w = [&](uint4 (&wc)[RG][CH], int c) {
#pragma unroll
            for (int g = 0; g < RG; ++g)
#pragma unroll
                for (int sg = 0; sg < CH; ++sg)
                    wc[g][sg] = load16(wb + g * 32 * I + (c * CH + sg) * 128 + lo);
        };
        // every h load of the pass goes out, then the first weight chunk;
        // the LDS stores wait for the h loads only
        uint4 w[3][RG][CH];
        moe::f32x4 hr[HV];
#pragma unroll
        for (int i = 0; i < HV; ++i) {
            // past the pass's last float4 a lane reloads that one (never stored)
            const int f = min(tid + i * kThreads, nt * I4 - 1);
            const int j = f / I4, r = h_src(f - j * I4);
            hr[i] = *reinterpret_cast<const moe::f32x4 *>(a.h + (size_t)(p0 + s0 + j) * I + r * 4);
        }
        __builtin_amdgcn_sched_barrier(0);
        load_w(w[0], 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < HV; ++i) {
            const int f = tid + i * kThreads;
            if (f < nt * I4) reinterpret_cast<moe::f32x4 *>(hl)[f] = hr[i];
        }
        __builtin_amdgcn_sched_barrier(0);
        if (NCH > 1) load_w(w[1], 1);
        moe::lds_barrier();
        float acc[ST][RG];
#pragma unroll
        for (int j = 0; j < ST; ++j)
#pragma unroll
            for (int g = 0; g < RG; ++g) acc[j][g] = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (c + 2 < NCH) load_w(w[(c + 2) % 3], c + 2);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int sg = 0; sg < CH; ++sg) {
                const int seg = c * CH + sg;
                const float s = seg < 64 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                               __builtin_bit_cast(int, sc_lo), seg))
                                         : __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                               __builtin_bit_cast(int, sc_hi), seg - 64));
                float d[ST][RG];
#pragma unroll
                for (int j = 0; j < ST; ++j)
#pragma unroll
                    for (int g = 0; g < RG; ++g) d[j][g] = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x2 w01[RG], w23[RG];
#pragma unroll
                    for (int g = 0; g < RG; ++g) {
                        const uint4 wv = w[c % 3][g][sg];
                        const uint32_t dw = q == 0 ? wv.x : q == 1 ? wv.y : q == 2 ? wv.z : wv.w;
                        w01[g] = __builtin_amdgcn_cvt_pk_f32_fp8((int)dw, false);
                        w23[g] = __builtin_amdgcn_cvt_pk_f32_fp8((int)dw, true);
                    }
#pragma unroll
                    for (int j = 0; j < ST; ++j) {
                        if (j < nt) {
                            const float4 hv = hl[j * I4 + seg * 32 + q * 8 + sub];
#pragma unroll
                            for (int g = 0; g < RG; ++g) {
                                d[j][g] = fmaf(w01[g].x, hv.x, d[j][g]);
                                d[j][g] = fmaf(w01[g].y, hv.y, d[j][g]);
                                d[j][g] = fmaf(w23[g].x, hv.z, d[j][g]);
                                d[j][g] = fmaf(w23[g].y, hv.w, d[j][g]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < ST; ++j)
                    if (j < nt)
#pragma unroll
                        for (int g = 0; g < RG; ++g) {
                            acc[j][g] = fmaf(d[j][g], s, acc[j][g]);
                            asm volatile("" : "+v"(acc[j][g]));   // (keeps the sums per segment)
                        }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int j = 0; j < ST; ++j)
            if (j < nt)
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    const float v = moe::sum8_lanes(acc[j][g]);
                    if (sub == 0) a.y[(size_t)(p0 + s0 + j) * H + row0 + g * 32 + wave * 8 + grp] = v;
                }
        moe::lds_barrier();                           // h is reused by the next pass
    }
}

// ---------------------------------------------------------------------------
// down + combine of one token
// ---------------------------------------------------------------------------
// With one token the layer's k <= 8 slots all feed the same output row, so
// the down projection and the combine run in one launch without any hand-off
// between blocks: a block owns 8*RG output rows for EVERY slot.  Wave j
// streams those rows of slot j's expert (8 lanes per row as in the down
// item, the same products in the same order: y is bit-identical) against
// slot j's h row, which it stages in an LDS region of its own; the block then
// sums the slots' rows of its tile in slot order, each product rounded before
// its add (the combine's arithmetic), and writes the output rows.
template <int CH, int NCH, int RG>
__global__ __launch_bounds__(512, RG <= 2 ? 4 : 2) void gemv_down1_e4m3_kernel(Down1Args a)
{
    extern __shared__ float4 hl[];                   // [8][I/4] h rows, [8][8*RG] row sums, slot table
    constexpr int ROWS = 8 * RG;
    constexpr int I4 = NCH * CH * 32, I = I4 * 4;    // float4 per h row, K
    constexpr int NSEG = I / 128, HV = I4 / 64;      // 128-wide segments; h float4 per lane
    static_assert(I4 % 64 == 0 && NSEG <= 128, "K must be a multiple of 256 up to 16384");
    const int tid = threadIdx.x, lane = tid & 63;
    const int j = moe::uniform(tid >> 6);            // this wave's slot
    const int grp = lane >> 3, sub = lane & 7;
    const int H = a.H, row0 = blockIdx.x * ROWS;
    float *sums = reinterpret_cast<float *>(hl + 8 * I4);
    // the combine's slot table (packed row, weight) goes out first; its
    // lanes store it in LDS once their rows are done
    const int pc = tid < a.k ? a.t2p[tid] : -1;
    const float wc = tid < a.k ? a.w[tid] : 0.0f;
    const int p = j < a.k ? moe::uniform(a.t2p[j]) : -1;   // packed row; -1: no slot
    const int e = j < a.k ? moe::uniform(a.ids[j]) : 0;     // (loaded beside p, not after it)
    const bool live = p >= 0;
    moe::f32x4 *hw = reinterpret_cast<moe::f32x4 *>(hl + j * I4);
    const uint8_t *wb = moe::uniform_ptr(a.codes + ((size_t)e * H + row0) * I);
    uint32_t lo = (uint32_t)grp * I + sub * 16;
    asm volatile("" : "+s"(wb), "+v"(lo));
    auto load_w = [&](uint4 (&wc)[RG][CH], int c) {
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int sg = 0; sg < CH; ++sg)
                wc[g][sg] = load16(wb + g * 8 * I + (c * CH + sg) * 128 + lo);
    };
    if (live) {
        // h row loads, then the first weight chunk, then the h stores
        uint4 w[3][RG][CH];
        moe::f32x4 hr[HV];
#pragma unroll
        for (int i = 0; i < HV; ++i)
            hr[i] = *reinterpret_cast<const moe::f32x4 *>(a.h + (size_t)p * I + h_src(lane + i * 64) * 4);
        const float *scb = a.scales + ((size_t)e * (H >> 7) + (row0 >> 7)) * NSEG;
        const float sc_lo = lane < NSEG ? scb[lane] : 0.0f;
        const float sc_hi = lane + 64 < NSEG ? scb[lane + 64] : 0.0f;
        __builtin_amdgcn_sched_barrier(0);
        load_w(w[0], 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < HV; ++i) hw[lane + i * 64] = hr[i];
        __builtin_amdgcn_sched_barrier(0);
        if (NCH > 1) load_w(w[1], 1);
        // the h region is this wave's own: a wave-level barrier orders its
        // LDS stores before the reads of the other lanes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float acc[RG];
#pragma unroll
        for (int g = 0; g < RG; ++g) acc[g] = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (c + 2 < NCH) load_w(w[(c + 2) % 3], c + 2);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int sg = 0; sg < CH; ++sg) {
                const int seg = c * CH + sg;
                const float s = seg < 64 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                               __builtin_bit_cast(int, sc_lo), seg))
                                         : __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                               __builtin_bit_cast(int, sc_hi), seg - 64));
                float d[RG];
#pragma unroll
                for (int g = 0; g < RG; ++g) d[g] = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const moe::f32x4 hv = hw[seg * 32 + q * 8 + sub];
#pragma unroll
                    for (int g = 0; g < RG; ++g) {
                        const uint4 wv = w[c % 3][g][sg];
                        const uint32_t dw = q == 0 ? wv.x : q == 1 ? wv.y : q == 2 ? wv.z : wv.w;
                        const f32x2 w01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)dw, false);
                        const f32x2 w23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)dw, true);
                        d[g] = fmaf(w01.x, hv.x, d[g]);
                        d[g] = fmaf(w01.y, hv.y, d[g]);
                        d[g] = fmaf(w23.x, hv.z, d[g]);
                        d[g] = fmaf(w23.y, hv.w, d[g]);
                    }
                }
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    acc[g] = fmaf(d[g], s, acc[g]);
                    // (pins the row groups' sums here: left alone, the
                    // compiler sinks the later groups' products to the end of
                    // the loop and keeps every h value live until then)
                    asm volatile("" : "+v"(acc[g]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const float v = moe::sum8_lanes(acc[g]);
            if (sub == 0) {
                a.y[(size_t)p * H + row0 + g * 8 + grp] = v;
                sums[j * ROWS + g * 8 + grp] = v;
            }
        }
    }
    int *cp = reinterpret_cast<int *>(sums + 8 * ROWS);
    float *cw = reinterpret_cast<float *>(cp + 8);
    if (tid < 8) {
        cp[tid] = pc;
        cw[tid] = wc;
    }
    moe::lds_barrier();
    if (tid < ROWS) {
        float o = 0.0f;
        for (int jj = 0; jj < a.k; ++jj)
            if (cp[jj] >= 0) o = __fadd_rn(o, __fmul_rn(cw[jj], sums[jj * ROWS + tid]));
        a.out[row0 + tid] = o;
    }
}

// The same for hidden sizes that are multiples of 28 (7168 = 256 x 28), where
// 16-row blocks leave the CUs unevenly loaded: at 7168 rows they make 448
// blocks, two on most CUs and one on the rest, and the CUs with one block
// finish early and sit idle while those with two stream on.  Here a block
// owns 28 output rows for every slot (one block per CU at 7168) and has two
// waves per slot.  Rows stay in 8-row groups aligned to 8 with 8 lanes per
// row, as in the down item: the block's rows lie in the four aligned groups
// from base8 = row0 rounded down to 8, and wave 2j + hh takes groups 2hh and
// 2hh + 1 of slot j.  When row0 is not a multiple of 8, the first group holds
// 4 rows of the previous block, else the last group holds 4 rows of the next
// one; the lanes of those rows load the same bytes as the lanes 4 rows away
// (no extra traffic) and store nothing.  Each wave stages slot j's h row
// in an LDS region of its own.  Every row's products and their order are the
// down item's (y is bit-identical), and the block adds the slots' rows in
// slot order.
template <int CH, int NCH>
__global__ __launch_bounds__(1024, 4) void gemv_down1p_e4m3_kernel(Down1Args a)
{
    extern __shared__ float4 hl[];                   // [16][I/4] h rows, [8][28] row sums, slot table
    constexpr int ROWS = 28;
    constexpr int I4 = NCH * CH * 32, I = I4 * 4;    // float4 per h row, K
    constexpr int NSEG = I / 128, HV = I4 / 64;      // 128-wide segments; h float4 per lane
    static_assert(I4 % 64 == 0 && NSEG <= 64, "K must be a multiple of 256 up to 8192");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = moe::uniform(tid >> 6);
    const int j = wv >> 1, hh = wv & 1;              // this wave's slot and half
    const int grp = lane >> 3, sub = lane & 7;
    const int H = a.H, row0 = blockIdx.x * ROWS, base8 = row0 & ~7;
    float *sums = reinterpret_cast<float *>(hl + 16 * I4);
    const int pc = tid < a.k ? a.t2p[tid] : -1;
    const float wc = tid < a.k ? a.w[tid] : 0.0f;
    const int p = j < a.k ? moe::uniform(a.t2p[j]) : -1;   // packed row; -1: no slot
    const int e = j < a.k ? moe::uniform(a.ids[j]) : 0;     // (loaded beside p, not after it)
    const bool live = p >= 0;
    // the lane's row in each of its two groups; rows outside the block read
    // the row 4 away, inside the same group
    const int g0 = base8 + hh * 16;                  // first row of the wave's first group
    int own[2], src[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int r = g0 + g * 8 + grp;
        own[g] = r >= row0 && r < row0 + ROWS;
        src[g] = own[g] ? grp : grp ^ 4;
    }
    moe::f32x4 *hw = reinterpret_cast<moe::f32x4 *>(hl + wv * I4);
    const uint8_t *wb = moe::uniform_ptr(a.codes + ((size_t)e * H + g0) * I);
    uint32_t lo0 = (uint32_t)src[0] * I + sub * 16, lo1 = (uint32_t)(8 + src[1]) * I + sub * 16;
    asm volatile("" : "+s"(wb), "+v"(lo0), "+v"(lo1));
    auto load_w = [&](uint4 (&wc)[2][CH], int c) {
#pragma unroll
        for (int sg = 0; sg < CH; ++sg) {
            wc[0][sg] = load16(wb + (c * CH + sg) * 128 + lo0);
            wc[1][sg] = load16(wb + (c * CH + sg) * 128 + lo1);
        }
    };
    if (live) {
        // h row loads, then the first weight chunk, then the h stores
        uint4 w[3][2][CH];
        moe::f32x4 hr[HV];
#pragma unroll
        for (int i = 0; i < HV; ++i)
            hr[i] = *reinterpret_cast<const moe::f32x4 *>(a.h + (size_t)p * I + h_src(lane + i * 64) * 4);
        // each aligned 8-row group lies inside one 128-row scale block
        const float *scb = a.scales + (size_t)e * (H >> 7) * NSEG;
        const float sc0 = lane < NSEG ? scb[(g0 >> 7) * NSEG + lane] : 0.0f;
        const float sc1 = lane < NSEG ? scb[((g0 + 8) >> 7) * NSEG + lane] : 0.0f;
        __builtin_amdgcn_sched_barrier(0);
        load_w(w[0], 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < HV; ++i) hw[lane + i * 64] = hr[i];
        __builtin_amdgcn_sched_barrier(0);
        if (NCH > 1) load_w(w[1], 1);
        // the h region is this wave's own: a wave-level barrier orders its
        // LDS stores before the reads of the other lanes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float acc[2] = {0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (c + 2 < NCH) load_w(w[(c + 2) % 3], c + 2);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int sg = 0; sg < CH; ++sg) {
                const int seg = c * CH + sg;
                const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc0), seg));
                const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc1), seg));
                float d[2] = {0.0f, 0.0f};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const moe::f32x4 hv = hw[seg * 32 + q * 8 + sub];
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        const uint4 wq = w[c % 3][g][sg];
                        const uint32_t dw = q == 0 ? wq.x : q == 1 ? wq.y : q == 2 ? wq.z : wq.w;
                        const f32x2 w01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)dw, false);
                        const f32x2 w23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)dw, true);
                        d[g] = fmaf(w01.x, hv.x, d[g]);
                        d[g] = fmaf(w01.y, hv.y, d[g]);
                        d[g] = fmaf(w23.x, hv.z, d[g]);
                        d[g] = fmaf(w23.y, hv.w, d[g]);
                    }
                }
                acc[0] = fmaf(d[0], s0, acc[0]);
                acc[1] = fmaf(d[1], s1, acc[1]);
                // (pins the groups' sums here, as in the 16-row kernel)
                asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const float v = moe::sum8_lanes(acc[g]);
            const int r = g0 + g * 8 + grp;
            if (sub == 0 && own[g]) {
                a.y[(size_t)p * H + r] = v;
                sums[j * ROWS + r - row0] = v;
            }
        }
    }
    int *cp = reinterpret_cast<int *>(sums + 8 * ROWS);
    float *cw = reinterpret_cast<float *>(cp + 8);
    if (tid < 8) {
        cp[tid] = pc;
        cw[tid] = wc;
    }
    moe::lds_barrier();
    if (tid < ROWS) {
        float o = 0.0f;
        for (int jj = 0; jj < a.k; ++jj)
            if (cp[jj] >= 0) o = __fadd_rn(o, __fmul_rn(cw[jj], sums[jj * ROWS + tid]));
        a.out[row0 + tid] = o;
    }
}

// ---------------------------------------------------------------------------
// fused decode layer: route pack, gate/up + SwiGLU, down and combine in one launch
// ---------------------------------------------------------------------------
// The route, flags, waits and launch are in fused_common.h; the items below
// are this file's gate/up and down items.
static_assert(kThreads == kFusedThreads, "fused kernels use the GEMV block size");
using FusedArgs = FusedArgsT<GateUpArgs, DownArgs>;

// GCH/GNCH and DCH/DNCH: the chunking of the gate/up and down items (NCH > 0
// fully unrolled, 0 looped).
template <int GCH, int GNCH, int GST, int DCH, int DNCH, int DST>
__global__ __launch_bounds__(kThreads, 4) void moe_fused_decode_e4m3_kernel(FusedArgs a)
{
    extern __shared__ uint4 dyn[];                   // x tile (gate/up), then h tile (down)
    __shared__ FusedRoute R;
    __shared__ float ush[GST][16];
    const int tid = threadIdx.x;
    fused_route(a, R, tid < a.M * a.k ? a.ids[tid] : -1);
    fused_route_status(a, R);
    const int na = moe::uniform(R.na);
    const int H = a.dn.H, I = a.gu.I;
    if (na == 0) {                                   // no valid slot: every output row is zero
        for (size_t q = (size_t)blockIdx.x * kThreads + tid; q < (size_t)a.M * H;
             q += (size_t)gridDim.x * kThreads)
            a.out[q] = 0.0f;
    }

    // gate/up + SwiGLU items: expert-major
    const int ntg = I / 16;
    for (int it = blockIdx.x; it < na * ntg; it += gridDim.x) {
        const int ai = it / ntg, tile = it - ai * ntg;
        const int e = moe::uniform(R.ae[ai]), p0 = moe::uniform(R.ap0[ai]);
        const int ne = moe::uniform(R.acnt[ai]);
        gateup_e4m3_item<GCH, GNCH, GST, true>(a.gu, e, tile, p0, ne, R.tok + p0, dyn, ush);
        moe::wait_vm0();                             // this wave's h stores are written
        __syncthreads();
        if (tid == 0) publish(a.flag_gu + it, a.epoch);
    }

    // down items: tile-major, so the experts of one row tile run together
    const int ntd = H / 32;
    for (int it = blockIdx.x; it < na * ntd; it += gridDim.x) {
        const int tile = it / na, ai = it - tile * na;
        const int e = moe::uniform(R.ae[ai]), p0 = moe::uniform(R.ap0[ai]);
        const int ne = moe::uniform(R.acnt[ai]);
        const FusedWait wait_h{a.flag_gu + ai * ntg, ntg, a.epoch, &R.flag};
        down_e4m3_item<DCH, DNCH, DST, true>(a.dn, e, tile, p0, ne, reinterpret_cast<float4 *>(dyn),
                                             wait_h);
        moe::wait_vm0();                             // this wave's y stores are written
        __syncthreads();
        uint32_t *fl = a.flag_dn + (size_t)tile * a.A;
        if (ai + 1 < na) {
            if (tid == 0) publish(fl + ai, a.epoch);
            continue;
        }
        // the tile's last expert: wait for the others' y rows, then combine rows
        // tile*32 .. +32 of every token
        const FusedWait wait_y{fl, na - 1, a.epoch, &R.flag};
        wait_y();
        for (int q = tid; q < a.M * 32; q += kThreads) {
            const int t = q >> 5, m = tile * 32 + (q & 31);
            float acc = 0.0f;
            for (int j = 0; j < a.k; ++j) {
                const int pr = R.t2p[t * a.k + j];
                if (pr < 0) continue;
                acc = __fadd_rn(acc, __fmul_rn(a.w[t * a.k + j], moe::load_dev(a.dn.y + (size_t)pr * H + m)));
            }
            a.out[(size_t)t * H + m] = acc;
        }
    }
    fused_route_tables(a, R);
    __syncthreads();
    if (tid == 0 && R.flag) atomicAdd(a.r.status, (int)kFusedTimeoutFlag);
}

// ---------------------------------------------------------------------------
// fused decode layer for one token (M == 1)
// ---------------------------------------------------------------------------
// The same phases with gate/up items of 2 h rows: wave w streams row
// 2r + (w & 1) of the gate (w < 2) or up (w >= 2) bank of one expert over the
// whole of K, 64 lanes x 16 bytes per load (1 KB, 8 K segments).  Items are
// numbered expert-major (q = expert * inter/2 + r) and block b takes q = b,
// b + grid, ..., so every block walks the experts in order and the experts'
// h are completed one after another rather than all at the end; the down items (32 rows of one
// expert) run expert-major, so those of the first experts overlap the gate/up
// of the last.  The token's x row sits in LDS for the whole gate/up phase;
// each item's weights are in flight while the previous item is multiplied.
// Gate/up flags are per item ([A][inter/2]).  Products are summed per lane
// over its K segments, then over the 64 lanes, so g and u agree with the
// three-call path to rounding, not bit for bit.
template <int NJ>
__device__ __forceinline__ void thin_issue(const FusedArgs &a, const FusedRoute &R, bool is_up,
                                           int wave, int lane, int ai, int r, uint4 (&w)[NJ],
                                           float &sc)
{
    const int H = a.gu.H, I = a.gu.I;
    const int e = moe::uniform(R.ae[ai]);
    const int row = 2 * r + (wave & 1);
    const uint8_t *rp = moe::uniform_ptr((is_up ? a.gu.ucodes : a.gu.gcodes) + ((size_t)e * I + row) * H);
#pragma unroll
    for (int j = 0; j < NJ; ++j) w[j] = load16(rp + j * 1024 + lane * 16);
    const int nseg = H >> 7;
    const float *sp = (is_up ? a.gu.uscales : a.gu.gscales) + ((size_t)e * (I >> 7) + (row >> 7)) * nseg;
    sc = lane < nseg ? sp[lane] : 0.0f;
}

// one row's sum over K, every lane of the wave ends with it
template <int NJ>
__device__ __forceinline__ float thin_row(const uint4 (&w)[NJ], float sc, const uint4 *xl, int lane)
{
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const float s = __shfl(sc, j * 8 + (lane >> 3), 64);
        bf16x2 wb[8];
        e4m3x4_to_bf16(w[j].x, wb[0], wb[1]);
        e4m3x4_to_bf16(w[j].y, wb[2], wb[3]);
        e4m3x4_to_bf16(w[j].z, wb[4], wb[5]);
        e4m3x4_to_bf16(w[j].w, wb[6], wb[7]);
        const uint4 xa = xl[j * 128 + lane * 2];
        const uint4 xb = xl[j * 128 + lane * 2 + 1];
        float d = dot2(wb[0], xa.x, 0.0f);
        d = dot2(wb[1], xa.y, d);
        d = dot2(wb[2], xa.z, d);
        d = dot2(wb[3], xa.w, d);
        d = dot2(wb[4], xb.x, d);
        d = dot2(wb[5], xb.y, d);
        d = dot2(wb[6], xb.z, d);
        d = dot2(wb[7], xb.w, d);
        acc = fmaf(d, s, acc);
    }
    acc = moe::sum8_lanes(acc);
    acc += __shfl_xor(acc, 8, 64);
    acc += __shfl_xor(acc, 16, 64);
    acc += __shfl_xor(acc, 32, 64);
    return acc;
}

template <int NJ, int DCH, int DNCH, int DST>
__global__ __launch_bounds__(kThreads, 4) void moe_fused_decode1_e4m3_kernel(FusedArgs a)
{
    extern __shared__ uint4 dyn[];                   // x row (gate/up), then h tile (down)
    __shared__ FusedRoute R;
    __shared__ float ush[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int H = a.dn.H, I = a.gu.I;
    const int id_in = tid < a.k ? a.ids[tid] : -1;
    fused_route(a, R, id_in);
    fused_route_status(a, R);
    const int na = moe::uniform(R.na);
    if (na == 0) {                                   // no valid slot: the output row is zero
        for (int q = blockIdx.x * kThreads + tid; q < H; q += gridDim.x * kThreads) a.out[q] = 0.0f;
    }

    // gate/up + SwiGLU items, expert by expert
    const int nr = I >> 1;
    const bool is_up = wave >= 2;
    const int nq = na * nr;                          // item q: expert q / nr, rows 2(q % nr), +1
    int q = blockIdx.x, ai = q / nr, r = q - ai * nr;
    bool have = q < nq;
    int pq = -1;                                     // item whose h waits for its flag
    uint4 w0[NJ], w1[NJ];
    float sc0 = 0.0f, sc1 = 0.0f;
    if (have) thin_issue<NJ>(a, R, is_up, wave, lane, ai, r, w0, sc0);
    for (int f = tid; f < (H >> 3); f += kThreads)
        dyn[f] = *reinterpret_cast<const uint4 *>(a.gu.x + (size_t)f * 8);
    auto step = [&](uint4 (&wc)[NJ], float &scc, uint4 (&wn)[NJ], float &scn) {
        moe::wait_vm0();                             // this item's weights, the last h stores
        moe::lds_barrier();
        if (tid == 0 && pq >= 0) publish(a.flag_gu + pq, a.epoch);
        const int q2 = q + (int)gridDim.x, ai2 = q2 / nr, r2 = q2 - ai2 * nr;
        const bool have2 = q2 < nq;
        if (have2) thin_issue<NJ>(a, R, is_up, wave, lane, ai2, r2, wn, scn);
        const float v = thin_row<NJ>(wc, scc, dyn, lane);
        if (is_up && lane == 0) ush[wave - 2] = v;
        moe::lds_barrier();
        if (!is_up && lane == 0) {
            const float hv = swiglu_clamp(v, ush[wave], a.gu.limit);
            const int p0 = R.ap0[ai], ne = R.acnt[ai];
            const int row = 2 * r + wave;
            for (int j = 0; j < ne; ++j) moe::store_dev(a.gu.h + (size_t)(p0 + j) * I + row, hv);
        }
        pq = q; q = q2; ai = ai2; r = r2; have = have2;
    };
    if (have) {
        for (;;) {
            step(w0, sc0, w1, sc1);
            if (!have) break;
            step(w1, sc1, w0, sc0);
            if (!have) break;
        }
        moe::wait_vm0();
        moe::lds_barrier();
        if (tid == 0) publish(a.flag_gu + pq, a.epoch);
    } else {
        moe::lds_barrier();                          // x is in LDS before the down items
    }

    // down items, expert-major
    const int ntd = H / 32, nd = na * ntd;
    for (int d = blockIdx.x; d < nd; d += gridDim.x) {
        const int dai = d / ntd, tile = d - dai * ntd;
        const int e = moe::uniform(R.ae[dai]), p0 = moe::uniform(R.ap0[dai]);
        const int ne = moe::uniform(R.acnt[dai]);
        const FusedWait wait_h{a.flag_gu + (size_t)dai * nr, nr, a.epoch, &R.flag};
        down_e4m3_item<DCH, DNCH, DST, true>(a.dn, e, tile, p0, ne, reinterpret_cast<float4 *>(dyn),
                                             wait_h);
        moe::wait_vm0();                             // this wave's y stores are written
        __syncthreads();
        uint32_t *fl = a.flag_dn + (size_t)tile * a.A;
        if (dai + 1 < na) {
            if (tid == 0) publish(fl + dai, a.epoch);
            continue;
        }
        // the tile's last expert: wait for the others' y rows, then combine
        const FusedWait wait_y{fl, na - 1, a.epoch, &R.flag};
        wait_y();
        for (int q = tid; q < 32; q += kThreads) {
            const int m = tile * 32 + q;
            float acc = 0.0f;
            for (int j = 0; j < a.k; ++j) {
                const int pr2 = R.t2p[j];
                if (pr2 < 0) continue;
                acc = __fadd_rn(acc, __fmul_rn(a.w[j], moe::load_dev(a.dn.y + (size_t)pr2 * H + m)));
            }
            a.out[m] = acc;
        }
    }
    fused_route_tables(a, R);
    __syncthreads();
    if (tid == 0 && R.flag) atomicAdd(a.r.status, (int)kFusedTimeoutFlag);
}

}  // namespace

// Launch shapes.  Grid = (upper bound on active experts) x (row tiles) x
// (K slices); blocks whose active index is past num_active exit at once, so
// the host never needs the routing.
namespace {

template <int CH, int NCH, int ST, bool ROUTE>
void gateup_launch(const GateUpArgs &a, int grid, hipStream_t st)
{
    // x rows of a pass (with the route built in, at least block 0's route)
    size_t lds = (size_t)a.st * a.H * 2;
    if (ROUTE && lds < sizeof(FusedRoute)) lds = sizeof(FusedRoute);
    hipLaunchKernelGGL((gemv_gateup_e4m3_kernel<CH, NCH, ST, ROUTE>), dim3(grid), dim3(kThreads),
                       lds, st, a);
}

// Unrolled kernels for CH-segment chunks, for the chunk counts that fit 128
// VGPRs at each pass size; every other shape runs the looped kernel.  Passes
// of one slot take 4-segment chunks (hidden a multiple of 512, up to 16
// chunks), two slots 8-segment chunks (up to 8), more slots 8-segment chunks
// (up to 2).  At one token the launch is a single round of blocks, and the
// smaller chunks start multiplying sooner: 37.9 against 38.3 us at hidden
// 7168.
template <int CH, int ST, int MAXN, bool ROUTE, int N = 1>
bool gateup_launch_unrolled(const GateUpArgs &a, int nch, int grid, hipStream_t st)
{
    if constexpr (N > MAXN) {
        return false;
    } else {
        if (nch == N) {
            gateup_launch<CH, N, ST, ROUTE>(a, grid, st);
            return true;
        }
        return gateup_launch_unrolled<CH, ST, MAXN, ROUTE, N + 1>(a, nch, grid, st);
    }
}

// More slots than whole x rows fit (the pages' verify shape, hidden 7168 =
// 14 chunks of 512): one pass of up to MOE_E4M3_GU_ST slots, x staged per
// chunk (XW).  False for other shapes.
template <bool ROUTE>
bool gateup_launch_xw(const GateUpArgs &a, int grid, hipStream_t st)
{
    if (a.H != 7168) return false;
    size_t lds = 2 * (size_t)MOE_E4M3_GU_ST * 4 * 16 * sizeof(uint4);
    if (ROUTE && lds < sizeof(FusedRoute)) lds = sizeof(FusedRoute);
    hipLaunchKernelGGL((gemv_gateup_e4m3_kernel<4, 14, MOE_E4M3_GU_ST, ROUTE, true>), dim3(grid),
                       dim3(kThreads), lds, st, a);
    return true;
}

template <bool ROUTE>
void gateup_dispatch(const GateUpArgs &a, int grid, hipStream_t st)
{
    if (a.st > gemv_gateup_pass_slots(a.st, a.H, MOE_E4M3_GU_ST) && gateup_launch_xw<ROUTE>(a, grid, st))
        return;
    if (a.st <= 1 && a.H % 512 == 0 && gateup_launch_unrolled<4, 1, 16, ROUTE>(a, a.H / 512, grid, st))
        return;
    const int ch = gemv_chunk_segs(kFmtE4M3, a.H), nch = a.H / 128 / ch;
    bool done = false;
    if (ch == 8 && a.st > 1) {
        if (a.st <= 2) done = gateup_launch_unrolled<8, 2, 8, ROUTE>(a, nch, grid, st);
        else done = gateup_launch_unrolled<8, MOE_E4M3_GU_ST, 2, ROUTE>(a, nch, grid, st);
    }
    if (!done) {
        switch (ch) {
        case 8: gateup_launch<8, 0, MOE_E4M3_GU_ST, ROUTE>(a, grid, st); break;
        case 7: gateup_launch<7, 0, MOE_E4M3_GU_ST, ROUTE>(a, grid, st); break;
        case 6: gateup_launch<6, 0, MOE_E4M3_GU_ST, ROUTE>(a, grid, st); break;
        case 5: gateup_launch<5, 0, MOE_E4M3_GU_ST, ROUTE>(a, grid, st); break;
        case 4: gateup_launch<4, 0, MOE_E4M3_GU_ST, ROUTE>(a, grid, st); break;
        case 3: gateup_launch<3, 0, MOE_E4M3_GU_ST, ROUTE>(a, grid, st); break;
        case 2: gateup_launch<2, 0, MOE_E4M3_GU_ST, ROUTE>(a, grid, st); break;
        default: gateup_launch<1, 0, MOE_E4M3_GU_ST, ROUTE>(a, grid, st); break;
        }
    }
}

template <int CH, int NCH, int ST>
void down_launch(const DownArgs &a, int grid, hipStream_t st)
{
    hipLaunchKernelGGL((gemv_down_e4m3_kernel<CH, NCH, ST>), dim3(grid), dim3(kThreads),
                       (size_t)a.st * a.I * 4, st, a);
}

// Unrolled kernels for 4-segment chunks, for the chunk counts that fit the
// register budget of each pass size (up to 5 chunks, inter <= 2560, with one
// slot; 8 with two; 3 with more); every other shape runs the looped kernel.
template <int ST, int MAXN, int N = 1>
bool down_launch_unrolled(const DownArgs &a, int nch, int grid, hipStream_t st)
{
    if constexpr (N > MAXN) {
        return false;
    } else {
        if (nch == N) {
            down_launch<4, N, ST>(a, grid, st);
            return true;
        }
        return down_launch_unrolled<ST, MAXN, N + 1>(a, nch, grid, st);
    }
}

template <int NCH>
void down_rg_launch(const DownArgs &a, int grid, hipStream_t st)
{
    hipLaunchKernelGGL((gemv_down_rg_e4m3_kernel<1, 2 * NCH, 4, 2>), dim3(grid), dim3(kThreads),
                       (size_t)a.st * a.I * 4, st, a);
}

template <int CH, int NCH, int RG>
void down1_launch(const Down1Args &a, hipStream_t st)
{
    constexpr int I = NCH * CH * 128;
    hipLaunchKernelGGL((gemv_down1_e4m3_kernel<CH, NCH, RG>), dim3(a.H / (8 * RG)), dim3(512),
                       (size_t)8 * I * 4 + 8 * 8 * RG * 4 + 64, st, a);
}

template <int CH, int NCH>
void down1p_launch(const Down1Args &a, hipStream_t st)
{
    constexpr int I = NCH * CH * 128;
    hipLaunchKernelGGL((gemv_down1p_e4m3_kernel<CH, NCH>), dim3(a.H / 28), dim3(1024),
                       (size_t)16 * I * 4 + 8 * 28 * 4 + 64, st, a);
}

}  // namespace

hipError_t launch_gemv_gateup_e4m3(const GemvBankDev &gate, const GemvBankDev &up,
                                   const uint16_t *x, const MoeRouteDev &r, int32_t M, int32_t S,
                                   int32_t E, int32_t hidden, int32_t inter, float limit, float *h,
                                   hipStream_t st, const int32_t *route_ids, int32_t top_k)
{
    GateUpArgs a{};
    // whole x rows of as many slots as fit the tile; the chunk-staged form
    // takes every slot of an expert (up to the cap) where it is built
    a.st = gemv_gateup_pass_slots(M, hidden, MOE_E4M3_GU_ST);
    if (a.st < (M < MOE_E4M3_GU_ST ? M : MOE_E4M3_GU_ST) && hidden == 7168)
        a.st = M < MOE_E4M3_GU_ST ? M : MOE_E4M3_GU_ST;
    a.gcodes = gate.codes; a.ucodes = up.codes;
    a.gscales = (const float *)gate.scales; a.uscales = (const float *)up.scales;
    a.x = x; a.offsets = r.offsets; a.sorted_token = r.sorted_token; a.active = r.active;
    a.h = h; a.H = hidden; a.I = inter; a.limit = limit;
    a.ntiles = inter / 16;
    a.ids = route_ids; a.M = M; a.k = top_k; a.E = E; a.r = r;
    const int grid = (S < E ? S : E) * a.ntiles;
    if (route_ids) {
        if (S > 128) return hipErrorInvalidValue;
        gateup_dispatch<true>(a, grid, st);
    } else {
        gateup_dispatch<false>(a, grid, st);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_down_e4m3(const GemvBankDev &down, const float *h, const MoeRouteDev &r,
                                 int32_t M, int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                 float *y, hipStream_t st)
{
    DownArgs a;
    a.st = gemv_down_pass_slots(M, inter, MOE_E4M3_DN_ST);
    a.codes = down.codes; a.scales = (const float *)down.scales; a.h = h;
    a.offsets = r.offsets; a.active = r.active; a.y = y;
    a.H = hidden; a.I = inter;
    if (M >= 3 && a.st < 4 && inter % 256 == 0 && inter <= 2560 && hidden % 64 == 0) {
        // four slots a pass, two row groups per wave (64-row tiles)
        a.st = M < 4 ? M : 4;
        a.ntiles = hidden / 64;
        const int grid = (S < E ? S : E) * a.ntiles;
        switch (inter / 256) {
        case 1: down_rg_launch<1>(a, grid, st); break;
        case 2: down_rg_launch<2>(a, grid, st); break;
        case 3: down_rg_launch<3>(a, grid, st); break;
        case 4: down_rg_launch<4>(a, grid, st); break;
        case 5: down_rg_launch<5>(a, grid, st); break;
        case 6: down_rg_launch<6>(a, grid, st); break;
        case 7: down_rg_launch<7>(a, grid, st); break;
        case 8: down_rg_launch<8>(a, grid, st); break;
        case 9: down_rg_launch<9>(a, grid, st); break;
        default: down_rg_launch<10>(a, grid, st); break;
        }
        return hipGetLastError();
    }
    a.ntiles = hidden / 32;
    const int grid = (S < E ? S : E) * a.ntiles;
    const int ch = gemv_down_chunk_segs(kFmtE4M3, inter), nch = inter / 128 / ch;
    bool done = false;
    if (ch == 4) {
        if (a.st <= 1) done = down_launch_unrolled<1, 5>(a, nch, grid, st);
        else if (a.st <= 2) done = down_launch_unrolled<2, 8>(a, nch, grid, st);
        else done = down_launch_unrolled<MOE_E4M3_DN_ST, 3>(a, nch, grid, st);
    }
    if (!done) {
        switch (ch) {
        case 4: down_launch<4, 0, MOE_E4M3_DN_ST>(a, grid, st); break;
        case 3: down_launch<3, 0, MOE_E4M3_DN_ST>(a, grid, st); break;
        case 2: down_launch<2, 0, MOE_E4M3_DN_ST>(a, grid, st); break;
        default: down_launch<1, 0, MOE_E4M3_DN_ST>(a, grid, st); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_gemv_down1_e4m3(const GemvBankDev &down, const float *h, const int32_t *ids,
                                  const int32_t *t2p, const float *w, int32_t k, int32_t hidden,
                                  int32_t inter, float *y, float *out, hipStream_t st)
{
    if (!gemv_down1_fits(kFmtE4M3, 1, k, hidden, inter)) return hipErrorInvalidValue;
    Down1Args a;
    a.codes = down.codes; a.scales = (const float *)down.scales; a.h = h;
    a.ids = ids; a.t2p = t2p; a.w = w; a.y = y; a.out = out;
    a.H = hidden; a.k = k;
    // The grid is a single round, so the CU with the most rows sets the
    // length: 28-row blocks (16 waves, an h row per wave, so inter up to
    // 2048) where hidden is a multiple of 28 and they leave the busiest CU
    // fewer rows than 16-row blocks do.  Their waves stream 2-segment
    // chunks (20.7 against 21.2 us with 4 at 7168 x 2048).
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    auto busiest = [&](int rows) { return (hidden / rows + cus - 1) / cus * rows; };
    if (hidden % 28 == 0 && inter <= 2048 && busiest(28) < busiest(16)) {
        switch (inter / 512) {
        case 1: down1p_launch<2, 2>(a, st); break;
        case 2: down1p_launch<2, 4>(a, st); break;
        case 3: down1p_launch<2, 6>(a, st); break;
        default: down1p_launch<2, 8>(a, st); break;
        }
        return hipGetLastError();
    }
    switch (inter / 512) {
    case 1: down1_launch<4, 1, 2>(a, st); break;
    case 2: down1_launch<4, 2, 2>(a, st); break;
    case 3: down1_launch<4, 3, 2>(a, st); break;
    case 4: down1_launch<4, 4, 2>(a, st); break;
    default: down1_launch<4, 5, 2>(a, st); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fused decode layer launch
// ---------------------------------------------------------------------------
namespace {

template <int GCH, int GNCH, int GST, int DCH, int DNCH, int DST>
hipError_t fused_launch(const FusedArgs &a, size_t lds, hipStream_t st)
{
    return resident_launch<moe_fused_decode_e4m3_kernel<GCH, GNCH, GST, DCH, DNCH, DST>>(a, lds, st);
}

// Unrolled chunking for the pages' decode shape (hidden 7168 = 7 chunks of
// 1024, inter 2048 = 4 chunks of 512); single-segment looped items otherwise.
template <int GST, int DST>
hipError_t fused_dispatch(const FusedArgs &a, size_t lds, hipStream_t st)
{
    if (a.gu.H == 7168 && a.gu.I == 2048) return fused_launch<8, 7, GST, 4, 4, DST>(a, lds, st);
    return fused_launch<1, 0, GST, 1, 0, DST>(a, lds, st);
}

// One token: 2-row gate/up items (H a multiple of 1024), unrolled down items
// for the pages' decode shape.
template <int NJ>
hipError_t fused1_dispatch(const FusedArgs &a, size_t lds, hipStream_t st)
{
    if (a.gu.H == 7168 && a.gu.I == 2048)
        return resident_launch<moe_fused_decode1_e4m3_kernel<NJ, 4, 4, 1>>(a, lds, st);
    return resident_launch<moe_fused_decode1_e4m3_kernel<NJ, 1, 0, 1>>(a, lds, st);
}

}  // namespace

int fused_decode_max_slots() { return kFusedMaxSlots; }

hipError_t launch_fused_decode_e4m3(const GemvBankDev &gate, const GemvBankDev &up,
                                    const GemvBankDev &down, const uint16_t *x, const int32_t *ids,
                                    const float *w, int32_t M, int32_t k, int32_t E, int32_t hidden,
                                    int32_t inter, float limit, const MoeRouteDev &r, float *h,
                                    float *y, float *out, void *flags, uint32_t epoch,
                                    hipStream_t st)
{
    FusedArgs a{};
    a.gu.gcodes = gate.codes; a.gu.ucodes = up.codes;
    a.gu.gscales = (const float *)gate.scales; a.gu.uscales = (const float *)up.scales;
    a.gu.x = x; a.gu.h = h; a.gu.H = hidden; a.gu.I = inter; a.gu.limit = limit;
    a.gu.st = gemv_gateup_pass_slots(M, hidden, 2);
    a.dn.codes = down.codes; a.dn.scales = (const float *)down.scales; a.dn.h = h; a.dn.y = y;
    a.dn.H = hidden; a.dn.I = inter;
    a.dn.st = gemv_down_pass_slots(M, inter, 2);
    a.ids = ids; a.w = w; a.M = M; a.k = k; a.E = E; a.epoch = epoch;
    a.A = M * k < E ? M * k : E;
    a.flag_gu = (uint32_t *)flags;
    a.flag_dn = a.flag_gu + (size_t)a.A * (inter / 2);
    a.out = out; a.r = r;
    const size_t xl = (size_t)a.gu.st * hidden * 2, hl = (size_t)a.dn.st * inter * 4;
    const size_t lds = xl > hl ? xl : hl;
    if (M == 1 && hidden % 1024 == 0 && hidden <= 8192 && a.dn.st == 1) {
        switch (hidden / 1024) {
        case 1: return fused1_dispatch<1>(a, lds, st);
        case 2: return fused1_dispatch<2>(a, lds, st);
        case 3: return fused1_dispatch<3>(a, lds, st);
        case 4: return fused1_dispatch<4>(a, lds, st);
        case 5: return fused1_dispatch<5>(a, lds, st);
        case 6: return fused1_dispatch<6>(a, lds, st);
        case 7: return fused1_dispatch<7>(a, lds, st);
        default: return fused1_dispatch<8>(a, lds, st);
        }
    }
    if (a.gu.st == 1 && a.dn.st == 1) return fused_dispatch<1, 1>(a, lds, st);
    if (a.gu.st == 1) return fused_dispatch<1, 2>(a, lds, st);
    if (a.dn.st == 1) return fused_dispatch<2, 1>(a, lds, st);
    return fused_dispatch<2, 2>(a, lds, st);
}
