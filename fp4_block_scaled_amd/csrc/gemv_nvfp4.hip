// gemv_nvfp4.hip -- dequant-GEMV tier for NVFP4 expert banks.
//
// NVFP4 weight = E2M1 code x E4M3 scale (one per 16 inputs) x FP32 scale_2
// (one per expert projection): "memra-engine src/dsv4_ep.rs", fn chain (code
// stride inter*hidden/2, scale stride inter*hidden/16, a scale_2 per expert)
// and "spark_model glm5next_mlp/forward.rs", fn w4a16_gemv (the NVFP4 operand
// triple, scale_2 by value).  Same work layout as the E4M3 GEMV: 8 lanes per
// weight row, 16 code bytes (32 weights) per lane per 128-byte segment, one
// pass over each active expert for all of its slots; gate/up covers the
// whole of K per block and ends in the clamped SwiGLU.
//
// Decode: gfx950 converts E2M1 pairs straight to bf16 (gate/up, against bf16
// activations with v_dot2) or to f32 (down, against FP32 h); the E2M1 values
// are exact in both.  The two E4M3 group scales of a lane's 32 weights are
// applied once per 16 products; scale_2 once per output.
#include <type_traits>

#include "moe_internal.h"
#include "fused_common.h"

namespace {

using moe::bf16x2;
using moe::f32x2;

constexpr int kThreads = 256;
constexpr int kSegK = 256;                          // K values per 128-byte segment

struct GateUpArgs {
    const uint8_t *gcodes, *ucodes, *gscales, *uscales;
    const float *gscale2, *uscale2;
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
    const uint8_t *codes, *scales;
    const float *scale2;
    const float *h;                     // [S][I]
    const int32_t *offsets, *active;
    float *y;                           // [S][H]
    int32_t H, I, ntiles, st;           // st: slots per weight pass (<= ST)
};

// Down projection and combine of one token (gemv_down1_nvfp4_kernel).
struct Down1Args {
    const uint8_t *codes, *scales;
    const float *scale2;
    const float *h;                     // [S][I]
    const int32_t *ids, *t2p;           // [k]: the token's expert ids and packed rows (-1: none)
    const float *w;                     // [k]: its top-k weights
    float *y, *out;                     // y [S][H] packed rows, out [H]
    int32_t H, k;
};

// Codes and group scales are streamed once per call (non-temporal loads).
__device__ __forceinline__ uint4 load16(const uint8_t *p)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = moe::load_nt_global<u32x4>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Activation rows sit in LDS permuted per 256-wide segment so that the 8
// lanes of a weight row read 128 contiguous bytes: bf16 x keeps uint4 q*8 +
// sub of a segment for the source uint4 sub*4 + q, FP32 h keeps float4 q*8 +
// sub for the source float4 sub*8 + q.  Staging walks the LDS positions in
// order (each 64-lane store is one contiguous 1 KB, free of bank conflicts)
// and loads the source element of each position.
__device__ __forceinline__ int x_src(int pos)
{
    return (pos & ~31) | ((pos & 7) << 2) | ((pos >> 3) & 3);
}
__device__ __forceinline__ int h_src(int pos)
{
    return (pos & ~63) | ((pos & 7) << 3) | ((pos >> 3) & 7);
}

__device__ __forceinline__ uint32_t load2(const uint8_t *p)
{
    return moe::load_nt_global<uint16_t>(p);
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

// silu(min(g, L)) * clamp(u, -L, L), silu(z) = z / (1 + e^-z)
__device__ __forceinline__ float swiglu_clamp(float g, float u, float L)
{
    const float gc = fminf(g, L);
    const float uc = fminf(fmaxf(u, -L), L);
    return gc / (1.0f + expf(-gc)) * uc;
}

// gate + up + SwiGLU: one block = 16 h rows of one active expert over the
// whole of K; waves 0-1 stream those rows of the gate bank, waves 2-3 of the
// up bank.  At the start of a pass the bf16 x rows of up to a.st slots go to
// LDS for the whole of K (uint4 q of lane sub in segment sg at sg*32 + q*8 +
// sub, so the 8 lanes of a row read 128 contiguous bytes); the K loop then
// only streams codes and group scales, in chunks of CH 256-wide segments.
// With NCH > 0 (chunk count known at compile time) the loop is fully
// unrolled with the next two chunks in flight (straight-line code: the
// compiler waits for exactly the chunk it multiplies); NCH == 0 is the
// generic looped form with one chunk in flight.  The up sums reach the gate
// waves through LDS; they apply scale_2, the clamped SwiGLU, and write h.
// ROUTE: the route of the S <= 128 slots comes from the ids inside the launch
// (the same stable pack as route_pack) instead of from the tables of a route
// pack launched before: every block works out its own expert; block 0 also
// builds the whole route and writes the tables for the down and combine
// launches that follow.
struct NoRoute {};

template <class Args, class Route>
__device__ __forceinline__ void route_tables_block0(const Args &a, Route &R)
{
    if (blockIdx.x != 0) return;
    const int id_in = (int)threadIdx.x < a.M * a.k ? a.ids[threadIdx.x] : -1;
    fused_route(a, R, id_in);
    fused_route_status(a, R);
    fused_route_tables(a, R);
}

// XW (unrolled form, more slots than whole x rows fit): the x rows of the
// pass go to LDS one K chunk at a time into two buffers ([2][ST][CH * 32]
// uint4, permuted per segment as above), chunk c+1's loaded into VGPRs while
// chunk c is multiplied, so one weight pass serves every slot of the expert
// (up to ST); the scale rows follow the two buffers.
template <int CH, int NCH, int ST, bool ROUTE, bool XW = false>
__global__ __launch_bounds__(kThreads, 4) void gemv_gateup_nvfp4_kernel(GateUpArgs a)
{
    static_assert(!XW || NCH > 0, "chunked x staging is an unrolled form");
    extern __shared__ uint4 xl[];                    // [a.st][H / 8], permuted per segment
    __shared__ float ush[ST][16];
    // with the route built in, block 0's route goes to the x tile's LDS once
    // its item has ended (the launch sizes it for both)
    auto &R = *reinterpret_cast<typename std::conditional<ROUTE, FusedRoute, NoRoute>::type *>(xl);
    __shared__ int32_t tokl[ROUTE ? 128 : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int grp = lane >> 3, sub = lane & 7;
    const int tile = blockIdx.x % a.ntiles;
    const int ai = blockIdx.x / a.ntiles;
    int e, p0, ne;
    const int32_t *tok;
    if constexpr (ROUTE) {
        const LightRoute lr = light_route(a.ids, a.M * a.k, a.E, ai);
        light_route_tokens(lr, a.k, tokl);
        moe::lds_barrier();
        if (lr.e < 0) {
            route_tables_block0(a, R);
            return;
        }
        e = moe::uniform(lr.e);
        p0 = moe::uniform(lr.p0);
        ne = moe::uniform(lr.ne);
        tok = tokl;
    } else {
        e = moe::uniform(a.active[ai]);              // -1 past the active experts
        if (e < 0) return;
        p0 = moe::uniform(a.offsets[e]);
        ne = moe::uniform(a.offsets[e + 1]) - p0;
        tok = a.sorted_token + p0;
    }
    const int H = a.H, I = a.I, H8 = H >> 3;
    const int nch = NCH > 0 ? NCH : H / (kSegK * CH);
    const bool is_up = wave >= 2;
    const int hrow0 = tile * 16;
    const int hrow = hrow0 + (wave & 1) * 8 + grp;
    const int rowb = H / 2, rows = H / 16;
    const float s2 = (is_up ? a.uscale2 : a.gscale2)[e];
    // code and group-scale addresses = wave-uniform base + fixed lane offset
    const size_t row0 = (size_t)e * I + hrow0 + (wave & 1) * 8;
    const uint8_t *cb0 = (is_up ? a.ucodes : a.gcodes) + row0 * rowb;
    const uint8_t *sb0 = (is_up ? a.uscales : a.gscales) + row0 * rows;
    const uint32_t coff = (uint32_t)grp * rowb + sub * 16, soff = (uint32_t)grp * rows + sub * 2;
    // Unrolled form: the group scales of the wave's 8 rows (contiguous in
    // memory) go to LDS with the x rows, in 16-byte loads, each row padded by
    // 16 bytes so the rows of one read fall in different banks; the K loop
    // then reads a lane's 2 scale bytes from LDS instead of issuing a 2-byte
    // load per segment.
    constexpr bool kScLds = NCH > 0;
    const int srow = rows + 16;
    constexpr int XC = CH * 32;                      // XW: uint4 of one slot's x per chunk
    constexpr int XB = ST * XC;                      // XW: uint4 per buffer
    const moe::u32x4 *xsrc[XW ? (XB + kThreads - 1) / kThreads : 1];   // XW: each x load's source in chunk 0
    const size_t xbytes = XW ? 2 * (size_t)XB * 16 : (size_t)a.st * H * 2;
    uint8_t *scl = reinterpret_cast<uint8_t *>(xl) + xbytes + wave * 8 * srow;

    for (int s0 = 0; s0 < ne; s0 += a.st) {          // passes over the weights
        const int nt = min(a.st, ne - s0);
        // opaque copies keep the per-chunk address arithmetic inside the pass
        const uint8_t *cbp = moe::uniform_ptr(cb0), *sbp = moe::uniform_ptr(sb0);
        uint32_t co = coff, so = soff;
        asm volatile("" : "+s"(cbp), "+s"(sbp), "+v"(co), "+v"(so));
        auto load_w = [&](uint4 (&wb)[CH], uint32_t (&sb)[CH], int c) {
#pragma unroll
            for (int sg = 0; sg < CH; ++sg) {
                wb[sg] = load16(cbp + (c * CH + sg) * 128 + co);
                if constexpr (!kScLds) sb[sg] = load2(sbp + (c * CH + sg) * 16 + so);
            }
        };
        float acc[ST];
#pragma unroll
        for (int j = 0; j < ST; ++j) acc[j] = 0.0f;
        // x tile as mul_chunk reads it: base, row stride (uint4), first segment
        const uint4 *xcur = xl;
        int xstr = H8, xseg0 = 0;
        auto mul_chunk = [&](const uint4 (&wc)[CH], const uint32_t (&vc)[CH], int c) {
#pragma unroll
            for (int sg = 0; sg < CH; ++sg) {
                const int seg = c * CH + sg;
                uint32_t vs;
                if constexpr (kScLds)
                    vs = *reinterpret_cast<const uint16_t *>(scl + grp * srow + seg * 16 + sub * 2);
                else
                    vs = vc[sg];
                const f32x2 sc = __builtin_amdgcn_cvt_pk_f32_fp8((int)vs, false);
                const uint4 wv = wc[sg];
#pragma unroll
                for (int j = 0; j < ST; ++j) {
                    if (j < nt) {
                        const uint4 *xv = &xcur[j * xstr + (seg - xseg0) * 32 + sub];
                        float d0 = dot8_fp4_bf16(wv.x, xv[0], 0.0f);
                        d0 = dot8_fp4_bf16(wv.y, xv[8], d0);
                        float d1 = dot8_fp4_bf16(wv.z, xv[16], 0.0f);
                        d1 = dot8_fp4_bf16(wv.w, xv[24], d1);
                        acc[j] = fmaf(d0, sc.x, acc[j]);
                        acc[j] = fmaf(d1, sc.y, acc[j]);
                    }
                }
                if constexpr (NCH > 0) __builtin_amdgcn_sched_barrier(0);
            }
        };

        if constexpr (NCH > 0) {
            constexpr int H8C = NCH * CH * 32;       // uint4 per x row (H8)
            constexpr int XV = (ST * H8C + kThreads - 1) / kThreads;
            uint4 w[3][CH];
            uint32_t v[3][CH];
            // the wave's scale rows: 8 * H/16 bytes, 1 KB per wave-wide load
            constexpr int SRB = NCH * CH * 16;       // scale bytes per row (H/16)
            constexpr int SV = (8 * SRB + 1023) / 1024;
            moe::u32x4 sr[SV];
#pragma unroll
            for (int i = 0; i < SV; ++i) {
                // past the rows' last 16 bytes a lane reloads those (never stored)
                const int o = min(lane * 16 + i * 1024, 8 * SRB - 16);
                sr[i] = moe::load_nt_global<moe::u32x4>(sbp + o);
            }
            if constexpr (XW) {
                // the first chunk's x rows (the rest go chunk by chunk below)
                xstr = XC;
                moe::u32x4 xr[(XB + kThreads - 1) / kThreads];
#pragma unroll
                for (int i = 0; i < (XB + kThreads - 1) / kThreads; ++i) {
                    // past the pass's last uint4 a lane reloads that one (never stored)
                    const int f = min(tid + i * kThreads, nt * XC - 1);
                    const int j = f / XC, r = x_src(f - j * XC);
                    // (the chunks of a load differ by XC uint4: looked up once per pass)
                    xsrc[i] = reinterpret_cast<const moe::u32x4 *>(a.x + (size_t)tok[s0 + j] * H + (size_t)r * 8);
                    xr[i] = xsrc[i][0];
                }
                load_w(w[0], v[0], 0);
#pragma unroll
                for (int i = 0; i < (XB + kThreads - 1) / kThreads; ++i) {
                    const int f = tid + i * kThreads;
                    if (f < nt * XC) reinterpret_cast<moe::u32x4 *>(xl)[f] = xr[i];
                }
            } else if constexpr (XV <= 4) {
                // x rows to LDS: every x load goes out at once, then the first
                // weight chunk; the LDS stores wait for the x loads only
                moe::u32x4 xr[XV];                   // (native vectors stay in VGPRs)
#pragma unroll
                for (int i = 0; i < XV; ++i) {
                    // past the pass's last uint4 a lane reloads that one (never stored)
                    const int f = min(tid + i * kThreads, nt * H8C - 1);
                    const int j = f / H8C, r = x_src(f - j * H8C);
                    xr[i] = *reinterpret_cast<const moe::u32x4 *>(a.x + (size_t)tok[s0 + j] * H + r * 8);
                }
                __builtin_amdgcn_sched_barrier(0);
                load_w(w[0], v[0], 0);
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
                    const int j = f / H8, r = x_src(f - j * H8);
                    xl[f] = *reinterpret_cast<const uint4 *>(a.x + (size_t)tok[s0 + j] * H + r * 8);
                }
                load_w(w[0], v[0], 0);
            }
#pragma unroll
            for (int i = 0; i < SV; ++i) {
                const int o = lane * 16 + i * 1024;
                if (o < 8 * SRB) {
                    const int r = o / SRB, cc = o - r * SRB;
                    *reinterpret_cast<moe::u32x4 *>(scl + r * srow + cc) = sr[i];
                }
            }
            if (NCH > 1) load_w(w[1], v[1], 1);
            moe::lds_barrier();
            if constexpr (XW) {
                constexpr int XR = (XB + kThreads - 1) / kThreads;
                moe::u32x4 xr[XR];
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    // x of chunk c+1 before the weights of c+2, so the wait for the
                    // x leaves those weight loads in flight
                    if (c + 1 < NCH) {
#pragma unroll
                        for (int i = 0; i < XR; ++i) xr[i] = xsrc[i][(c + 1) * XC];
                    }
                    if (c + 2 < NCH) load_w(w[(c + 2) % 3], v[(c + 2) % 3], c + 2);
                    __builtin_amdgcn_sched_barrier(0);
                    xcur = xl + (c & 1) * XB;
                    xseg0 = c * CH;
                    mul_chunk(w[c % 3], v[c % 3], c);
                    __builtin_amdgcn_sched_barrier(0);
                    if (c + 1 < NCH) {
                        moe::u32x4 *buf = reinterpret_cast<moe::u32x4 *>(xl) + ((c + 1) & 1) * XB;
#pragma unroll
                        for (int i = 0; i < XR; ++i) {
                            const int f = tid + i * kThreads;
                            if (f < nt * XC) buf[f] = xr[i];
                        }
                        moe::lds_barrier();
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    if (c + 2 < NCH) load_w(w[(c + 2) % 3], v[(c + 2) % 3], c + 2);
                    __builtin_amdgcn_sched_barrier(0);
                    mul_chunk(w[c % 3], v[c % 3], c);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            for (int f = tid; f < nt * H8; f += kThreads) {
                const int j = f / H8, r = x_src(f - j * H8); // r: source uint4 (8 K values)
                xl[f] = *reinterpret_cast<const uint4 *>(a.x + (size_t)tok[s0 + j] * H + r * 8);
            }
            uint4 w0[CH], w1[CH];
            uint32_t v0[CH], v1[CH];
            load_w(w0, v0, 0);
            moe::lds_barrier();
            auto step = [&](int c, uint4 (&wc)[CH], uint32_t (&vc)[CH], uint4 (&wn)[CH],
                            uint32_t (&vn)[CH]) {
                moe::wait_vm0();
                if (c + 1 < nch) load_w(wn, vn, c + 1);
                mul_chunk(wc, vc, c);
            };
            for (int c = 0; c < nch; c += 2) {
                step(c, w0, v0, w1, v1);
                if (c + 1 >= nch) break;
                step(c + 1, w1, v1, w0, v0);
            }
        }

        float v[ST];
#pragma unroll
        for (int j = 0; j < ST; ++j) v[j] = j < nt ? moe::sum8_lanes(acc[j]) * s2 : 0.0f;
        if (is_up && sub == 0) {
#pragma unroll
            for (int j = 0; j < ST; ++j)
                if (j < nt) ush[j][(wave & 1) * 8 + grp] = v[j];
        }
        moe::lds_barrier();
        if (!is_up && sub == 0) {
#pragma unroll
            for (int j = 0; j < ST; ++j)
                if (j < nt)
                    a.h[(size_t)(p0 + s0 + j) * I + hrow] =
                        swiglu_clamp(v[j], ush[j][(wave & 1) * 8 + grp], a.limit);
        }
        moe::lds_barrier();                           // x and ush are reused by the next pass
    }
    if constexpr (ROUTE) route_tables_block0(a, R);
}

// down: one block = 32 output rows of one active expert over the whole of K
// (= inter), 8 rows per wave.  At the start of a pass the FP32 h rows of up
// to a.st slots go to LDS (float4 q of lane sub in segment sg at sg*64 + q*8
// + sub); the K loop then streams codes and group scales in chunks of CH
// 256-wide segments, fully unrolled with the next two chunks in flight when
// NCH > 0, looped with one chunk in flight when NCH == 0.
// down_nvfp4_item does one (expert e, 32-row tile) item for the ne slots of
// e (packed rows p0..p0+ne) with hl the LDS h tile ([a.st][I / 4] float4).
// FUSED (the one-launch layer's item): the first weight chunks go out, then
// wait_h() runs (the wait for the expert's h), and h and y move through
// device-coherent accesses; otherwise the h loads go out first (in the
// unrolled form all of them, followed by the first chunk's loads before h is
// written to LDS).
struct NoWait {
    __device__ void operator()() const {}
};

template <int CH, int NCH, int ST, bool FUSED, class WaitH>
__device__ __forceinline__ void down_nvfp4_item(const DownArgs &a, int e, int tile, int p0, int ne,
                                                float4 *hl, const WaitH &wait_h)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int grp = lane >> 3, sub = lane & 7;
    const int H = a.H, I = a.I, I4 = I >> 2;
    const int nch = NCH > 0 ? NCH : I / (kSegK * CH);
    const int rowb = I / 2, rows = I / 16;
    const float s2 = a.scale2[e];
    const int row0 = tile * 32;
    const int row = row0 + wave * 8 + grp;
    const size_t r0 = (size_t)e * H + row0 + wave * 8;
    const uint8_t *cb0 = a.codes + r0 * rowb, *sb0 = a.scales + r0 * rows;
    const uint32_t coff = (uint32_t)grp * rowb + sub * 16, soff = (uint32_t)grp * rows + sub * 2;
    // Unrolled standalone form: the group scales of the wave's 8 rows go to
    // LDS after the h rows (as in the gate/up kernel: 16-byte loads, rows
    // padded by 16 bytes) and the K loop reads them from there.
    constexpr bool kScLds = NCH > 0 && !FUSED;
    const int srow = rows + 16;
    uint8_t *scl = reinterpret_cast<uint8_t *>(hl) + (size_t)a.st * I * 4 + wave * 8 * srow;

    for (int s0 = 0; s0 < ne; s0 += a.st) {          // passes over the weights
        const int nt = min(a.st, ne - s0);
        const uint8_t *cbp = moe::uniform_ptr(cb0), *sbp = moe::uniform_ptr(sb0);
        uint32_t co = coff, so = soff;
        asm volatile("" : "+s"(cbp), "+s"(sbp), "+v"(co), "+v"(so));
        auto load_w = [&](uint4 (&wb)[CH], uint32_t (&sb)[CH], int c) {
#pragma unroll
            for (int sg = 0; sg < CH; ++sg) {
                wb[sg] = load16(cbp + (c * CH + sg) * 128 + co);
                if constexpr (!kScLds) sb[sg] = load2(sbp + (c * CH + sg) * 16 + so);
            }
        };
        float acc[ST];
#pragma unroll
        for (int j = 0; j < ST; ++j) acc[j] = 0.0f;
        auto mul_chunk = [&](const uint4 (&wc)[CH], const uint32_t (&vc)[CH], int c) {
#pragma unroll
            for (int sg = 0; sg < CH; ++sg) {
                const int seg = c * CH + sg;
                uint32_t vs;
                if constexpr (kScLds)
                    vs = *reinterpret_cast<const uint16_t *>(scl + grp * srow + seg * 16 + sub * 2);
                else
                    vs = vc[sg];
                const f32x2 sc = __builtin_amdgcn_cvt_pk_f32_fp8((int)vs, false);
                const uint4 wv = wc[sg];
#pragma unroll
                for (int j = 0; j < ST; ++j) {
                    if (j < nt) {
                        const float4 *hv = &hl[j * I4 + seg * 64 + sub];
                        float d0 = dot8_fp4_f32(wv.x, hv[0], hv[8], 0.0f);
                        d0 = dot8_fp4_f32(wv.y, hv[16], hv[24], d0);
                        float d1 = dot8_fp4_f32(wv.z, hv[32], hv[40], 0.0f);
                        d1 = dot8_fp4_f32(wv.w, hv[48], hv[56], d1);
                        acc[j] = fmaf(d0, sc.x, acc[j]);
                        acc[j] = fmaf(d1, sc.y, acc[j]);
                    }
                }
                if constexpr (NCH > 0) __builtin_amdgcn_sched_barrier(0);
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
            uint32_t v[3][CH];
            constexpr int I4C = NCH * CH * 64;       // float4 per h row (I4)
            constexpr int HV = (ST * I4C + kThreads - 1) / kThreads;
            if constexpr (FUSED) {
                load_w(w[0], v[0], 0);
                if (NCH > 1) load_w(w[1], v[1], 1);
                wait_h();
                stage_h();
            } else if constexpr (HV <= 4) {
                // every h load goes out at once, then the first weight chunk;
                // the LDS stores wait for the h loads only (up to 4 per thread:
                // the two-slot passes of a 16-token layer too)
                constexpr int SRB = NCH * CH * 16;   // scale bytes per row (I/16)
                constexpr int SV = (8 * SRB + 1023) / 1024;
                moe::u32x4 sr[SV];
#pragma unroll
                for (int i = 0; i < SV; ++i) {
                    // past the rows' last 16 bytes a lane reloads those (never stored)
                    const int o = min(lane * 16 + i * 1024, 8 * SRB - 16);
                    sr[i] = moe::load_nt_global<moe::u32x4>(sbp + o);
                }
                moe::f32x4 hr[HV];                   // (native vectors stay in VGPRs)
#pragma unroll
                for (int i = 0; i < HV; ++i) {
                    // past the pass's last float4 a lane reloads that one (never stored)
                    const int f = min(tid + i * kThreads, nt * I4C - 1);
                    const int j = f / I4C, r = h_src(f - j * I4C);
                    hr[i] = *reinterpret_cast<const moe::f32x4 *>(a.h + (size_t)(p0 + s0 + j) * I + r * 4);
                }
                __builtin_amdgcn_sched_barrier(0);
                load_w(w[0], v[0], 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < HV; ++i) {
                    const int f = tid + i * kThreads;
                    if (f < nt * I4C) reinterpret_cast<moe::f32x4 *>(hl)[f] = hr[i];
                }
#pragma unroll
                for (int i = 0; i < SV; ++i) {
                    const int o = lane * 16 + i * 1024;
                    if (o < 8 * SRB) {
                        const int r = o / SRB, cc = o - r * SRB;
                        *reinterpret_cast<moe::u32x4 *>(scl + r * srow + cc) = sr[i];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if (NCH > 1) load_w(w[1], v[1], 1);
            } else {
                // (larger passes: h in a loop; the scales still go to LDS)
                stage_h();
                for (int o = lane * 16; o < 8 * rows; o += 1024) {
                    const int r = o / rows, cc = o - r * rows;
                    *reinterpret_cast<moe::u32x4 *>(scl + r * srow + cc) =
                        moe::load_nt_global<moe::u32x4>(sbp + o);
                }
                load_w(w[0], v[0], 0);
                if (NCH > 1) load_w(w[1], v[1], 1);
            }
            moe::lds_barrier();
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                if (c + 2 < NCH) load_w(w[(c + 2) % 3], v[(c + 2) % 3], c + 2);
                __builtin_amdgcn_sched_barrier(0);
                mul_chunk(w[c % 3], v[c % 3], c);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            if constexpr (!FUSED) stage_h();
            uint4 w0[CH], w1[CH];
            uint32_t v0[CH], v1[CH];
            load_w(w0, v0, 0);
            if constexpr (FUSED) {
                wait_h();
                stage_h();
            }
            moe::lds_barrier();
            auto step = [&](int c, uint4 (&wc)[CH], uint32_t (&vc)[CH], uint4 (&wn)[CH],
                            uint32_t (&vn)[CH]) {
                moe::wait_vm0();
                if (c + 1 < nch) load_w(wn, vn, c + 1);
                mul_chunk(wc, vc, c);
            };
            for (int c = 0; c < nch; c += 2) {
                step(c, w0, v0, w1, v1);
                if (c + 1 >= nch) break;
                step(c + 1, w1, v1, w0, v0);
            }
        }
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            if (j < nt) {
                const float v = moe::sum8_lanes(acc[j]) * s2;
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
__global__ __launch_bounds__(kThreads) void gemv_down_nvfp4_kernel(DownArgs a)
{
    extern __shared__ float4 hl[];                   // [a.st][I / 4], permuted per segment
    const int tile = blockIdx.x % a.ntiles;
    const int ai = blockIdx.x / a.ntiles;
    const int e = moe::uniform(a.active[ai]);       // -1 past the active experts
    if (e < 0) return;
    const int p0 = moe::uniform(a.offsets[e]);
    const int ne = moe::uniform(a.offsets[e + 1]) - p0;
    down_nvfp4_item<CH, NCH, ST, false>(a, e, tile, p0, ne, hl, NoWait{});
}

// ---------------------------------------------------------------------------
// down, several slots a pass
// ---------------------------------------------------------------------------
// As the E4M3 kernel of the same name: each wave takes RG row groups 32 rows
// apart (a block: 32*RG output rows), so every h value it reads from LDS
// serves all of them and four slots a pass cost the LDS reads per weight byte
// of two.  The group scales of the wave's rows go to LDS with the h rows.  The
// products of a slot are the down item's, in the same order.
template <int CH, int NCH, int ST, int RG>
__global__ __launch_bounds__(kThreads, 4) void gemv_down_rg_nvfp4_kernel(DownArgs a)
{
    extern __shared__ float4 hl[];                   // [a.st][I / 4] h rows, then the scale rows
    constexpr int I4 = NCH * CH * 64, I = I4 * 4;    // float4 per h row, K
    constexpr int HV = (ST * I4 + kThreads - 1) / kThreads;
    constexpr int RB = I / 2, SB = I / 16;           // code and scale bytes per row
    constexpr int SROW = SB + 16;                    // LDS scale row (padded)
    constexpr int SV = (8 * SB + 1023) / 1024;       // 16-byte scale loads per lane and row group
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
    const float s2 = a.scale2[e];
    uint8_t *scl = reinterpret_cast<uint8_t *>(hl) + (size_t)a.st * I * 4 + wave * 8 * RG * SROW;

    for (int s0 = 0; s0 < ne; s0 += a.st) {          // passes over the weights
        const int nt = min(a.st, ne - s0);
        const size_t r0 = (size_t)e * H + row0 + wave * 8;
        const uint8_t *cb = moe::uniform_ptr(a.codes + r0 * RB);
        const uint8_t *sb = moe::uniform_ptr(a.scales + r0 * SB);
        uint32_t co = (uint32_t)grp * RB + sub * 16;
        asm volatile("" : "+s"(cb), "+s"(sb), "+v"(co));
        auto load_w = [&](uint4 (&wc)[RG][CH], int c) {
#pragma unroll
            for (int g = 0; g < RG; ++g)
#pragma unroll
                for (int sg = 0; sg < CH; ++sg)
                    wc[g][sg] = load16(cb + g * 32 * RB + (c * CH + sg) * 128 + co);
        };
        // scale rows and every h load of the pass, then the first weight
        // chunk, then the LDS stores
        uint4 w[3][RG][CH];
        moe::u32x4 sr[RG][SV];
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int i = 0; i < SV; ++i) {
                // past the rows' last 16 bytes a lane reloads those (never stored)
                const int o = min(lane * 16 + i * 1024, 8 * SB - 16);
                sr[g][i] = moe::load_nt_global<moe::u32x4>(sb + g * 32 * SB + o);
            }
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
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int i = 0; i < SV; ++i) {
                const int o = lane * 16 + i * 1024;
                if (o < 8 * SB) {
                    const int r = o / SB, cc = o - r * SB;
                    *reinterpret_cast<moe::u32x4 *>(scl + (g * 8 + r) * SROW + cc) = sr[g][i];
                }
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
                f32x2 sc[RG];
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    const uint32_t vs =
                        *reinterpret_cast<const uint16_t *>(scl + (g * 8 + grp) * SROW + seg * 16 + sub * 2);
                    sc[g] = __builtin_amdgcn_cvt_pk_f32_fp8((int)vs, false);
                }
#pragma unroll
                for (int j = 0; j < ST; ++j) {
                    if (j < nt) {
                        const float4 *hv = &hl[j * I4 + seg * 64 + sub];
                        float d0[RG], d1[RG];
#pragma unroll
                        for (int qq = 0; qq < 4; ++qq) {
                            const float4 ha = hv[qq * 16], hb = hv[qq * 16 + 8];
#pragma unroll
                            for (int g = 0; g < RG; ++g) {
                                const uint4 wv = w[c % 3][g][sg];
                                const uint32_t dw = qq == 0 ? wv.x : qq == 1 ? wv.y : qq == 2 ? wv.z : wv.w;
                                if (qq == 0) d0[g] = dot8_fp4_f32(dw, ha, hb, 0.0f);
                                else if (qq == 1) d0[g] = dot8_fp4_f32(dw, ha, hb, d0[g]);
                                else if (qq == 2) d1[g] = dot8_fp4_f32(dw, ha, hb, 0.0f);
                                else d1[g] = dot8_fp4_f32(dw, ha, hb, d1[g]);
                            }
                        }
#pragma unroll
                        for (int g = 0; g < RG; ++g) {
                            acc[j][g] = fmaf(d0[g], sc[g].x, acc[j][g]);
                            acc[j][g] = fmaf(d1[g], sc[g].y, acc[j][g]);
                            asm volatile("" : "+v"(acc[j][g]));   // (keeps the sums per segment)
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int j = 0; j < ST; ++j)
            if (j < nt)
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    const float v = moe::sum8_lanes(acc[j][g]) * s2;
                    if (sub == 0) a.y[(size_t)(p0 + s0 + j) * H + row0 + g * 32 + wave * 8 + grp] = v;
                }
        moe::lds_barrier();                           // h and the scales are reused by the next pass
    }
}

// ---------------------------------------------------------------------------
// down + combine of one token
// ---------------------------------------------------------------------------
// As the E4M3 kernel of the same name: a block owns 8*RG output rows for
// every one of the token's k <= 8 slots, wave j streams those rows of slot
// j's expert (codes from HBM; its h row and its rows' group scales staged in
// an LDS region of its own) with the down item's products in the down item's
// order, and the block adds the slots' rows in slot order.
template <int CH, int NCH, int RG>
__global__ __launch_bounds__(512, RG <= 2 ? 4 : 2) void gemv_down1_nvfp4_kernel(Down1Args a)
{
    extern __shared__ float4 hl[];                   // per wave: h row, scale rows; row sums, slot table
    constexpr int ROWS = 8 * RG;
    constexpr int I4 = NCH * CH * 64, I = I4 * 4;    // float4 per h row, K
    constexpr int HV = I4 / 64;                      // h float4 per lane
    constexpr int RB = I / 2, SB = I / 16;           // code and scale bytes per row
    constexpr int SROW = SB + 16;                    // LDS scale row (padded)
    constexpr int SV = (ROWS * SB + 1023) / 1024;    // 16-byte scale loads per lane
    constexpr int WL = I * 4 + ROWS * SROW;          // LDS bytes per wave
    static_assert(WL % 16 == 0, "wave regions stay 16-byte aligned");
    const int tid = threadIdx.x, lane = tid & 63;
    const int j = moe::uniform(tid >> 6);            // this wave's slot
    const int grp = lane >> 3, sub = lane & 7;
    const int H = a.H, row0 = blockIdx.x * ROWS;
    uint8_t *wl = reinterpret_cast<uint8_t *>(hl) + j * WL;
    moe::f32x4 *hw = reinterpret_cast<moe::f32x4 *>(wl);
    uint8_t *scl = wl + I * 4;
    float *sums = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(hl) + 8 * WL);
    // the combine's slot table (packed row, weight) goes out first; its
    // lanes store it in LDS once their rows are done
    const int pc = tid < a.k ? a.t2p[tid] : -1;
    const float wc = tid < a.k ? a.w[tid] : 0.0f;
    const int p = j < a.k ? moe::uniform(a.t2p[j]) : -1;   // packed row; -1: no slot
    const int e = j < a.k ? moe::uniform(a.ids[j]) : 0;     // (loaded beside p, not after it)
    if (p >= 0) {
        const size_t r0 = (size_t)e * H + row0;
        const uint8_t *cb = moe::uniform_ptr(a.codes + r0 * RB);
        const uint8_t *sb = moe::uniform_ptr(a.scales + r0 * SB);
        uint32_t co = (uint32_t)grp * RB + sub * 16;
        asm volatile("" : "+s"(cb), "+v"(co));
        auto load_w = [&](uint4 (&wc)[RG][CH], int c) {
#pragma unroll
            for (int g = 0; g < RG; ++g)
#pragma unroll
                for (int sg = 0; sg < CH; ++sg)
                    wc[g][sg] = load16(cb + g * 8 * RB + (c * CH + sg) * 128 + co);
        };
        // scale rows and h row loads, then the first weight chunk, then the
        // LDS stores
        uint4 w[3][RG][CH];
        moe::u32x4 sr[SV];
#pragma unroll
        for (int i = 0; i < SV; ++i) {
            // past the rows' last 16 bytes a lane reloads those (never stored)
            const int o = min(lane * 16 + i * 1024, ROWS * SB - 16);
            sr[i] = moe::load_nt_global<moe::u32x4>(sb + o);
        }
        moe::f32x4 hr[HV];
#pragma unroll
        for (int i = 0; i < HV; ++i)
            hr[i] = *reinterpret_cast<const moe::f32x4 *>(a.h + (size_t)p * I + h_src(lane + i * 64) * 4);
        const float s2 = a.scale2[e];
        __builtin_amdgcn_sched_barrier(0);
        load_w(w[0], 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < HV; ++i) hw[lane + i * 64] = hr[i];
#pragma unroll
        for (int i = 0; i < SV; ++i) {
            const int o = lane * 16 + i * 1024;
            if (o < ROWS * SB) {
                const int r = o / SB, cc = o - r * SB;
                *reinterpret_cast<moe::u32x4 *>(scl + r * SROW + cc) = sr[i];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (NCH > 1) load_w(w[1], 1);
        // the LDS region is this wave's own: a wave-level barrier orders its
        // stores before the reads of the other lanes
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
                const float4 *hv = reinterpret_cast<const float4 *>(hw) + seg * 64 + sub;
                // each pair of h float4 serves every row group
                float d0[RG], d1[RG];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 ha = hv[q * 16], hb = hv[q * 16 + 8];
#pragma unroll
                    for (int g = 0; g < RG; ++g) {
                        const uint4 wv = w[c % 3][g][sg];
                        const uint32_t dw = q == 0 ? wv.x : q == 1 ? wv.y : q == 2 ? wv.z : wv.w;
                        if (q == 0) d0[g] = dot8_fp4_f32(dw, ha, hb, 0.0f);
                        else if (q == 1) d0[g] = dot8_fp4_f32(dw, ha, hb, d0[g]);
                        else if (q == 2) d1[g] = dot8_fp4_f32(dw, ha, hb, 0.0f);
                        else d1[g] = dot8_fp4_f32(dw, ha, hb, d1[g]);
                    }
                }
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    const uint32_t vs =
                        *reinterpret_cast<const uint16_t *>(scl + (g * 8 + grp) * SROW + seg * 16 + sub * 2);
                    const f32x2 sc = __builtin_amdgcn_cvt_pk_f32_fp8((int)vs, false);
                    acc[g] = fmaf(d0[g], sc.x, acc[g]);
                    acc[g] = fmaf(d1[g], sc.y, acc[g]);
                    // (pins each row group's sum here, so the compiler does
                    // not sink the later groups' products to the end of the
                    // loop and keep every h value live until then)
                    asm volatile("" : "+v"(acc[g]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const float v = moe::sum8_lanes(acc[g]) * s2;
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

// ---------------------------------------------------------------------------
// fused decode layer for one token (M == 1), NVFP4 banks
// ---------------------------------------------------------------------------
// The one-launch layer of fused_common.h with gate/up items of 2 h rows: wave
// w streams row 2r + (w & 1) of the gate (w < 2) or up (w >= 2) bank over the
// whole of K, 64 lanes x 16 code bytes per load (2048 K values); every block
// walks the experts in order, so their h complete one after another; the down
// items (32 rows of one expert) run expert-major.  The token's x row stays in
// LDS, permuted so that the lanes of one load read consecutive 16-byte words:
// word q (q < 4) of lane l in load j sits at j*256 + q*64 + l.  A lane's two
// group scales of a load come from one dword of the row's scale bytes, read
// once per item (lane l holds dwords l, l + 64, ...).  The gate/up sums run in
// another order than the three-call path's (per lane over its K, then over 64
// lanes), so they agree with it to rounding.
using FusedArgs = FusedArgsT<GateUpArgs, DownArgs>;
static_assert(kThreads == kFusedThreads, "fused kernels use the GEMV block size");

template <int NJ>
__device__ __forceinline__ void thin_issue_nv(const FusedArgs &a, const FusedRoute &R, bool is_up,
                                              int wave, int lane, int ai, int r, uint4 (&w)[NJ],
                                              uint32_t (&sd)[(NJ + 1) / 2])
{
    const int H = a.gu.H, I = a.gu.I;
    const int e = moe::uniform(R.ae[ai]);
    const size_t rr = (size_t)e * I + 2 * r + (wave & 1);
    const uint8_t *cp = moe::uniform_ptr((is_up ? a.gu.ucodes : a.gu.gcodes) + rr * (H / 2));
#pragma unroll
    for (int j = 0; j < NJ; ++j) w[j] = load16(cp + j * 1024 + lane * 16);
    const uint32_t *sp = reinterpret_cast<const uint32_t *>(
        moe::uniform_ptr((is_up ? a.gu.uscales : a.gu.gscales) + rr * (H / 16)));
    const int ndw = H / 64;                          // scale dwords of the row
#pragma unroll
    for (int q = 0; q < (NJ + 1) / 2; ++q) {
        const int d = lane + 64 * q;
        sd[q] = d < ndw ? moe::load_nt_global<uint32_t>(sp + d) : 0u;
    }
}

// one row's sum over K (before scale_2), every lane of the wave ends with it
template <int NJ>
__device__ __forceinline__ float thin_row_nv(const uint4 (&w)[NJ], const uint32_t (&sd)[(NJ + 1) / 2],
                                             const uint4 *xl, int lane)
{
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        // group scales of K j*2048 + lane*32 .. +32: bytes j*128 + 2*lane, +1
        const uint32_t dw = __shfl(sd[j / 2], (j * 32 + (lane >> 1)) & 63, 64);
        const uint32_t s16 = (lane & 1) ? (dw >> 16) : (dw & 0xFFFFu);
        const f32x2 sc = __builtin_amdgcn_cvt_pk_f32_fp8((int)s16, false);
        const uint4 *xv = xl + j * 256 + lane;
        float d0 = dot8_fp4_bf16(w[j].x, xv[0], 0.0f);
        d0 = dot8_fp4_bf16(w[j].y, xv[64], d0);
        float d1 = dot8_fp4_bf16(w[j].z, xv[128], 0.0f);
        d1 = dot8_fp4_bf16(w[j].w, xv[192], d1);
        acc = fmaf(d0, sc.x, acc);
        acc = fmaf(d1, sc.y, acc);
    }
    acc = moe::sum8_lanes(acc);
    acc += __shfl_xor(acc, 8, 64);
    acc += __shfl_xor(acc, 16, 64);
    acc += __shfl_xor(acc, 32, 64);
    return acc;
}

template <int NJ, int DCH, int DNCH>
__global__ __launch_bounds__(kThreads, 4) void moe_fused_decode1_nvfp4_kernel(FusedArgs a)
{
    extern __shared__ uint4 dyn[];                   // x row (gate/up), then h tile (down)
    __shared__ FusedRoute R;
    __shared__ float ush[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int H = a.dn.H, I = a.gu.I;
    fused_route(a, R, tid < a.k ? a.ids[tid] : -1);
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
    uint32_t s0[(NJ + 1) / 2], s1[(NJ + 1) / 2];
    if (have) thin_issue_nv<NJ>(a, R, is_up, wave, lane, ai, r, w0, s0);
    for (int u = tid; u < (H >> 3); u += kThreads)   // x, permuted per load
        dyn[(u & ~255) + (u & 3) * 64 + ((u & 255) >> 2)] =
            *reinterpret_cast<const uint4 *>(a.gu.x + (size_t)u * 8);
    auto step = [&](uint4 (&wc)[NJ], uint32_t (&sc)[(NJ + 1) / 2], uint4 (&wn)[NJ],
                    uint32_t (&sn)[(NJ + 1) / 2]) {
        moe::wait_vm0();                             // this item's weights, the last h stores
        moe::lds_barrier();
        if (tid == 0 && pq >= 0) publish(a.flag_gu + pq, a.epoch);
        const int q2 = q + (int)gridDim.x, ai2 = q2 / nr, r2 = q2 - ai2 * nr;
        const bool have2 = q2 < nq;
        if (have2) thin_issue_nv<NJ>(a, R, is_up, wave, lane, ai2, r2, wn, sn);
        const int e = moe::uniform(R.ae[ai]);
        const float v = thin_row_nv<NJ>(wc, sc, dyn, lane) * (is_up ? a.gu.uscale2 : a.gu.gscale2)[e];
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
            step(w0, s0, w1, s1);
            if (!have) break;
            step(w1, s1, w0, s0);
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
        down_nvfp4_item<DCH, DNCH, 1, true>(a.dn, e, tile, p0, ne, reinterpret_cast<float4 *>(dyn),
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

// Unrolled down items for the pages' NVFP4 shape (inter 1536 = 3 chunks of
// 2 segments), looped single-segment items otherwise.
template <int NJ>
hipError_t fused1_nv_dispatch(const FusedArgs &a, size_t lds, hipStream_t st)
{
    if (a.dn.I == 1536) return resident_launch<moe_fused_decode1_nvfp4_kernel<NJ, 2, 3>>(a, lds, st);
    return resident_launch<moe_fused_decode1_nvfp4_kernel<NJ, 1, 0>>(a, lds, st);
}

}  // namespace

namespace {

constexpr int kGUST = 8, kDNST = 8;

template <int CH, int NCH, int ST, bool ROUTE>
void gateup_launch(const GateUpArgs &a, int grid, hipStream_t st)
{
    // x rows of a pass, then (unrolled form) the scale rows of the 4 waves
    size_t lds = (size_t)a.st * a.H * 2 + (NCH > 0 ? 32 * (size_t)(a.H / 16 + 16) : 0);
    if (ROUTE && lds < sizeof(FusedRoute)) lds = sizeof(FusedRoute);
    hipLaunchKernelGGL((gemv_gateup_nvfp4_kernel<CH, NCH, ST, ROUTE>), dim3(grid), dim3(kThreads),
                       lds, st, a);
}

// Passes of one slot: unrolled kernels for 2-segment chunks (hidden a
// multiple of 512 up to 8192).  At one token the launch is a single round of
// blocks, and the smaller chunks start multiplying sooner: 16.8-17.0 against
// 17.0-17.3 us with 4-segment chunks at hidden 6144.
template <bool ROUTE, int N = 1>
bool gateup_launch_unrolled1(const GateUpArgs &a, int nch, int grid, hipStream_t st)
{
    if constexpr (N > 16) {
        return false;
    } else {
        if (nch == N) {
            gateup_launch<2, N, 1, ROUTE>(a, grid, st);
            return true;
        }
        return gateup_launch_unrolled1<ROUTE, N + 1>(a, nch, grid, st);
    }
}

// Unrolled kernels for 4-segment chunks (hidden a multiple of 1024 up to
// 8192) per pass size; every other shape runs the looped kernel.
template <int ST, bool ROUTE>
bool gateup_launch_unrolled(const GateUpArgs &a, int nch, int grid, hipStream_t st)
{
    switch (nch) {
    case 1: gateup_launch<4, 1, ST, ROUTE>(a, grid, st); return true;
    case 2: gateup_launch<4, 2, ST, ROUTE>(a, grid, st); return true;
    case 3: gateup_launch<4, 3, ST, ROUTE>(a, grid, st); return true;
    case 4: gateup_launch<4, 4, ST, ROUTE>(a, grid, st); return true;
    case 5: gateup_launch<4, 5, ST, ROUTE>(a, grid, st); return true;
    case 6: gateup_launch<4, 6, ST, ROUTE>(a, grid, st); return true;
    case 7: gateup_launch<4, 7, ST, ROUTE>(a, grid, st); return true;
    case 8: gateup_launch<4, 8, ST, ROUTE>(a, grid, st); return true;
    default: return false;
    }
}

// More slots than whole x rows fit (the pages' NVFP4 shape, hidden 6144 = 6
// chunks of 1024): one pass of up to kGUXW slots, x staged per chunk (XW).
// False for other shapes.
constexpr int kGUXW = 6;
template <bool ROUTE>
bool gateup_launch_xw(const GateUpArgs &a, int grid, hipStream_t st)
{
    if (a.H != 6144) return false;
    size_t lds = 2 * (size_t)kGUXW * 4 * 32 * sizeof(uint4) + 32 * (size_t)(a.H / 16 + 16);
    if (ROUTE && lds < sizeof(FusedRoute)) lds = sizeof(FusedRoute);
    hipLaunchKernelGGL((gemv_gateup_nvfp4_kernel<4, 6, kGUXW, ROUTE, true>), dim3(grid), dim3(kThreads),
                       lds, st, a);
    return true;
}

template <bool ROUTE>
void gateup_dispatch(const GateUpArgs &a, int grid, hipStream_t st)
{
    if (a.st > gemv_gateup_pass_slots(a.st, a.H, kGUST) && a.st <= kGUXW && gateup_launch_xw<ROUTE>(a, grid, st))
        return;
    if (a.st <= 1 && a.H % 512 == 0 && gateup_launch_unrolled1<ROUTE>(a, a.H / 512, grid, st)) return;
    const int ch = gemv_chunk_segs(kFmtNVFP4, a.H), nch = a.H / kSegK / ch;
    bool done = false;
    if (ch == 4 && a.st > 1) {
        if (a.st <= 2) done = gateup_launch_unrolled<2, ROUTE>(a, nch, grid, st);
        else done = gateup_launch_unrolled<8, ROUTE>(a, nch, grid, st);
    }
    if (!done) {
        switch (ch) {
        case 4: gateup_launch<4, 0, kGUST, ROUTE>(a, grid, st); break;
        case 3: gateup_launch<3, 0, kGUST, ROUTE>(a, grid, st); break;
        case 2: gateup_launch<2, 0, kGUST, ROUTE>(a, grid, st); break;
        default: gateup_launch<1, 0, kGUST, ROUTE>(a, grid, st); break;
        }
    }
}

template <int CH, int NCH, int ST>
void down_launch(const DownArgs &a, int grid, hipStream_t st)
{
    // h rows of a pass, then (unrolled form) the scale rows of the 4 waves
    const size_t lds = (size_t)a.st * a.I * 4 + (NCH > 0 ? 32 * (size_t)(a.I / 16 + 16) : 0);
    hipLaunchKernelGGL((gemv_down_nvfp4_kernel<CH, NCH, ST>), dim3(grid), dim3(kThreads), lds, st, a);
}

// Unrolled kernels for 2-segment chunks (inter a multiple of 512 up to 4096)
// per pass size; every other shape runs the looped kernel.
template <int ST>
bool down_launch_unrolled(const DownArgs &a, int nch, int grid, hipStream_t st)
{
    switch (nch) {
    case 1: down_launch<2, 1, ST>(a, grid, st); return true;
    case 2: down_launch<2, 2, ST>(a, grid, st); return true;
    case 3: down_launch<2, 3, ST>(a, grid, st); return true;
    case 4: down_launch<2, 4, ST>(a, grid, st); return true;
    case 5: down_launch<2, 5, ST>(a, grid, st); return true;
    case 6: down_launch<2, 6, ST>(a, grid, st); return true;
    case 7: down_launch<2, 7, ST>(a, grid, st); return true;
    case 8: down_launch<2, 8, ST>(a, grid, st); return true;
    default: return false;
    }
}

template <int NCH>
void down_rg_launch(const DownArgs &a, int grid, hipStream_t st)
{
    constexpr int RG = 2;
    const size_t lds = (size_t)a.st * a.I * 4 + 4 * 8 * RG * (size_t)(a.I / 16 + 16);
    hipLaunchKernelGGL((gemv_down_rg_nvfp4_kernel<1, 2 * NCH, 4, RG>), dim3(grid), dim3(kThreads), lds,
                       st, a);
}

template <int CH, int NCH, int RG>
void down1_launch(const Down1Args &a, hipStream_t st)
{
    constexpr int I = NCH * CH * 256, ROWS = 8 * RG;
    constexpr size_t lds = 8 * ((size_t)I * 4 + ROWS * (I / 16 + 16)) + 8 * ROWS * 4 + 64;
    hipLaunchKernelGGL((gemv_down1_nvfp4_kernel<CH, NCH, RG>), dim3(a.H / ROWS), dim3(512), lds, st,
                       a);
}

// (the 24-row blocks stream 1-segment chunks: 10.7 against 11.2 us with 2
// at 6144 x 1536)
template <int NCH>
void down1_launch_rg(const Down1Args &a, int rg, hipStream_t st)
{
    if (rg == 3) down1_launch<1, 2 * NCH, 3>(a, st);
    else down1_launch<2, NCH, 2>(a, st);
}

}  // namespace

hipError_t launch_gemv_gateup_nvfp4(const GemvBankDev &gate, const GemvBankDev &up,
                                    const uint16_t *x, const MoeRouteDev &r, int32_t M, int32_t S,
                                    int32_t E, int32_t hidden, int32_t inter, float limit, float *h,
                                    hipStream_t st, const int32_t *route_ids, int32_t top_k)
{
    GateUpArgs a{};
    // whole x rows of as many slots as fit the tile; the chunk-staged form
    // takes up to kGUXW slots of an expert in one pass where it is built
    a.st = gemv_gateup_pass_slots(M, hidden, kGUST);
    if (a.st < (M < kGUXW ? M : kGUXW) && hidden == 6144) a.st = M < kGUXW ? M : kGUXW;
    a.gcodes = gate.codes; a.ucodes = up.codes;
    a.gscales = (const uint8_t *)gate.scales; a.uscales = (const uint8_t *)up.scales;
    a.gscale2 = gate.scale2; a.uscale2 = up.scale2;
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

hipError_t launch_gemv_down_nvfp4(const GemvBankDev &down, const float *h, const MoeRouteDev &r,
                                  int32_t M, int32_t S, int32_t E, int32_t hidden, int32_t inter,
                                  float *y, hipStream_t st)
{
    DownArgs a;
    a.st = gemv_down_pass_slots(M, inter, kDNST);
    a.codes = down.codes; a.scales = (const uint8_t *)down.scales; a.scale2 = down.scale2;
    a.h = h; a.offsets = r.offsets; a.active = r.active; a.y = y;
    a.H = hidden; a.I = inter;
    if (M >= 3 && a.st < 4 && inter % 512 == 0 && inter <= 4096 && hidden % 64 == 0) {
        // four slots a pass, two row groups per wave (64-row tiles)
        a.st = M < 4 ? M : 4;
        a.ntiles = hidden / 64;
        const int grid = (S < E ? S : E) * a.ntiles;
        switch (inter / 512) {
        case 1: down_rg_launch<1>(a, grid, st); break;
        case 2: down_rg_launch<2>(a, grid, st); break;
        case 3: down_rg_launch<3>(a, grid, st); break;
        case 4: down_rg_launch<4>(a, grid, st); break;
        case 5: down_rg_launch<5>(a, grid, st); break;
        case 6: down_rg_launch<6>(a, grid, st); break;
        case 7: down_rg_launch<7>(a, grid, st); break;
        default: down_rg_launch<8>(a, grid, st); break;
        }
        return hipGetLastError();
    }
    a.ntiles = hidden / 32;
    const int grid = (S < E ? S : E) * a.ntiles;
    const int ch = gemv_down_chunk_segs(kFmtNVFP4, inter), nch = inter / kSegK / ch;
    bool done = false;
    if (ch == 2) {
        if (a.st <= 1) done = down_launch_unrolled<1>(a, nch, grid, st);
        else if (a.st <= 2) done = down_launch_unrolled<2>(a, nch, grid, st);
        else done = down_launch_unrolled<kDNST>(a, nch, grid, st);
    }
    if (!done) {
        if (ch == 2) down_launch<2, 0, kDNST>(a, grid, st);
        else down_launch<1, 0, kDNST>(a, grid, st);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_down1_nvfp4(const GemvBankDev &down, const float *h, const int32_t *ids,
                                   const int32_t *t2p, const float *w, int32_t k, int32_t hidden,
                                   int32_t inter, float *y, float *out, hipStream_t st)
{
    if (!gemv_down1_fits(kFmtNVFP4, 1, k, hidden, inter)) return hipErrorInvalidValue;
    Down1Args a;
    a.codes = down.codes; a.scales = (const uint8_t *)down.scales; a.scale2 = down.scale2;
    a.h = h; a.ids = ids; a.t2p = t2p; a.w = w; a.y = y; a.out = out;
    a.H = hidden; a.k = k;
    // A block owns 8 x RG output rows for every slot and the grid is a single
    // round, so the busiest CU holds ceil(blocks / CUs) x RG row groups per
    // slot.  Three row groups per wave where that is fewer than with two: at
    // 6144 rows, 256 blocks of 24 rows (one per CU) instead of 384 blocks of
    // 16 (two on half of the CUs, one on the rest).
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    auto busiest = [&](int rg) { return (hidden / (8 * rg) + cus - 1) / cus * rg; };
    const int rg = hidden % 24 == 0 && busiest(3) < busiest(2) ? 3 : 2;
    switch (inter / 512) {
    case 1: down1_launch_rg<1>(a, rg, st); break;
    case 2: down1_launch_rg<2>(a, rg, st); break;
    case 3: down1_launch_rg<3>(a, rg, st); break;
    default: down1_launch_rg<4>(a, rg, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_fused_decode_nvfp4(const GemvBankDev &gate, const GemvBankDev &up,
                                     const GemvBankDev &down, const uint16_t *x, const int32_t *ids,
                                     const float *w, int32_t M, int32_t k, int32_t E, int32_t hidden,
                                     int32_t inter, float limit, const MoeRouteDev &r, float *h,
                                     float *y, float *out, void *flags, uint32_t epoch,
                                     hipStream_t st)
{
    if (M != 1 || hidden % 2048 != 0 || hidden > 16384) return hipErrorInvalidValue;
    FusedArgs a{};
    a.gu.gcodes = gate.codes; a.gu.ucodes = up.codes;
    a.gu.gscales = (const uint8_t *)gate.scales; a.gu.uscales = (const uint8_t *)up.scales;
    a.gu.gscale2 = gate.scale2; a.gu.uscale2 = up.scale2;
    a.gu.x = x; a.gu.h = h; a.gu.H = hidden; a.gu.I = inter; a.gu.limit = limit; a.gu.st = 1;
    a.dn.codes = down.codes; a.dn.scales = (const uint8_t *)down.scales; a.dn.scale2 = down.scale2;
    a.dn.h = h; a.dn.y = y; a.dn.H = hidden; a.dn.I = inter; a.dn.st = 1;
    a.ids = ids; a.w = w; a.M = M; a.k = k; a.E = E; a.epoch = epoch;
    a.A = k < E ? k : E;
    a.flag_gu = (uint32_t *)flags;
    a.flag_dn = a.flag_gu + (size_t)a.A * (inter / 2);
    a.out = out; a.r = r;
    const size_t xl = (size_t)hidden * 2, hl = (size_t)inter * 4;
    const size_t lds = xl > hl ? xl : hl;
    switch (hidden / 2048) {
    case 1: return fused1_nv_dispatch<1>(a, lds, st);
    case 2: return fused1_nv_dispatch<2>(a, lds, st);
    case 3: return fused1_nv_dispatch<3>(a, lds, st);
    case 4: return fused1_nv_dispatch<4>(a, lds, st);
    case 5: return fused1_nv_dispatch<5>(a, lds, st);
    case 6: return fused1_nv_dispatch<6>(a, lds, st);
    case 7: return fused1_nv_dispatch<7>(a, lds, st);
    default: return fused1_nv_dispatch<8>(a, lds, st);
    }
}
