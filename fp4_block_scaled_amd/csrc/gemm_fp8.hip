// gemm_fp8.hip -- grouped FP8 MFMA GEMM tier for wide M (prefill).
//
// With thousands of tokens every expert holds many rows, so the projections
// become dense contractions per expert ("spark_model glm5next_mlp/forward.rs",
// grouped-prefill arm of fn forward_moe: sort slots by expert, then one
// grouped GEMM per projection, worth it above 64-128 rows).  Activations enter
// the matrix cores as E4M3 with one FP32 scale per 1x128 group, like the
// xq/xs and hq/hs buffers of "memra-engine src/dsv4_ep.rs" (EpScratch and
// the act_quant_fp8 step of fn chain).
//
// Kernels:
//   quant_act_kernel    x bf16 -> E4M3 codes + FP32 scale per 1x128 group
//                       (scale = amax/448, code = RNE(x/scale) saturated).
//   gemm_tiles_kernel   per-expert 128-row tiles over the expert-sorted rows,
//                       built on the device from expert_offsets.
//   gemm_gateup_kernel  one block = 128 packed rows x 128 h-columns: it runs
//                       the gate AND the up projection for those columns on
//                       v_mfma_f32_16x16x128_f8f6f4 (one MFMA = one 128-wide
//                       K block, so each product is promoted into the FP32
//                       accumulator with its activation scale x weight block
//                       scale), then applies the clamped SwiGLU and quantizes
//                       the 128-wide h row segment (exactly one 1x128 group)
//                       to E4M3 + scale in the epilogue.
//   gemm_down_kernel    one block = 128 packed rows x 128 outputs of y.
// Tiles: 4 waves as 2x2, 64x64 (x2 for gate/up) per wave; A and B staged
// through LDS with a 16-byte row pad (conflict-free operand reads), two LDS
// stages and a two-deep register prefetch of the global tiles.
#include "moe_internal.h"

namespace {

using moe::f32x4;
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BM = 128;       // packed rows per tile
constexpr int BK = 128;       // K per step = one scale block = one MFMA
constexpr int PITCH = 144;    // LDS row pitch in bytes (128 + 16 pad)

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

__device__ __forceinline__ float max8_lanes(float v)
{
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
    return v;
}

// E4M3 (OCP, RNE) of v, saturated to +-448 first so the convert never sees an
// out-of-range input.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b)
{
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// ---------------------------------------------------------------------------
// activation quantization: 8 lanes per 128-wide group, 16 values per lane
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t *__restrict__ x,
                                                        int64_t n16, uint8_t *__restrict__ q,
                                                        float *__restrict__ s)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 16-value chunk
    const bool ok = i < n16;
    uint4 u0 = make_uint4(0, 0, 0, 0), u1 = u0;
    if (ok) {
        u0 = reinterpret_cast<const uint4 *>(x)[2 * i];
        u1 = reinterpret_cast<const uint4 *>(x)[2 * i + 1];
    }
    const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float v[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
        v[2 * j + 1] = bf16_to_f32(w[j] >> 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = max8_lanes(amax);
    const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        c[j] = e4m3_pair(v[4 * j] / scale, v[4 * j + 1] / scale) |
               (e4m3_pair(v[4 * j + 2] / scale, v[4 * j + 3] / scale) << 16);
    if (ok) {
        reinterpret_cast<uint4 *>(q)[i] = make_uint4(c[0], c[1], c[2], c[3]);
        if ((threadIdx.x & 7) == 0) s[i >> 3] = scale;
    }
}

// ---------------------------------------------------------------------------
// tile schedule: tiles[t] = (expert, first packed row), t < *ntiles
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void gemm_tiles_kernel(const int32_t *__restrict__ offsets,
                                                          int32_t E, int32_t tmax,
                                                          int2 *__restrict__ tiles,
                                                          int32_t *__restrict__ ntiles)
{
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = tid;
    const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
    const int nt = (cnt + BM - 1) / BM;
    int inc = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    const int first = base + inc - nt;
    if (e < E) {
        const int p0 = offsets[e];
        for (int m = 0; m < nt && first + m < tmax; ++m) tiles[first + m] = make_int2(e, p0 + m * BM);
    }
    if (tid == 1023) *ntiles = min(base + inc, tmax);
}

// ---------------------------------------------------------------------------
// shared pieces of the two GEMMs
// ---------------------------------------------------------------------------
struct GemmArgs {
    const uint8_t *a;          // gate/up: xq [M][K]; down: hq [S][K]
    const float *as;           // activation scales [rows][K/128]
    const int32_t *sorted_token;   // gate/up gathers A rows through it (null for down)
    const uint8_t *w0, *w1;    // gate and up codes (down: w0 only), [E][N][K]
    const float *ws0, *ws1;    // their block scales [E][N/128][K/128]
    const int32_t *offsets;
    const int2 *tiles;
    const int32_t *ntiles;
    uint8_t *hq;               // gate/up output codes [S][N]
    float *hs;                 // gate/up output scales [S][N/128]
    float *y;                  // down output [S][N]
    int32_t K, N, ntn;         // N: h columns (gate/up) or outputs (down); ntn = N/128
    float limit;
};

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8 &a, const i32x8 &b)
{
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 lds_op(const uint8_t *lds_tile, int row, int lane)
{
    const uint8_t *p = lds_tile + row * PITCH + (lane >> 4) * 32;
    const uint4 lo = *reinterpret_cast<const uint4 *>(p);
    const uint4 hi = *reinterpret_cast<const uint4 *>(p + 16);
    i32x8 r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

__device__ __forceinline__ uint4 ldg_nt(const uint8_t *p)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float swiglu_clamp(float g, float u, float L)
{
    const float gc = fminf(g, L);
    const float uc = fminf(fmaxf(u, -L), L);
    return gc / (1.0f + expf(-gc)) * uc;
}

// ---------------------------------------------------------------------------
// gate + up (+ SwiGLU + h quantization)
// ---------------------------------------------------------------------------
// 512 threads = 8 waves as 2 (rows) x 4 (columns); a wave owns 64 rows x 32
// h-columns of both the gate and the up product (64 FP32 accumulators per
// lane), so SwiGLU is elementwise in registers.
// LDS stage: A [128][PITCH] | B [256][PITCH] (rows 0-127 gate, 128-255 up) | as[128] floats
constexpr int GU_THREADS = 512;
constexpr int GU_A = 0, GU_B = BM * PITCH, GU_S = GU_B + 256 * PITCH, GU_STAGE = GU_S + BM * 4;

__global__ __launch_bounds__(GU_THREADS, 1) void gemm_gateup_kernel(GemmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int t = blockIdx.x / a.ntn, nb = blockIdx.x - t * a.ntn;
    if (t >= *a.ntiles) return;
    const int2 tile = a.tiles[t];
    const int e = tile.x, p0 = tile.y;
    const int rows = min(BM, a.offsets[e + 1] - p0);
    const int K = a.K, N = a.N, KB = K / BK;
    const int n0 = nb * 128;

    // loaders: A 2 chunks, B 4 chunks (2 gate rows, 2 up rows) of 16 bytes per
    // thread and K step; 32-bit offsets from per-expert bases
    uint32_t aoff[2];
    bool aok[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = tid + GU_THREADS * j, r = c >> 3;
        aok[j] = r < rows;
        const int tok = aok[j] ? a.sorted_token[p0 + r] : 0;
        aoff[j] = (uint32_t)tok * K + (c & 7) * 16;
    }
    const uint8_t *gbase = a.w0 + (size_t)e * N * K;
    const uint8_t *ubase = a.w1 + (size_t)e * N * K;
    // B chunk j: rows (tid >> 3) + 64 * (j & 1) of gate (j < 2) or up (j >= 2)
    const uint32_t boff = (uint32_t)(n0 + (tid >> 3)) * K + (tid & 7) * 16;
    const uint32_t brow64 = (uint32_t)64 * K;
    uint32_t soff = 0;
    bool sok = false;
    if (tid < BM) {
        sok = tid < rows;
        soff = (uint32_t)(sok ? a.sorted_token[p0 + tid] : 0) * KB;
    }
    const float *sw0 = a.ws0 + ((size_t)e * (N / 128) + nb) * KB;
    const float *sw1 = a.ws1 + ((size_t)e * (N / 128) + nb) * KB;

    uint4 ra[2][2], rb[2][4];
    float rs[2];
    auto gload = [&](int buf, int kb) {
        const uint32_t ko = (uint32_t)kb * BK;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            ra[buf][j] = aok[j] ? *reinterpret_cast<const uint4 *>(a.a + aoff[j] + ko) : make_uint4(0, 0, 0, 0);
        rb[buf][0] = ldg_nt(gbase + boff + ko);
        rb[buf][1] = ldg_nt(gbase + boff + brow64 + ko);
        rb[buf][2] = ldg_nt(ubase + boff + ko);
        rb[buf][3] = ldg_nt(ubase + boff + brow64 + ko);
        rs[buf] = sok ? a.as[soff + kb] : 0.0f;
    };
    auto sstore = [&](int buf, int stage) {
        uint8_t *st = lds + stage * GU_STAGE;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = tid + GU_THREADS * j;
            *reinterpret_cast<uint4 *>(st + GU_A + (c >> 3) * PITCH + (c & 7) * 16) = ra[buf][j];
        }
        const int r = tid >> 3, part = (tid & 7) * 16;
        *reinterpret_cast<uint4 *>(st + GU_B + r * PITCH + part) = rb[buf][0];
        *reinterpret_cast<uint4 *>(st + GU_B + (r + 64) * PITCH + part) = rb[buf][1];
        *reinterpret_cast<uint4 *>(st + GU_B + (r + 128) * PITCH + part) = rb[buf][2];
        *reinterpret_cast<uint4 *>(st + GU_B + (r + 192) * PITCH + part) = rb[buf][3];
        if (tid < BM) reinterpret_cast<float *>(st + GU_S)[tid] = rs[buf];
    };

    f32x4 accg[4][2], accu[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) { accg[i][j] = f32x4{0.f, 0.f, 0.f, 0.f}; accu[i][j] = accg[i][j]; }

    auto compute = [&](int stage, int kb) {
        const uint8_t *st = lds + stage * GU_STAGE;
        const float swg = sw0[kb], swu = sw1[kb];
        i32x8 av[4];
        f32x4 fa[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            av[mt] = lds_op(st + GU_A, wm * 64 + mt * 16 + (lane & 15), lane);
            fa[mt] = *reinterpret_cast<const f32x4 *>(st + GU_S + (wm * 64 + mt * 16 + (lane >> 4) * 4) * 4);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const i32x8 bg = lds_op(st + GU_B, wn * 32 + nt * 16 + (lane & 15), lane);
            const i32x8 bu = lds_op(st + GU_B, 128 + wn * 32 + nt * 16 + (lane & 15), lane);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const f32x4 pg = mfma_fp8(av[mt], bg);
                const f32x4 pu = mfma_fp8(av[mt], bu);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    accg[mt][nt][i] = fmaf(pg[i], fa[mt][i] * swg, accg[mt][nt][i]);
                    accu[mt][nt][i] = fmaf(pu[i], fa[mt][i] * swu, accu[mt][nt][i]);
                }
            }
        }
    };

    // prologue: tiles 0 and 1 in flight, tile 0 staged
    gload(0, 0);
    if (KB > 1) gload(1, 1);
    sstore(0, 0);
    __syncthreads();
    for (int kb = 0; kb < KB; kb += 2) {
        // even step: compute stage 0, prefetch kb+2 into regs 0, stage kb+1 from regs 1
        if (kb + 2 < KB) gload(0, kb + 2);
        compute(0, kb);
        if (kb + 1 < KB) sstore(1, 1);
        __syncthreads();
        if (kb + 1 >= KB) break;
        if (kb + 3 < KB) gload(1, kb + 3);
        compute(1, kb + 1);
        if (kb + 2 < KB) sstore(0, 0);
        __syncthreads();
    }

    // epilogue: h = SwiGLU(g, u); per-row amax over the block's 128 columns
    float h[4][2][4];
    float rmax[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = 0.0f;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                h[mt][nt][i] = swiglu_clamp(accg[mt][nt][i], accu[mt][nt][i], a.limit);
                m = fmaxf(m, fabsf(h[mt][nt][i]));
            }
            // max over the 16 lanes holding this row's columns
#pragma unroll
            for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
            rmax[mt][i] = m;
        }
    // combine the four column quarters (wn = 0..3) through LDS
    float *xm = reinterpret_cast<float *>(lds);   // [4][128]
    if ((lane & 15) == 0) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) xm[wn * 128 + wm * 64 + mt * 16 + (lane >> 4) * 4 + i] = rmax[mt][i];
    }
    __syncthreads();
    uint8_t *ct = lds + 2048;                      // codes tile [128][PITCH]
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + mt * 16 + (lane >> 4) * 4 + i;
            const float amax = fmaxf(fmaxf(xm[r], xm[128 + r]), fmaxf(xm[256 + r], xm[384 + r]));
            const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const uint32_t code = e4m3_pair(h[mt][nt][i] / scale, 0.0f) & 0xFFu;
                ct[r * PITCH + wn * 32 + nt * 16 + (lane & 15)] = (uint8_t)code;
            }
            if (wn == 0 && (lane & 15) == 0 && r < rows) a.hs[(size_t)(p0 + r) * a.ntn + nb] = scale;
        }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = tid + GU_THREADS * j, r = c >> 3, part = c & 7;
        if (r < rows)
            *reinterpret_cast<uint4 *>(a.hq + (size_t)(p0 + r) * N + n0 + part * 16) =
                *reinterpret_cast<const uint4 *>(ct + r * PITCH + part * 16);
    }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------
constexpr int DN_A = 0, DN_B = BM * PITCH, DN_S = DN_B + 128 * PITCH, DN_STAGE = DN_S + BM * 4;

__global__ __launch_bounds__(kThreads, 1) void gemm_down_kernel(GemmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int t = blockIdx.x / a.ntn, nb = blockIdx.x - t * a.ntn;
    if (t >= *a.ntiles) return;
    const int2 tile = a.tiles[t];
    const int e = tile.x, p0 = tile.y;
    const int rows = min(BM, a.offsets[e + 1] - p0);
    const int K = a.K, N = a.N, KB = K / BK;
    const int n0 = nb * 128;

    const uint8_t *asrc[4];
    bool aok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = tid + 256 * j, r = c >> 3;
        aok[j] = r < rows;
        asrc[j] = a.a + (size_t)(p0 + (aok[j] ? r : 0)) * K + (c & 7) * 16;
    }
    const uint8_t *bsrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = tid + 256 * j, r = c >> 3;
        bsrc[j] = a.w0 + ((size_t)e * N + n0 + r) * K + (c & 7) * 16;
    }
    const float *ssrc = a.as + (size_t)(p0 + (tid < rows ? tid : 0)) * KB;
    const float *sw0 = a.ws0 + ((size_t)e * (N / 128) + nb) * KB;

    uint4 ra[2][4], rb[2][4];
    float rs[2];
    auto gload = [&](int buf, int kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) ra[buf][j] = aok[j] ? *reinterpret_cast<const uint4 *>(asrc[j] + kb * BK) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) rb[buf][j] = ldg_nt(bsrc[j] + kb * BK);
        rs[buf] = (tid < BM && tid < rows) ? ssrc[kb] : 0.0f;
    };
    auto sstore = [&](int buf, int stage) {
        uint8_t *st = lds + stage * DN_STAGE;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = tid + 256 * j;
            *reinterpret_cast<uint4 *>(st + DN_A + (c >> 3) * PITCH + (c & 7) * 16) = ra[buf][j];
            *reinterpret_cast<uint4 *>(st + DN_B + (c >> 3) * PITCH + (c & 7) * 16) = rb[buf][j];
        }
        if (tid < BM) reinterpret_cast<float *>(st + DN_S)[tid] = rs[buf];
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int stage, int kb) {
        const uint8_t *st = lds + stage * DN_STAGE;
        const float sw = sw0[kb];
        i32x8 av[4];
        f32x4 fa[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            av[mt] = lds_op(st + DN_A, wm * 64 + mt * 16 + (lane & 15), lane);
            fa[mt] = *reinterpret_cast<const f32x4 *>(st + DN_S + (wm * 64 + mt * 16 + (lane >> 4) * 4) * 4);
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const i32x8 bv = lds_op(st + DN_B, wn * 64 + nt * 16 + (lane & 15), lane);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const f32x4 p = mfma_fp8(av[mt], bv);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mt][nt][i] = fmaf(p[i], fa[mt][i] * sw, acc[mt][nt][i]);
            }
        }
    };

    gload(0, 0);
    if (KB > 1) gload(1, 1);
    sstore(0, 0);
    __syncthreads();
    for (int kb = 0; kb < KB; kb += 2) {
        if (kb + 2 < KB) gload(0, kb + 2);
        compute(0, kb);
        if (kb + 1 < KB) sstore(1, 1);
        __syncthreads();
        if (kb + 1 >= KB) break;
        if (kb + 3 < KB) gload(1, kb + 3);
        compute(1, kb + 1);
        if (kb + 2 < KB) sstore(0, 0);
        __syncthreads();
    }

#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + mt * 16 + (lane >> 4) * 4 + i;
            if (r < rows) {
                float *yr = a.y + (size_t)(p0 + r) * N + n0 + wn * 64 + (lane & 15);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) yr[nt * 16] = acc[mt][nt][i];
            }
        }
}

}  // namespace

int gemm_max_tiles(int32_t S, int32_t E) { return (S < E ? S : E) + (S + BM - 1) / BM; }

hipError_t launch_quant_act(const uint16_t *x, int32_t M, int32_t hidden, uint8_t *xq, float *xs,
                            hipStream_t st)
{
    const int64_t n16 = (int64_t)M * hidden / 16;
    hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st, x,
                       n16, xq, xs);
    return hipGetLastError();
}

hipError_t launch_gemm_tiles(const int32_t *offsets, int32_t E, int32_t tmax, int2 *tiles,
                             int32_t *ntiles, hipStream_t st)
{
    hipLaunchKernelGGL(gemm_tiles_kernel, dim3(1), dim3(1024), 0, st, offsets, E, tmax, tiles,
                       ntiles);
    return hipGetLastError();
}

hipError_t launch_gemm_gateup(const uint8_t *xq, const float *xs, const int32_t *sorted_token,
                              const uint8_t *gcodes, const float *gscales, const uint8_t *ucodes,
                              const float *uscales, const int32_t *offsets, const int2 *tiles,
                              const int32_t *ntiles, int32_t tmax, int32_t hidden, int32_t inter,
                              float limit, uint8_t *hq, float *hs, hipStream_t st)
{
    GemmArgs a{};
    a.a = xq; a.as = xs; a.sorted_token = sorted_token;
    a.w0 = gcodes; a.w1 = ucodes; a.ws0 = gscales; a.ws1 = uscales;
    a.offsets = offsets; a.tiles = tiles; a.ntiles = ntiles;
    a.hq = hq; a.hs = hs; a.K = hidden; a.N = inter; a.ntn = inter / 128; a.limit = limit;
    const size_t lds = 2 * GU_STAGE;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_gateup_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL(gemm_gateup_kernel, dim3((unsigned)(tmax * a.ntn)), dim3(GU_THREADS), lds, st,
                       a);
    return hipGetLastError();
}

hipError_t launch_gemm_down(const uint8_t *hq, const float *hs, const uint8_t *dcodes,
                            const float *dscales, const int32_t *offsets, const int2 *tiles,
                            const int32_t *ntiles, int32_t tmax, int32_t hidden, int32_t inter,
                            float *y, hipStream_t st)
{
    GemmArgs a{};
    a.a = hq; a.as = hs; a.w0 = dcodes; a.ws0 = dscales;
    a.offsets = offsets; a.tiles = tiles; a.ntiles = ntiles;
    a.y = y; a.K = inter; a.N = hidden; a.ntn = hidden / 128;
    const size_t lds = 2 * DN_STAGE;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_down_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL(gemm_down_kernel, dim3((unsigned)(tmax * a.ntn)), dim3(kThreads), lds, st, a);
    return hipGetLastError();
}
