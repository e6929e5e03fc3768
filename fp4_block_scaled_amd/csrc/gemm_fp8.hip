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
// Tiles: 4 waves as 2x2, 64x64 (x2 for gate/up) per wave; A and B move from
// global memory straight into a ring of swizzled LDS stages (see below).
#include "gemm_common.h"

namespace {

using moe::f32x4;
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BM = 128;       // packed rows per tile
constexpr int BK = 128;       // K per step = one scale block = one MFMA

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
                                                          int4 *__restrict__ tiles,
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
        for (int m = 0; m < nt && first + m < tmax; ++m) tiles[first + m] = make_int4(e, p0 + m * BM, first, nt);
    }
    if (tid == 1023) *ntiles = min(base + inc, tmax);
}

// ---------------------------------------------------------------------------
// shared pieces of the two GEMMs
// ---------------------------------------------------------------------------
// Block: 256 threads = 4 waves as 2 (rows) x 2 (columns).  Tiles move from
// global memory straight into LDS (global_load_lds_dwordx4: lane i of one
// instruction fills bytes 16i..16i+15 of a 1 KB run = 8 rows x 128 bytes),
// in a ring of LDS stages (three for gate/up: two K steps in flight; two for
// down, whose two blocks per CU cover each other's waits), holding no VGPRs.  Inside a stage a row's eight 16-byte chunks are stored
// XOR-swizzled (swz below), so the lanes that feed one MFMA operand half (16
// rows, same K chunk) read without bank conflicts.  Each wave
// loads the activation scales of its own 64 rows into its own 256-byte slot.
// Every wave issues the same number of DMA instructions per stage, so an
// immediate vmcnt wait tells a wave its share of a stage has landed; one
// barrier per K step publishes the stage to all waves and retires the stage
// that the next DMA overwrites.
struct GemmArgs {
    const uint8_t *a;          // gate/up: xq [M][K]; down: hq [S][K]
    const float *as;           // activation scales [rows][K/128]
    const int32_t *sorted_token;   // gate/up gathers A rows through it (null for down)
    const uint8_t *w0, *w1;    // gate and up codes (down: w0 only), [E][N][K]
    const float *ws0, *ws1;    // their block scales [E][N/128][K/128]
    const int32_t *offsets;
    const int4 *tiles;         // (expert, first packed row, expert's first tile, its tile count)
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

// 32-byte MFMA operand of lane `lane` for tile row `row` (K chunks 2q, 2q+1, q = lane/16)
// (one byte offset per 16-byte read, so every LDS access stays a direct
// offset of its stage array and the compiler can tell the stages apart when
// it places waits for the DMA)
__device__ __forceinline__ i32x8 lds_op(const uint8_t *tile, int row, int lane)
{
    const int c = (lane >> 4) * 2;
    const i32x4 lo = *reinterpret_cast<const i32x4 *>(tile + (row * 128 + swz(row, c) * 16));
    const i32x4 hi = *reinterpret_cast<const i32x4 *>(tile + (row * 128 + swz(row, c + 1) * 16));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
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
// 512 threads = 8 waves as 4 (32 rows each) x 2 (64 h columns each, gate and
// up both), two waves per SIMD.
// Stage: A [128 rows][128 B] | B [256 rows][128 B] (0-127 gate, 128-255 up) | S [8 waves][64] f32
constexpr int kGuThreads = 512;
constexpr int GU_A = 0, GU_B = 128 * 128, GU_S = GU_B + 256 * 128, GU_STAGE = GU_S + 8 * 256;
constexpr int GU_DMA = 2 + 4 + 1;   // DMA instructions per wave per stage

constexpr int GU_NST = 3;           // LDS stages of the gate/up GEMM (2 K steps in flight)
static_assert(GU_NST * GU_STAGE <= 160 * 1024, "gate/up stages exceed LDS");

__global__ __launch_bounds__(kGuThreads, 1) void gemm_gateup_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t sm[GU_NST * GU_STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int wm = wave & 3, wn = wave >> 2;
    int4 tile;
    int nb;
    if (!gemm_item(a, tile, nb)) return;
    const int e = tile.x, p0 = tile.y;
    const int rows = moe::uniform(min(BM, a.offsets[e + 1] - p0));
    const int K = a.K, N = a.N, KB = K / BK;
    const int n0 = nb * 128;

    // per-lane byte offsets of this wave's DMA runs (rows past the tile read
    // the tile's first row and are never stored)
    uint32_t aoff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = (wave * 2 + j) * 8 + (lane >> 3);
        const int tok = a.sorted_token[p0 + (r < rows ? r : 0)];
        aoff[j] = (uint32_t)tok * K + swz(r, lane & 7) * 16;
    }
    const uint8_t *wbase = (wave < 4 ? a.w0 : a.w1) + ((size_t)e * N + n0) * K;
    uint32_t boff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int rb = (wave * 4 + j) * 8 + (lane >> 3);   // 0..255
        boff[j] = (uint32_t)(rb & 127) * K + swz(rb, lane & 7) * 16;
    }
    const int srow = wm * 32 + (lane & 31);             // both half-waves load the same 32 rows
    const uint32_t soff = (uint32_t)a.sorted_token[p0 + (srow < rows ? srow : 0)] * KB * 4;
    // weight block scales of this column block, K block j in lane j % 64 of
    // register j / 64 (K <= 16384); a uniform readlane picks one per K step
    const float *sw0 = a.ws0 + ((size_t)e * (N / 128) + nb) * KB;
    const float *sw1 = a.ws1 + ((size_t)e * (N / 128) + nb) * KB;
    const float g_lo = lane < KB ? sw0[lane] : 0.0f, g_hi = lane + 64 < KB ? sw0[lane + 64] : 0.0f;
    const float u_lo = lane < KB ? sw1[lane] : 0.0f, u_hi = lane + 64 < KB ? sw1[lane + 64] : 0.0f;

    auto issue = [&](int kb, uint8_t *st) {
        const uint8_t *ab = a.a + (size_t)kb * BK, *bb = wbase + (size_t)kb * BK;
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(ab, aoff[j], lds_addr(st + GU_A + (wave * 2 + j) * 1024));
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(bb, boff[j], lds_addr(st + GU_B + (wave * 4 + j) * 1024));
        dma4(a.as + kb, soff, lds_addr(st + GU_S + wave * 256));
    };

    f32x4 accg[2][4], accu[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) { accg[i][j] = f32x4{0.f, 0.f, 0.f, 0.f}; accu[i][j] = accg[i][j]; }

    auto compute = [&](const uint8_t *st, int kb) {
        const float swg = kb < 64 ? lane_f(g_lo, kb) : lane_f(g_hi, kb - 64);
        const float swu = kb < 64 ? lane_f(u_lo, kb) : lane_f(u_hi, kb - 64);
        const float *sa = reinterpret_cast<const float *>(st + GU_S) + wave * 64;
        i32x8 av[2];
        f32x4 fg[2], fu[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            av[mt] = lds_op(st + GU_A, wm * 32 + mt * 16 + (lane & 15), lane);
            const f32x4 fa = *reinterpret_cast<const f32x4 *>(sa + mt * 16 + (lane >> 4) * 4);
            fg[mt] = fa * swg;
            fu[mt] = fa * swu;
        }
        // per column group: four independent products, then their scaled
        // accumulation (the block scales change every K step)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const i32x8 bg = lds_op(st + GU_B, wn * 64 + nt * 16 + (lane & 15), lane);
            const i32x8 bu = lds_op(st + GU_B, 128 + wn * 64 + nt * 16 + (lane & 15), lane);
            f32x4 pg[2], pu[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                pg[mt] = mfma_fp8(av[mt], bg);
                pu[mt] = mfma_fp8(av[mt], bu);
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    accg[mt][nt][i] = fmaf(pg[mt][i], fg[mt][i], accg[mt][nt][i]);
                    accu[mt][nt][i] = fmaf(pu[mt][i], fu[mt][i], accu[mt][nt][i]);
                }
        }
    };

    k_loop<GU_NST, GU_DMA>(KB, sm, GU_STAGE, issue, compute);
    __syncthreads();

    // epilogue: h = SwiGLU(g, u); per-row amax over the block's 128 columns
    float h[2][4][4];
    float rmax[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = 0.0f;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                h[mt][nt][i] = swiglu_clamp(accg[mt][nt][i], accu[mt][nt][i], a.limit);
                m = fmaxf(m, fabsf(h[mt][nt][i]));
            }
#pragma unroll
            for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
            rmax[mt][i] = m;
        }
    float *xm = reinterpret_cast<float *>(sm);     // [2 column halves][128 rows]
    if ((lane & 15) == 0) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) xm[wn * 128 + wm * 32 + mt * 16 + (lane >> 4) * 4 + i] = rmax[mt][i];
    }
    __syncthreads();
    uint8_t *ct = sm + GU_STAGE;                   // codes tile [128][144]
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 32 + mt * 16 + (lane >> 4) * 4 + i;
            const float amax = fmaxf(xm[r], xm[128 + r]);
            const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const uint32_t code = e4m3_pair(h[mt][nt][i] / scale, 0.0f) & 0xFFu;
                ct[r * 144 + wn * 64 + nt * 16 + (lane & 15)] = (uint8_t)code;
            }
            if (wn == 0 && (lane & 15) == 0 && r < rows) a.hs[(size_t)(p0 + r) * a.ntn + nb] = scale;
        }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = tid + kGuThreads * j, r = c >> 3, part = c & 7;
        if (r < rows)
            *reinterpret_cast<uint4 *>(a.hq + (size_t)(p0 + r) * N + n0 + part * 16) =
                *reinterpret_cast<const uint4 *>(ct + r * 144 + part * 16);
    }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------
// Stage: A [128][128 B] | B [128][128 B] | S [4 waves][64] f32
constexpr int DN_A = 0, DN_B = 128 * 128, DN_S = DN_B + 128 * 128, DN_STAGE = DN_S + 4 * 256;
constexpr int DN_DMA = 4 + 4 + 1;

// LDS stages of the down GEMM: two (one K step in flight) in 66 KB, so two
// blocks share a CU.  A down block runs only K/128 = 16 K steps; with one
// block per CU the ramp of every block's first stages stood exposed, with two
// one block's ramp runs under the other's MFMAs (1.61 -> 1.11 ms at M=4096).
constexpr int DN_NST = 2;
static_assert(2 * DN_NST * DN_STAGE <= 160 * 1024, "two down blocks exceed LDS");

__global__ __launch_bounds__(kThreads, 2) void gemm_down_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t sm[DN_NST * DN_STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    int4 tile;
    int nb;
    if (!gemm_item(a, tile, nb)) return;
    const int e = tile.x, p0 = tile.y;
    const int rows = moe::uniform(min(BM, a.offsets[e + 1] - p0));
    const int K = a.K, N = a.N, KB = K / BK;
    const int n0 = nb * 128;

    uint32_t aoff[4], boff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (wave * 4 + j) * 8 + (lane >> 3);
        aoff[j] = (uint32_t)(p0 + (r < rows ? r : 0)) * K + swz(r, lane & 7) * 16;
        boff[j] = (uint32_t)r * K + swz(r, lane & 7) * 16;
    }
    const uint8_t *wbase = a.w0 + ((size_t)e * N + n0) * K;
    const int srow = wm * 64 + lane;
    const uint32_t soff = (uint32_t)(p0 + (srow < rows ? srow : 0)) * KB * 4;
    const float *sw0 = a.ws0 + ((size_t)e * (N / 128) + nb) * KB;
    const float w_lo = lane < KB ? sw0[lane] : 0.0f, w_hi = lane + 64 < KB ? sw0[lane + 64] : 0.0f;

    auto issue = [&](int kb, uint8_t *st) {
        const uint8_t *ab = a.a + (size_t)kb * BK, *bb = wbase + (size_t)kb * BK;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(ab, aoff[j], lds_addr(st + DN_A + (wave * 4 + j) * 1024));
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(bb, boff[j], lds_addr(st + DN_B + (wave * 4 + j) * 1024));
        dma4(a.as + kb, soff, lds_addr(st + DN_S + wave * 256));
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const uint8_t *st, int kb) {
        const float sw = kb < 64 ? lane_f(w_lo, kb) : lane_f(w_hi, kb - 64);
        const float *sa = reinterpret_cast<const float *>(st + DN_S) + wave * 64;
        i32x8 av[4];
        f32x4 fa[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            av[mt] = lds_op(st + DN_A, wm * 64 + mt * 16 + (lane & 15), lane);
            fa[mt] = *reinterpret_cast<const f32x4 *>(sa + mt * 16 + (lane >> 4) * 4) * sw;
        }
        f32x4 p[4][4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const i32x8 bv = lds_op(st + DN_B, wn * 64 + nt * 16 + (lane & 15), lane);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) p[mt][nt] = mfma_fp8(av[mt], bv);
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mt][nt][i] = fmaf(p[mt][nt][i], fa[mt][i], acc[mt][nt][i]);
    };

    k_loop<DN_NST, DN_DMA>(KB, sm, DN_STAGE, issue, compute);

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

hipError_t launch_gemm_tiles(const int32_t *offsets, int32_t E, int32_t tmax, int4 *tiles,
                             int32_t *ntiles, hipStream_t st)
{
    hipLaunchKernelGGL(gemm_tiles_kernel, dim3(1), dim3(1024), 0, st, offsets, E, tmax, tiles,
                       ntiles);
    return hipGetLastError();
}

hipError_t launch_gemm_gateup(const uint8_t *xq, const float *xs, const int32_t *sorted_token,
                              const uint8_t *gcodes, const float *gscales, const uint8_t *ucodes,
                              const float *uscales, const int32_t *offsets, const int4 *tiles,
                              const int32_t *ntiles, int32_t tmax, int32_t hidden, int32_t inter,
                              float limit, uint8_t *hq, float *hs, hipStream_t st)
{
    GemmArgs a{};
    a.a = xq; a.as = xs; a.sorted_token = sorted_token;
    a.w0 = gcodes; a.w1 = ucodes; a.ws0 = gscales; a.ws1 = uscales;
    a.offsets = offsets; a.tiles = tiles; a.ntiles = ntiles;
    a.hq = hq; a.hs = hs; a.K = hidden; a.N = inter; a.ntn = inter / 128; a.limit = limit;
    hipLaunchKernelGGL(gemm_gateup_kernel, dim3((unsigned)(tmax * a.ntn)), dim3(kGuThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gemm_down(const uint8_t *hq, const float *hs, const uint8_t *dcodes,
                            const float *dscales, const int32_t *offsets, const int4 *tiles,
                            const int32_t *ntiles, int32_t tmax, int32_t hidden, int32_t inter,
                            float *y, hipStream_t st)
{
    GemmArgs a{};
    a.a = hq; a.as = hs; a.w0 = dcodes; a.ws0 = dscales;
    a.offsets = offsets; a.tiles = tiles; a.ntiles = ntiles;
    a.y = y; a.K = inter; a.N = hidden; a.ntn = hidden / 128;
    hipLaunchKernelGGL(gemm_down_kernel, dim3((unsigned)(tmax * a.ntn)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}
