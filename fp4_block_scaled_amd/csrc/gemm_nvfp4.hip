// gemm_nvfp4.hip -- grouped bf16 MFMA GEMM tier for NVFP4 banks at wide M.
//
// With thousands of tokens every expert holds many rows and the projections
// become dense contractions per expert, as in the FP8 tier ("spark_model
// glm5next_mlp/forward.rs", grouped-prefill arm of fn forward_moe).  NVFP4
// experts keep the pages' W4A16 form (fn w4a16_gemv and its batched variant:
// 4-bit weights, bf16 activations), so x enters the matrix cores as the bf16
// it is, with no activation quantization.
//
// Exact weights in bf16: an NVFP4 weight is e2m1 x (E4M3 group scale) x
// scale_2.  An E2M1 value has at most 2 significant bits and an E4M3 scale at
// most 4, so their product has at most 6 and is a bf16 value exactly (the
// exponents stay far inside bf16's range).  The kernels decode the codes and
// group scales of each MFMA operand to bf16 in registers right before the
// MFMA and multiply the FP32 sums by scale_2 at the end: every product is
// exact and only the order of the FP32 sums differs from the definition.
//
// h between the projections: the gate/up epilogue computes h = SwiGLU(g, u)
// in FP32 and stores it as two bf16 arrays, hi = bf16(h) and lo = bf16(h -
// hi), so that hi + lo carries h to about 2^-16 relative; the down GEMM runs
// the MFMA on both (y = W hi + W lo), keeping the FP32 h of the GEMV tier.
//
// Kernels (tiles from gemm_tiles_kernel: 128 expert-sorted rows each):
//   gemm_gateup_nvfp4_kernel  one block = 128 rows x 64 h columns: 64 gate and
//                             64 up weight rows per K step, SwiGLU, hi/lo h.
//   gemm_down_nvfp4_kernel    one block = 128 rows x 128 outputs of y.
// Block: 256 threads = 4 waves as 2 (64 rows each) x 2 (column halves).  Per
// K step of 64: the A rows (128 bytes of bf16 each) move from global memory
// straight into swizzled LDS, with the B codes (32 bytes per weight row) and
// group scales (4 bytes per row) beside them, four stages deep.  Each wave
// decodes its own B operands from LDS: lane l of a 16x16x32 MFMA operand
// needs 8 consecutive K values of one weight row, i.e. one code dword and one
// group scale.
#include "gemm_common.h"

namespace {

using moe::f32x2;
using moe::f32x4;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int TM = 128;      // rows per tile
constexpr int KS = 64;       // K per step (128 bytes of a bf16 row)

struct NvGemmArgs {
    const uint16_t *a;            // gate/up: x [M][K]; down: h hi [S][K]
    const uint16_t *a2;           // down: h lo [S][K]
    const int32_t *sorted_token;  // gate/up gathers A rows through it
    const uint8_t *c0, *c1;       // gate and up codes (down: c0), [E][N][K/2]
    const uint8_t *s0, *s1;       // their group scales [E][N][K/16]
    const float *g0, *g1;         // their scale_2 [E]
    const int32_t *offsets;
    const int4 *tiles;
    const int32_t *ntiles;
    uint16_t *hhi, *hlo;          // gate/up output [S][N]
    float *y;                     // down output [S][N]
    int32_t K, N, ntn;            // ntn: column blocks
    float limit;
};

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight consecutive K values of one weight row: code dword c (element 2i in
// the low nibble of byte i) times the decoded group scale sc, as bf16.  The
// products are exact in FP32 and representable in bf16, so keeping the high
// half of each FP32 word is the exact conversion.
__device__ __forceinline__ bf16x8 dequant8(uint32_t c, float sc)
{
    auto pair = [sc](f32x2 v) {
        return __builtin_amdgcn_perm(__float_as_uint(v.y * sc), __float_as_uint(v.x * sc), 0x07060302u);
    };
    const u32x4 o = {pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)c, 1.0f, 0)),
                     pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)c, 1.0f, 1)),
                     pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)c, 1.0f, 2)),
                     pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)c, 1.0f, 3))};
    return __builtin_bit_cast(bf16x8, o);
}

// 16-byte A operand of lane `lane` (K values 8(lane/16) .. +7 of K half ks)
// for tile row `row`
__device__ __forceinline__ bf16x8 a_op(const uint8_t *tile, int row, int ks, int lane)
{
    return *reinterpret_cast<const bf16x8 *>(tile + row * 128 + swz(row, ks * 4 + (lane >> 4)) * 16);
}

// B operand of lane `lane` for B row `br` and K half ks: the code dword of
// its 8 K values and the scale of their 16-group, from the stage's code and
// scale regions (codes row-major 32 bytes per row; scales one dword per row,
// rows in runs of 32 per 256 bytes)
__device__ __forceinline__ bf16x8 b_op(const uint8_t *codes, const uint8_t *scales, int br, int ks,
                                       int lane)
{
    const uint32_t c = *reinterpret_cast<const uint32_t *>(codes + br * 32 + ks * 16 + (lane >> 4) * 4);
    const uint32_t sd = *reinterpret_cast<const uint32_t *>(scales + (br >> 5) * 256 + (br & 31) * 4);
    const uint32_t sb = sd >> ((lane >> 5) * 8);       // group 2 ks + lane/32 in byte 2 ks
    const float sc = ks == 0 ? __builtin_amdgcn_cvt_f32_fp8((int)sb, 0)
                             : __builtin_amdgcn_cvt_f32_fp8((int)sb, 2);
    return dequant8(c, sc);
}

__device__ __forceinline__ float swiglu_clamp(float g, float u, float L)
{
    const float gc = fminf(g, L);
    const float uc = fminf(fmaxf(u, -L), L);
    return gc / (1.0f + expf(-gc)) * uc;
}

// bf16 of a finite float, round to nearest even
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    const uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// vmcnt wait that leaves `ahead` stages of `per` DMA instructions in flight
#define NV_WAIT_AHEAD(kb, KB, per)                        \
    do {                                                  \
        if ((kb) + 2 < (KB)) MOE_WAIT_VM(2 * (per));      \
        else if ((kb) + 1 < (KB)) MOE_WAIT_VM(per);       \
        else MOE_WAIT_VM(0);                              \
    } while (0)

// ---------------------------------------------------------------------------
// gate + up (+ SwiGLU, h as hi/lo bf16)
// ---------------------------------------------------------------------------
// Stage: A [128 rows][128 B] | B codes [128 rows][32 B] (0-63 gate, 64-127 up)
//        | B scales [4 runs][256 B]
constexpr int GA = 0, GC = TM * 128, GS = GC + 128 * 32, GSTAGE = GS + 4 * 256;
constexpr int G_DMA = 4 + 1 + 1;   // DMA instructions per wave per stage

__global__ __launch_bounds__(kThreads, 1) void gemm_gateup_nvfp4_kernel(NvGemmArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t st0[GSTAGE], st1[GSTAGE], st2[GSTAGE], st3[GSTAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    int4 tile;
    int nb;
    if (!gemm_item(a, tile, nb)) return;
    const int e = tile.x, p0 = tile.y;
    const int rows = moe::uniform(min(TM, a.offsets[e + 1] - p0));
    const int K = a.K, N = a.N, KB = K / KS;
    const int n0 = nb * 64;
    const float sg = a.g0[e], su = a.g1[e];

    // A: four runs of 8 rows per wave (rows past the tile read its first row
    // and are never stored)
    uint32_t aoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (wave * 4 + j) * 8 + (lane >> 3);
        const int tok = a.sorted_token[p0 + (r < rows ? r : 0)];
        aoff[j] = (uint32_t)tok * (uint32_t)(K * 2) + swz(r, lane & 7) * 16;
    }
    // B: wave w loads B rows 32w..32w+31 (gate rows n0 + 32w.. for w < 2, up
    // rows n0 + 32(w-2).. otherwise): codes 16 bytes per lane, scales one
    // dword per lane (lanes 32-63 repeat lanes 0-31)
    const size_t brow = (size_t)e * N + n0 + (wave & 1) * 32;
    const uint8_t *cbase = (wave < 2 ? a.c0 : a.c1) + brow * (K / 2);
    const uint8_t *sbase = (wave < 2 ? a.s0 : a.s1) + brow * (K / 16);
    const uint32_t coff = (uint32_t)(lane >> 1) * (K / 2) + (lane & 1) * 16;
    const uint32_t soff = (uint32_t)(lane & 31) * (K / 16);

    auto issue = [&](int kb, uint8_t *st) {
        const uint8_t *ab = reinterpret_cast<const uint8_t *>(a.a) + (size_t)kb * 128;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(ab, aoff[j], lds_addr(st + GA + (wave * 4 + j) * 1024));
        dma16(cbase + (size_t)kb * 32, coff, lds_addr(st + GC + wave * 1024));
        dma4(sbase + (size_t)kb * 4, soff, lds_addr(st + GS + wave * 256));
    };

    f32x4 accg[4][2], accu[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) { accg[i][j] = f32x4{0.f, 0.f, 0.f, 0.f}; accu[i][j] = accg[i][j]; }

    auto compute = [&](const uint8_t *st) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 av[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) av[mt] = a_op(st + GA, wm * 64 + mt * 16 + (lane & 15), ks, lane);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int rg = wn * 32 + nt * 16 + (lane & 15);
                const bf16x8 bg = b_op(st + GC, st + GS, rg, ks, lane);
                const bf16x8 bu = b_op(st + GC, st + GS, 64 + rg, ks, lane);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    accg[mt][nt] = mfma_bf16(av[mt], bg, accg[mt][nt]);
                    accu[mt][nt] = mfma_bf16(av[mt], bu, accu[mt][nt]);
                }
            }
        }
    };

    auto step = [&](int kb, const uint8_t *cur, uint8_t *later) {
        NV_WAIT_AHEAD(kb, KB, G_DMA);
        MOE_WAIT_LGKM0();
        MOE_BARRIER();
        if (kb + 3 < KB) issue(kb + 3, later);
        compute(cur);
    };

    MOE_WAIT_VM(0);    // retire the offset and scale_2 loads above before the DMA starts
    issue(0, st0);
    if (KB > 1) issue(1, st1);
    if (KB > 2) issue(2, st2);
    for (int kb = 0; kb < KB; kb += 4) {
        step(kb, st0, st3);
        if (kb + 1 >= KB) break;
        step(kb + 1, st1, st0);
        if (kb + 2 >= KB) break;
        step(kb + 2, st2, st1);
        if (kb + 3 >= KB) break;
        step(kb + 3, st3, st2);
    }
    MOE_WAIT_VM(0);
    __syncthreads();

    // epilogue: h = SwiGLU(sg g, su u) -> hi, lo tiles [128][64] bf16 in LDS,
    // then 16-byte stores of the valid rows
    uint16_t *th = reinterpret_cast<uint16_t *>(st0);
    uint16_t *tl = reinterpret_cast<uint16_t *>(st1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + mt * 16 + (lane >> 4) * 4 + i;
                const int c = wn * 32 + nt * 16 + (lane & 15);
                const float h = swiglu_clamp(accg[mt][nt][i] * sg, accu[mt][nt][i] * su, a.limit);
                const uint32_t hi = bf16_rne(h);
                th[r * 64 + c] = (uint16_t)hi;
                tl[r * 64 + c] = (uint16_t)bf16_rne(h - __uint_as_float(hi << 16));
            }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ch = tid + kThreads * j, r = ch >> 3, part = ch & 7;
        if (r < rows) {
            const size_t o = (size_t)(p0 + r) * N + n0 + part * 8;
            *reinterpret_cast<uint4 *>(a.hhi + o) = *reinterpret_cast<const uint4 *>(th + r * 64 + part * 8);
            *reinterpret_cast<uint4 *>(a.hlo + o) = *reinterpret_cast<const uint4 *>(tl + r * 64 + part * 8);
        }
    }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------
// Stage: A hi [128][128 B] | A lo [128][128 B] | B codes [128][32 B] | B scales
constexpr int DA = 0, DA2 = TM * 128, DC = 2 * TM * 128, DS = DC + 128 * 32, DSTAGE = DS + 4 * 256;
constexpr int D_DMA = 8 + 1 + 1;

__global__ __launch_bounds__(kThreads, 1) void gemm_down_nvfp4_kernel(NvGemmArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t st0[DSTAGE], st1[DSTAGE], st2[DSTAGE], st3[DSTAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    int4 tile;
    int nb;
    if (!gemm_item(a, tile, nb)) return;
    const int e = tile.x, p0 = tile.y;
    const int rows = moe::uniform(min(TM, a.offsets[e + 1] - p0));
    const int K = a.K, N = a.N, KB = K / KS;
    const int n0 = nb * 128;
    const float sd = a.g0[e];

    uint32_t aoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (wave * 4 + j) * 8 + (lane >> 3);
        aoff[j] = (uint32_t)(p0 + (r < rows ? r : 0)) * (uint32_t)(K * 2) + swz(r, lane & 7) * 16;
    }
    const size_t brow = (size_t)e * N + n0 + wave * 32;
    const uint8_t *cbase = a.c0 + brow * (K / 2);
    const uint8_t *sbase = a.s0 + brow * (K / 16);
    const uint32_t coff = (uint32_t)(lane >> 1) * (K / 2) + (lane & 1) * 16;
    const uint32_t soff = (uint32_t)(lane & 31) * (K / 16);

    auto issue = [&](int kb, uint8_t *st) {
        const uint8_t *ab = reinterpret_cast<const uint8_t *>(a.a) + (size_t)kb * 128;
        const uint8_t *ab2 = reinterpret_cast<const uint8_t *>(a.a2) + (size_t)kb * 128;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(ab, aoff[j], lds_addr(st + DA + (wave * 4 + j) * 1024));
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(ab2, aoff[j], lds_addr(st + DA2 + (wave * 4 + j) * 1024));
        dma16(cbase + (size_t)kb * 32, coff, lds_addr(st + DC + wave * 1024));
        dma4(sbase + (size_t)kb * 4, soff, lds_addr(st + DS + wave * 256));
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const uint8_t *st) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 ah[4], al[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int r = wm * 64 + mt * 16 + (lane & 15);
                ah[mt] = a_op(st + DA, r, ks, lane);
                al[mt] = a_op(st + DA2, r, ks, lane);
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const bf16x8 b = b_op(st + DC, st + DS, wn * 64 + nt * 16 + (lane & 15), ks, lane);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    acc[mt][nt] = mfma_bf16(ah[mt], b, acc[mt][nt]);
                    acc[mt][nt] = mfma_bf16(al[mt], b, acc[mt][nt]);
                }
            }
        }
    };

    auto step = [&](int kb, const uint8_t *cur, uint8_t *later) {
        NV_WAIT_AHEAD(kb, KB, D_DMA);
        MOE_WAIT_LGKM0();
        MOE_BARRIER();
        if (kb + 3 < KB) issue(kb + 3, later);
        compute(cur);
    };

    MOE_WAIT_VM(0);
    issue(0, st0);
    if (KB > 1) issue(1, st1);
    if (KB > 2) issue(2, st2);
    for (int kb = 0; kb < KB; kb += 4) {
        step(kb, st0, st3);
        if (kb + 1 >= KB) break;
        step(kb + 1, st1, st0);
        if (kb + 2 >= KB) break;
        step(kb + 2, st2, st1);
        if (kb + 3 >= KB) break;
        step(kb + 3, st3, st2);
    }

#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + mt * 16 + (lane >> 4) * 4 + i;
            if (r < rows) {
                float *yr = a.y + (size_t)(p0 + r) * N + n0 + wn * 64 + (lane & 15);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) yr[nt * 16] = acc[mt][nt][i] * sd;
            }
        }
}

}  // namespace

hipError_t launch_gemm_gateup_nvfp4(const uint16_t *x, const int32_t *sorted_token,
                                    const GemvBankDev &gate, const GemvBankDev &up,
                                    const int32_t *offsets, const int4 *tiles,
                                    const int32_t *ntiles, int32_t tmax, int32_t hidden,
                                    int32_t inter, float limit, uint16_t *hhi, uint16_t *hlo,
                                    hipStream_t st)
{
    NvGemmArgs a{};
    a.a = x; a.sorted_token = sorted_token;
    a.c0 = gate.codes; a.c1 = up.codes;
    a.s0 = (const uint8_t *)gate.scales; a.s1 = (const uint8_t *)up.scales;
    a.g0 = gate.scale2; a.g1 = up.scale2;
    a.offsets = offsets; a.tiles = tiles; a.ntiles = ntiles;
    a.hhi = hhi; a.hlo = hlo; a.K = hidden; a.N = inter; a.ntn = inter / 64; a.limit = limit;
    hipLaunchKernelGGL(gemm_gateup_nvfp4_kernel, dim3((unsigned)(tmax * a.ntn)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gemm_down_nvfp4(const uint16_t *hhi, const uint16_t *hlo, const GemvBankDev &down,
                                  const int32_t *offsets, const int4 *tiles, const int32_t *ntiles,
                                  int32_t tmax, int32_t hidden, int32_t inter, float *y,
                                  hipStream_t st)
{
    NvGemmArgs a{};
    a.a = hhi; a.a2 = hlo;
    a.c0 = down.codes; a.s0 = (const uint8_t *)down.scales; a.g0 = down.scale2;
    a.offsets = offsets; a.tiles = tiles; a.ntiles = ntiles;
    a.y = y; a.K = inter; a.N = hidden; a.ntn = hidden / 128;
    hipLaunchKernelGGL(gemm_down_nvfp4_kernel, dim3((unsigned)(tmax * a.ntn)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}
