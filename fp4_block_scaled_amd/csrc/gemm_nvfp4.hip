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
// h between the projections is a 16-bit activation, as in the W4A16 form,
// held as FP16 rather than bf16: the gate/up epilogue computes h = SwiGLU(g,
// u) in FP32 and rounds h * 2^-k to FP16 (RNE), with the power of two chosen
// from the clamp limit so that the bound on |h| lands in (16384, 32768]: no
// overflow, and h keeps FP16's full 11-bit significand down to 2^-15 of its
// bound instead of falling into FP16's subnormals under a small limit (k = -9
// for the limit 7).  FP16 then keeps the layer's output within about 2e-4
// relative L2 of the exact one, where a bf16 h would cost about 1e-3.  The
// down GEMM decodes its NVFP4 weights to FP16, exactly (a product of at most
// 6 significant bits between 2^-10 and 2688), runs the FP16 MFMA once, and
// multiplies the FP32 sums by 2^k (exact), then by scale_2.
//
// Kernels (tiles from gemm_tiles_kernel: 128 expert-sorted rows each):
//   gemm_gateup_nvfp4_kernel  one block = 128 rows x 64 h columns: 64 gate and
//                             64 up weight rows per K step, SwiGLU, FP16 h.
//   gemm_down_nvfp4_kernel    one block = 128 rows x 128 outputs of y.
// Block: 256 threads = 4 waves as 2 (64 rows each) x 2 (column halves).  Per
// K step of 64: the A rows (128 bytes of bf16 x or FP16 h) move from global memory
// straight into swizzled LDS, with the B codes (32 bytes per weight row) and
// group scales (4 bytes per row) beside them, four stages deep.  Each wave
// decodes its own B operands from LDS: lane l of a 16x16x32 MFMA operand
// needs 8 consecutive K values of one weight row, i.e. one code dword and one
// group scale.
#include "gemm_common.h"

#include <cmath>

namespace {

using moe::f32x2;
using moe::f32x4;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int TM = 128;      // rows per tile
constexpr int KS = 64;       // K per step (128 bytes of a bf16 row)

struct NvGemmArgs {
    const uint16_t *a;            // gate/up: x bf16 [M][K]; down: h FP16 [S][K]
    const int32_t *sorted_token;  // gate/up gathers A rows through it
    const uint8_t *c0, *c1;       // gate and up codes (down: c0), [E][N][K/2]
    const uint8_t *s0, *s1;       // their group scales [E][N][K/16]
    const float *g0, *g1;         // their scale_2 [E]
    const int32_t *offsets;
    const int4 *tiles;
    const int32_t *ntiles;
    uint16_t *h;                  // gate/up output, FP16 h * hscale [S][N]
    float *y;                     // down output [S][N]
    int32_t K, N, ntn;            // ntn: column blocks
    float limit;
    float hscale;                 // gate/up: 2^-k; down: 2^k
};

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(const f16x8 &a, const f16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
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

// The same eight weights as FP16: E2M1 pairs convert exactly and the E4M3
// group scale is an FP16 value, so the packed products are exact too.
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t c, float sc)
{
    const _Float16 h = (_Float16)sc;
    const f16x2 s2 = {h, h};
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((int)c, 1.0f, 0) * s2;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((int)c, 1.0f, 1) * s2;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((int)c, 1.0f, 2) * s2;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((int)c, 1.0f, 3) * s2;
    return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// 16-byte A operand of lane `lane` (K values 8(lane/16) .. +7 of K half ks)
// for tile row `row`
template <typename T>
__device__ __forceinline__ T a_op(const uint8_t *tile, int row, int ks, int lane)
{
    return *reinterpret_cast<const T *>(tile + row * 128 + swz(row, ks * 4 + (lane >> 4)) * 16);
}

// FP16 B operand of lane `lane` for B row `br` and K half ks: the code dword
// of its 8 K values and the scale of their 16-group, from the stage's code and
// scale regions (codes row-major 32 bytes per row; scales one dword per row,
// rows in runs of 32 per 256 bytes)
__device__ __forceinline__ f16x8 b_op16(const uint8_t *codes, const uint8_t *scales, int br, int ks,
                                        int lane)
{
    const uint32_t c = *reinterpret_cast<const uint32_t *>(codes + br * 32 + ks * 16 + (lane >> 4) * 4);
    const uint32_t sd = *reinterpret_cast<const uint32_t *>(scales + (br >> 5) * 256 + (br & 31) * 4);
    const uint32_t sb = sd >> ((lane >> 5) * 8);       // group 2 ks + lane/32 in byte 2 ks
    const float sc = ks == 0 ? __builtin_amdgcn_cvt_f32_fp8((int)sb, 0)
                             : __builtin_amdgcn_cvt_f32_fp8((int)sb, 2);
    return dequant8_f16(c, sc);
}

__device__ __forceinline__ float swiglu_clamp(float g, float u, float L)
{
    const float gc = fminf(g, L);
    const float uc = fminf(fmaxf(u, -L), L);
    return gc / (1.0f + expf(-gc)) * uc;
}

// ---------------------------------------------------------------------------
// gate + up (+ SwiGLU, h as FP16)
// ---------------------------------------------------------------------------
// Block: W waves; wave w = all 128 rows x h columns 32w..32w+31 of both gate
// and up, so each decoded B operand feeds 8 MFMAs (one per 16-row group).
// The tile is 128 rows x 32W h columns: 64W B rows, gate rows first, then up
// rows; wave w loads B rows 64w..64w+63.
// Stage: A [128][128 B] | B codes [64W][32 B] | B scales [64W][4 B]
template <int W>
struct GuLayout {
    static constexpr int threads = 64 * W;
    static constexpr int cols = 32 * W;
    static constexpr int A = 0, C = TM * 128, S = C + 64 * W * 32, STAGE = S + 64 * W * 4;
    static constexpr int arun = 16 / W;          // A runs of 8 rows per wave
    static constexpr int dma = arun + 2 + 1;     // DMA instructions per wave per stage
};

// B operand of lane `lane` for B row `br` and K half ks, scales stored one
// dword per row
__device__ __forceinline__ bf16x8 b_op_lin(const uint8_t *codes, const uint8_t *scales, int br,
                                           int ks, int lane)
{
    const uint32_t c = *reinterpret_cast<const uint32_t *>(codes + br * 32 + ks * 16 + (lane >> 4) * 4);
    const uint32_t sd = *reinterpret_cast<const uint32_t *>(scales + br * 4);
    const uint32_t sb = sd >> ((lane >> 5) * 8);
    const float sc = ks == 0 ? __builtin_amdgcn_cvt_f32_fp8((int)sb, 0)
                             : __builtin_amdgcn_cvt_f32_fp8((int)sb, 2);
    return dequant8(c, sc);
}

template <int W, int NST, int OCC>
__global__ __launch_bounds__(GuLayout<W>::threads, OCC) void gemm_gateup_nvfp4_kernel(NvGemmArgs a)
{
    using Lo = GuLayout<W>;
    __shared__ __attribute__((aligned(16))) uint8_t sm[NST * Lo::STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    int4 tile;
    int nb;
    if (!gemm_item(a, tile, nb)) return;
    const int e = tile.x, p0 = tile.y;
    const int rows = moe::uniform(min(TM, a.offsets[e + 1] - p0));
    const int K = a.K, N = a.N, KB = K / KS;
    const int n0 = nb * Lo::cols;
    const float sg = a.g0[e], su = a.g1[e];

    // A: runs of 8 rows (rows past the tile read its first row and are
    // never stored)
    uint32_t aoff[Lo::arun];
#pragma unroll
    for (int j = 0; j < Lo::arun; ++j) {
        const int r = (wave * Lo::arun + j) * 8 + (lane >> 3);
        const int tok = a.sorted_token[p0 + (r < rows ? r : 0)];
        aoff[j] = (uint32_t)tok * (uint32_t)(K * 2) + swz(r, lane & 7) * 16;
    }
    // B rows 64w..64w+63: the first W/2 waves gate rows n0 + 64w.., the
    // others up rows n0 + 64(w - W/2)..; codes in two runs of 32 rows (16
    // bytes per lane), scales one dword per lane
    const bool gate_rows = wave < W / 2;
    const size_t brow = (size_t)e * N + n0 + (gate_rows ? wave : wave - W / 2) * 64;
    const uint8_t *cbase = (gate_rows ? a.c0 : a.c1) + brow * (K / 2);
    const uint8_t *sbase = (gate_rows ? a.s0 : a.s1) + brow * (K / 16);
    const uint32_t coff0 = (uint32_t)(lane >> 1) * (K / 2) + (lane & 1) * 16;
    const uint32_t coff1 = coff0 + 32 * (uint32_t)(K / 2);
    const uint32_t soff = (uint32_t)lane * (K / 16);

    auto issue = [&](int kb, uint8_t *st) {
        const uint8_t *ab = reinterpret_cast<const uint8_t *>(a.a) + (size_t)kb * 128;
#pragma unroll
        for (int j = 0; j < Lo::arun; ++j)
            dma16(ab, aoff[j], lds_addr(st + Lo::A + (wave * Lo::arun + j) * 1024));
        const uint8_t *cb = cbase + (size_t)kb * 32;
        dma16(cb, coff0, lds_addr(st + Lo::C + wave * 2048));
        dma16(cb, coff1, lds_addr(st + Lo::C + wave * 2048 + 1024));
        dma4(sbase + (size_t)kb * 4, soff, lds_addr(st + Lo::S + wave * 256));
    };

    f32x4 accg[8][2], accu[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) { accg[i][j] = f32x4{0.f, 0.f, 0.f, 0.f}; accu[i][j] = accg[i][j]; }

    auto compute = [&](const uint8_t *st, int) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 av[8];
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) av[mt] = a_op<bf16x8>(st + Lo::A, mt * 16 + (lane & 15), ks, lane);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int rg = wave * 32 + nt * 16 + (lane & 15);
                const bf16x8 bg = b_op_lin(st + Lo::C, st + Lo::S, rg, ks, lane);
                const bf16x8 bu = b_op_lin(st + Lo::C, st + Lo::S, Lo::cols + rg, ks, lane);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    accg[mt][nt] = mfma_bf16(av[mt], bg, accg[mt][nt]);
                    accu[mt][nt] = mfma_bf16(av[mt], bu, accu[mt][nt]);
                }
            }
        }
    };

    k_loop<NST, Lo::dma>(KB, sm, Lo::STAGE, issue, compute);
    __syncthreads();

    // epilogue: h = SwiGLU(sg g, su u) -> FP16 tile [128][128] in LDS (rows
    // padded to 136 elements), then 16-byte stores of the valid rows
    constexpr int C = Lo::cols, CP = C + 8;
    static_assert(TM * CP * 2 <= NST * Lo::STAGE, "the h tile exceeds the stages");
    uint16_t *th = reinterpret_cast<uint16_t *>(sm);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = mt * 16 + (lane >> 4) * 4 + i;
                const int c = wave * 32 + nt * 16 + (lane & 15);
                const float h = swiglu_clamp(accg[mt][nt][i] * sg, accu[mt][nt][i] * su, a.limit);
                th[r * CP + c] = __builtin_bit_cast(uint16_t, (_Float16)(h * a.hscale));
            }
    __syncthreads();
    constexpr int cpr = C / 8;                        // 16-byte chunks per row
#pragma unroll
    for (int j = 0; j < TM * cpr / Lo::threads; ++j) {
        const int ch = tid + Lo::threads * j, r = ch / cpr, part = ch % cpr;
        if (r < rows) {
            const size_t o = (size_t)(p0 + r) * N + n0 + part * 8;
            *reinterpret_cast<uint4 *>(a.h + o) = *reinterpret_cast<const uint4 *>(th + r * CP + part * 8);
        }
    }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------
// Block: 2 x NW waves, wave (wm, wn) = 64 rows x 64 outputs; the tile is
// 128 rows x 64 NW outputs.  Wave w loads B rows 32w..32w+31.
// Stage: A (FP16 h) [128][128 B] | B codes [64 NW][32 B] | B scales
template <int NW>
struct DnLayout {
    static constexpr int threads = 128 * NW;
    static constexpr int cols = 64 * NW;
    static constexpr int A = 0, C = TM * 128, S = C + 64 * NW * 32, STAGE = S + 2 * NW * 256;
    static constexpr int arun = 8 / NW;          // runs of 8 rows per wave
    static constexpr int dma = arun + 2;
};

template <int NW, int NST, int OCC>
__global__ __launch_bounds__(DnLayout<NW>::threads, OCC) void gemm_down_nvfp4_kernel(NvGemmArgs a)
{
    using Lo = DnLayout<NW>;
    __shared__ __attribute__((aligned(16))) uint8_t sm[NST * Lo::STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    int4 tile;
    int nb;
    if (!gemm_item(a, tile, nb)) return;
    const int e = tile.x, p0 = tile.y;
    const int rows = moe::uniform(min(TM, a.offsets[e + 1] - p0));
    const int K = a.K, N = a.N, KB = K / KS;
    const int n0 = nb * Lo::cols;
    const float sd = a.g0[e], hk = a.hscale;       // scale_2, 2^k

    uint32_t aoff[Lo::arun];
#pragma unroll
    for (int j = 0; j < Lo::arun; ++j) {
        const int r = (wave * Lo::arun + j) * 8 + (lane >> 3);
        aoff[j] = (uint32_t)(p0 + (r < rows ? r : 0)) * (uint32_t)(K * 2) + swz(r, lane & 7) * 16;
    }
    const size_t brow = (size_t)e * N + n0 + wave * 32;
    const uint8_t *cbase = a.c0 + brow * (K / 2);
    const uint8_t *sbase = a.s0 + brow * (K / 16);
    const uint32_t coff = (uint32_t)(lane >> 1) * (K / 2) + (lane & 1) * 16;
    const uint32_t soff = (uint32_t)(lane & 31) * (K / 16);

    auto issue = [&](int kb, uint8_t *st) {
        const uint8_t *ab = reinterpret_cast<const uint8_t *>(a.a) + (size_t)kb * 128;
#pragma unroll
        for (int j = 0; j < Lo::arun; ++j)
            dma16(ab, aoff[j], lds_addr(st + Lo::A + (wave * Lo::arun + j) * 1024));
        dma16(cbase + (size_t)kb * 32, coff, lds_addr(st + Lo::C + wave * 1024));
        dma4(sbase + (size_t)kb * 4, soff, lds_addr(st + Lo::S + wave * 256));
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const uint8_t *st, int) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            f16x8 ah[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) ah[mt] = a_op<f16x8>(st + Lo::A, wm * 64 + mt * 16 + (lane & 15), ks, lane);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const f16x8 b = b_op16(st + Lo::C, st + Lo::S, wn * 64 + nt * 16 + (lane & 15), ks, lane);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma_f16(ah[mt], b, acc[mt][nt]);
            }
        }
    };

    k_loop<NST, Lo::dma>(KB, sm, Lo::STAGE, issue, compute);

#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + mt * 16 + (lane >> 4) * 4 + i;
            if (r < rows) {
                float *yr = a.y + (size_t)(p0 + r) * N + n0 + wn * 64 + (lane & 15);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) yr[nt * 16] = acc[mt][nt][i] * hk * sd;
            }
        }
}

// launch shapes: gate/up 4 waves (128 h columns) over 3 stages, down 4 waves
// (128 outputs) over 2 stages, two blocks of each per CU (the LDS of both
// within the 160 KB of a CU), so every SIMD runs waves of two blocks whose
// barriers and waits do not line up
constexpr int GU_W = 4, GU_NST = 3, GU_OCC = 2, DN_NW = 2, DN_NST = 2, DN_OCC = 2;
static_assert(GU_OCC * GU_NST * GuLayout<GU_W>::STAGE <= 160 * 1024, "gate/up stages exceed LDS");
static_assert(DN_OCC * DN_NST * DnLayout<DN_NW>::STAGE <= 160 * 1024, "down stages exceed LDS");

// k for the FP16 h: |silu(gc)| <= max(L, 0.28) and |uc| <= L, so with the
// bound in (16384, 32768] after the factor 2^-k, |h| * 2^-k stays below FP16's
// largest finite value (65504) with room for the rounding of the FP32 SwiGLU
int h16_shift(float limit)
{
    const double bound = (limit > 0.28f ? (double)limit : 0.28) * (double)limit;
    int k = 0;
    while (k < 100 && bound > std::ldexp(32768.0, k)) ++k;
    while (k > -100 && bound <= std::ldexp(16384.0, k)) --k;
    return k;
}

}  // namespace

hipError_t launch_gemm_gateup_nvfp4(const uint16_t *x, const int32_t *sorted_token,
                                    const GemvBankDev &gate, const GemvBankDev &up,
                                    const int32_t *offsets, const int4 *tiles,
                                    const int32_t *ntiles, int32_t tmax, int32_t hidden,
                                    int32_t inter, float limit, uint16_t *h16, hipStream_t st)
{
    using Lo = GuLayout<GU_W>;
    if (inter % Lo::cols || hidden % KS) return hipErrorInvalidValue;
    NvGemmArgs a{};
    a.a = x; a.sorted_token = sorted_token;
    a.c0 = gate.codes; a.c1 = up.codes;
    a.s0 = (const uint8_t *)gate.scales; a.s1 = (const uint8_t *)up.scales;
    a.g0 = gate.scale2; a.g1 = up.scale2;
    a.offsets = offsets; a.tiles = tiles; a.ntiles = ntiles;
    a.h = h16; a.K = hidden; a.N = inter; a.ntn = inter / Lo::cols; a.limit = limit;
    a.hscale = std::ldexp(1.0f, -h16_shift(limit));
    hipLaunchKernelGGL((gemm_gateup_nvfp4_kernel<GU_W, GU_NST, GU_OCC>), dim3((unsigned)(tmax * a.ntn)),
                       dim3(Lo::threads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gemm_down_nvfp4(const uint16_t *h16, const GemvBankDev &down,
                                  const int32_t *offsets, const int4 *tiles, const int32_t *ntiles,
                                  int32_t tmax, int32_t hidden, int32_t inter, float limit, float *y,
                                  hipStream_t st)
{
    using Lo = DnLayout<DN_NW>;
    if (hidden % Lo::cols || inter % KS) return hipErrorInvalidValue;
    NvGemmArgs a{};
    a.a = h16;
    a.c0 = down.codes; a.s0 = (const uint8_t *)down.scales; a.g0 = down.scale2;
    a.offsets = offsets; a.tiles = tiles; a.ntiles = ntiles;
    a.y = y; a.K = inter; a.N = hidden; a.ntn = hidden / Lo::cols;
    a.hscale = std::ldexp(1.0f, h16_shift(limit));
    hipLaunchKernelGGL((gemm_down_nvfp4_kernel<DN_NW, DN_NST, DN_OCC>), dim3((unsigned)(tmax * a.ntn)),
                       dim3(Lo::threads), 0, st, a);
    return hipGetLastError();
}
