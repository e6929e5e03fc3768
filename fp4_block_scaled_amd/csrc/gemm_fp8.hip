// gemm_fp8.hip -- grouped GEMM tier for E4M3 banks at wide M (prefill).
//
// With thousands of tokens every expert holds many rows, so the projections
// become dense contractions per expert ("spark_model glm5next_mlp/forward.rs",
// grouped-prefill arm of fn forward_moe: sort slots by expert, then one
// grouped GEMM per projection, worth it above 64-128 rows).  Activations are
// E4M3 with one FP32 scale per 1x128 group, like the xq/xs and hq/hs buffers
// of "memra-engine src/dsv4_ep.rs" (EpScratch and the act_quant_fp8 step of
// fn chain).
//
// Kernels:
//   quant_act_kernel    x bf16 -> E4M3 codes + FP32 scale per 1x128 group
//                       (scale = amax/448, code = RNE(x/scale) saturated).
//   gemm_tiles_kernel   per-expert row chunks over the expert-sorted rows,
//                       built on the device from expert_offsets.
//   gemm_gateup8_kernel one block (8 waves) = one chunk of <= 128 rows of
//                       one expert x 128 h columns: the gate AND the up
//                       projection of those columns, the clamped SwiGLU, and
//                       the E4M3 quantization of the 128-wide h row segment
//                       (exactly one 1x128 group) in the epilogue.
//   gemm_down_kernel    persistent: a block per CU runs a fixed list of
//                       (chunk, 128 outputs of y) items as one pipeline.
//
// Matrix-core precision.  gfx950's FP8 MFMA sums its products in groups of
// eight, each group in a fixed-point window about 13 bits below the group's
// largest product; smaller products lose their low bits (measured on
// MI355X: single products are exact, a 1x1 product beside a 448x448 one in
// the same group of eight vanishes, and the error reaches 3e-4 of the
// largest term on layer-like operands).  Every h code is a rounding decision
// taken on g and u, so gate/up runs on the bf16 MFMA instead, whose products
// are exact and whose sums are FP32 (E4M3 codes of x and of the weights are
// bf16 values exactly): g and u then carry only FP32 rounding and the h codes
// agree with the exact layer's except at true ties.  y decides nothing, so
// down keeps the FP8 MFMA (one v_mfma_f32_16x16x128_f8f6f4 per 128-wide K
// block), whose error stays far inside the output tolerance.
//
// Data movement.  Gate/up: weights are read once per chunk straight from
// global memory into VGPRs, in exactly the lane layout of the MFMA operand
// (lane l: row l % 16, 32 bytes of K), several K steps ahead; they never
// touch LDS.  The activation rows of the chunk, shared by every wave, go to
// LDS (XOR swizzled, two stages) through VGPRs.  All its loads are ordinary
// compiler-visible loads, so the compiler's waits are exact.  Down: both
// operands go from global memory straight into LDS stages (DMA), with
// explicit waits.
//
// K order inside a 128-wide block: a lane's 32 bytes are K offsets
// 16q..16q+15 and 64+16q..64+16q+15 (q = lane / 16), so each half is one
// 16-byte load of a row; A and B use the same order, and a dot product over
// the block does not depend on the order of its terms.
#include "gemm_common.h"

#include <algorithm>

namespace {

using moe::f32x4;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 128;       // K per step = one scale block
constexpr int RMAX = 128;     // rows per chunk of the E4M3 tier
constexpr int TILE_ROWS = 128;   // rows per tile of the NVFP4 tier's schedule
constexpr int kThreads = 256;

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
// tile schedule: tiles[t] = (expert, first packed row, expert's first tile,
// its tile count), t < *ntiles.  An expert with n rows gets ceil(n / rmax)
// tiles; balanced: all but the last hold ceil(n / tiles) rows (so no tile is
// much shorter than the others), else rmax rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void gemm_tiles_kernel(const int32_t *__restrict__ offsets,
                                                          int32_t E, int32_t tmax, int32_t rmax,
                                                          int32_t balanced,
                                                          int4 *__restrict__ tiles,
                                                          int32_t *__restrict__ ntiles)
{
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = tid;
    const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
    const int nt = (cnt + rmax - 1) / rmax;
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
    if (e < E && nt > 0) {
        const int p0 = offsets[e];
        const int cs = balanced ? (cnt + nt - 1) / nt : rmax;
        for (int m = 0; m < nt && first + m < tmax; ++m) tiles[first + m] = make_int4(e, p0 + m * cs, first, nt);
    }
    if (tid == 1023) *ntiles = min(base + inc, tmax);
}

// Rows of a balanced chunk starting at packed row p0 of expert e whose
// tiles number n (<= 0 for a chunk past the expert's rows).
__device__ __forceinline__ int chunk_rows(const int32_t *offsets, int e, int p0, int n)
{
    const int lo = moe::uniform(offsets[e]), hi = moe::uniform(offsets[e + 1]);
    const int cs = (hi - lo + n - 1) / n;
    return min(cs, hi - p0);
}

// Eight E4M3 codes (bytes of lo then hi) as bf16 values, exactly (every
// E4M3 value is a bf16 value).
__device__ __forceinline__ bf16x8 cvt8(uint32_t lo, uint32_t hi)
{
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8 &a, const i32x8 &b)
{
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float swiglu_clamp(float g, float u, float L)
{
    const float gc = fminf(g, L);
    const float uc = fminf(fmaxf(u, -L), L);
    return gc / (1.0f + expf(-gc)) * uc;
}

// ---------------------------------------------------------------------------
// activation rows of a chunk in LDS
// ---------------------------------------------------------------------------
// A stage holds a chunk's activation rows for one K step of 128 as bf16
// values (256 bytes a row: 16 chunks of 16 bytes, XOR swizzled), then the
// two promotion factors of each row.  Rows past the chunk's hold its first
// row: their products land in output rows that are never stored.
template <int RB>
struct AStage {
    static constexpr int C = RB / 16;                 // 16-byte chunks per row
    static constexpr int S_OFF = RMAX * RB;           // factors after the rows
    // physical chunk of logical chunk c in row r: an XOR with the row's low
    // bits, so the 16 rows an operand read touches at one logical chunk land
    // on distinct chunks (distinct banks)
    static __device__ __forceinline__ int swz(int r, int c)
    {
        if constexpr (C == 16) return c ^ (r & 15);
        else return ::swz(r, c);
    }
};

// ---------------------------------------------------------------------------
// gate + up (+ SwiGLU + h quantization), bf16 MFMA
// ---------------------------------------------------------------------------
struct GuArgs {
    const uint8_t *xq;         // x codes [M][K]
    const float *xs;           // x scales [M][K/128]
    const int32_t *sorted_token;
    const uint8_t *w0, *w1;    // gate and up codes, [E][N][K]
    const float *ws0, *ws1;    // their block scales [E][N/128][K/128]
    const int32_t *offsets;
    const int4 *tiles;
    const int32_t *ntiles;
    uint8_t *hq;               // h codes [S][N] (packed rows)
    float *hs;                 // h scales [S][N/128]
    int32_t K, N, ntn;         // ntn = N/128 column blocks
    float limit;
};

constexpr int GU_RB = 256;    // activation bytes per row and K step (bf16)
using GuStage = AStage<GU_RB>;
constexpr int GU_STAGE = GuStage::S_OFF + 2 * RMAX * 4;   // rows, gate factors, up factors

// K order inside a step (the same for both operands of every MFMA): MFMA k
// of lane group q takes K 16q + 8k .. +7 for k = 0, 1 and 64 + 16q + 8(k-2)
// .. +7 for k = 2, 3, i.e. 16-byte bf16 chunks 2q, 2q+1, 8+2q, 9+2q of the
// activation row and bytes 16q.., 64+16q.. of the weight row.
__device__ __forceinline__ int gu_chunk(int q, int k) { return (k < 2 ? 0 : 8) + 2 * q + (k & 1); }

// Block: 8 waves, two per SIMD, so one wave's weight conversions and
// promotions issue while the other's MFMAs run.  Wave w = every row of the
// chunk x h columns n0 + 16w .. +15 of gate and of up (two 16-column operand
// tiles), so gate and up of one h element sit in the same lane and the
// SwiGLU needs no exchange.  Every wave reads the chunk's whole activation
// tile from LDS; the weights stream from global memory straight into VGPRs in
// the MFMA operand layout, G8_D K steps ahead, and are converted to bf16 in
// registers once per wave.  The activation codes of step kb+1 move global ->
// VGPRs -> LDS (converted to bf16 once per block) while step kb multiplies;
// they are loaded two steps ahead.
constexpr int G8_THREADS = 512;
constexpr int G8_D = 2;       // K steps of weights in flight per wave

struct G8B {
    u32x4 v[4];               // [tile: gate, up][half]
};

struct G8A {
    u32x4 v[2];               // 16 codes of rows t/8 and t/8 + 64
    float s;                  // activation scale of row t % 128
};

template <int NJ>
__device__ __forceinline__ G8A g8_load_a(const uint8_t *xq, const float *xs, const uint32_t (&off)[2],
                                         uint32_t soff, int kb)
{
    G8A r;
#pragma unroll
    for (int j = 0; j < NJ; ++j) r.v[j] = moe::load_global<u32x4>(xq + (off[j] + (uint32_t)kb * BK));
    r.s = moe::load_global<float>(xs + (soff + (uint32_t)kb));
    return r;
}

// thread t: bf16 chunks 2(t % 8), 2(t % 8) + 1 of rows t / 8 (+ 64), and the
// promotion factor t % 256 (gate factors of the 128 rows, then up factors)
template <int NJ>
__device__ __forceinline__ void g8_store_a(uint8_t *st, const G8A &r, int tid, float swg, float swu)
{
    using L = AStage<256>;
    const int r0 = (tid >> 3) & 63, c8 = tid & 7;
    const uint32_t lo = r0 * 256 + L::swz(r0, 2 * c8) * 16;
    const uint32_t hi = r0 * 256 + L::swz(r0, 2 * c8 + 1) * 16;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const u32x4 v = r.v[j];
        *reinterpret_cast<bf16x8 *>(st + lo + 64 * 256 * j) = cvt8(v[0], v[1]);
        *reinterpret_cast<bf16x8 *>(st + hi + 64 * 256 * j) = cvt8(v[2], v[3]);
    }
    // threads t and t + 256 hold the same factor: both store it
    reinterpret_cast<float *>(st + L::S_OFF)[tid & 255] = r.s * ((tid & 128) ? swu : swg);
}

template <int NRS>
__device__ __forceinline__ void gateup8_chunk(const GuArgs &a, int e, int p0, int rows, int nb,
                                              uint8_t *sm)
{
    constexpr int NJ = NRS <= 4 ? 1 : 2;     // 64-row groups of A codes moved per step
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int q = lane >> 4, r16 = lane & 15;
    const int K = a.K, N = a.N, KB = K / BK;
    const int n0 = nb * 128;

    uint32_t off[2] = {0u, 0u}, soff;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int row = 64 * j + ((tid >> 3) & 63);
        off[j] = (uint32_t)a.sorted_token[p0 + (row < rows ? row : 0)] * (uint32_t)K + (tid & 7) * 16;
    }
    {
        const int row = tid & (RMAX - 1);
        soff = (uint32_t)a.sorted_token[p0 + (row < rows ? row : 0)] * KB;
    }
    uint32_t aoff[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) aoff[k] = r16 * GU_RB + GuStage::swz(r16, gu_chunk(q, k)) * 16;

    const uint8_t *gbase = moe::uniform_ptr(a.w0 + ((size_t)e * N + n0 + 16 * wave) * K);
    const uint8_t *ubase = moe::uniform_ptr(a.w1 + ((size_t)e * N + n0 + 16 * wave) * K);
    const uint32_t boff = (uint32_t)r16 * K + 16 * q;
    auto load_b = [&](int kb) {
        G8B b;
        const uint32_t k0 = (uint32_t)kb * BK;
        b.v[0] = moe::load_global<u32x4>(gbase + (boff + k0));
        b.v[1] = moe::load_global<u32x4>(gbase + (boff + k0 + 64));
        b.v[2] = moe::load_global<u32x4>(ubase + (boff + k0));
        b.v[3] = moe::load_global<u32x4>(ubase + (boff + k0 + 64));
        return b;
    };

    const float *sg = a.ws0 + ((size_t)e * a.ntn + nb) * KB;
    const float *su = a.ws1 + ((size_t)e * a.ntn + nb) * KB;
    const float g_lo = lane < KB ? sg[lane] : 0.0f, g_hi = lane + 64 < KB ? sg[lane + 64] : 0.0f;
    const float u_lo = lane < KB ? su[lane] : 0.0f, u_hi = lane + 64 < KB ? su[lane + 64] : 0.0f;

    f32x4 acc[NRS][2];
#pragma unroll
    for (int i = 0; i < NRS; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int klast = KB - 1;
    G8B b[G8_D];
    G8A ar[2];
    if constexpr (G8_D == 4) b[0] = load_b(0);
    ar[0] = g8_load_a<NJ>(a.xq, a.xs, off, soff, 0);
    if constexpr (G8_D == 4) b[1] = load_b(min(1, klast));
    ar[1] = g8_load_a<NJ>(a.xq, a.xs, off, soff, min(1, klast));
    b[G8_D - 2] = load_b(min(G8_D - 2, klast));
    g8_store_a<NJ>(sm, ar[0], tid, lane_f(g_lo, 0), lane_f(u_lo, 0));
    ar[0] = g8_load_a<NJ>(a.xq, a.xs, off, soff, min(2, klast));
    b[G8_D - 1] = load_b(min(G8_D - 1, klast));
    moe::lds_barrier();

    auto step = [&](int kb, G8B &bk, G8A &an, uint8_t *cur, uint8_t *nxt) {
        {
            const int kn = kb + 1;
            g8_store_a<NJ>(nxt, an, tid, lane_f(kn < 64 ? g_lo : g_hi, kn & 63),
                           lane_f(kn < 64 ? u_lo : u_hi, kn & 63));
        }
        an = g8_load_a<NJ>(a.xq, a.xs, off, soff, min(kb + 3, klast));
        // this step's weights as bf16 operands; their registers take the
        // load of step kb + G8_D at once
        bf16x8 bw[2][4];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const u32x4 &v = bk.v[2 * c + (k >> 1)];
                bw[c][k] = cvt8(v[2 * (k & 1)], v[2 * (k & 1) + 1]);
            }
        bk = load_b(min(kb + G8_D, klast));
        // Row tiles in pairs, K-outer inside a pair: the 2 x 2 block sums of a
        // pair are independent MFMA chains, four deep.  Software pipeline,
        // fenced so the scheduler keeps it: the activation operands of the
        // next K slice (or of the next pair's first) are read while this
        // slice's MFMAs run, and a pair is promoted beside the next pair's
        // first MFMAs.
        const float *ss = reinterpret_cast<const float *>(cur + GuStage::S_OFF);
        auto a_op = [&](int k, int rs) {
            return *reinterpret_cast<const bf16x8 *>(cur + aoff[k] + 16 * GU_RB * rs);
        };
        f32x4 tp[2][2], fgp[2], fup[2];
        auto promote = [&](int rs0) {
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[rs0 + r][0][i] = fmaf(tp[r][0][i], fgp[r][i], acc[rs0 + r][0][i]);
                    acc[rs0 + r][1][i] = fmaf(tp[r][1][i], fup[r][i], acc[rs0 + r][1][i]);
                }
        };
        bf16x8 acur[2], anxt[2];
        acur[0] = a_op(0, 0);
        acur[1] = a_op(0, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g0 = 0; g0 < NRS; g0 += 2) {
            f32x4 t[2][2], fg[2], fu[2];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool more = k < 3 || g0 + 2 < NRS;
                if (more) {
#pragma unroll
                    for (int r = 0; r < 2; ++r) anxt[r] = k < 3 ? a_op(k + 1, g0 + r) : a_op(0, g0 + 2 + r);
                }
                if (k == 0) {
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        fg[r] = *reinterpret_cast<const f32x4 *>(ss + (g0 + r) * 16 + 4 * q);
                        fu[r] = *reinterpret_cast<const f32x4 *>(ss + RMAX + (g0 + r) * 16 + 4 * q);
                    }
                }
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const f32x4 zg = k == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : t[r][0];
                    const f32x4 zu = k == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : t[r][1];
                    t[r][0] = mfma_bf16(acur[r], bw[0][k], zg);
                    t[r][1] = mfma_bf16(acur[r], bw[1][k], zu);
                }
                if (k == 0 && g0 > 0) promote(g0 - 2);
                if (more) {
                    acur[0] = anxt[0];
                    acur[1] = anxt[1];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                tp[r][0] = t[r][0];
                tp[r][1] = t[r][1];
                fgp[r] = fg[r];
                fup[r] = fu[r];
            }
        }
        promote(NRS - 2);
        moe::lds_barrier();
    };

    uint8_t *s0 = sm, *s1 = sm + GU_STAGE;
    static_assert(G8_D == 2 || G8_D == 4, "the K loop is unrolled by 4");
#pragma unroll 1
    for (int kb0 = 0; kb0 < KB; kb0 += 4) {
        step(kb0, b[0], ar[1], s0, s1);
        step(kb0 + 1, b[1 % G8_D], ar[0], s1, s0);
        step(kb0 + 2, b[2 % G8_D], ar[1], s0, s1);
        step(kb0 + 3, b[3 % G8_D], ar[0], s1, s0);
    }

    // epilogue: h = SwiGLU(g, u); per-row amax of the wave's 16 columns, then
    // over the 8 waves through LDS
    float *rmax = reinterpret_cast<float *>(sm);          // [8 waves][RMAX]
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[rs][0][i] = swiglu_clamp(acc[rs][0][i], acc[rs][1][i], a.limit);
            float m = fabsf(acc[rs][0][i]);
#pragma unroll
            for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
            if (r16 == 0) rmax[wave * RMAX + rs * 16 + 4 * q + i] = m;
        }
    }
    __syncthreads();
    uint8_t *ct = sm + 8 * RMAX * 4;                      // codes tile [RMAX][144]
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rs * 16 + 4 * q + i;
            float amax = rmax[r];
#pragma unroll
            for (int w = 1; w < 8; ++w) amax = fmaxf(amax, rmax[w * RMAX + r]);
            const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;
            ct[r * 144 + 16 * wave + r16] = (uint8_t)(e4m3_pair(acc[rs][0][i] / scale, 0.0f) & 0xFFu);
            if (wave == 0 && r16 == 0 && r < rows) a.hs[(size_t)(p0 + r) * a.ntn + nb] = scale;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < (NRS + 3) / 4; ++j) {
        const int r = 64 * j + (tid >> 3), part = tid & 7;
        if (r < rows)
            *reinterpret_cast<uint4 *>(a.hq + (size_t)(p0 + r) * N + n0 + part * 16) =
                *reinterpret_cast<const uint4 *>(ct + r * 144 + part * 16);
    }
}

__global__ __launch_bounds__(G8_THREADS, 1) void gemm_gateup8_kernel(GuArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t sm[2 * GU_STAGE];
    int4 tile;
    int nb;
    if (!gemm_item(a, tile, nb)) return;
    const int e = tile.x, p0 = tile.y;
    const int rows = moe::uniform(chunk_rows(a.offsets, e, p0, tile.w));
    if (rows <= 0) return;
    switch ((rows + 31) >> 5) {
    case 1: gateup8_chunk<2>(a, e, p0, rows, nb, sm); break;
    case 2: gateup8_chunk<4>(a, e, p0, rows, nb, sm); break;
    case 3: gateup8_chunk<6>(a, e, p0, rows, nb, sm); break;
    default: gateup8_chunk<8>(a, e, p0, rows, nb, sm); break;
    }
}

// ---------------------------------------------------------------------------
// down, FP8 MFMA, persistent
// ---------------------------------------------------------------------------
// The W = chunks x (N/128) items (one chunk of <= 128 rows x 128 outputs of
// y each) split into 8 contiguous runs in the order of gemm_item, one per XCD
// (block b runs on XCD b % 8), and the blocks of an XCD deal its run out
// round-robin: the items in flight on an XCD at any time are neighbours (the
// chunks of one expert on one weight block, then the next column block), so
// they share weight blocks and h rows in that XCD's L2.  A block runs its
// items as one continuous K-step pipeline: every step's operands (128 h rows,
// 128 weight rows, the h scales and the weight block scale) go from global
// memory straight into a ring of LDS stages (DMA), and the loads of the next
// item's first steps are in flight while the current item finishes and
// stores its y block, so no item pays the ramp of its first loads.  Only the
// descriptors are read before the pipeline starts: each block decodes its
// items into LDS once.  Waves as 2 x 2, 64 x 64 outputs each.
struct DnArgs {
    const uint8_t *hq;         // h codes [S][K] (packed rows)
    const float *hs;           // h scales [S][K/128]
    const uint8_t *w0;         // down codes [E][N][K]
    const float *ws0;          // block scales [E][N/128][K/128]
    const int32_t *offsets;
    const int4 *tiles;
    const int32_t *ntiles;
    float *y;                  // [S][N]
    int32_t K, N, ntn;
};

constexpr int DN_NST = 2;                 // LDS stages (DN_NST - 1 K steps in flight)
constexpr int DN_BPC = 2;                 // blocks per CU
constexpr int DN_MAXI = 256;              // items per block (the host sizes the grid for it)
constexpr int DN_A = 0, DN_B = 128 * 128, DN_S = DN_B + 128 * 128, DN_W = DN_S + 4 * 256;
constexpr int DN_STAGE = DN_W + 4 * 256;
constexpr int DN_PER = 4 + 4 + 1 + 1;     // DMA instructions per stage and wave
static_assert(DN_BPC * (DN_NST * DN_STAGE + DN_MAXI * 16) <= 160 * 1024, "down stages exceed LDS");
static_assert((DN_NST - 2) * DN_PER < 64, "vmcnt is 6 bits");

// A 16 x 128 FP8 operand from a swizzled 128-byte-row tile: lane l takes
// row l % 16, bytes 32 (l / 16) .. +31.
__device__ __forceinline__ i32x8 lds_op(const uint8_t *tile, int row, int lane)
{
    const int c = (lane >> 4) * 2;
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(tile + (row * 128 + swz(row, c) * 16));
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(tile + (row * 128 + swz(row, c + 1) * 16));
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__global__ __launch_bounds__(kThreads, DN_BPC) void gemm_down_kernel(DnArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t sm[DN_NST * DN_STAGE];
    __shared__ int4 s_item[DN_MAXI];       // (expert, first row, rows, column block)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int K = a.K, N = a.N, KB = K / BK;

    // this block's items: L = begin + bi + t * nbx, t < T
    const int W = moe::uniform(*a.ntiles) * a.ntn;
    const int x = blockIdx.x & 7, bi = blockIdx.x >> 3, nbx = gridDim.x >> 3;
    const int q = W >> 3, rr = W & 7;
    const int begin = x * q + min(x, rr), len = q + (x < rr ? 1 : 0);
    const int T = bi < len ? min((len - bi + nbx - 1) / nbx, DN_MAXI) : 0;
    if (T == 0) return;
    if (tid < T) {
        const int L = begin + bi + tid * nbx;
        const int4 head = a.tiles[L / a.ntn];
        const int local = L - head.z * a.ntn;
        const int4 tl = a.tiles[head.z + local % head.w];
        const int lo = a.offsets[tl.x], hi = a.offsets[tl.x + 1];
        const int cs = (hi - lo + head.w - 1) / head.w;
        const int rows = min(cs, hi - tl.y);
        // a chunk with no rows loads the expert's first row and stores nothing
        s_item[tid] = make_int4(tl.x, rows > 0 ? tl.y : lo, rows, local / head.w);
    }
    __syncthreads();

    // issue side: per-thread sources of the item being loaded
    uint32_t aoff[4], boff[4], soff = 0;
    const uint8_t *wbase = nullptr;
    const float *wsb = nullptr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (wave * 4 + j) * 8 + (lane >> 3);
        boff[j] = (uint32_t)r * K + swz(r, lane & 7) * 16;
        aoff[j] = 0;
    }
    auto set_issue = [&](int t) {
        const int4 d = s_item[t];
        const int e = moe::uniform(d.x), p0 = moe::uniform(d.y), rows = moe::uniform(d.z);
        const int nb = moe::uniform(d.w);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = (wave * 4 + j) * 8 + (lane >> 3);
            aoff[j] = (uint32_t)(p0 + (r < rows ? r : 0)) * K + swz(r, lane & 7) * 16;
        }
        const int srow = wm * 64 + lane;
        soff = (uint32_t)(p0 + (srow < rows ? srow : 0)) * KB * 4;
        wbase = moe::uniform_ptr(a.w0 + ((size_t)e * N + (size_t)nb * 128) * K);
        wsb = moe::uniform_ptr(a.ws0 + ((size_t)e * a.ntn + nb) * KB);
    };
    auto issue = [&](int kb, uint8_t *st) {
        const uint8_t *ab = a.hq + (size_t)kb * BK, *bb = wbase + (size_t)kb * BK;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(ab, aoff[j], lds_addr(st + DN_A + (wave * 4 + j) * 1024));
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(bb, boff[j], lds_addr(st + DN_B + (wave * 4 + j) * 1024));
        dma4(a.hs + kb, soff, lds_addr(st + DN_S + wave * 256));
        dma4(wsb + kb, 0u, lds_addr(st + DN_W + wave * 256));     // one float, every lane
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const uint8_t *st) {
        const float sw = *reinterpret_cast<const float *>(st + DN_W + wave * 256);
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
    auto store_y = [&](int t) {
        const int4 d = s_item[t];
        const int p0 = moe::uniform(d.y), rows = moe::uniform(d.z), nb = moe::uniform(d.w);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + mt * 16 + (lane >> 4) * 4 + i;
                if (r < rows) {
                    float *yr = a.y + (size_t)(p0 + r) * N + nb * 128 + wn * 64 + (lane & 15);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) yr[nt * 16] = acc[mt][nt][i];
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) acc[mt][nt][i] = 0.0f;
            }
    };

    // the block's T x KB steps as one ring of DN_NST stages
    const int G = T * KB;
    int it = 0, ikb = 0;                 // next step to load: item it, K step ikb
    set_issue(0);
    auto advance = [&]() {
        if (++ikb == KB) {
            ikb = 0;
            if (++it < T) set_issue(it);
        }
    };
    MOE_WAIT_VM(0);
#pragma unroll
    for (int j = 0; j < DN_NST - 1; ++j)
        if (j < G) {
            issue(ikb, sm + j * DN_STAGE);
            advance();
        }
    int cs = 0, is = DN_NST - 1, ckb = 0, ct = 0;
    for (int g = 0; g < G; ++g) {
        wait_stages<DN_PER, DN_NST - 2>(G - 1 - g);
        MOE_WAIT_LGKM0();
        MOE_BARRIER();
        if (g + DN_NST - 1 < G) {
            issue(ikb, sm + is * DN_STAGE);
            advance();
        }
        // y of the item finished last step, stored under the loads in flight
        if (ckb == 0 && g > 0) store_y(ct - 1);
        compute(sm + cs * DN_STAGE);
        cs = cs + 1 == DN_NST ? 0 : cs + 1;
        is = is + 1 == DN_NST ? 0 : is + 1;
        if (++ckb == KB) {
            ckb = 0;
            ++ct;
        }
    }
    store_y(T - 1);
}

}  // namespace

int gemm_max_tiles(int32_t S, int32_t E) { return (S < E ? S : E) + (S + TILE_ROWS - 1) / TILE_ROWS; }

hipError_t launch_quant_act(const uint16_t *x, int32_t M, int32_t hidden, uint8_t *xq, float *xs,
                            hipStream_t st)
{
    const int64_t n16 = (int64_t)M * hidden / 16;
    hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st, x,
                       n16, xq, xs);
    return hipGetLastError();
}

hipError_t launch_gemm_tiles(const int32_t *offsets, int32_t E, int32_t tmax, int4 *tiles,
                             int32_t *ntiles, hipStream_t st, bool balanced)
{
    static_assert(RMAX == TILE_ROWS, "both tiers share gemm_max_tiles");
    hipLaunchKernelGGL(gemm_tiles_kernel, dim3(1), dim3(1024), 0, st, offsets, E, tmax,
                       balanced ? RMAX : TILE_ROWS, balanced ? 1 : 0, tiles, ntiles);
    return hipGetLastError();
}

hipError_t launch_gemm_gateup(const uint8_t *xq, const float *xs, const int32_t *sorted_token,
                              const uint8_t *gcodes, const float *gscales, const uint8_t *ucodes,
                              const float *uscales, const int32_t *offsets, const int4 *tiles,
                              const int32_t *ntiles, int32_t tmax, int32_t hidden, int32_t inter,
                              float limit, uint8_t *hq, float *hs, hipStream_t st)
{
    GuArgs a{};
    a.xq = xq; a.xs = xs; a.sorted_token = sorted_token;
    a.w0 = gcodes; a.w1 = ucodes; a.ws0 = gscales; a.ws1 = uscales;
    a.offsets = offsets; a.tiles = tiles; a.ntiles = ntiles;
    a.hq = hq; a.hs = hs; a.K = hidden; a.N = inter; a.ntn = inter / 128; a.limit = limit;
    hipLaunchKernelGGL(gemm_gateup8_kernel, dim3((unsigned)(tmax * a.ntn)), dim3(G8_THREADS), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gemm_down(const uint8_t *hq, const float *hs, const uint8_t *dcodes,
                            const float *dscales, const int32_t *offsets, const int4 *tiles,
                            const int32_t *ntiles, int32_t tmax, int32_t hidden, int32_t inter,
                            float *y, hipStream_t st)
{
    DnArgs a{};
    a.hq = hq; a.hs = hs; a.w0 = dcodes; a.ws0 = dscales;
    a.offsets = offsets; a.tiles = tiles; a.ntiles = ntiles;
    a.y = y; a.K = inter; a.N = hidden; a.ntn = hidden / 128;
    // DN_BPC blocks per CU, more where a block would hold over DN_MAXI items
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    const int64_t wmax = (int64_t)tmax * a.ntn;
    const int64_t per_xcd = (wmax + 7) / 8;
    const int64_t nbx = std::max<int64_t>((DN_BPC * cus + 7) / 8, (per_xcd + DN_MAXI - 1) / DN_MAXI);
    hipLaunchKernelGGL(gemm_down_kernel, dim3((unsigned)(8 * nbx)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}
