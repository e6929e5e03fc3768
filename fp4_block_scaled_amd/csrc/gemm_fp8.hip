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
//   gemm_gateup_kernel  one block = one chunk of <= 128 rows of one expert x
//                       128 h columns: the gate AND the up projection of
//                       those columns, the clamped SwiGLU, and the E4M3
//                       quantization of the 128-wide h row segment (exactly
//                       one 1x128 group) in the epilogue.
//   gemm_down_kernel    one block = one chunk x 128 outputs of y.
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
// Data movement.  Weights are read once per chunk straight from global
// memory into VGPRs, in exactly the lane layout of the MFMA operand (lane l:
// row l % 16, 32 bytes of K), several K steps ahead; they never touch LDS.
// The activation rows of the chunk, shared by every wave, go to LDS (XOR
// swizzled, two stages) through VGPRs.  All loads are ordinary compiler-
// visible loads, so the compiler's waits are exact.
//
// K order inside a 128-wide block: a lane's 32 bytes are K offsets
// 16q..16q+15 and 64+16q..64+16q+15 (q = lane / 16), so each half is one
// 16-byte load of a row; A and B use the same order, and a dot product over
// the block does not depend on the order of its terms.
#include "gemm_common.h"

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
// A chunk's activation rows for one K step of 128 move global -> VGPRs ->
// LDS.  RB = bytes of one row's K step: 256 for gate/up (bf16 values of the
// x codes), 128 for down (E4M3 h codes).  A row is RB/16 16-byte chunks;
// thread t moves chunk t % C of rows G*j + t / C (C = RB/16, G = 256/C row
// groups per pass), j = 0..NJ-1, and thread t the activation scale of row
// t % RMAX.  Rows past the chunk's read its first row: their products land
// in output rows that are never stored.
template <int RB>
struct AStage {
    static constexpr int C = RB / 16;                 // 16-byte chunks per row
    static constexpr int G = kThreads / C;            // rows per pass
    static constexpr int S_OFF = RMAX * RB;           // scales after the rows
    static constexpr int BYTES = S_OFF + RMAX * 4;
    // physical chunk of logical chunk c in row r: an XOR with the row's low
    // bits, so the 16 rows an operand read touches at one logical chunk land
    // on distinct chunks (distinct banks), and so do the chunks of one row
    // written by consecutive threads
    static __device__ __forceinline__ int swz(int r, int c)
    {
        if constexpr (C == 16) return c ^ (r & 15);
        else return ::swz(r, c);
    }
};

template <int RB, int NJ>
struct ARegs {
    u32x4 v[NJ];
    float s;
};

// Per-thread sources: byte offsets at K step 0 of its row chunks and of its
// scale.
template <int NJ>
struct ASrc {
    uint32_t off[NJ];
    uint32_t soff;
};

template <int RB, int NJ>
__device__ __forceinline__ ARegs<RB, NJ> load_a(const uint8_t *a, const float *as,
                                                const ASrc<NJ> &src, int kb)
{
    ARegs<RB, NJ> r;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        r.v[j] = moe::load_global<u32x4>(a + (src.off[j] + (uint32_t)kb * RB));
    r.s = moe::load_global<float>(as + (src.soff + (uint32_t)kb));
    return r;
}

// Byte offset in a stage where thread t stores its chunk of row group 0; row
// group j is G*j rows (G*j*RB bytes) further, and the swizzle depends only on
// the row's low bits, which j does not change.
template <int RB>
__device__ __forceinline__ uint32_t a_store_base(int tid)
{
    using L = AStage<RB>;
    const int row = tid / L::C;
    return row * RB + L::swz(row, tid % L::C) * 16;
}

template <int RB, int NJ>
__device__ __forceinline__ void store_a(uint8_t *st, const ARegs<RB, NJ> &r, int tid, uint32_t sbase)
{
    using L = AStage<RB>;
#pragma unroll
    for (int j = 0; j < NJ; ++j) *reinterpret_cast<u32x4 *>(st + sbase + L::G * RB * j) = r.v[j];
    // threads t and t + RMAX hold the same row's scale: both store it
    reinterpret_cast<float *>(st + L::S_OFF)[tid & (RMAX - 1)] = r.s;
}

// Gate/up staging: thread t loaded 16 E4M3 codes (chunk t % 8) of rows 32j +
// t / 8 and stores them as 32 bytes of bf16 values (bf16 chunks 2(t % 8) and
// 2(t % 8) + 1 of the 256-byte bf16 row).  Each code is converted once per
// block.
template <int NJ>
__device__ __forceinline__ void store_a_bf16(uint8_t *st, const ARegs<128, NJ> &r, int tid)
{
    using L = AStage<256>;
    const int r0 = tid >> 3, c8 = tid & 7;
    const uint32_t lo = r0 * 256 + L::swz(r0, 2 * c8) * 16;
    const uint32_t hi = r0 * 256 + L::swz(r0, 2 * c8 + 1) * 16;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const u32x4 v = r.v[j];
        *reinterpret_cast<bf16x8 *>(st + lo + 32 * 256 * j) = cvt8(v[0], v[1]);
        *reinterpret_cast<bf16x8 *>(st + hi + 32 * 256 * j) = cvt8(v[2], v[3]);
    }
    reinterpret_cast<float *>(st + L::S_OFF)[tid & (RMAX - 1)] = r.s;
}

// ---------------------------------------------------------------------------
// gate + up (+ SwiGLU + h quantization), bf16 MFMA
// ---------------------------------------------------------------------------
// Block: 4 waves, one per SIMD; wave w = every row of the chunk x h columns
// n0 + 32w .. +31 of gate and of up (four 16-column operand tiles: gate
// 0-15, gate 16-31, up 0-15, up 16-31), so gate and up of one h element sit
// in the same lane and the SwiGLU needs no exchange.  One activation operand
// (read from LDS) feeds the four tiles.
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

constexpr int GU_D = 4;       // K steps of weights in flight per wave (2 or 4)
constexpr int GU_RB = 256;    // activation bytes per row and K step (bf16)
using GuStage = AStage<GU_RB>;

struct GuB {
    u32x4 v[8];               // [operand tile c][half]: weight rows' 32 bytes of K
};

// K order inside a step (the same for both operands of every MFMA): MFMA k
// of lane group q takes K 16q + 8k .. +7 for k = 0, 1 and 64 + 16q + 8(k-2)
// .. +7 for k = 2, 3, i.e. 16-byte bf16 chunks 2q, 2q+1, 8+2q, 9+2q of the
// activation row and bytes 16q.., 64+16q.. of the weight row.
__device__ __forceinline__ int gu_chunk(int q, int k) { return (k < 2 ? 0 : 8) + 2 * q + (k & 1); }

// Chunk body for NRS 16-row operand tiles (rows <= 16 * NRS).
template <int NRS>
__device__ __forceinline__ void gateup_chunk(const GuArgs &a, int e, int p0, int rows, int nb,
                                             uint8_t *sm)
{
    constexpr int NJ = (NRS + 1) / 2;         // 32-row groups of A codes moved per step
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int q = lane >> 4, r16 = lane & 15;
    const int K = a.K, N = a.N, KB = K / BK;
    const int n0 = nb * 128;

    // activation sources (gathered token rows, 16 codes per thread and row group)
    ASrc<NJ> src;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int row = 32 * j + (tid >> 3);
        src.off[j] = (uint32_t)a.sorted_token[p0 + (row < rows ? row : 0)] * (uint32_t)K + (tid & 7) * 16;
    }
    {
        const int row = tid & (RMAX - 1);
        src.soff = (uint32_t)a.sorted_token[p0 + (row < rows ? row : 0)] * KB;
    }
    uint32_t aoff[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) aoff[k] = r16 * GU_RB + GuStage::swz(r16, gu_chunk(q, k)) * 16;
    const uint8_t *xa = a.xq;

    // weight rows of this wave: gate n0+32w+r16 (+16), up likewise; lane
    // offset within a 16-row operand tile: row r16, bytes 16q
    const uint8_t *gbase = moe::uniform_ptr(a.w0 + ((size_t)e * N + n0 + 32 * wave) * K);
    const uint8_t *ubase = moe::uniform_ptr(a.w1 + ((size_t)e * N + n0 + 32 * wave) * K);
    const uint32_t boff = (uint32_t)r16 * K + 16 * q;
    const uint32_t boff16 = boff + 16u * K;
    auto load_b = [&](int kb) {
        GuB b;
        const uint32_t k0 = (uint32_t)kb * BK;
        b.v[0] = moe::load_global<u32x4>(gbase + (boff + k0));
        b.v[1] = moe::load_global<u32x4>(gbase + (boff + k0 + 64));
        b.v[2] = moe::load_global<u32x4>(gbase + (boff16 + k0));
        b.v[3] = moe::load_global<u32x4>(gbase + (boff16 + k0 + 64));
        b.v[4] = moe::load_global<u32x4>(ubase + (boff + k0));
        b.v[5] = moe::load_global<u32x4>(ubase + (boff + k0 + 64));
        b.v[6] = moe::load_global<u32x4>(ubase + (boff16 + k0));
        b.v[7] = moe::load_global<u32x4>(ubase + (boff16 + k0 + 64));
        return b;
    };

    // weight block scales of this column block, K block j in lane j % 64 of
    // register j / 64 (K <= 16384); a uniform readlane picks one per K step
    const float *sg = a.ws0 + ((size_t)e * a.ntn + nb) * KB;
    const float *su = a.ws1 + ((size_t)e * a.ntn + nb) * KB;
    const float g_lo = lane < KB ? sg[lane] : 0.0f, g_hi = lane + 64 < KB ? sg[lane + 64] : 0.0f;
    const float u_lo = lane < KB ? su[lane] : 0.0f, u_hi = lane + 64 < KB ? su[lane + 64] : 0.0f;

    f32x4 acc[NRS][4];
#pragma unroll
    for (int i = 0; i < NRS; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Step kb: store A(kb+1) into the other stage, load A(kb+3), convert the
    // weights of kb, load those of kb+4, multiply, barrier.  Every step runs
    // unconditionally: loads past the last K step re-read it (valid memory),
    // and a step past the end adds nothing (its weight block scale, a lane
    // past KB, is 0).  The prologue issues the loads of steps -4..-1 in the
    // same order, so the waits the compiler places are those of the steady
    // state.
    const int klast = KB - 1;
    GuB b[GU_D];
    ARegs<128, NJ> ar[2];
    // steps -4..-1 of the pattern: A loads of steps 0..2, weight loads of
    // steps 0..D-1 (each after the A load issued in the same step)
    if constexpr (GU_D == 4) b[0] = load_b(0);
    ar[0] = load_a<128, NJ>(xa, a.xs, src, 0);
    if constexpr (GU_D == 4) b[1] = load_b(min(1, klast));
    ar[1] = load_a<128, NJ>(xa, a.xs, src, min(1, klast));
    b[GU_D - 2] = load_b(min(GU_D - 2, klast));
    store_a_bf16<NJ>(sm, ar[0], tid);
    ar[0] = load_a<128, NJ>(xa, a.xs, src, min(2, klast));
    b[GU_D - 1] = load_b(min(GU_D - 1, klast));
    moe::lds_barrier();

    auto step = [&](int kb, GuB &bk, ARegs<128, NJ> &an, uint8_t *cur, uint8_t *nxt) {
        __builtin_amdgcn_sched_barrier(0);
        // A of step kb+1 (loaded two steps ago) into the other stage, whose
        // last reader (step kb-1) every wave has passed
        store_a_bf16<NJ>(nxt, an, tid);
        an = load_a<128, NJ>(xa, a.xs, src, min(kb + 3, klast));
        // this step's weights as bf16 operands, then the next load into the registers
        bf16x8 bw[4][4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const u32x4 &v = bk.v[2 * c + t];
                bw[c][2 * t] = cvt8(v[0], v[1]);
                bw[c][2 * t + 1] = cvt8(v[2], v[3]);
            }
        bk = load_b(min(kb + GU_D, klast));
        const float swg = lane_f(kb < 64 ? g_lo : g_hi, kb & 63);
        const float swu = lane_f(kb < 64 ? u_lo : u_hi, kb & 63);
        const float *ss = reinterpret_cast<const float *>(cur + GuStage::S_OFF);
        // operand tile rs: its MFMAs, the promotion of tile rs-1 (independent
        // VALU work beside them), and the LDS reads of tile rs+1; then a
        // scheduling fence, so no tile's reads are hoisted further
        bf16x8 av[4], an4[4];
        f32x4 sx, snx, t[4], tp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) av[k] = *reinterpret_cast<const bf16x8 *>(cur + aoff[k]);
        sx = *reinterpret_cast<const f32x4 *>(ss + 4 * q);
        auto promote = [&](int r, const f32x4 (&tt)[4], const f32x4 &sxr) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float fg = sxr[i] * swg, fu = sxr[i] * swu;
                acc[r][0][i] = fmaf(tt[0][i], fg, acc[r][0][i]);
                acc[r][1][i] = fmaf(tt[1][i], fg, acc[r][1][i]);
                acc[r][2][i] = fmaf(tt[2][i], fu, acc[r][2][i]);
                acc[r][3][i] = fmaf(tt[3][i], fu, acc[r][3][i]);
            }
        };
        f32x4 sp;
#pragma unroll
        for (int rs = 0; rs < NRS; ++rs) {
            if (rs + 1 < NRS) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    an4[k] = *reinterpret_cast<const bf16x8 *>(cur + aoff[k] + 16 * GU_RB * (rs + 1));
                snx = *reinterpret_cast<const f32x4 *>(ss + (rs + 1) * 16 + 4 * q);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) t[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int c = 0; c < 4; ++c) t[c] = mfma_bf16(av[k], bw[c][k], t[c]);
            if (rs > 0) promote(rs - 1, tp, sp);
#pragma unroll
            for (int c = 0; c < 4; ++c) tp[c] = t[c];
            sp = sx;
            if (rs + 1 < NRS) {
#pragma unroll
                for (int k = 0; k < 4; ++k) av[k] = an4[k];
                sx = snx;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        promote(NRS - 1, tp, sp);
        moe::lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    uint8_t *s0 = sm, *s1 = sm + GuStage::BYTES;
    static_assert(GU_D == 2 || GU_D == 4, "the K loop is unrolled by 4");
#pragma unroll 1
    for (int kb0 = 0; kb0 < KB; kb0 += 4) {
        step(kb0, b[0], ar[1], s0, s1);
        step(kb0 + 1, b[1 % GU_D], ar[0], s1, s0);
        step(kb0 + 2, b[2 % GU_D], ar[1], s0, s1);
        step(kb0 + 3, b[3 % GU_D], ar[0], s1, s0);
    }

    // epilogue: h = SwiGLU(g, u) in place of the gate sums; per-row amax of
    // the wave's 32 columns, then over the 4 waves through LDS
    float *rmax = reinterpret_cast<float *>(sm);          // [4 waves][RMAX]
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[rs][0][i] = swiglu_clamp(acc[rs][0][i], acc[rs][2][i], a.limit);
            acc[rs][1][i] = swiglu_clamp(acc[rs][1][i], acc[rs][3][i], a.limit);
            float m = fmaxf(fabsf(acc[rs][0][i]), fabsf(acc[rs][1][i]));
#pragma unroll
            for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
            if (r16 == 0) rmax[wave * RMAX + rs * 16 + 4 * q + i] = m;
        }
    }
    __syncthreads();
    uint8_t *ct = sm + 4 * RMAX * 4;                      // codes tile [RMAX][144]
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rs * 16 + 4 * q + i;
            const float amax = fmaxf(fmaxf(rmax[r], rmax[RMAX + r]),
                                     fmaxf(rmax[2 * RMAX + r], rmax[3 * RMAX + r]));
            const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;
            const uint32_t c2 = e4m3_pair(acc[rs][0][i] / scale, acc[rs][1][i] / scale);
            ct[r * 144 + 32 * wave + r16] = (uint8_t)(c2 & 0xFFu);
            ct[r * 144 + 32 * wave + 16 + r16] = (uint8_t)(c2 >> 8);
            if (wave == 0 && r16 == 0 && r < rows) a.hs[(size_t)(p0 + r) * a.ntn + nb] = scale;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < (NRS + 1) / 2; ++j) {
        const int r = 32 * j + (tid >> 3), part = tid & 7;
        if (r < rows)
            *reinterpret_cast<uint4 *>(a.hq + (size_t)(p0 + r) * N + n0 + part * 16) =
                *reinterpret_cast<const uint4 *>(ct + r * 144 + part * 16);
    }
}

__global__ __launch_bounds__(kThreads, 1) void gemm_gateup_kernel(GuArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t sm[2 * GuStage::BYTES];
    int4 tile;
    int nb;
    if (!gemm_item(a, tile, nb)) return;
    const int e = tile.x, p0 = tile.y;
    const int rows = moe::uniform(chunk_rows(a.offsets, e, p0, tile.w));
    if (rows <= 0) return;
    // rows rounded up to a multiple of 32
    switch ((rows + 31) >> 5) {
    case 1: gateup_chunk<2>(a, e, p0, rows, nb, sm); break;
    case 2: gateup_chunk<4>(a, e, p0, rows, nb, sm); break;
    case 3: gateup_chunk<6>(a, e, p0, rows, nb, sm); break;
    default: gateup_chunk<8>(a, e, p0, rows, nb, sm); break;
    }
}

// ---------------------------------------------------------------------------
// down, FP8 MFMA
// ---------------------------------------------------------------------------
// Block: 4 waves; wave w = every row of the chunk x outputs n0 + 32w .. +31
// (two 16-column operand tiles).  Two blocks share a CU: a down block runs
// only K/128 = 16 K steps, and one block's ramp runs under another's stream.
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

constexpr int DN_D = 4;
constexpr int DN_RB = 128;    // activation bytes per row and K step (E4M3)
using DnStage = AStage<DN_RB>;

struct DnB {
    u32x4 v[4];               // [operand tile c][half]
};

template <int NRS>
__device__ __forceinline__ void down_chunk(const DnArgs &a, int e, int p0, int rows, int nb,
                                           uint8_t *sm)
{
    constexpr int NJ = (NRS + 1) / 2;         // 32-row groups of A moved per step
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int q = lane >> 4, r16 = lane & 15;
    const int K = a.K, N = a.N, KB = K / BK;
    const int n0 = nb * 128;

    ASrc<NJ> src;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int row = DnStage::G * j + tid / DnStage::C;
        src.off[j] = (uint32_t)(p0 + (row < rows ? row : 0)) * K + (tid % DnStage::C) * 16;
    }
    {
        const int row = tid & (RMAX - 1);
        src.soff = (uint32_t)(p0 + (row < rows ? row : 0)) * KB;
    }
    const uint32_t sbase = a_store_base<DN_RB>(tid);
    // A operand halves of lane (row r16): logical chunks q and 4+q (K 16q..
    // and 64+16q..), the weight rows' byte order
    const uint32_t ao0 = r16 * DN_RB + DnStage::swz(r16, q) * 16;
    const uint32_t ao1 = r16 * DN_RB + DnStage::swz(r16, 4 + q) * 16;

    const uint8_t *wbase = moe::uniform_ptr(a.w0 + ((size_t)e * N + n0 + 32 * wave) * K);
    const uint32_t boff = (uint32_t)r16 * K + 16 * q;
    const uint32_t boff16 = boff + 16u * K;
    auto load_b = [&](int kb) {
        DnB b;
        const uint32_t k0 = (uint32_t)kb * BK;
        b.v[0] = moe::load_nt_global<u32x4>(wbase + (boff + k0));
        b.v[1] = moe::load_nt_global<u32x4>(wbase + (boff + k0 + 64));
        b.v[2] = moe::load_nt_global<u32x4>(wbase + (boff16 + k0));
        b.v[3] = moe::load_nt_global<u32x4>(wbase + (boff16 + k0 + 64));
        return b;
    };
    const float *sw0 = a.ws0 + ((size_t)e * a.ntn + nb) * KB;
    const float w_lo = lane < KB ? sw0[lane] : 0.0f, w_hi = lane + 64 < KB ? sw0[lane + 64] : 0.0f;

    f32x4 acc[NRS][2];
#pragma unroll
    for (int i = 0; i < NRS; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the K loop of the gate/up kernel, with FP8 operands taken as they are
    const int klast = KB - 1;
    DnB b[DN_D];
    ARegs<DN_RB, NJ> ar[2];
    b[0] = load_b(0);
    ar[0] = load_a<DN_RB, NJ>(a.hq, a.hs, src, 0);
    b[1] = load_b(min(1, klast));
    ar[1] = load_a<DN_RB, NJ>(a.hq, a.hs, src, min(1, klast));
    b[2] = load_b(min(2, klast));
    store_a<DN_RB, NJ>(sm, ar[0], tid, sbase);
    ar[0] = load_a<DN_RB, NJ>(a.hq, a.hs, src, min(2, klast));
    b[3] = load_b(min(3, klast));
    moe::lds_barrier();

    auto step = [&](int kb, DnB &bk, ARegs<DN_RB, NJ> &an, uint8_t *cur, uint8_t *nxt) {
        __builtin_amdgcn_sched_barrier(0);
        store_a<DN_RB, NJ>(nxt, an, tid, sbase);
        an = load_a<DN_RB, NJ>(a.hq, a.hs, src, min(kb + 3, klast));
        i32x8 bv[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
            bv[c] = __builtin_bit_cast(i32x8, __builtin_shufflevector(bk.v[2 * c], bk.v[2 * c + 1],
                                                                      0, 1, 2, 3, 4, 5, 6, 7));
        bk = load_b(min(kb + DN_D, klast));
        const float sw = lane_f(kb < 64 ? w_lo : w_hi, kb & 63);
        const float *ss = reinterpret_cast<const float *>(cur + DnStage::S_OFF);
#pragma unroll
        for (int rs = 0; rs < NRS; ++rs) {
            const u32x4 a0 = *reinterpret_cast<const u32x4 *>(cur + ao0 + 16 * DN_RB * rs);
            const u32x4 a1 = *reinterpret_cast<const u32x4 *>(cur + ao1 + 16 * DN_RB * rs);
            const i32x8 av = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
            const f32x4 sx = *reinterpret_cast<const f32x4 *>(ss + rs * 16 + 4 * q);
            const f32x4 t0 = mfma_fp8(av, bv[0]);
            const f32x4 t1 = mfma_fp8(av, bv[1]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float f = sx[i] * sw;
                acc[rs][0][i] = fmaf(t0[i], f, acc[rs][0][i]);
                acc[rs][1][i] = fmaf(t1[i], f, acc[rs][1][i]);
            }
        }
        moe::lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    uint8_t *s0 = sm, *s1 = sm + DnStage::BYTES;
    static_assert(DN_D == 4, "the K loop is unrolled by the weight registers' rotation");
#pragma unroll 1
    for (int kb0 = 0; kb0 < KB; kb0 += 4) {
        step(kb0, b[0], ar[1], s0, s1);
        step(kb0 + 1, b[1], ar[0], s1, s0);
        step(kb0 + 2, b[2], ar[1], s0, s1);
        step(kb0 + 3, b[3], ar[0], s1, s0);
    }

#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rs * 16 + 4 * q + i;
            if (r < rows) {
                float *yr = a.y + (size_t)(p0 + r) * N + n0 + 32 * wave + r16;
                yr[0] = acc[rs][0][i];
                yr[16] = acc[rs][1][i];
            }
        }
    }
}

__global__ __launch_bounds__(kThreads, 2) void gemm_down_kernel(DnArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t sm[2 * DnStage::BYTES];
    int4 tile;
    int nb;
    if (!gemm_item(a, tile, nb)) return;
    const int e = tile.x, p0 = tile.y;
    const int rows = moe::uniform(chunk_rows(a.offsets, e, p0, tile.w));
    if (rows <= 0) return;
    switch ((rows + 31) >> 5) {
    case 1: down_chunk<2>(a, e, p0, rows, nb, sm); break;
    case 2: down_chunk<4>(a, e, p0, rows, nb, sm); break;
    case 3: down_chunk<6>(a, e, p0, rows, nb, sm); break;
    default: down_chunk<8>(a, e, p0, rows, nb, sm); break;
    }
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
    hipLaunchKernelGGL(gemm_gateup_kernel, dim3((unsigned)(tmax * a.ntn)), dim3(kThreads), 0, st, a);
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
    hipLaunchKernelGGL(gemm_down_kernel, dim3((unsigned)(tmax * a.ntn)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}
