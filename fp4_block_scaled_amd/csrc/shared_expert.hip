// shared_expert.hip -- the shared expert for up to 16 tokens: a dense bf16
// SwiGLU MLP of width W applied to every token with weight 1 ("spark_model
// glm5next_mlp/forward.rs", fn forward_dense: down(clamped_swiglu(gate(x),
// up(x))), the same math as a routed expert with its own clamp, and the
// shared-expert step of fn forward_moe).
//
// One expert of width W gives only W/16 blocks in the GEMV layout of the
// routed tiers, so both projections here give a whole wave to one weight row:
//   gate/up: a block = 2R h rows; wave w streams R rows of the gate (w < 2)
//            or up (w >= 2) bank, rows 2Rb + R(w & 1) + r, lane l holding bytes
//            1024 j + 16 l of each row for j < H/512 in registers, then loops
//            over the tokens, reading their x from L2 once per R rows (R up to
//            2 for H <= 7168, else 1), and reduces over the 64 lanes; the gate
//            waves apply the clamped SwiGLU and write h (FP32).
//   down:    a block = 4 waves of R output rows each, the same way over W
//            with the FP32 h rows read from L2 once per R rows (R up to 4 for
//            W <= 2048, 2 for W <= 4096, else 1: the weights of a wave's rows
//            stay in registers).
// Products are bf16 x bf16 in v_dot2_f32_bf16 (gate/up) and FP32 (down), so
// only the summation order differs from the FP64 definition.
#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxTok = 16;

__device__ __forceinline__ uint4 load16(const void *p)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(moe::bf16x2, a),
                                          __builtin_bit_cast(moe::bf16x2, b), c, false);
}

__device__ __forceinline__ float wave_sum(float v)
{
    v = moe::sum8_lanes(v);
    v += __shfl_xor(v, 8, 64);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

__device__ __forceinline__ float swiglu_clamp(float g, float u, float L)
{
    const float gc = fminf(g, L);
    const float uc = fminf(fmaxf(u, -L), L);
    return gc / (1.0f + expf(-gc)) * uc;
}

// NJ = H / 512 loads of 16 bytes per lane and row; R rows per wave
template <int NJ, int R>
__global__ __launch_bounds__(kThreads) void shared_gateup_kernel(const uint16_t *__restrict__ gate,
                                                                 const uint16_t *__restrict__ up,
                                                                 const uint16_t *__restrict__ x,
                                                                 int32_t M, int32_t H, int32_t W,
                                                                 float limit, float *__restrict__ h)
{
    __shared__ float gu[4][R][kMaxTok];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int row0 = 2 * R * blockIdx.x + R * (wave & 1);
    const uint8_t *rp = reinterpret_cast<const uint8_t *>(moe::uniform_ptr(wave < 2 ? gate : up) +
                                                          (size_t)row0 * H);
    uint4 w[R][NJ];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < NJ; ++j) w[r][j] = load16(rp + (size_t)r * H * 2 + j * 1024 + lane * 16);
    for (int t = 0; t < M; ++t) {
        const uint8_t *xp = reinterpret_cast<const uint8_t *>(x + (size_t)t * H);
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(xp + j * 1024 + lane * 16);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                acc[r] = dot2(w[r][j].x, xv.x, acc[r]);
                acc[r] = dot2(w[r][j].y, xv.y, acc[r]);
                acc[r] = dot2(w[r][j].z, xv.z, acc[r]);
                acc[r] = dot2(w[r][j].w, xv.w, acc[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = wave_sum(acc[r]);
            if (lane == 0) gu[wave][r][t] = v;
        }
    }
    __syncthreads();
    if (wave < 2 && lane < M) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            h[(size_t)lane * W + row0 + r] = swiglu_clamp(gu[wave][r][lane], gu[wave + 2][r][lane], limit);
    }
}

// NJ = W / 512 loads of 16 bytes per lane and row; R rows per wave.  LH
// (one token, one row per wave, where each wave's h reads from L2 are twice
// its weight bytes): the block's 4 waves share the h row through LDS (W
// floats of dynamic LDS): 16.6 against 17.1 us for the whole shared expert at
// H7168 W2048.  With two rows per wave (H6144 W1536) it ran 0.25 us slower.
template <int NJ, int R, bool LH>
__global__ __launch_bounds__(kThreads) void shared_down_kernel(const uint16_t *__restrict__ down,
                                                               const float *__restrict__ h,
                                                               int32_t M, int32_t H, int32_t W,
                                                               float *__restrict__ out)
{
    extern __shared__ float hsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int row0 = (4 * blockIdx.x + wave) * R;    // < H: the grid is H / (4R) blocks
    const uint8_t *rp = reinterpret_cast<const uint8_t *>(moe::uniform_ptr(down) + (size_t)row0 * W);
    uint4 w[R][NJ];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < NJ; ++j) w[r][j] = load16(rp + (size_t)r * W * 2 + j * 1024 + lane * 16);
    if constexpr (LH) {
        for (int i = tid * 4; i < W; i += kThreads * 4)
            *reinterpret_cast<float4 *>(hsm + i) = *reinterpret_cast<const float4 *>(h + i);
        __syncthreads();
    }
    for (int t = 0; t < M; ++t) {
        const float *hp = LH ? hsm : h + (size_t)t * W;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const float4 a = *reinterpret_cast<const float4 *>(hp + j * 512 + lane * 8);
            const float4 b = *reinterpret_cast<const float4 *>(hp + j * 512 + lane * 8 + 4);
            const float hv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t q[4] = {w[r][j].x, w[r][j].y, w[r][j].z, w[r][j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[r] = fmaf(__uint_as_float(q[i] << 16), hv[2 * i], acc[r]);
                    acc[r] = fmaf(__uint_as_float(q[i] & 0xFFFF0000u), hv[2 * i + 1], acc[r]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = wave_sum(acc[r]);
            if (lane == 0) out[(size_t)t * H + row0 + r] = v;
        }
    }
}

// Rows per wave: with several tokens the largest R the registers allow (the
// x or h reads from L2 shrink by R); with one token the R whose grid puts the
// fewest rows on the busiest CU, the larger R on a tie (1536 gate/up rows:
// 3 blocks of 2 on the busiest CU with R = 1 against 2 of 4 with R = 2).
int pick_rows(int32_t M, int rows, int rows_per_block_r1, int rmax)
{
    if (M > 1) return rmax;
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
    }
    int best = 1, best_rows = 1 << 30;
    for (int r = 1; r <= rmax; r *= 2) {
        const int per = rows_per_block_r1 * r;
        const int busiest = (rows / per + cus - 1) / cus * per;
        if (busiest <= best_rows) best = r, best_rows = busiest;
    }
    return best;
}

template <int NJ, int R>
void gateup_launch_r(const uint16_t *gate, const uint16_t *up, const uint16_t *x, int32_t M, int32_t H,
                     int32_t W, float limit, float *h, hipStream_t st)
{
    hipLaunchKernelGGL((shared_gateup_kernel<NJ, R>), dim3((unsigned)(W / (2 * R))), dim3(kThreads), 0, st,
                       gate, up, x, M, H, W, limit, h);
}

template <int NJ>
void gateup_launch(const uint16_t *gate, const uint16_t *up, const uint16_t *x, int32_t M,
                   int32_t H, int32_t W, float limit, float *h, hipStream_t st)
{
    constexpr int RMAX = NJ <= 14 ? 2 : 1;
    if (pick_rows(M, W, 2, RMAX) == 2) gateup_launch_r<NJ, RMAX>(gate, up, x, M, H, W, limit, h, st);
    else gateup_launch_r<NJ, 1>(gate, up, x, M, H, W, limit, h, st);
}

template <int NJ, int R>
void down_launch_r(const uint16_t *down, const float *h, int32_t M, int32_t H, int32_t W, float *out,
                   hipStream_t st)
{
    if (M == 1 && R == 1)
        hipLaunchKernelGGL((shared_down_kernel<NJ, R, true>), dim3((unsigned)(H / (4 * R))), dim3(kThreads),
                           (size_t)W * 4, st, down, h, M, H, W, out);
    else
        hipLaunchKernelGGL((shared_down_kernel<NJ, R, false>), dim3((unsigned)(H / (4 * R))), dim3(kThreads),
                           0, st, down, h, M, H, W, out);
}

template <int NJ>
void down_launch(const uint16_t *down, const float *h, int32_t M, int32_t H, int32_t W, float *out,
                 hipStream_t st)
{
    constexpr int RMAX = NJ <= 4 ? 4 : NJ <= 8 ? 2 : 1;
    const int r = pick_rows(M, H, 4, RMAX);
    if (r == 4) down_launch_r<NJ, RMAX>(down, h, M, H, W, out, st);
    else if (r == 2) down_launch_r<NJ, (RMAX >= 2 ? 2 : 1)>(down, h, M, H, W, out, st);
    else down_launch_r<NJ, 1>(down, h, M, H, W, out, st);
}

template <int... N>
bool gateup_switch(int nj, const uint16_t *gate, const uint16_t *up, const uint16_t *x, int32_t M,
                   int32_t H, int32_t W, float limit, float *h, hipStream_t st)
{
    return ((nj == N ? (gateup_launch<N>(gate, up, x, M, H, W, limit, h, st), true) : false) || ...);
}

template <int... N>
bool down_switch(int nj, const uint16_t *down, const float *h, int32_t M, int32_t H, int32_t W,
                 float *out, hipStream_t st)
{
    return ((nj == N ? (down_launch<N>(down, h, M, H, W, out, st), true) : false) || ...);
}

}  // namespace

hipError_t launch_shared_expert(const uint16_t *gate, const uint16_t *up, const uint16_t *down,
                                const uint16_t *x, int32_t M, int32_t hidden, int32_t W,
                                float limit, float *h, float *out, hipStream_t st)
{
    if (M < 1 || M > kMaxTok || hidden % 512 || W % 512 || hidden > 8192 || W > 8192)
        return hipErrorInvalidValue;
    if (!gateup_switch<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(
            hidden / 512, gate, up, x, M, hidden, W, limit, h, st))
        return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!down_switch<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(W / 512, down, h, M,
                                                                           hidden, W, out, st))
        return hipErrorInvalidValue;
    return hipGetLastError();
}
