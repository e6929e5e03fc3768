// shared_expert.hip -- the shared expert for up to 16 tokens: a dense bf16
// SwiGLU MLP of width W applied to every token with weight 1 ("spark_model
// glm5next_mlp/forward.rs", fn forward_dense: down(clamped_swiglu(gate(x),
// up(x))), the same math as a routed expert with its own clamp, and the
// shared-expert step of fn forward_moe).
//
// One expert of width W gives only W/16 blocks in the GEMV layout of the
// routed tiers, so both projections here give a whole wave to one weight row:
//   gate/up: a block = 2 h rows; wave w streams row 2r + (w & 1) of the gate
//            (w < 2) or up (w >= 2) bank, lane l holding bytes 1024 j + 16 l of
//            the row for j < H/512 in registers, then loops over the tokens,
//            reading their x from L2, and reduces over the 64 lanes; the gate
//            waves apply the clamped SwiGLU and write h (FP32).
//   down:    a block = 4 output rows, one per wave, the same way over W with
//            the FP32 h rows read from L2.
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

// NJ = H / 512 loads of 16 bytes per lane
template <int NJ>
__global__ __launch_bounds__(kThreads) void shared_gateup_kernel(const uint16_t *__restrict__ gate,
                                                                 const uint16_t *__restrict__ up,
                                                                 const uint16_t *__restrict__ x,
                                                                 int32_t M, int32_t H, int32_t W,
                                                                 float limit, float *__restrict__ h)
{
    __shared__ float gu[4][kMaxTok];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int row = 2 * blockIdx.x + (wave & 1);
    const uint8_t *rp = reinterpret_cast<const uint8_t *>(moe::uniform_ptr(wave < 2 ? gate : up) +
                                                          (size_t)row * H);
    uint4 w[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) w[j] = load16(rp + j * 1024 + lane * 16);
    for (int t = 0; t < M; ++t) {
        const uint8_t *xp = reinterpret_cast<const uint8_t *>(x + (size_t)t * H);
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(xp + j * 1024 + lane * 16);
            acc = dot2(w[j].x, xv.x, acc);
            acc = dot2(w[j].y, xv.y, acc);
            acc = dot2(w[j].z, xv.z, acc);
            acc = dot2(w[j].w, xv.w, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) gu[wave][t] = acc;
    }
    __syncthreads();
    if (wave < 2 && lane < M) h[(size_t)lane * W + row] = swiglu_clamp(gu[wave][lane], gu[wave + 2][lane], limit);
}

// NJ = W / 512 loads of 16 bytes per lane
template <int NJ>
__global__ __launch_bounds__(kThreads) void shared_down_kernel(const uint16_t *__restrict__ down,
                                                               const float *__restrict__ h,
                                                               int32_t M, int32_t H, int32_t W,
                                                               float *__restrict__ out)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::uniform(tid >> 6);
    const int row = 4 * blockIdx.x + wave;
    if (row >= H) return;                            // whole wave
    const uint8_t *rp = reinterpret_cast<const uint8_t *>(moe::uniform_ptr(down) + (size_t)row * W);
    uint4 w[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) w[j] = load16(rp + j * 1024 + lane * 16);
    for (int t = 0; t < M; ++t) {
        const float *hp = h + (size_t)t * W;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const float4 a = *reinterpret_cast<const float4 *>(hp + j * 512 + lane * 8);
            const float4 b = *reinterpret_cast<const float4 *>(hp + j * 512 + lane * 8 + 4);
            const uint32_t q[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
            const float hv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc = fmaf(__uint_as_float(q[i] << 16), hv[2 * i], acc);
                acc = fmaf(__uint_as_float(q[i] & 0xFFFF0000u), hv[2 * i + 1], acc);
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) out[(size_t)t * H + row] = acc;
    }
}

template <int NJ>
void gateup_launch(const uint16_t *gate, const uint16_t *up, const uint16_t *x, int32_t M,
                   int32_t H, int32_t W, float limit, float *h, hipStream_t st)
{
    hipLaunchKernelGGL(shared_gateup_kernel<NJ>, dim3((unsigned)(W / 2)), dim3(kThreads), 0, st, gate,
                       up, x, M, H, W, limit, h);
}

template <int NJ>
void down_launch(const uint16_t *down, const float *h, int32_t M, int32_t H, int32_t W, float *out,
                 hipStream_t st)
{
    hipLaunchKernelGGL(shared_down_kernel<NJ>, dim3((unsigned)((H + 3) / 4)), dim3(kThreads), 0, st,
                       down, h, M, H, W, out);
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
