// elementwise.hip -- clamped SwiGLU over gate/up slice partials, and the
// per-token weighted combine.
//
// SwiGLU: h = silu(min(g, L)) * clamp(u, -L, L) with silu(z) = z / (1 + e^-z)
// ("spark_model glm5next_mlp/forward.rs", doc of swiglu_rows: the clamp is
// asymmetric -- the gate is only capped from above).  g and u arrive as FP32
// partial rows of the K slices of the gate/up GEMV; they are added here in
// slice order, so the result does not depend on scheduling.
//
// Combine: out[t] = sum_j w[t, j] * y[token_to_perm[t*k + j]], j = 0..k-1, each
// product rounded before the add ("memra-engine
// src/bin/ep_step_fp8_gate.rs", fn combine_down_rows_host and the
// "separate-rn-mul-add, canonical" combine label), reading the expert-sorted
// rows through token_to_perm like the indexed combine of "spark_model
// glm5next_mlp/forward.rs" (fn forward_moe).  One launch for every token.
#include "moe_internal.h"

namespace {

__device__ __forceinline__ float swiglu_clamp(float g, float u, float L)
{
    const float gc = fminf(g, L);
    const float uc = fminf(fmaxf(u, -L), L);
    const float silu = gc / (1.0f + expf(-gc));
    return silu * uc;
}

__global__ __launch_bounds__(256) void swiglu_partials_kernel(
    const float *__restrict__ part, int32_t nks, int32_t S, int32_t I,
    const int32_t *__restrict__ offsets, int32_t E, float L, float *__restrict__ h)
{
    const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;   // float4 index into h
    const int q = I >> 2;
    const size_t p = i4 / q;
    if (p >= (size_t)offsets[E]) return;
    const int n = (int)(i4 - p * q) * 4;
    const size_t pst = (size_t)2 * I;
    const size_t sst = (size_t)S * pst;
    float4 g = *reinterpret_cast<const float4 *>(part + p * pst + n);
    float4 u = *reinterpret_cast<const float4 *>(part + p * pst + I + n);
    for (int ks = 1; ks < nks; ++ks) {
        const float4 gg = *reinterpret_cast<const float4 *>(part + ks * sst + p * pst + n);
        const float4 uu = *reinterpret_cast<const float4 *>(part + ks * sst + p * pst + I + n);
        g.x += gg.x; g.y += gg.y; g.z += gg.z; g.w += gg.w;
        u.x += uu.x; u.y += uu.y; u.z += uu.z; u.w += uu.w;
    }
    float4 r;
    r.x = swiglu_clamp(g.x, u.x, L);
    r.y = swiglu_clamp(g.y, u.y, L);
    r.z = swiglu_clamp(g.z, u.z, L);
    r.w = swiglu_clamp(g.w, u.w, L);
    *reinterpret_cast<float4 *>(h + p * I + n) = r;
}

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const int32_t *__restrict__ t2p,
                                                      const float *__restrict__ w, int32_t k,
                                                      int32_t H, int32_t bx, float *__restrict__ out)
{
    const int t = blockIdx.x / bx;
    const int m = ((blockIdx.x - t * bx) * 256 + threadIdx.x) * 4;
    if (m >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const int p = t2p[(size_t)t * k + j];
        if (p < 0) continue;
        const float wt = w[(size_t)t * k + j];
        const float4 v = *reinterpret_cast<const float4 *>(y + (size_t)p * H + m);
        acc.x = __fadd_rn(acc.x, __fmul_rn(wt, v.x));
        acc.y = __fadd_rn(acc.y, __fmul_rn(wt, v.y));
        acc.z = __fadd_rn(acc.z, __fmul_rn(wt, v.z));
        acc.w = __fadd_rn(acc.w, __fmul_rn(wt, v.w));
    }
    *reinterpret_cast<float4 *>(out + (size_t)t * H + m) = acc;
}

}  // namespace

hipError_t launch_swiglu_partials(const float *partials, int32_t nks, int32_t S, int32_t inter,
                                  const int32_t *offsets, int32_t E, float limit, float *h,
                                  hipStream_t st)
{
    const size_t n4 = (size_t)S * inter / 4;
    hipLaunchKernelGGL(swiglu_partials_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                       st, partials, nks, S, inter, offsets, E, limit, h);
    return hipGetLastError();
}

hipError_t launch_combine(const float *y, const int32_t *token_to_perm, const float *w, int32_t M,
                          int32_t k, int32_t hidden, float *out, hipStream_t st)
{
    const int bx = (hidden / 4 + 255) / 256;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(bx * M)), dim3(256), 0, st, y, token_to_perm,
                       w, k, hidden, bx, out);
    return hipGetLastError();
}
