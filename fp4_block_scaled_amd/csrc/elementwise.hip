// elementwise.hip -- the per-token weighted combine.
//
// Combine: out[t] = sum_j w[t, j] * y[token_to_perm[t*k + j]], j = 0..k-1, each
// product rounded before the add ("memra-engine
// src/bin/ep_step_fp8_gate.rs", fn combine_down_rows_host and the
// "separate-rn-mul-add, canonical" combine label), reading the expert-sorted
// rows through token_to_perm like the indexed combine of "spark_model
// glm5next_mlp/forward.rs" (fn forward_moe).  One launch for every token.
// With a shared-expert row and a residual, each is then added in that order,
// one rounded addition each (the final add order routed-plus-shared-then-
// residual of "memra-engine src/bin/ep_step_fp8_gate.rs", full-layer gate).
#include "moe_internal.h"

namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const int32_t *__restrict__ t2p,
                                                      const float *__restrict__ w, int32_t k,
                                                      int32_t H, int32_t bx,
                                                      const float *__restrict__ shared,
                                                      const float *__restrict__ residual,
                                                      float *__restrict__ out)
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
    const size_t o = (size_t)t * H + m;
    if (shared) {
        const float4 v = *reinterpret_cast<const float4 *>(shared + o);
        acc.x = __fadd_rn(acc.x, v.x); acc.y = __fadd_rn(acc.y, v.y);
        acc.z = __fadd_rn(acc.z, v.z); acc.w = __fadd_rn(acc.w, v.w);
    }
    if (residual) {
        const float4 v = *reinterpret_cast<const float4 *>(residual + o);
        acc.x = __fadd_rn(acc.x, v.x); acc.y = __fadd_rn(acc.y, v.y);
        acc.z = __fadd_rn(acc.z, v.z); acc.w = __fadd_rn(acc.w, v.w);
    }
    *reinterpret_cast<float4 *>(out + o) = acc;
}

}  // namespace

hipError_t launch_combine(const float *y, const int32_t *token_to_perm, const float *w, int32_t M,
                          int32_t k, int32_t hidden, const float *shared, const float *residual,
                          float *out, hipStream_t st)
{
    const int bx = (hidden / 4 + 255) / 256;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(bx * M)), dim3(256), 0, st, y, token_to_perm,
                       w, k, hidden, bx, shared, residual, out);
    return hipGetLastError();
}
