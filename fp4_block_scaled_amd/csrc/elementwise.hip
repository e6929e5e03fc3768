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

// y rows are read once: non-temporal loads keep them out of the way.
__device__ __forceinline__ float4 load_once(const float *p)
{
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void add_row(float4 &acc, const float4 v)
{
    acc.x = __fadd_rn(acc.x, v.x); acc.y = __fadd_rn(acc.y, v.y);
    acc.z = __fadd_rn(acc.z, v.z); acc.w = __fadd_rn(acc.w, v.w);
}

// KMAX > 0: top_k <= KMAX, the slot loop unrolled so that every y load is in
// flight before the first product; KMAX == 0: any top_k, one slot at a time.
// Either way the products are added in slot order.
template <int KMAX>
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
    if constexpr (KMAX > 0) {
        int p[KMAX];
        float wt[KMAX];
        float4 v[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            p[j] = j < k ? t2p[(size_t)t * k + j] : -1;
            wt[j] = j < k ? w[(size_t)t * k + j] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (p[j] >= 0) v[j] = load_once(y + (size_t)p[j] * H + m);
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (p[j] >= 0)
                add_row(acc, make_float4(__fmul_rn(wt[j], v[j].x), __fmul_rn(wt[j], v[j].y),
                                         __fmul_rn(wt[j], v[j].z), __fmul_rn(wt[j], v[j].w)));
    } else {
        for (int j = 0; j < k; ++j) {
            const int pj = t2p[(size_t)t * k + j];
            if (pj < 0) continue;
            const float wj = w[(size_t)t * k + j];
            const float4 vj = load_once(y + (size_t)pj * H + m);
            add_row(acc, make_float4(__fmul_rn(wj, vj.x), __fmul_rn(wj, vj.y), __fmul_rn(wj, vj.z),
                                     __fmul_rn(wj, vj.w)));
        }
    }
    const size_t o = (size_t)t * H + m;
    if (shared) add_row(acc, *reinterpret_cast<const float4 *>(shared + o));
    if (residual) add_row(acc, *reinterpret_cast<const float4 *>(residual + o));
    *reinterpret_cast<float4 *>(out + o) = acc;
}

}  // namespace

hipError_t launch_combine(const float *y, const int32_t *token_to_perm, const float *w, int32_t M,
                          int32_t k, int32_t hidden, const float *shared, const float *residual,
                          float *out, hipStream_t st)
{
    const int bx = (hidden / 4 + 255) / 256;
    const dim3 grid((unsigned)(bx * M));
    if (k <= 8)
        hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, st, y, token_to_perm, w, k, hidden,
                           bx, shared, residual, out);
    else
        hipLaunchKernelGGL(combine_kernel<0>, grid, dim3(256), 0, st, y, token_to_perm, w, k, hidden,
                           bx, shared, residual, out);
    return hipGetLastError();
}
