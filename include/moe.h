/*
 * moe.h -- C ABI of libmoe, the routed mixture-of-experts FFN layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (one token t, its k routed slots s = t*k + j, expert e = ids[s]):
 *   g = Wg[e] x[t],  u = Wu[e] x[t]                        gate and up
 *   h = silu(min(g, L)) * clamp(u, -L, L)                  clamped SwiGLU
 *   y[s] = Wd[e] h                                         down
 *   out[t] = sum_{j=0..k-1} w[t, j] * y[t*k + j]           combine
 * Sources: "memra-engine src/dsv4_ep.rs" (fn chain: gate/up, clamped SwiGLU,
 * FP8 h, down, per routed slot); "spark_model glm5next_mlp/forward.rs" (doc
 * of swiglu_rows for the activation, struct Glm5NextMlpWorkspace for the
 * expert-sorted route tables, the combine kernels of fn forward_moe);
 * "memra-engine src/bin/ep_step_fp8_gate.rs" (fn combine_down_rows_host for
 * the slot-order combine, fn expert_matrix for the bank layout).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns
 *     every buffer and keeps it alive until the work queued on `stream`
 *     completes.  `stream` is a hipStream_t (NULL = the null stream).
 *   - The library never allocates, frees, synchronises the stream or copies
 *     device -> host inside these calls, so the three layer calls can be
 *     captured in a HIP graph.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed check returns a non-zero status and launches nothing.
 *     moe_last_error() then describes it (thread-local).
 *   - A launch failure returns MOE_ERR_HIP with HIP's message.
 *   - Ids outside [0, E) never fault: -1 marks an unfilled slot and any other
 *     out-of-range id is counted in route.status; both contribute zero.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status_t;
enum {
    MOE_OK = 0,
    MOE_ERR_ARG = 1,         /* null pointer or inconsistent argument        */
    MOE_ERR_SHAPE = 2,       /* a size rule below is broken                  */
    MOE_ERR_FORMAT = 3,      /* weight formats disagree / scale2 misuse      */
    MOE_ERR_WORKSPACE = 4,   /* ws_bytes below moe_workspace_bytes()         */
    MOE_ERR_HIP = 5,         /* a HIP launch failed                          */
    MOE_ERR_UNSUPPORTED = 6  /* valid request the library does not serve    */
};

/* Weight formats. */
enum {
    /* E4M3FN codes, one FP32 scale per 128x128 block ("memra-engine
     * src/bin/ep_step_fp8_gate.rs", fn expert_matrix: expert-major codes and
     * a scale_rows x scale_cols grid per expert). */
    MOE_W_E4M3_B128 = 1,
    /* NVFP4: E2M1 codes two per byte (element 2i in the low nibble), one E4M3
     * scale byte per 16 consecutive inputs, one FP32 scale_2 per expert
     * ("memra-engine src/dsv4_ep.rs", fn chain strides inter*hidden/2 and
     * inter*hidden/16; "spark_model glm5next_mlp/forward.rs", fn w4a16_gemv,
     * scale_2 as a scalar). */
    MOE_W_NVFP4_B16 = 2
};

/* Execution tiers. */
enum {
    MOE_MODE_AUTO = 0,      /* GEMV_A16 for M <= MOE_GEMV_MAX_M; above that
                               GEMM_A8 for E4M3 banks, GEMM_A16 for NVFP4     */
    /* Dequant-GEMV, bf16 activations, each active expert's weights streamed
     * once for all slots routed to it ("spark_model glm5next_mlp/forward.rs",
     * fn w4a16_gemv_moe_batchm: the union of the rows' experts, each swept
     * once). */
    MOE_MODE_GEMV_A16 = 1,
    /* Grouped FP8 MFMA GEMM over expert-sorted rows, activations and h
     * quantized to E4M3 per 1x128 group ("spark_model glm5next_mlp/forward.rs",
     * grouped prefill arm of fn forward_moe; "memra-engine src/dsv4_ep.rs",
     * EpScratch xq/xs/hq/hs).  E4M3 banks only. */
    MOE_MODE_GEMM_A8 = 2,
    /* Not a tier of moe_expert_ffn: the workspace mode of moe_layer_fused
     * (route pack, gate/up, SwiGLU, down and combine in one launch). */
    MOE_MODE_FUSED = 3,
    /* Grouped 16-bit MFMA GEMM over expert-sorted rows for NVFP4 banks: the
     * pages' W4A16 form (16-bit activations; "spark_model
     * glm5next_mlp/forward.rs", fn w4a16_gemv and its batched variant) at
     * prefill widths.  gate/up takes x as the bf16 it is; h passes between
     * the projections as FP16 (rounded once from the FP32 SwiGLU, times a
     * power of two picked from the clamp limit so that it neither overflows
     * nor falls into FP16's subnormals).  Each
     * E2M1 code times its E4M3 group scale is exact in bf16 and in FP16;
     * scale_2 multiplies the FP32 sums.  NVFP4 banks only; scales must be
     * 4-byte aligned. */
    MOE_MODE_GEMM_A16 = 4
};

/* Routers of moe_router_topk. */
enum {
    /* p = softmax(logits) over the experts; the top_k largest p, which are
     * the top_k largest logits. */
    MOE_ROUTER_SOFTMAX = 0,
    /* s = sigmoid(logits); the top_k largest binary32(s) + bias (one binary32
     * addition); the bias only selects, the weights come from s. */
    MOE_ROUTER_SIGMOID = 1
};

#define MOE_GEMV_MAX_M 16
/* Largest M * top_k moe_layer_fused takes. */
#define MOE_FUSED_MAX_SLOTS 256
#define MOE_MAX_EXPERTS 512
/* Largest hidden and inter (128 blocks of 128 along K, and the bf16 x rows
 * of a GEMV pass held in LDS). */
#define MOE_MAX_DIM 16384

/* One projection bank holding every expert, expert-major (host struct of
 * device pointers).  n_out x k_in is the matrix shape per expert:
 *   gate, up: n_out = inter,  k_in = hidden
 *   down:     n_out = hidden, k_in = inter
 * E4M3:  codes  uint8 [E][n_out][k_in]
 *        scales float [E][n_out/128][k_in/128]
 *        scale2 must be NULL
 * NVFP4: codes  uint8 [E][n_out][k_in/2]
 *        scales uint8 (E4M3) [E][n_out][k_in/16]
 *        scale2 float [E]                                                    */
typedef struct {
    int32_t fmt;
    int32_t num_experts;
    int32_t n_out;
    int32_t k_in;
    const uint8_t *codes;
    const void *scales;
    const float *scale2;
} moe_bank_t;

/* Expert-sorted route tables (host struct of device pointers into the
 * caller's workspace; "spark_model glm5next_mlp/forward.rs", struct
 * Glm5NextMlpWorkspace: expert_offsets, sorted_token_ids, token_to_perm).
 * S = M * top_k slots; slot s = t*top_k + j.  A slot's packed row is its
 * position in the expert-sorted order; within one expert, rows keep
 * ascending slot order.
 *   expert_offsets [E+1]  exclusive prefix sum of per-expert slot counts;
 *                         expert_offsets[E] = number of valid slots
 *   sorted_slot    [S]    packed row -> slot          (first expert_offsets[E]
 *   sorted_token   [S]    packed row -> token          rows; the rest of both
 *                         arrays holds unspecified values)
 *   token_to_perm  [S]    slot -> packed row, -1 for an invalid/unfilled id
 *   active_experts [min(E,S)]  ascending ids of experts with >= 1 slot,
 *                         then -1 up to min(E,S)
 *   num_active     [1]    number of experts with >= 1 slot
 *   status         [1]    number of ids outside [0, E) other than -1       */
typedef struct {
    int32_t M;
    int32_t top_k;
    int32_t num_experts;
    int32_t num_slots;
    int32_t *expert_offsets;
    int32_t *sorted_slot;
    int32_t *sorted_token;
    int32_t *token_to_perm;
    int32_t *active_experts;
    int32_t *num_active;
    int32_t *status;
} moe_route_t;

/* Bytes of device workspace one layer call sequence needs for any M <= max_M
 * (route tables first, then the FFN's scratch), so a caller sizes and
 * allocates it once, before any call, without a GPU ("spark_model
 * glm5next_mlp/forward.rs", fns mlp_ws_bytes / mlp_ws_total_bytes: the MLP
 * workspace computed from the config and the largest row count, split out of
 * the constructor so it can be checked with no device).  0 if the sizes
 * break a rule of moe_route_pack / moe_expert_ffn.  Needs no GPU. */
size_t moe_workspace_bytes(int32_t max_M, int32_t top_k, int32_t num_experts,
                           int32_t hidden, int32_t inter, int32_t fmt,
                           int32_t mode);

/* Router: the top_k experts of every token row and their weights, all rows
 * in one launch ("spark_model glm5next_mlp/forward.rs", fn forward_moe: one
 * top-k launch for every row, with router bias, routed_scale, renormalize and
 * one expert group; "memra-engine src/bin/ep_step_fp8_gate.rs", the full-layer
 * gate's sigmoid top-k router with router bias, router scale and route norm).
 * Its outputs feed moe_route_pack directly, with no host round trip.
 *   logits        float [M][num_experts], row-major (device)
 *   bias          float [num_experts] (device) for MOE_ROUTER_SIGMOID, or NULL
 *                 (no bias); must be NULL for MOE_ROUTER_SOFTMAX; its values
 *                 must be finite (a NaN bias leaves the order undefined)
 *   topk_ids      int32 [M][top_k] out (device): slot j holds rank j
 *   topk_weights  float [M][top_k] out (device)
 * Definition, per row (l = the row's logits; a NaN counts as -FLT_MAX and
 * +-inf as +-FLT_MAX):
 *   SOFTMAX: choose the top_k largest l; renormalize != 0:
 *            w[j] = exp(l[j] - l[0]) / sum_{i<top_k} exp(l[i] - l[0]), which is
 *            p[j] / sum of the chosen p; renormalize == 0: w[j] = p[j] (the
 *            full softmax, denominator summed over experts in ascending order).
 *   SIGMOID: s = 1 / (1 + exp(-l)); choose the top_k largest binary32(s) + bias;
 *            w[j] = s[j], divided by sum_{i<top_k} s[i] if renormalize != 0
 *            (all 0 if that sum is 0: every chosen s underflowed).
 *   Equal keys go to the lower expert id.  w[j] is then multiplied by
 *   routed_scale and rounded once to binary32; everything before that is
 *   double, and sums over the chosen experts run in rank order.
 * Rules: M >= 1, 1 <= top_k <= num_experts <= MOE_MAX_EXPERTS, routed_scale
 * finite and > 0, renormalize 0 or 1; else MOE_ERR_SHAPE / MOE_ERR_ARG, with
 * nothing launched.  Allocates nothing; capturable in a HIP graph. */
moe_status_t moe_router_topk(const float *logits, int32_t M, int32_t num_experts, int32_t top_k,
                             int32_t kind, const float *bias, float routed_scale,
                             int32_t renormalize, int32_t *topk_ids, float *topk_weights,
                             void *stream);

/* The tier moe_expert_ffn runs for `requested` at M tokens: a non-AUTO
 * request is returned as is; AUTO gives MOE_MODE_GEMV_A16 for M <=
 * MOE_GEMV_MAX_M, else MOE_MODE_GEMM_A8 for E4M3 banks and MOE_MODE_GEMM_A16
 * for NVFP4 banks.  A caller can ask which kernel family a row count takes
 * before it runs ("spark_model glm5next_mlp/forward.rs", fn gemm: one token
 * to the GEMV, a few rows to one weight read for all rows, wider shapes to
 * the tile GEMM; fn forward_moe and its announce_* helpers, which report
 * which routed-expert arm a row count took).  Needs no GPU. */
int32_t moe_resolve_mode(int32_t M, int32_t fmt, int32_t requested);

/* Route pack: stable counting sort of the M*top_k slots of topk_ids
 * (int32 [M][top_k], device) by expert, into the route region at the start
 * of `ws`.  Fills *route (host) with pointers into ws.
 * Rules: M >= 1, 1 <= top_k <= num_experts <= MOE_MAX_EXPERTS, M*top_k
 * < 2^31; ws_bytes >= moe_workspace_bytes(M, top_k, num_experts, 128, 128,
 * MOE_W_E4M3_B128, MOE_MODE_GEMV_A16) at least (the route region). */
moe_status_t moe_route_pack(const int32_t *topk_ids, int32_t M, int32_t top_k,
                            int32_t num_experts, void *ws, size_t ws_bytes,
                            moe_route_t *route, void *stream);

/* Expert FFN ("memra-engine src/dsv4_ep.rs", fn chain: per routed slot the
 * gate and up projections, the clamped SwiGLU, then the down projection into
 * an FP32 row; "spark_model glm5next_mlp/forward.rs", fn forward_moe: the
 * routed sweep over expert-sorted rows).  For every valid slot, in packed
 * order,
 *   y_packed[row] = Wd[e] (silu(min(Wg[e] x[t], L)) * clamp(Wu[e] x[t], -L, L))
 * x_bf16: bf16 [M][hidden]; y_packed: float [M*top_k][hidden], rows past
 * expert_offsets[E] are left untouched.  `route` (host) must come from
 * moe_route_pack on this same `ws`.
 * Rules: hidden % 128 == 0, inter % 128 == 0 (% 256 for NVFP4), both
 * <= MOE_MAX_DIM; gate/up are inter x hidden,
 * down is hidden x inter; all banks share one format and num_experts;
 * hidden, inter <= MOE_MAX_DIM; GEMM_A8 needs E4M3 banks, and M*hidden
 * and M*top_k*inter < 2^31 (MOE_ERR_SHAPE otherwise); GEMM_A16 needs NVFP4
 * banks with 4-byte aligned scales, and 2*M*hidden and 2*M*top_k*inter
 * < 2^31 (a tier that does not serve the banks' format returns
 * MOE_ERR_UNSUPPORTED);
 * ws_bytes >= moe_workspace_bytes(route->M, ..., mode). */
moe_status_t moe_expert_ffn(const moe_bank_t *gate, const moe_bank_t *up,
                            const moe_bank_t *down, const uint16_t *x_bf16,
                            const moe_route_t *route, int32_t hidden,
                            int32_t inter, float limit, int32_t mode,
                            float *y_packed, void *ws, size_t ws_bytes,
                            void *stream);

/* Combine: out[t][m] = sum_{j=0..top_k-1} w[t][j] * y_packed[token_to_perm[t*top_k+j]][m],
 * in slot order j, each product rounded before it is added (FP32); slots
 * with token_to_perm = -1 contribute nothing ("memra-engine
 * src/bin/ep_step_fp8_gate.rs", fn combine_down_rows_host).
 * topk_weights: float [M][top_k]; out: float [M][hidden]; hidden % 4 == 0. */
moe_status_t moe_combine(const float *y_packed, const moe_route_t *route,
                         const float *topk_weights, int32_t hidden, float *out,
                         void *stream);

/* The whole layer in one call: the route pack, the expert FFN of tier `mode`
 * and the combine, with the outputs (route tables in *route, y_packed, out)
 * of moe_route_pack + moe_expert_ffn + moe_combine, bit for bit.  For the
 * GEMV tier and M*top_k <= 128 slots (E4M3; 64 for NVFP4) the route pack runs
 * inside the gate/up launch (every block builds the route of the slots from
 * the ids in LDS; block 0 writes the tables for the down and combine
 * launches), so the layer is three launches; with one token (M == 1,
 * top_k <= 8, inter a multiple of 512 up to 2560 for E4M3 or 2048 for
 * NVFP4, out 16-byte aligned) the down launch also does the combine (each
 * block owns some output rows for every slot and adds them in slot order),
 * two launches; otherwise the three calls' launches run in sequence.  No
 * host state: capturable in a HIP graph.
 * Rules and workspace: those of the three calls (ws_bytes >=
 * moe_workspace_bytes(M, top_k, E, hidden, inter, fmt, mode)); a failed
 * check launches nothing of the failing call. */
moe_status_t moe_layer(const moe_bank_t *gate, const moe_bank_t *up, const moe_bank_t *down,
                       const uint16_t *x_bf16, const int32_t *topk_ids, const float *topk_weights,
                       int32_t M, int32_t top_k, int32_t hidden, int32_t inter, float limit,
                       int32_t mode, float *y_packed, float *out, void *ws, size_t ws_bytes,
                       moe_route_t *route, void *stream);

/* Bytes of the library's static scratch for moe_layer_static, per GPU. */
#define MOE_STATIC_SCRATCH_BYTES (8u << 20)

/* moe_layer for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call, kernels and outputs (route tables in *route, y_packed, out) as
 * moe_layer, bit for bit, but the workspace is the library's own static
 * device array of MOE_STATIC_SCRATCH_BYTES on the current device
 * (hipGetDevice; `stream` must belong to it) instead of a caller buffer.
 * The caller still passes inputs and outputs.  *route points into that
 * array and stays valid until the next moe_layer_static call on the same
 * GPU.  Nothing in the array needs clearing: every call writes the route
 * tables and all the scratch it then reads.  The array is shared by every
 * call on one GPU and keeps the last call's contents, so calls that overlap
 * on one GPU (other streams, other threads) race; order them on one stream.
 * Rules: those of moe_layer; a layer whose workspace
 * (moe_workspace_bytes(M, top_k, E, hidden, inter, fmt, mode)) exceeds
 * MOE_STATIC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE and launches nothing
 * (at decode shapes it needs about 1 MB at M = 16).  Allocates nothing and
 * calls no allocating routine; the array's device address is looked up once
 * per device (hipGetSymbolAddress) on the first call there. */
moe_status_t moe_layer_static(const moe_bank_t *gate, const moe_bank_t *up, const moe_bank_t *down,
                              const uint16_t *x_bf16, const int32_t *topk_ids,
                              const float *topk_weights, int32_t M, int32_t top_k, int32_t hidden,
                              int32_t inter, float limit, int32_t mode, float *y_packed, float *out,
                              moe_route_t *route, void *stream);

/* Fused decode layer: moe_route_pack, moe_expert_ffn on the GEMV tier and
 * moe_combine as ONE kernel launch of resident blocks ("spark_model
 * glm5next_mlp/forward.rs", doc of forward_moe: the per-row MoE path without
 * host round trips and its launch count; "memra-engine src/dsv4_ep.rs", fn
 * chain: gate/up, activation, down and weighting as one chain per expert).
 * Each block builds the route in LDS; gate/up items publish per expert, down
 * items wait for their expert's h, and the last down item of each 32-row
 * output tile applies the top-k weights for every token.  One token (M = 1,
 * hidden a multiple of 1024 for E4M3, 2048 for NVFP4) runs gate/up items of
 * two h rows taken expert by expert; their sums run in another order than
 * the three calls', so outputs agree with those to rounding.  Otherwise
 * (E4M3 only) the items are the three-call path's and outputs are
 * bit-identical to it.
 * Inputs and outputs as for the three calls: topk_ids int32 [M][top_k],
 * topk_weights float [M][top_k], x bf16 [M][hidden]; y_packed float
 * [M*top_k][hidden] (expert-sorted rows), out float [M][hidden]; *route
 * (host) describes the route tables in ws, as moe_route_pack fills them.
 * Rules: E4M3 banks with M*top_k <= MOE_FUSED_MAX_SLOTS, or NVFP4 banks
 * with M = 1 and hidden a multiple of 2048 up to 16384 (other NVFP4 sizes:
 * MOE_ERR_UNSUPPORTED); the moe_expert_ffn shape rules; num_experts is the
 * banks'; ws_bytes >= moe_workspace_bytes(M, top_k, E, hidden, inter, fmt,
 * MOE_MODE_FUSED), ws 256-byte aligned.  The workspace needs no clearing,
 * and calls on one ws must be ordered on one stream.  The kernel assumes its
 * blocks can all be resident on the GPU at once (no other kernel holding the
 * CUs); a wait that does not end within about a second gives up and adds
 * 2^30 to route->status.  Each call takes a fresh epoch on the host, so the
 * call cannot be captured into a HIP graph: on a capturing stream it returns
 * MOE_ERR_UNSUPPORTED and launches nothing (the three calls above can be
 * captured). */
moe_status_t moe_layer_fused(const moe_bank_t *gate, const moe_bank_t *up, const moe_bank_t *down,
                             const uint16_t *x_bf16, const int32_t *topk_ids,
                             const float *topk_weights, int32_t M, int32_t top_k,
                             int32_t hidden, int32_t inter, float limit, float *y_packed,
                             float *out, void *ws, size_t ws_bytes, moe_route_t *route,
                             void *stream);

/* Shared expert: a dense SwiGLU MLP of width shared_width with bf16 weights,
 * applied to every token with weight 1 ("spark_model
 * glm5next_mlp/forward.rs", fn forward_dense: down(clamped_swiglu(gate(x),
 * up(x))), the same math as a routed expert with its own clamp, and the
 * shared-expert step of fn forward_moe, not routed-scaled).
 *   gate_bf16, up_bf16  bf16 [shared_width][hidden]
 *   down_bf16           bf16 [hidden][shared_width]
 *   x_bf16              bf16 [M][hidden]
 *   shared_out          float [M][hidden] out
 *   ws                  >= moe_shared_workspace_bytes(M, hidden, shared_width)
 *                       bytes, 256-byte aligned (h [M][shared_width] FP32)
 * g, u, h and the outputs are FP32.  Rules: 1 <= M <= MOE_GEMV_MAX_M (wider M:
 * MOE_ERR_UNSUPPORTED); hidden and shared_width positive multiples of 512 up
 * to 8192; limit > 0; pointers 16-byte aligned.  Two launches on `stream`;
 * allocates nothing. */
size_t moe_shared_workspace_bytes(int32_t max_M, int32_t hidden, int32_t shared_width);
moe_status_t moe_shared_expert(const uint16_t *gate_bf16, const uint16_t *up_bf16,
                               const uint16_t *down_bf16, const uint16_t *x_bf16, int32_t M,
                               int32_t hidden, int32_t shared_width, float limit,
                               float *shared_out, void *ws, size_t ws_bytes, void *stream);

/* Combine with the shared expert and the residual:
 *   out[t][m] = ((sum_j w[t][j] * y[perm(t, j)][m]) + shared_out[t][m]) + residual[t][m]
 * the routed combine of moe_combine (slot order, multiply then add), then one
 * rounded FP32 addition of the shared expert's row, then one of the residual
 * ("memra-engine src/bin/ep_step_fp8_gate.rs", the full-layer gate's final
 * add order routed-plus-shared-then-residual).  shared_out and residual are
 * float [M][hidden] (device) and may each be NULL (not added); with both NULL
 * this is moe_combine.  Same rules as moe_combine. */
moe_status_t moe_combine_residual(const float *y_packed, const moe_route_t *route,
                                  const float *topk_weights, const float *shared_out,
                                  const float *residual, int32_t hidden, float *out,
                                  void *stream);

/* Stage timing (optional, thread-local).  With events != NULL, later
 * moe_expert_ffn calls on this thread record events[0] on their stream before
 * the first kernel and events[i] after the i-th kernel, for at most
 * n_events events; NULL turns it off.  The handles are the caller's
 * hipEvent_t.  Returns the number of stages the tier `mode` records (2 for
 * MOE_MODE_GEMV_A16: gate/up with SwiGLU, down; 1 for MOE_MODE_FUSED, where
 * moe_layer_fused records around its single launch; 3 otherwise: for
 * MOE_MODE_GEMM_A8 activation quantization + tile schedule, gate/up with
 * SwiGLU, down; for MOE_MODE_GEMM_A16 tile schedule, gate/up with SwiGLU,
 * down), so n_events = 4 covers every tier.  Mirrors the
 * per-stage timers of "spark_model glm5next_mlp/forward.rs" (profile::start /
 * profile::end around the MoE stages). */
int32_t moe_set_stage_events(void *const *events, int32_t n_events, int32_t fmt,
                             int32_t hidden, int32_t inter, int32_t mode);

/* Message for the last non-OK status returned on this thread: the call and
 * the check that failed, or HIP's message for a failed launch.  Every
 * non-OK status says which step failed and why, as the labelled launch
 * checks of "memra-engine src/dsv4_ep.rs" do (fn chain: each kernel call
 * wrapped with its stage name, e.g. "EP w1/w3").  Thread-local; the pointer
 * stays valid until the next failing call on the same thread. */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
