/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU definition of one routed
 * mixture-of-experts FFN layer with block-scaled expert weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or constant generator with the
 * HIP library.
 *
 * Arithmetic: every value is decoded exactly and every sum is taken in IEEE
 * double precision, in plain loops, in the order the definition states.
 * Compile without -ffast-math and with -ffp-contract=off so that each float
 * operation the definition names is exactly one rounded operation.
 *
 * What is computed (sources are the three pages the method is described on):
 *   - the expert chain gate -> clamped SwiGLU -> down, per routed slot
 *     ("memra-engine src/dsv4_ep.rs", fn chain; "memra-engine
 *     src/bin/ep_step_fp8_gate.rs", fn reference_expert and
 *     fn reference_grouped_projections);
 *   - the clamped activation silu(min(g, L)) * clamp(u, -L, L)
 *     ("spark_model glm5next_mlp/forward.rs", doc of swiglu_rows);
 *   - the per-token combine in canonical slot order with a separate multiply
 *     and add ("memra-engine src/bin/ep_step_fp8_gate.rs",
 *     fn combine_down_rows_host and the combine_numeric label of
 *     run_dynamic_owner_grouped_fp8_combine_gate);
 *   - the expert-sorted route tables: per-expert prefix offsets, sorted row ->
 *     token, slot -> sorted row ("spark_model glm5next_mlp/forward.rs",
 *     struct Glm5NextMlpWorkspace);
 *   - block-scaled E4M3 banks (one FP32 scale per 128x128 block, expert-major,
 *     "memra-engine src/bin/ep_step_fp8_gate.rs", fn expert_matrix) and NVFP4
 *     banks (E2M1 nibbles, one E4M3 scale per 16, one FP32 scale_2 per expert
 *     projection; "memra-engine src/dsv4_ep.rs", fn chain strides, and
 *     "spark_model glm5next_mlp/forward.rs", fn w4a16_gemv);
 *   - per 1x128 group FP8 quantization of activations for the wide-M tier
 *     ("memra-engine src/dsv4_ep.rs", EpScratch xq/xs and the act_quant_fp8
 *     step of fn chain);
 *   - the shared expert (a dense bf16 SwiGLU MLP applied to every token) and
 *     the final add order routed, then shared, then residual ("spark_model
 *     glm5next_mlp/forward.rs", fn forward_dense; "memra-engine
 *     src/bin/ep_step_fp8_gate.rs", the full-layer gate);
 *   - the router before the layer: softmax, or sigmoid with a selection bias,
 *     top-k per token, renormalized and scaled weights ("spark_model
 *     glm5next_mlp/forward.rs", the router launch of fn forward_moe;
 *     "memra-engine src/bin/ep_step_fp8_gate.rs", the full-layer gate's
 *     sigmoid top-k router).
 * Readings of points the pages leave open are listed beside the function
 * that takes them.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Code tables                                                               */
/* ------------------------------------------------------------------------ */

/* OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinity;
 * the only NaN encodings are S.1111.111.  Subnormals: m * 2^-9. */
double oracle_e4m3_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* OCP E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; subnormal m/2. */
double oracle_e2m1_value(uint8_t nib)
{
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* bfloat16 bits -> value (the upper half of an IEEE binary32). */
double oracle_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a binary32 value to E4M3FN, nearest with ties to the even code,
 * saturating to +-448 (finite inputs only; NaN maps to 0x7F).  The search is a
 * plain walk over the 127 non-negative finite codes, which are increasing in
 * value, so the result is the nearest code by construction. */
uint8_t oracle_e4m3_encode(float v)
{
    double a = fabs((double)v);
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    uint8_t best = 0;
    if (isnan(v)) return 0x7F;
    if (a >= 448.0) return sign | 0x7E;
    for (int c = 0; c <= 0x7E; ++c) {
        double lo = oracle_e4m3_value((uint8_t)c);
        double hi;
        if (c == 0x7E) { best = 0x7E; break; }
        hi = oracle_e4m3_value((uint8_t)(c + 1));
        if (a >= lo && a <= hi) {
            double dlo = a - lo, dhi = hi - a;
            if (dlo < dhi) best = (uint8_t)c;
            else if (dhi < dlo) best = (uint8_t)(c + 1);
            else best = (c & 1) ? (uint8_t)(c + 1) : (uint8_t)c; /* tie: even */
            break;
        }
    }
    return sign | best;
}

/* ------------------------------------------------------------------------ */
/* Activation quantization for the FP8 tier                                  */
/* ------------------------------------------------------------------------ */

/* Per row and per group of 128 consecutive columns: amax = max |x| over the
 * group (binary32, exact); scale = amax / 448 in binary32 (1.0 when amax is 0);
 * code = E4M3(binary32(x / scale)).  The pages give the layout (one FP32 scale
 * per 128 activations) but not the rule; this is the plain reading where the
 * group maximum lands on the largest finite E4M3 magnitude. */
void oracle_quant_1x128(const float *x, int64_t rows, int64_t cols,
                        uint8_t *q, float *s)
{
    int64_t groups = cols / 128;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < groups; ++g) {
            const float *xg = x + r * cols + g * 128;
            float amax = 0.0f, scale;
            for (int i = 0; i < 128; ++i) {
                float a = fabsf(xg[i]);
                if (a > amax) amax = a;
            }
            scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;
            s[r * groups + g] = scale;
            for (int i = 0; i < 128; ++i) {
                float t = xg[i] / scale;
                q[r * cols + g * 128 + i] = oracle_e4m3_encode(t);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Route pack                                                                */
/* ------------------------------------------------------------------------ */

/* Stable counting sort of the S = M*k route slots by expert id.
 * Slot s = t*k + j is token t's j-th choice.  Ids in [0, E) are valid; -1
 * means "slot unfilled"; anything else is invalid.  Neither of the latter is
 * placed, and token_to_perm holds -1 for them.  Within an expert, slots keep
 * ascending flat slot order (the pages name the tables but not their order
 * inside one expert; ascending slot order makes the result unique).
 * Returns the number of invalid ids (not counting -1). */
int oracle_route_pack(const int32_t *ids, int32_t M, int32_t k, int32_t E,
                      int32_t *offsets, int32_t *sorted_slot,
                      int32_t *sorted_token, int32_t *token_to_perm,
                      int32_t *active, int32_t *num_active)
{
    int64_t S = (int64_t)M * k;
    int32_t *count = calloc((size_t)E, sizeof(int32_t));
    int32_t *fill = calloc((size_t)E, sizeof(int32_t));
    int invalid = 0, na = 0;
    for (int64_t s = 0; s < S; ++s) {
        int32_t e = ids[s];
        if (e >= 0 && e < E) count[e]++;
        else if (e != -1) invalid++;
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + count[e];
    for (int64_t s = 0; s < S; ++s) {
        int32_t e = ids[s];
        if (e >= 0 && e < E) {
            int32_t pos = offsets[e] + fill[e]++;
            sorted_slot[pos] = (int32_t)s;
            sorted_token[pos] = (int32_t)(s / k);
            token_to_perm[s] = pos;
        } else {
            token_to_perm[s] = -1;
        }
    }
    for (int32_t e = 0; e < E; ++e)
        if (count[e] > 0) active[na++] = e;
    *num_active = na;
    free(count);
    free(fill);
    return invalid;
}

/* ------------------------------------------------------------------------ */
/* Expert banks                                                              */
/* ------------------------------------------------------------------------ */

enum { ORACLE_E4M3_B128 = 1, ORACLE_NVFP4_B16 = 2 };

/* One projection bank for every expert, expert-major.
 * E4M3:  codes [E][n][k] bytes; scales float [E][n/128][k/128].
 * NVFP4: codes [E][n][k/2] bytes, element 2i in the low nibble of byte i and
 *        element 2i+1 in the high nibble (the pages do not fix the nibble
 *        order; low-first is the OCP packing convention); scales are E4M3
 *        bytes [E][n][k/16]; scale2 float [E]. */
typedef struct {
    int32_t fmt, num_experts, n_out, k_in;
    const uint8_t *codes;
    const void *scales;
    const float *scale2;
} oracle_bank_t;

/* The decode functions above, evaluated once per code so that the matrix
 * loops do not call ldexp per element.  Filled before any parallel region. */
static double e4m3_tab[256], e2m1_tab[16];
static int tabs_ready = 0;
static void fill_tables(void)
{
    if (tabs_ready) return;
    for (int c = 0; c < 256; ++c) e4m3_tab[c] = oracle_e4m3_value((uint8_t)c);
    for (int c = 0; c < 16; ++c) e2m1_tab[c] = oracle_e2m1_value((uint8_t)c);
    tabs_ready = 1;
}

/* Exact value of W[e][n][kk]. */
static double bank_weight(const oracle_bank_t *b, int64_t e, int64_t n,
                          int64_t kk)
{
    int64_t N = b->n_out, K = b->k_in;
    if (b->fmt == ORACLE_E4M3_B128) {
        const float *sc = (const float *)b->scales;
        uint8_t c = b->codes[(e * N + n) * K + kk];
        double sblk = sc[(e * (N / 128) + n / 128) * (K / 128) + kk / 128];
        return e4m3_tab[c] * sblk;
    } else {
        const uint8_t *sc = (const uint8_t *)b->scales;
        uint8_t byte = b->codes[(e * N + n) * (K / 2) + kk / 2];
        uint8_t nib = (kk & 1) ? (byte >> 4) : (byte & 15);
        double s16 = e4m3_tab[sc[(e * N + n) * (K / 16) + kk / 16]];
        return e2m1_tab[nib] * s16 * (double)b->scale2[e];
    }
}

/* Dense dequantized copy of one expert's matrix, [n][k] doubles. */
void oracle_dequant_expert(const oracle_bank_t *b, int32_t e, double *out)
{
    fill_tables();
    for (int64_t n = 0; n < b->n_out; ++n)
        for (int64_t kk = 0; kk < b->k_in; ++kk)
            out[n * b->k_in + kk] = bank_weight(b, e, n, kk);
}

/* y[n] = sum_kk W[e][n][kk] * v[kk], FP64, kk ascending. */
static void expert_matvec(const oracle_bank_t *b, int32_t e, const double *v,
                          double *y)
{
    int64_t N = b->n_out, K = b->k_in;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t kk = 0; kk < K; ++kk) acc += bank_weight(b, e, n, kk) * v[kk];
        y[n] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* The clamped SwiGLU                                                        */
/* ------------------------------------------------------------------------ */

/* silu(min(g, L)) * clamp(u, -L, L), silu(z) = z / (1 + exp(-z)). */
double oracle_swiglu_clamp(double g, double u, double limit)
{
    double gc = g < limit ? g : limit;
    double uc = u < -limit ? -limit : (u > limit ? limit : u);
    double silu = gc / (1.0 + exp(-gc));
    return silu * uc;
}

/* ------------------------------------------------------------------------ */
/* The expert FFN per routed slot                                            */
/* ------------------------------------------------------------------------ */

/* For every slot in slot_list (flat slot index s = t*k + j with a valid id):
 *   xhat = x[t] decoded from bf16             (act_fp8 == 0), or
 *   xhat = dec(q) * scale, (q, scale) = 1x128 quantization of x[t] (act_fp8)
 *   g = Wg[e] xhat,  u = Wu[e] xhat            (FP64 sums)
 *   h = swiglu_clamp(g, u, L)                  (FP64)
 *   act_fp8: h <- dec(q) * scale of the 1x128 quantization of binary32(h)
 *   y = Wd[e] h
 * Outputs are row-major per listed slot: g,u,h [n_list][inter], y [n_list][hidden].
 * Any output pointer may be NULL.  Slots whose id is not in [0, E) get zero
 * rows. */
void oracle_expert_slots(const oracle_bank_t *gate, const oracle_bank_t *up,
                         const oracle_bank_t *down, const uint16_t *x_bf16,
                         const int32_t *ids, int32_t M, int32_t k,
                         int32_t hidden, int32_t inter, float limit,
                         int32_t act_fp8, const int32_t *slot_list,
                         int32_t n_list, double *g_out, double *u_out,
                         double *h_out, double *y_out)
{
    double *xv = malloc(sizeof(double) * (size_t)hidden);
    double *g = malloc(sizeof(double) * (size_t)inter);
    double *u = malloc(sizeof(double) * (size_t)inter);
    double *h = malloc(sizeof(double) * (size_t)inter);
    double *y = malloc(sizeof(double) * (size_t)hidden);
    float *tmp = malloc(sizeof(float) * (size_t)(hidden > inter ? hidden : inter));
    uint8_t *q = malloc((size_t)(hidden > inter ? hidden : inter));
    float *qs = malloc(sizeof(float) * (size_t)(hidden > inter ? hidden : inter) / 128);
    (void)M;
    fill_tables();
    for (int32_t li = 0; li < n_list; ++li) {
        int32_t s = slot_list[li];
        int32_t t = s / k, e = ids[s];
        int valid = (e >= 0 && e < gate->num_experts);
        if (!valid) {
            if (g_out) memset(g_out + (int64_t)li * inter, 0, sizeof(double) * inter);
            if (u_out) memset(u_out + (int64_t)li * inter, 0, sizeof(double) * inter);
            if (h_out) memset(h_out + (int64_t)li * inter, 0, sizeof(double) * inter);
            if (y_out) memset(y_out + (int64_t)li * hidden, 0, sizeof(double) * hidden);
            continue;
        }
        if (!act_fp8) {
            for (int32_t i = 0; i < hidden; ++i)
                xv[i] = oracle_bf16_value(x_bf16[(int64_t)t * hidden + i]);
        } else {
            for (int32_t i = 0; i < hidden; ++i)
                tmp[i] = (float)oracle_bf16_value(x_bf16[(int64_t)t * hidden + i]);
            oracle_quant_1x128(tmp, 1, hidden, q, qs);
            for (int32_t i = 0; i < hidden; ++i)
                xv[i] = oracle_e4m3_value(q[i]) * (double)qs[i / 128];
        }
        expert_matvec(gate, e, xv, g);
        expert_matvec(up, e, xv, u);
        for (int32_t i = 0; i < inter; ++i)
            h[i] = oracle_swiglu_clamp(g[i], u[i], (double)limit);
        if (act_fp8) {
            for (int32_t i = 0; i < inter; ++i) tmp[i] = (float)h[i];
            oracle_quant_1x128(tmp, 1, inter, q, qs);
            for (int32_t i = 0; i < inter; ++i)
                h[i] = oracle_e4m3_value(q[i]) * (double)qs[i / 128];
        }
        expert_matvec(down, e, h, y);
        if (g_out) memcpy(g_out + (int64_t)li * inter, g, sizeof(double) * inter);
        if (u_out) memcpy(u_out + (int64_t)li * inter, u, sizeof(double) * inter);
        if (h_out) memcpy(h_out + (int64_t)li * inter, h, sizeof(double) * inter);
        if (y_out) memcpy(y_out + (int64_t)li * hidden, y, sizeof(double) * hidden);
    }
    free(xv); free(g); free(u); free(h); free(y); free(tmp); free(q); free(qs);
}

/* ------------------------------------------------------------------------ */
/* Combine                                                                   */
/* ------------------------------------------------------------------------ */

/* out[t][m] = sum over j = 0..k-1 of w[t][j] * y[t*k + j][m], slot order,
 * multiply then add.  y is indexed by flat slot; rows of slots whose valid[]
 * flag is 0 contribute nothing. */
void oracle_combine(const double *y_by_slot, const float *w,
                    const int32_t *valid, int32_t M, int32_t k, int32_t hidden,
                    double *out)
{
    for (int64_t t = 0; t < M; ++t) {
        for (int64_t m = 0; m < hidden; ++m) out[t * hidden + m] = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            int64_t s = t * k + j;
            double wt = (double)w[s];
            if (!valid[s]) continue;
            for (int64_t m = 0; m < hidden; ++m) {
                double prod = wt * y_by_slot[s * hidden + m];
                out[t * hidden + m] += prod;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Router: the top-k experts of each token and their weights                 */
/* ------------------------------------------------------------------------ */

/* Two routers are defined.
 *   kind 0, softmax (the routing of the benchmark workloads):
 *     p[e] = exp(l[e] - m) / sum_e' exp(l[e'] - m),  m = max_e l[e];
 *     the k experts with the largest p are chosen.  p is strictly increasing
 *     in the logit, so the order is the order of the logits themselves.
 *     Weights: renormalized, w[j] = exp(l[j] - l[0]) / sum_{i<k} exp(l[i] - l[0])
 *     (this is p[j] / sum of the chosen p), else w[j] = p[j].
 *   kind 1, sigmoid with a selection bias ("memra-engine
 *     src/bin/ep_step_fp8_gate.rs", the full-layer gate's sigmoid top-k router
 *     with router bias, router scale and route norm; "spark_model
 *     glm5next_mlp/forward.rs", the router launch in fn forward_moe with its
 *     bias, routed_scale and renormalize arguments):
 *     s[e] = 1 / (1 + exp(-l[e])); the key is binary32(s[e]) + bias[e], one
 *     binary32 addition; the k largest keys are chosen.  The bias only
 *     selects: w[j] = s[j], renormalized by the sum of the chosen s if asked.
 * Both: w[j] is then multiplied by routed_scale and rounded once to binary32.
 * Readings where the pages are silent:
 *   - ties in the key go to the lower expert id, and slot j holds rank j;
 *   - a NaN logit counts as -FLT_MAX and an infinite one as +-FLT_MAX, so
 *     every key and weight is finite;
 *   - the sigmoid weights renormalize by the sum of the chosen s; where that
 *     sum is 0 (every chosen s underflows, logits below about -745) the
 *     weights are 0.  The softmax sum is at least 1;
 *   - sums over the chosen experts run in rank order, the softmax
 *     denominator over e ascending, all in double. */
typedef struct {
    float key;
    int32_t id;
} router_key_t;

static int router_key_cmp(const void *pa, const void *pb)
{
    const router_key_t *a = pa, *b = pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

static double router_logit(float v)
{
    if (isnan(v)) return -(double)FLT_MAX;
    if (v > FLT_MAX) return (double)FLT_MAX;
    if (v < -FLT_MAX) return -(double)FLT_MAX;
    return (double)v;
}

int oracle_router_topk(const float *logits, int32_t M, int32_t E, int32_t k,
                       int32_t kind, const float *bias, float routed_scale,
                       int32_t renormalize, int32_t *ids, float *w)
{
    if (M < 1 || k < 1 || k > E || (kind != 0 && kind != 1)) return -1;
    double *l = malloc(sizeof(double) * (size_t)E);
    double *s = malloc(sizeof(double) * (size_t)E);
    router_key_t *keys = malloc(sizeof(router_key_t) * (size_t)E);
    for (int64_t t = 0; t < M; ++t) {
        for (int32_t e = 0; e < E; ++e) l[e] = router_logit(logits[t * E + e]);
        if (kind == 0) {
            double m = l[0];
            for (int32_t e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
            double den = 0.0;
            for (int32_t e = 0; e < E; ++e) den += exp(l[e] - m);
            for (int32_t e = 0; e < E; ++e) {
                s[e] = exp(l[e] - m) / den;
                keys[e].key = (float)l[e];
                keys[e].id = e;
            }
        } else {
            for (int32_t e = 0; e < E; ++e) {
                s[e] = 1.0 / (1.0 + exp(-l[e]));
                float b = bias ? bias[e] : 0.0f;
                volatile float sk = (float)s[e];      /* one rounding, then one addition */
                keys[e].key = sk + b;
                keys[e].id = e;
            }
        }
        qsort(keys, (size_t)E, sizeof(router_key_t), router_key_cmp);
        double sum = 0.0;
        if (renormalize) {
            for (int32_t j = 0; j < k; ++j) {
                int32_t e = keys[j].id;
                sum += kind == 0 ? exp(l[e] - l[keys[0].id]) : s[e];
            }
        }
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = keys[j].id;
            double v;
            if (!renormalize) v = s[e];
            else if (kind == 0) v = exp(l[e] - l[keys[0].id]) / sum;
            else v = sum > 0.0 ? s[e] / sum : 0.0;
            ids[t * k + j] = e;
            w[t * k + j] = (float)(v * (double)routed_scale);
        }
    }
    free(l); free(s); free(keys);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Shared expert and residual                                                */
/* ------------------------------------------------------------------------ */

/* The shared expert: a dense SwiGLU MLP of width W with bf16 weights, applied
 * to every token with weight 1 ("spark_model glm5next_mlp/forward.rs",
 * fn forward_dense: down(clamped_swiglu(gate(x), up(x))), the same math as a
 * routed expert with its own clamp, and the shared-expert step of
 * fn forward_moe, not routed-scaled).  For each token t:
 *   g = Wg x[t], u = Wu x[t]   (FP64 sums over decoded bf16 values)
 *   h = swiglu_clamp(g, u, L)  (FP64)
 *   out[t] = Wd h
 * gate, up: bf16 [W][H]; down: bf16 [H][W]; x: bf16 [M][H]; out [M][H]. */
void oracle_shared_expert(const uint16_t *gate, const uint16_t *up,
                          const uint16_t *down, const uint16_t *x, int32_t M,
                          int32_t H, int32_t W, float limit, double *out)
{
    double *xv = malloc(sizeof(double) * (size_t)H);
    double *h = malloc(sizeof(double) * (size_t)W);
    for (int64_t t = 0; t < M; ++t) {
        for (int64_t i = 0; i < H; ++i) xv[i] = oracle_bf16_value(x[t * H + i]);
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < W; ++n) {
            double g = 0.0, u = 0.0;
            for (int64_t i = 0; i < H; ++i) {
                g += oracle_bf16_value(gate[n * H + i]) * xv[i];
                u += oracle_bf16_value(up[n * H + i]) * xv[i];
            }
            h[n] = oracle_swiglu_clamp(g, u, (double)limit);
        }
#pragma omp parallel for schedule(static)
        for (int64_t m = 0; m < H; ++m) {
            double y = 0.0;
            for (int64_t n = 0; n < W; ++n) y += oracle_bf16_value(down[m * W + n]) * h[n];
            out[t * H + m] = y;
        }
    }
    free(xv); free(h);
}

/* out[t][m] = ((sum_j w[t][j] * y[t*k + j][m]) + shared[t][m]) + residual[t][m]:
 * the routed combine in slot order, then the shared expert's row, then the
 * residual ("memra-engine src/bin/ep_step_fp8_gate.rs", the full-layer gate's
 * final add order routed-plus-shared-then-residual).  Rows of slots whose
 * valid[] flag is 0 contribute nothing; shared or residual may be NULL. */
void oracle_combine_residual(const double *y_by_slot, const float *w,
                             const int32_t *valid, const double *shared,
                             const float *residual, int32_t M, int32_t k,
                             int32_t hidden, double *out)
{
    oracle_combine(y_by_slot, w, valid, M, k, hidden, out);
    for (int64_t t = 0; t < M; ++t)
        for (int64_t m = 0; m < hidden; ++m) {
            double v = out[t * hidden + m];
            if (shared) v += shared[t * hidden + m];
            if (residual) v += (double)residual[t * hidden + m];
            out[t * hidden + m] = v;
        }
}
