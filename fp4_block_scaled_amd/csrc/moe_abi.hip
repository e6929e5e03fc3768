// moe_abi.hip -- the C ABI of libmoe: argument checks, workspace carving and
// tier dispatch for the routed MoE FFN layer (declared in include/moe.h).
//
// Everything here runs on the host before any launch; a failed check returns
// a status without touching the GPU.  The calls never allocate, synchronise
// or read device memory back, so a caller may capture them in a HIP graph.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <chrono>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "moe_internal.h"

// The workspace of moe_layer_static: one array per GPU the library runs on,
// held until the process ends.  Host code never uses its name as an address
// (on the host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;
thread_local void *const *g_stage_events = nullptr;
thread_local int32_t g_stage_n = 0;

// Records stage event i (if stage timing is on and i is in range).
void stage_mark(int i, hipStream_t s)
{
    if (g_stage_events && i < g_stage_n && g_stage_events[i])
        (void)hipEventRecord((hipEvent_t)g_stage_events[i], s);
}

moe_status_t fail(moe_status_t code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

moe_status_t hip_fail(hipError_t e, const char *what)
{
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// FFN scratch of the GEMV tier for S slots.
// FFN scratch of the GEMV tier: h, the SwiGLU output [S][inter].
size_t gemv_scratch_bytes(int64_t S, int32_t inter)
{
    return moe::align256(sizeof(float) * (size_t)(S * inter));
}

bool sizes_ok(int32_t M, int32_t top_k, int32_t E)
{
    return M >= 1 && top_k >= 1 && E >= 1 && top_k <= E && E <= MOE_MAX_EXPERTS &&
           (int64_t)M * top_k < (1ll << 31);
}

int32_t resolve(int32_t M, int32_t fmt, int32_t requested)
{
    if (requested == MOE_MODE_GEMV_A16 || requested == MOE_MODE_GEMM_A8 ||
        requested == MOE_MODE_FUSED || requested == MOE_MODE_GEMM_A16)
        return requested;
    if (M <= MOE_GEMV_MAX_M) return MOE_MODE_GEMV_A16;
    return fmt == MOE_W_NVFP4_B16 ? MOE_MODE_GEMM_A16 : MOE_MODE_GEMM_A8;
}

bool valid_mode(int32_t mode)
{
    return mode >= MOE_MODE_AUTO && mode <= MOE_MODE_GEMM_A16;
}

bool ffn_dims_ok(int32_t fmt, int32_t hidden, int32_t inter)
{
    if (hidden <= 0 || inter <= 0 || hidden % 128 || inter % 128) return false;
    if (hidden > MOE_MAX_DIM || inter > MOE_MAX_DIM) return false;
    if (fmt == MOE_W_NVFP4_B16 && (hidden % 256 || inter % 256)) return false;
    return true;
}

// FFN scratch of the FP8 GEMM tier for M tokens and S slots.
struct GemmScratch {
    uint8_t *xq, *hq;
    float *xs, *hs;
    int4 *tiles;
    int32_t *ntiles;
};

size_t gemm_scratch_bytes(int64_t M, int64_t S, int32_t E, int32_t hidden, int32_t inter)
{
    const int64_t tmax = gemm_max_tiles((int32_t)S, E);
    return moe::align256((size_t)(M * hidden)) +                          // xq
           moe::align256(sizeof(float) * (size_t)(M * (hidden / 128))) +  // xs
           moe::align256((size_t)(S * inter)) +                           // hq
           moe::align256(sizeof(float) * (size_t)(S * (inter / 128))) +   // hs
           moe::align256(sizeof(int4) * (size_t)tmax) + 256;              // tiles, count
}

GemmScratch carve_gemm(char *p, int64_t M, int64_t S, int32_t E, int32_t hidden, int32_t inter)
{
    GemmScratch g;
    const int64_t tmax = gemm_max_tiles((int32_t)S, E);
    g.xq = (uint8_t *)p;  p += moe::align256((size_t)(M * hidden));
    g.xs = (float *)p;    p += moe::align256(sizeof(float) * (size_t)(M * (hidden / 128)));
    g.hq = (uint8_t *)p;  p += moe::align256((size_t)(S * inter));
    g.hs = (float *)p;    p += moe::align256(sizeof(float) * (size_t)(S * (inter / 128)));
    g.tiles = (int4 *)p;  p += moe::align256(sizeof(int4) * (size_t)tmax);
    g.ntiles = (int32_t *)p;
    return g;
}

// Scratch of moe_layer_fused after the route region: h [S][inter] FP32, then
// the epoch flags, one 32-bit word per gate/up item (A x inter/2: the
// one-token kernel's 2-row items; the general kernel uses the first A x
// inter/16) and per down item (hidden/32 x A), A = min(S, E).
size_t fused_scratch_bytes(int64_t S, int32_t E, int32_t hidden, int32_t inter)
{
    const size_t A = (size_t)(S < E ? S : E);
    return moe::align256(sizeof(float) * (size_t)(S * inter)) +
           moe::align256(4 * A * (size_t)(inter / 2 + hidden / 32));
}

// The fused layer serves NVFP4 banks for one token with hidden a multiple of
// 2048 (one 1 KB code load per 2048 K values) up to 16384.
bool nvfp4_fused_ok(int64_t M, int32_t hidden)
{
    return M == 1 && hidden % 2048 == 0 && hidden <= 16384;
}

// Points *route at the route tables at the start of ws.
void carve_route(void *ws, int32_t M, int32_t top_k, int32_t E, moe_route_t *route)
{
    const int64_t S = (int64_t)M * top_k;
    const int64_t A = S < E ? S : E;
    char *p = (char *)ws;
    route->M = M;
    route->top_k = top_k;
    route->num_experts = E;
    route->num_slots = (int32_t)S;
    route->expert_offsets = (int32_t *)p; p += moe::align256(sizeof(int32_t) * (E + 1));
    route->sorted_slot = (int32_t *)p;    p += moe::align256(sizeof(int32_t) * S);
    route->sorted_token = (int32_t *)p;   p += moe::align256(sizeof(int32_t) * S);
    route->token_to_perm = (int32_t *)p;  p += moe::align256(sizeof(int32_t) * S);
    route->active_experts = (int32_t *)p; p += moe::align256(sizeof(int32_t) * (A > 0 ? A : 1));
    route->num_active = (int32_t *)p;
    route->status = (int32_t *)p + 1;
}

// The GEMM tiers address activation rows with 32-bit byte offsets (bf16
// rows in the A16 tier: two bytes per element).
bool gemm_dims_ok(int64_t M, int64_t S, int32_t hidden, int32_t inter, int32_t elem_bytes = 1)
{
    return M * hidden * elem_bytes < (int64_t(1) << 31) &&
           S * inter * elem_bytes < (int64_t(1) << 31);
}

// Scratch of the 16-bit GEMM tier: h FP16 [S][inter], the tiles.
struct GemmA16Scratch {
    uint16_t *h16;
    int4 *tiles;
    int32_t *ntiles;
};

size_t gemm_a16_scratch_bytes(int64_t S, int32_t E, int32_t inter)
{
    const int64_t tmax = gemm_max_tiles((int32_t)S, E);
    return moe::align256(2 * (size_t)(S * inter)) + moe::align256(sizeof(int4) * (size_t)tmax) + 256;
}

GemmA16Scratch carve_gemm_a16(char *p, int64_t S, int32_t E, int32_t inter)
{
    GemmA16Scratch g;
    const int64_t tmax = gemm_max_tiles((int32_t)S, E);
    g.h16 = (uint16_t *)p;  p += moe::align256(2 * (size_t)(S * inter));
    g.tiles = (int4 *)p;    p += moe::align256(sizeof(int4) * (size_t)tmax);
    g.ntiles = (int32_t *)p;
    return g;
}

size_t ffn_bytes(int64_t M, int64_t S, int32_t E, int32_t hidden, int32_t inter, int32_t fmt,
                 int32_t mode)
{
    if (mode == MOE_MODE_GEMV_A16) return gemv_scratch_bytes(S, inter);
    if (mode == MOE_MODE_GEMM_A16) {
        if (fmt != MOE_W_NVFP4_B16 || !gemm_dims_ok(M, S, hidden, inter, 2)) return 0;
        return gemm_a16_scratch_bytes(S, E, inter);
    }
    if (fmt != MOE_W_E4M3_B128 || !gemm_dims_ok(M, S, hidden, inter)) return 0;
    return gemm_scratch_bytes(M, S, E, hidden, inter);
}

}  // namespace

extern "C" {

const char *moe_last_error(void) { return g_last_error.c_str(); }

int32_t moe_set_stage_events(void *const *events, int32_t n_events, int32_t fmt, int32_t hidden,
                             int32_t inter, int32_t mode)
{
    g_stage_events = events;
    g_stage_n = events ? n_events : 0;
    (void)fmt; (void)hidden; (void)inter;
    // GEMV tier: gate/up GEMV with SwiGLU, down GEMV
    // fused layer: its one launch
    // FP8 GEMM tier: activation quantization + tile schedule, gate/up GEMM, down GEMM
    // bf16 GEMM tier: tile schedule, gate/up GEMM, down GEMM
    return mode == MOE_MODE_GEMV_A16 ? 2 : mode == MOE_MODE_FUSED ? 1 : 3;
}

int32_t moe_resolve_mode(int32_t M, int32_t fmt, int32_t requested)
{
    return resolve(M, fmt, requested);
}

size_t moe_workspace_bytes(int32_t max_M, int32_t top_k, int32_t num_experts, int32_t hidden,
                           int32_t inter, int32_t fmt, int32_t mode)
{
    if (!sizes_ok(max_M, top_k, num_experts)) return 0;
    if (fmt != MOE_W_E4M3_B128 && fmt != MOE_W_NVFP4_B16) return 0;
    if (!valid_mode(mode)) return 0;
    if (!ffn_dims_ok(fmt, hidden, inter)) return 0;
    const int64_t S = (int64_t)max_M * top_k;
    if (mode == MOE_MODE_FUSED) {
        if (S > MOE_FUSED_MAX_SLOTS) return 0;
        if (fmt == MOE_W_NVFP4_B16 && !nvfp4_fused_ok(max_M, hidden)) return 0;
        return moe::route_region_bytes(S, num_experts) + fused_scratch_bytes(S, num_experts, hidden, inter);
    }
    size_t ffn;
    if (mode == MOE_MODE_AUTO) {
        const int64_t mg = max_M < MOE_GEMV_MAX_M ? max_M : MOE_GEMV_MAX_M;
        ffn = ffn_bytes(mg, mg * top_k, num_experts, hidden, inter, fmt, MOE_MODE_GEMV_A16);
        // GEMM scratch only where that tier can run (E4M3, within its
        // limits); a call above MOE_GEMV_MAX_M tokens outside them is
        // refused by moe_expert_ffn
        if (max_M > MOE_GEMV_MAX_M) {
            const size_t g = ffn_bytes(max_M, S, num_experts, hidden, inter, fmt,
                                       resolve(max_M, fmt, MOE_MODE_AUTO));
            ffn = g > ffn ? g : ffn;
        }
    } else {
        ffn = ffn_bytes(max_M, S, num_experts, hidden, inter, fmt, mode);
        if (ffn == 0) return 0;
    }
    return moe::route_region_bytes(S, num_experts) + ffn;
}

moe_status_t moe_route_pack(const int32_t *topk_ids, int32_t M, int32_t top_k, int32_t num_experts,
                            void *ws, size_t ws_bytes, moe_route_t *route, void *stream)
{
    if (!topk_ids || !ws || !route) return fail(MOE_ERR_ARG, "moe_route_pack: null pointer");
    if (!sizes_ok(M, top_k, num_experts))
        return fail(MOE_ERR_SHAPE,
                    "moe_route_pack: need M >= 1, 1 <= top_k <= num_experts <= %d, M*top_k < 2^31 "
                    "(M=%d top_k=%d E=%d)",
                    MOE_MAX_EXPERTS, M, top_k, num_experts);
    const int64_t S = (int64_t)M * top_k;
    const size_t need = moe::route_region_bytes(S, num_experts);
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "moe_route_pack: workspace %zu bytes < %zu", ws_bytes, need);
    if (((uintptr_t)ws & 255) != 0) return fail(MOE_ERR_ARG, "moe_route_pack: ws not 256-byte aligned");

    carve_route(ws, M, top_k, num_experts, route);

    MoeRouteDev r{route->expert_offsets, route->sorted_slot, route->sorted_token,
                  route->token_to_perm, route->active_experts, route->num_active, route->status};
    hipError_t e = launch_route_pack(topk_ids, M, top_k, num_experts, r, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "moe_route_pack: route_pack launch");
    return MOE_OK;
}

static moe_status_t check_bank(const char *fn, const moe_bank_t *b, const char *name, int32_t fmt,
                               int32_t E, int32_t n_out, int32_t k_in)
{
    if (!b || !b->codes || !b->scales)
        return fail(MOE_ERR_ARG, "%s: %s bank or its codes/scales is null", fn, name);
    if (b->fmt != fmt)
        return fail(MOE_ERR_FORMAT, "%s: %s bank format %d differs from gate's %d",
                    fn, name, b->fmt, fmt);
    if (fmt == MOE_W_E4M3_B128 && b->scale2)
        return fail(MOE_ERR_FORMAT, "%s: %s bank: scale2 must be NULL for E4M3", fn, name);
    if (fmt == MOE_W_NVFP4_B16 && !b->scale2)
        return fail(MOE_ERR_FORMAT, "%s: %s bank: NVFP4 needs scale2", fn, name);
    if (b->num_experts != E || b->n_out != n_out || b->k_in != k_in)
        return fail(MOE_ERR_SHAPE,
                    "%s: %s bank is E=%d %dx%d, expected E=%d %dx%d", fn, name,
                    b->num_experts, b->n_out, b->k_in, E, n_out, k_in);
    if (!aligned16(b->codes))
        return fail(MOE_ERR_ARG, "%s: %s codes not 16-byte aligned", fn, name);
    return MOE_OK;
}

// The expert FFN of moe_expert_ffn.  With route_ids, the route tables of
// `route` (carved, not yet filled) are built by the gate/up launch itself
// from the ids: only for the GEMV tier and S <= 128 (E4M3) or 64 (NVFP4).  With comb_out as well
// (moe_layer), one token whose shape gemv_down1_fits accepts gets the down
// projection and the combine in one launch (out = comb_out, weights comb_w),
// and *combined says so; otherwise the caller runs the combine.
static moe_status_t expert_ffn(const moe_bank_t *gate, const moe_bank_t *up, const moe_bank_t *down,
                               const uint16_t *x_bf16, const moe_route_t *route, int32_t hidden,
                               int32_t inter, float limit, int32_t mode, float *y_packed, void *ws,
                               size_t ws_bytes, void *stream, const int32_t *route_ids,
                               const float *comb_w = nullptr, float *comb_out = nullptr,
                               bool *combined = nullptr)
{
    if (combined) *combined = false;
    if (!gate || !up || !down || !x_bf16 || !route || !y_packed || !ws)
        return fail(MOE_ERR_ARG, "moe_expert_ffn: null pointer");
    const int32_t fmt = gate->fmt;
    if (fmt != MOE_W_E4M3_B128 && fmt != MOE_W_NVFP4_B16)
        return fail(MOE_ERR_FORMAT, "moe_expert_ffn: unknown weight format %d", fmt);
    if (!valid_mode(mode) || mode == MOE_MODE_FUSED)
        return fail(MOE_ERR_ARG, "moe_expert_ffn: unknown mode %d%s", mode,
                    mode == MOE_MODE_FUSED ? " (the fused layer is moe_layer_fused)" : "");
    if (!ffn_dims_ok(fmt, hidden, inter))
        return fail(MOE_ERR_SHAPE,
                    "moe_expert_ffn: hidden %d and inter %d must be positive multiples of %d, "
                    "at most %d", hidden, inter, fmt == MOE_W_NVFP4_B16 ? 256 : 128, MOE_MAX_DIM);
    if (route->expert_offsets != (int32_t *)ws || !sizes_ok(route->M, route->top_k, route->num_experts) ||
        route->num_slots != route->M * route->top_k)
        return fail(MOE_ERR_ARG, "moe_expert_ffn: route does not come from moe_route_pack on this ws");
    const int32_t E = route->num_experts;
    moe_status_t st;
    if ((st = check_bank("moe_expert_ffn", gate, "gate", fmt, E, inter, hidden))) return st;
    if ((st = check_bank("moe_expert_ffn", up, "up", fmt, E, inter, hidden))) return st;
    if ((st = check_bank("moe_expert_ffn", down, "down", fmt, E, hidden, inter))) return st;
    if (!aligned16(x_bf16) || !aligned16(y_packed))
        return fail(MOE_ERR_ARG, "moe_expert_ffn: x and y must be 16-byte aligned");
    if (!(limit > 0.0f)) return fail(MOE_ERR_ARG, "moe_expert_ffn: limit must be > 0");
    const int32_t M = route->M, k = route->top_k;
    const int32_t tier = resolve(M, fmt, mode);
    if (tier == MOE_MODE_GEMM_A8 && fmt != MOE_W_E4M3_B128)
        return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: the FP8 GEMM tier serves E4M3 banks only");
    if (tier == MOE_MODE_GEMM_A8 && !gemm_dims_ok(M, (int64_t)M * k, hidden, inter))
        return fail(MOE_ERR_SHAPE,
                    "moe_expert_ffn: GEMM tier needs M*hidden and M*top_k*inter < 2^31 "
                    "(M=%d top_k=%d hidden=%d inter=%d)", M, k, hidden, inter);
    if (tier == MOE_MODE_GEMM_A16 && fmt != MOE_W_NVFP4_B16)
        return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: the bf16 GEMM tier serves NVFP4 banks only");
    if (tier == MOE_MODE_GEMM_A16 && !gemm_dims_ok(M, (int64_t)M * k, hidden, inter, 2))
        return fail(MOE_ERR_SHAPE,
                    "moe_expert_ffn: bf16 GEMM tier needs 2*M*hidden and 2*M*top_k*inter < 2^31 "
                    "(M=%d top_k=%d hidden=%d inter=%d)", M, k, hidden, inter);
    if (tier == MOE_MODE_GEMM_A16 && (((uintptr_t)gate->scales | (uintptr_t)up->scales |
                                       (uintptr_t)down->scales) & 3))
        return fail(MOE_ERR_ARG, "moe_expert_ffn: the bf16 GEMM tier needs 4-byte aligned scales");
    const size_t need = moe_workspace_bytes(M, k, E, hidden, inter, fmt, tier);
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn: workspace %zu bytes < %zu", ws_bytes, need);

    const int64_t S = (int64_t)M * k;
    hipStream_t s = (hipStream_t)stream;
    MoeRouteDev r{route->expert_offsets, route->sorted_slot, route->sorted_token,
                  route->token_to_perm, route->active_experts, route->num_active, route->status};
    char *scratch = (char *)ws + moe::route_region_bytes(S, E);
    if (tier == MOE_MODE_GEMM_A8) {
        GemmScratch gs = carve_gemm(scratch, M, S, E, hidden, inter);
        const int32_t tmax = gemm_max_tiles((int32_t)S, E);
        hipError_t e;
        stage_mark(0, s);
        e = launch_quant_act(x_bf16, M, hidden, gs.xq, gs.xs, s);
        if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: activation quantization launch");
        e = launch_gemm_tiles(r.offsets, E, tmax, gs.tiles, gs.ntiles, s, true);
        if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: tile schedule launch");
        stage_mark(1, s);
        e = launch_gemm_gateup(gs.xq, gs.xs, r.sorted_token, gate->codes, (const float *)gate->scales,
                               up->codes, (const float *)up->scales, r.offsets, gs.tiles,
                               gs.ntiles, tmax, hidden, inter, limit, gs.hq, gs.hs, s);
        if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: gate/up GEMM launch");
        stage_mark(2, s);
        e = launch_gemm_down(gs.hq, gs.hs, down->codes, (const float *)down->scales, r.offsets,
                             gs.tiles, gs.ntiles, tmax, hidden, inter, y_packed, s);
        if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: down GEMM launch");
        stage_mark(3, s);
        return MOE_OK;
    }
    GemvBankDev bg{gate->codes, gate->scales, gate->scale2};
    GemvBankDev bu{up->codes, up->scales, up->scale2};
    GemvBankDev bd{down->codes, down->scales, down->scale2};
    hipError_t e;
    if (tier == MOE_MODE_GEMM_A16) {
        GemmA16Scratch gs = carve_gemm_a16(scratch, S, E, inter);
        const int32_t tmax = gemm_max_tiles((int32_t)S, E);
        stage_mark(0, s);
        e = launch_gemm_tiles(r.offsets, E, tmax, gs.tiles, gs.ntiles, s, false);
        if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: tile schedule launch");
        stage_mark(1, s);
        e = launch_gemm_gateup_nvfp4(x_bf16, r.sorted_token, bg, bu, r.offsets, gs.tiles, gs.ntiles,
                                     tmax, hidden, inter, limit, gs.h16, s);
        if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: gate/up GEMM launch");
        stage_mark(2, s);
        e = launch_gemm_down_nvfp4(gs.h16, bd, r.offsets, gs.tiles, gs.ntiles, tmax, hidden, inter,
                                   limit, y_packed, s);
        if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: down GEMM launch");
        stage_mark(3, s);
        return MOE_OK;
    }
    float *h = (float *)scratch;
    stage_mark(0, s);
    if (fmt == MOE_W_E4M3_B128)
        e = launch_gemv_gateup_e4m3(bg, bu, x_bf16, r, M, (int32_t)S, E, hidden, inter, limit, h, s,
                                    route_ids, k);
    else
        e = launch_gemv_gateup_nvfp4(bg, bu, x_bf16, r, M, (int32_t)S, E, hidden, inter, limit, h, s,
                                     route_ids, k);
    if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: gate/up GEMV launch");
    stage_mark(1, s);
    const int kfmt = fmt == MOE_W_E4M3_B128 ? kFmtE4M3 : kFmtNVFP4;
    if (route_ids && comb_w && comb_out && gemv_down1_fits(kfmt, M, k, hidden, inter)) {
        if (fmt == MOE_W_E4M3_B128)
            e = launch_gemv_down1_e4m3(bd, h, route_ids, r.token_to_perm, comb_w, k, hidden, inter,
                                       y_packed, comb_out, s);
        else
            e = launch_gemv_down1_nvfp4(bd, h, route_ids, r.token_to_perm, comb_w, k, hidden, inter,
                                        y_packed, comb_out, s);
        if (e != hipSuccess) return hip_fail(e, "moe_layer: down + combine GEMV launch");
        *combined = true;
        stage_mark(2, s);
        return MOE_OK;
    }
    if (fmt == MOE_W_E4M3_B128)
        e = launch_gemv_down_e4m3(bd, h, r, M, (int32_t)S, E, hidden, inter, y_packed, s);
    else
        e = launch_gemv_down_nvfp4(bd, h, r, M, (int32_t)S, E, hidden, inter, y_packed, s);
    if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: down GEMV launch");
    stage_mark(2, s);
    return MOE_OK;
}

moe_status_t moe_expert_ffn(const moe_bank_t *gate, const moe_bank_t *up, const moe_bank_t *down,
                            const uint16_t *x_bf16, const moe_route_t *route, int32_t hidden,
                            int32_t inter, float limit, int32_t mode, float *y_packed, void *ws,
                            size_t ws_bytes, void *stream)
{
    return expert_ffn(gate, up, down, x_bf16, route, hidden, inter, limit, mode, y_packed, ws,
                      ws_bytes, stream, nullptr);
}

moe_status_t moe_layer(const moe_bank_t *gate, const moe_bank_t *up, const moe_bank_t *down,
                       const uint16_t *x_bf16, const int32_t *topk_ids, const float *topk_weights,
                       int32_t M, int32_t top_k, int32_t hidden, int32_t inter, float limit,
                       int32_t mode, float *y_packed, float *out, void *ws, size_t ws_bytes,
                       moe_route_t *route, void *stream)
{
    static const char *fn = "moe_layer";
    if (!gate || !up || !down || !x_bf16 || !topk_ids || !topk_weights || !y_packed || !out ||
        !ws || !route)
        return fail(MOE_ERR_ARG, "%s: null pointer", fn);
    const int32_t fmt = gate->fmt, E = gate->num_experts;
    if (!sizes_ok(M, top_k, E))
        return fail(MOE_ERR_SHAPE, "%s: need M >= 1, 1 <= top_k <= num_experts <= %d (M=%d top_k=%d E=%d)",
                    fn, MOE_MAX_EXPERTS, M, top_k, E);
    if (!valid_mode(mode) || mode == MOE_MODE_FUSED)
        return fail(MOE_ERR_ARG, "%s: unknown mode %d", fn, mode);
    const int64_t S = (int64_t)M * top_k;
    moe_status_t st;
    // (E4M3 up to 128 slots; the NVFP4 gate/up kernel with the route built in
    // ran slower at 128 slots than route_pack and the plain kernel together)
    if (S <= (fmt == MOE_W_E4M3_B128 ? 128 : 64) && resolve(M, fmt, mode) == MOE_MODE_GEMV_A16) {
        // the route pack runs inside the gate/up launch
        if (ws_bytes < moe::route_region_bytes(S, E))
            return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, ws_bytes,
                        moe::route_region_bytes(S, E));
        if (((uintptr_t)ws & 255) != 0) return fail(MOE_ERR_ARG, "%s: ws not 256-byte aligned", fn);
        carve_route(ws, M, top_k, E, route);
        bool combined = false;
        st = expert_ffn(gate, up, down, x_bf16, route, hidden, inter, limit, mode, y_packed, ws,
                        ws_bytes, stream, topk_ids, topk_weights, aligned16(out) ? out : nullptr,
                        &combined);
        if (st != MOE_OK || combined) return st;
    } else {
        st = moe_route_pack(topk_ids, M, top_k, E, ws, ws_bytes, route, stream);
        if (st == MOE_OK)
            st = expert_ffn(gate, up, down, x_bf16, route, hidden, inter, limit, mode, y_packed, ws,
                            ws_bytes, stream, nullptr);
    }
    if (st != MOE_OK) return st;
    return moe_combine(y_packed, route, topk_weights, hidden, out, stream);
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
static moe_status_t static_scratch(const char *fn, void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_static: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_UNSUPPORTED, "%s: device %d past the %d the static scratch serves", fn,
                    dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "moe_layer_static: hipGetSymbolAddress(scratch)");
        if (!p || ((uintptr_t)p & 255) != 0)
            return fail(MOE_ERR_HIP, "%s: static scratch at %p is not 256-byte aligned", fn, p);
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return MOE_OK;
}

moe_status_t moe_layer_static(const moe_bank_t *gate, const moe_bank_t *up, const moe_bank_t *down,
                              const uint16_t *x_bf16, const int32_t *topk_ids,
                              const float *topk_weights, int32_t M, int32_t top_k, int32_t hidden,
                              int32_t inter, float limit, int32_t mode, float *y_packed, float *out,
                              moe_route_t *route, void *stream)
{
    static const char *fn = "moe_layer_static";
    if (!gate || !up || !down || !route) return fail(MOE_ERR_ARG, "%s: null pointer", fn);
    if (!valid_mode(mode) || mode == MOE_MODE_FUSED)
        return fail(MOE_ERR_ARG, "%s: unknown mode %d", fn, mode);
    const int32_t fmt = gate->fmt, E = gate->num_experts;
    const size_t need = moe_workspace_bytes(M, top_k, E, hidden, inter, fmt, resolve(M, fmt, mode));
    if (need > MOE_STATIC_SCRATCH_BYTES)
        return fail(MOE_ERR_WORKSPACE,
                    "%s: the layer needs %zu bytes of scratch, more than the static %u; "
                    "call moe_layer with a workspace of your own", fn, need,
                    (unsigned)MOE_STATIC_SCRATCH_BYTES);
    void *ws = nullptr;
    moe_status_t st = static_scratch(fn, &ws);
    if (st != MOE_OK) return st;
    // moe_layer checks everything else (a zero `need` included) before any launch
    return moe_layer(gate, up, down, x_bf16, topk_ids, topk_weights, M, top_k, hidden, inter,
                     limit, mode, y_packed, out, ws, MOE_STATIC_SCRATCH_BYTES, route, stream);
}

moe_status_t moe_layer_fused(const moe_bank_t *gate, const moe_bank_t *up, const moe_bank_t *down,
                             const uint16_t *x_bf16, const int32_t *topk_ids,
                             const float *topk_weights, int32_t M, int32_t top_k, int32_t hidden,
                             int32_t inter, float limit, float *y_packed, float *out, void *ws,
                             size_t ws_bytes, moe_route_t *route, void *stream)
{
    static const char *fn = "moe_layer_fused";
    if (!gate || !up || !down || !x_bf16 || !topk_ids || !topk_weights || !y_packed || !out ||
        !ws || !route)
        return fail(MOE_ERR_ARG, "%s: null pointer", fn);
    const int32_t fmt = gate->fmt, E = gate->num_experts;
    if (fmt != MOE_W_E4M3_B128 && fmt != MOE_W_NVFP4_B16)
        return fail(MOE_ERR_FORMAT, "%s: unknown weight format %d", fn, fmt);
    if (!sizes_ok(M, top_k, E))
        return fail(MOE_ERR_SHAPE, "%s: need M >= 1, 1 <= top_k <= num_experts <= %d (M=%d top_k=%d E=%d)",
                    fn, MOE_MAX_EXPERTS, M, top_k, E);
    if ((int64_t)M * top_k > MOE_FUSED_MAX_SLOTS)
        return fail(MOE_ERR_SHAPE, "%s: M*top_k = %lld > %d", fn, (long long)M * top_k,
                    MOE_FUSED_MAX_SLOTS);
    if (!ffn_dims_ok(fmt, hidden, inter))
        return fail(MOE_ERR_SHAPE, "%s: hidden %d and inter %d must be positive multiples of %d, "
                    "at most %d", fn, hidden, inter, fmt == MOE_W_NVFP4_B16 ? 256 : 128, MOE_MAX_DIM);
    moe_status_t st;
    if ((st = check_bank(fn, gate, "gate", fmt, E, inter, hidden))) return st;
    if ((st = check_bank(fn, up, "up", fmt, E, inter, hidden))) return st;
    if ((st = check_bank(fn, down, "down", fmt, E, hidden, inter))) return st;
    if (fmt == MOE_W_NVFP4_B16 && !nvfp4_fused_ok(M, hidden))
        return fail(MOE_ERR_UNSUPPORTED, "%s: NVFP4 banks need M = 1 and hidden a multiple of 2048 "
                    "up to 16384 (M=%d hidden=%d)", fn, M, hidden);
    if (!aligned16(x_bf16) || !aligned16(y_packed) || !aligned16(out))
        return fail(MOE_ERR_ARG, "%s: x, y and out must be 16-byte aligned", fn);
    if (!(limit > 0.0f)) return fail(MOE_ERR_ARG, "%s: limit must be > 0", fn);
    if (((uintptr_t)ws & 255) != 0) return fail(MOE_ERR_ARG, "%s: ws not 256-byte aligned", fn);
    const size_t need = moe_workspace_bytes(M, top_k, E, hidden, inter, fmt, MOE_MODE_FUSED);
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, ws_bytes, need);

    hipStream_t s = (hipStream_t)stream;
    // the epoch is a launch argument: a captured launch would replay with the
    // same epoch, and flags left by an earlier replay could then end a wait
    // before the data behind them is written
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t ce = hipStreamIsCapturing(s, &cap);
    if (ce != hipSuccess) return hip_fail(ce, "moe_layer_fused: hipStreamIsCapturing");
    if (cap != hipStreamCaptureStatusNone)
        return fail(MOE_ERR_UNSUPPORTED, "%s: cannot be captured into a HIP graph (each call needs a "
                    "fresh epoch); capture moe_route_pack + moe_expert_ffn + moe_combine instead", fn);

    carve_route(ws, M, top_k, E, route);
    const int64_t S = (int64_t)M * top_k;
    char *scratch = (char *)ws + moe::route_region_bytes(S, E);
    float *h = (float *)scratch;
    void *flags = scratch + moe::align256(sizeof(float) * (size_t)(S * inter));
    // a fresh epoch per call: flags of any earlier call in this process never
    // match it
    static std::atomic<uint32_t> epoch{(uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() |
                                       1u};
    const uint32_t ep = epoch.fetch_add(1, std::memory_order_relaxed);
    MoeRouteDev r{route->expert_offsets, route->sorted_slot, route->sorted_token,
                  route->token_to_perm, route->active_experts, route->num_active, route->status};
    GemvBankDev bg{gate->codes, gate->scales, gate->scale2};
    GemvBankDev bu{up->codes, up->scales, up->scale2};
    GemvBankDev bd{down->codes, down->scales, down->scale2};
    stage_mark(0, s);
    hipError_t e = fmt == MOE_W_E4M3_B128
        ? launch_fused_decode_e4m3(bg, bu, bd, x_bf16, topk_ids, topk_weights, M, top_k, E, hidden,
                                   inter, limit, r, h, y_packed, out, flags, ep, s)
        : launch_fused_decode_nvfp4(bg, bu, bd, x_bf16, topk_ids, topk_weights, M, top_k, E, hidden,
                                    inter, limit, r, h, y_packed, out, flags, ep, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_fused: launch");
    stage_mark(1, s);
    return MOE_OK;
}

moe_status_t moe_router_topk(const float *logits, int32_t M, int32_t num_experts, int32_t top_k,
                             int32_t kind, const float *bias, float routed_scale,
                             int32_t renormalize, int32_t *topk_ids, float *topk_weights,
                             void *stream)
{
    static const char *fn = "moe_router_topk";
    if (!logits || !topk_ids || !topk_weights) return fail(MOE_ERR_ARG, "%s: null pointer", fn);
    if (!sizes_ok(M, top_k, num_experts))
        return fail(MOE_ERR_SHAPE, "%s: need M >= 1, 1 <= top_k <= num_experts <= %d (M=%d top_k=%d E=%d)",
                    fn, MOE_MAX_EXPERTS, M, top_k, num_experts);
    if (kind != MOE_ROUTER_SOFTMAX && kind != MOE_ROUTER_SIGMOID)
        return fail(MOE_ERR_ARG, "%s: unknown router kind %d", fn, kind);
    if (kind == MOE_ROUTER_SOFTMAX && bias)
        return fail(MOE_ERR_ARG, "%s: the softmax router takes no bias", fn);
    if (!(routed_scale > 0.0f) || !(routed_scale <= 3.4028234663852886e38f))
        return fail(MOE_ERR_ARG, "%s: routed_scale must be finite and > 0", fn);
    if (renormalize != 0 && renormalize != 1)
        return fail(MOE_ERR_ARG, "%s: renormalize must be 0 or 1", fn);
    hipError_t e = launch_router_topk(logits, M, num_experts, top_k, kind, bias, routed_scale,
                                      renormalize, topk_ids, topk_weights, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "moe_router_topk: launch");
    return MOE_OK;
}

moe_status_t moe_combine(const float *y_packed, const moe_route_t *route,
                         const float *topk_weights, int32_t hidden, float *out, void *stream)
{
    if (!y_packed || !route || !topk_weights || !out || !route->token_to_perm)
        return fail(MOE_ERR_ARG, "moe_combine: null pointer");
    if (!sizes_ok(route->M, route->top_k, route->num_experts))
        return fail(MOE_ERR_ARG, "moe_combine: route is not filled");
    if (hidden <= 0 || hidden % 4)
        return fail(MOE_ERR_SHAPE, "moe_combine: hidden %d must be a positive multiple of 4", hidden);
    if (!aligned16(y_packed) || !aligned16(out))
        return fail(MOE_ERR_ARG, "moe_combine: y and out must be 16-byte aligned");
    hipError_t e = launch_combine(y_packed, route->token_to_perm, topk_weights, route->M,
                                  route->top_k, hidden, nullptr, nullptr, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "moe_combine: launch");
    return MOE_OK;
}

moe_status_t moe_combine_residual(const float *y_packed, const moe_route_t *route,
                                  const float *topk_weights, const float *shared_out,
                                  const float *residual, int32_t hidden, float *out, void *stream)
{
    static const char *fn = "moe_combine_residual";
    if (!y_packed || !route || !topk_weights || !out || !route->token_to_perm)
        return fail(MOE_ERR_ARG, "%s: null pointer", fn);
    if (!sizes_ok(route->M, route->top_k, route->num_experts))
        return fail(MOE_ERR_ARG, "%s: route is not filled", fn);
    if (hidden <= 0 || hidden % 4)
        return fail(MOE_ERR_SHAPE, "%s: hidden %d must be a positive multiple of 4", fn, hidden);
    if (!aligned16(y_packed) || !aligned16(out) || (shared_out && !aligned16(shared_out)) ||
        (residual && !aligned16(residual)))
        return fail(MOE_ERR_ARG, "%s: y, out, shared_out and residual must be 16-byte aligned", fn);
    hipError_t e = launch_combine(y_packed, route->token_to_perm, topk_weights, route->M,
                                  route->top_k, hidden, shared_out, residual, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "moe_combine_residual: launch");
    return MOE_OK;
}

size_t moe_shared_workspace_bytes(int32_t max_M, int32_t hidden, int32_t shared_width)
{
    if (max_M < 1 || max_M > MOE_GEMV_MAX_M || hidden <= 0 || shared_width <= 0 ||
        hidden % 512 || shared_width % 512 || hidden > 8192 || shared_width > 8192)
        return 0;
    return moe::align256(sizeof(float) * (size_t)max_M * shared_width);
}

moe_status_t moe_shared_expert(const uint16_t *gate_bf16, const uint16_t *up_bf16,
                               const uint16_t *down_bf16, const uint16_t *x_bf16, int32_t M,
                               int32_t hidden, int32_t shared_width, float limit,
                               float *shared_out, void *ws, size_t ws_bytes, void *stream)
{
    static const char *fn = "moe_shared_expert";
    if (!gate_bf16 || !up_bf16 || !down_bf16 || !x_bf16 || !shared_out || !ws)
        return fail(MOE_ERR_ARG, "%s: null pointer", fn);
    if (M < 1) return fail(MOE_ERR_SHAPE, "%s: M must be >= 1 (M=%d)", fn, M);
    if (M > MOE_GEMV_MAX_M)
        return fail(MOE_ERR_UNSUPPORTED, "%s: M = %d > %d (the shared expert runs the GEMV form only)",
                    fn, M, MOE_GEMV_MAX_M);
    if (hidden <= 0 || shared_width <= 0 || hidden % 512 || shared_width % 512 || hidden > 8192 ||
        shared_width > 8192)
        return fail(MOE_ERR_SHAPE, "%s: hidden %d and shared_width %d must be positive multiples of 512, "
                    "at most 8192", fn, hidden, shared_width);
    if (!(limit > 0.0f)) return fail(MOE_ERR_ARG, "%s: limit must be > 0", fn);
    if (!aligned16(gate_bf16) || !aligned16(up_bf16) || !aligned16(down_bf16) || !aligned16(x_bf16) ||
        !aligned16(shared_out))
        return fail(MOE_ERR_ARG, "%s: weights, x and shared_out must be 16-byte aligned", fn);
    if (((uintptr_t)ws & 255) != 0) return fail(MOE_ERR_ARG, "%s: ws not 256-byte aligned", fn);
    const size_t need = moe_shared_workspace_bytes(M, hidden, shared_width);
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, ws_bytes, need);
    hipError_t e = launch_shared_expert(gate_bf16, up_bf16, down_bf16, x_bf16, M, hidden, shared_width,
                                        limit, (float *)ws, shared_out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "moe_shared_expert: launch");
    return MOE_OK;
}

}  // extern "C"
