"""GPU parity of the FP8 MFMA grouped-GEMM tier (wide M) against the oracle's
FP8 path (x and h quantized per 1x128 group): the activation codes and
scales bit for bit, layer outputs within max|err| <= 2e-3 * max|ref| and
relative L2 <= 1e-3, on reduced shapes with the full oracle and at the full
prefill size on sampled tokens."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads
from fp4_block_scaled_amd import binding as B
from moe_cases import (GpuCase, blockmax_sum, check_fp, check_h_codes, gemm_scratch_views,
                        h_error_bound, host_bank, x_bits)

pytestmark = pytest.mark.gpu

_cache = {}


def get_case(wl):
    key = (wl.name, wl.hidden, wl.inter, wl.experts, wl.top_k, wl.seed, wl.M)
    if key not in _cache:
        _cache.clear()
        gc.collect()
        torch.cuda.empty_cache()
        _cache[key] = GpuCase(wl)
    return _cache[key]


def run_gemm(case, ids, w, tokens=None, label=""):
    wl = case.wl
    out, y, tabs, L = case.run(ids, w, B.MOE_MODE_GEMM_A8)
    M, k = ids.shape
    S = M * k
    # activation codes and scales: bit-exact against the oracle's quantizer
    xq, xs, hq, hs = gemm_scratch_views(L.ws, M, S, wl.experts, wl.hidden, wl.inter)
    rows = np.arange(M) if tokens is None else np.asarray(tokens)
    xf = torch.from_numpy(x_bits(case.x[:M])[rows].view(np.int16)).view(torch.bfloat16).float().numpy()
    q_ref, s_ref = oracle.quant_1x128(xf)
    assert np.array_equal(xq.cpu().numpy()[rows], q_ref), f"{label}: x codes differ"
    assert np.array_equal(xs.cpu().numpy()[rows].view(np.uint32), s_ref.view(np.uint32)), f"{label}: x scales differ"

    # oracle FP8 path for the checked tokens: g, u, h (quantized), y, out
    E = wl.experts
    sel = ids[rows]
    valid = (sel >= 0) & (sel < E)
    used = np.unique(sel[valid])
    hb = [host_bank(b, used) for b in case.banks]
    remap = np.full(sel.shape, -1, np.int32)
    remap[valid] = np.searchsorted(used, sel[valid]).astype(np.int32)
    remap[~valid] = np.where(sel[~valid] == -1, -1, len(used) + 7)
    res = oracle.expert_slots(hb[0], hb[1], hb[2], x_bits(case.x[:M])[rows], remap, wl.limit, True,
                              want=("g", "u", "y"))
    t2p = tabs["token_to_perm"].reshape(ids.shape)
    pairs = [(t2p[t, j], i * k + j) for i, t in enumerate(rows) for j in range(k) if t2p[t, j] >= 0]
    p, sl = np.array(pairs).T
    hq_g, hs_g = hq.cpu().numpy()[p], hs.cpu().numpy()[p]
    # exact-arithmetic h of the oracle, the kernel's error bound on it (from
    # the l1 norms of the gate/up dot products), then each GPU code's validity
    sw = np.vectorize(oracle.swiglu_clamp)
    g_ex, u_ex = res["g"][sl], res["u"][sl]
    h_exact = sw(g_ex, u_ex, wl.limit)
    tab = oracle.e4m3_table()
    xhat = np.abs(tab[q_ref] * np.repeat(s_ref.astype(np.float64), 128, axis=1))   # |x| per checked token
    g_blk = np.zeros_like(g_ex)
    u_blk = np.zeros_like(u_ex)
    tok_of = np.repeat(np.arange(len(rows)), k)[sl]
    for e_local in np.unique(remap[remap >= 0]):
        idx = np.nonzero(remap.ravel()[sl] == e_local)[0]
        xa = xhat[tok_of[idx]]
        g_blk[idx] = blockmax_sum(np.abs(oracle.dequant_expert(hb[0], int(e_local))), xa)
        u_blk[idx] = blockmax_sum(np.abs(oracle.dequant_expert(hb[1], int(e_local))), xa)
    dh = h_error_bound(g_ex, u_ex, g_blk, u_blk, wl.limit)
    flip_rate = check_h_codes(hq_g, hs_g, h_exact, dh, label)
    assert flip_rate < 1e-2, f"{label}: h code flip rate {flip_rate:.2e}"
    # the oracle continues from the kernel's h codes: down projection and combine in FP64
    h_dq = tab[hq_g] * np.repeat(hs_g.astype(np.float64), 128, axis=1)
    y_ref = np.zeros((len(rows) * k, wl.hidden))
    for e_local in np.unique(remap[remap >= 0]):
        idx = np.nonzero(remap.ravel()[sl] == e_local)[0]
        y_ref[sl[idx]] = h_dq[idx] @ oracle.dequant_expert(hb[2], int(e_local)).T
    check_fp(y[p], y_ref[sl], f"{label} y rows")
    out_ref = oracle.combine(y_ref, w[rows], valid.astype(np.int32).ravel())
    r = check_fp(out[rows], out_ref, f"{label} out")
    # diagnostic: against the oracle's own h decisions end to end
    e2e = oracle.combine(res["y"], w[rows], valid.astype(np.int32).ravel())
    d = np.abs(out[rows] - e2e)
    print(f"  {label}: h code flips {flip_rate:.2e}; end-to-end vs oracle's own h codes: max err frac "
          f"{d.max() / np.abs(e2e).max():.2e}, rel L2 {np.linalg.norm(out[rows] - e2e) / np.linalg.norm(e2e):.2e}",
          flush=True)
    return r


REDUCED = [
    # name, overrides, M: several full and partial 128-row tiles per expert
    ("h512_i256_e8_k2", dict(hidden=512, inter=256, experts=8, top_k=2), 300),
    ("h256_i384_e5_k3", dict(hidden=256, inter=384, experts=5, top_k=3), 100),
    ("h1024_i128_e16_k4", dict(hidden=1024, inter=128, experts=16, top_k=4), 77),
    ("h384_i256_e3_k1", dict(hidden=384, inter=256, experts=3, top_k=1), 3),
]


@pytest.mark.parametrize("name,over,M", REDUCED, ids=[r[0] for r in REDUCED])
def test_gemm_tier_reduced_shapes_full_oracle(name, over, M):
    base = workloads.WORKLOADS["prefill_e4m3_m4096"]
    wl = workloads.with_shape(base, name=name, M=M, **over)
    case = get_case(wl)
    ids, w, info = workloads.make_routes(wl, 0)
    print(f"gemm tier {name} M={M} max load {info['max_load']}", flush=True)
    r = run_gemm(case, ids, w, label=name)
    print(f"  max err frac {r[0]:.2e}, rel L2 {r[1]:.2e}", flush=True)


def test_gemm_tier_skewed_and_invalid_ids():
    base = workloads.WORKLOADS["prefill_e4m3_m4096"]
    wl = workloads.with_shape(base, name="skew", hidden=256, inter=256, experts=6, top_k=2, M=400)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 0)
    ids[:, 0] = 2                      # one expert takes every token: 4 tiles
    ids[5, 1] = -1
    ids[9, 1] = 99
    ids[ids[:, 1] == 2, 1] = 3
    run_gemm(case, ids, w, label="skewed")


def test_gemm_tier_prefill_full_size_sampled_tokens():
    wl = workloads.WORKLOADS["prefill_e4m3_m4096"]
    case = get_case(wl)
    ids, w, info = workloads.make_routes(wl, 0)
    counts = np.bincount(ids.ravel(), minlength=wl.experts)
    heavy = int(np.argmax(counts))
    rng = np.random.default_rng(7)
    toks = set(rng.choice(wl.M, 5, replace=False).tolist())
    toks |= {0, wl.M - 1}
    toks.add(int(np.nonzero((ids == heavy).any(axis=1))[0][-1]))   # last row of the heaviest expert
    tokens = np.array(sorted(toks))
    print(f"prefill M=4096: max load {info['max_load']} (expert {heavy}), mean {info['mean_load']:.1f}, "
          f"checking tokens {tokens.tolist()}", flush=True)
    r = run_gemm(case, ids, w, tokens=tokens, label="prefill")
    print(f"  max err frac {r[0]:.2e}, rel L2 {r[1]:.2e}", flush=True)


def test_auto_mode_picks_gemm_above_16_tokens():
    assert B.moe_resolve_mode(17, B.MOE_W_E4M3_B128) == B.MOE_MODE_GEMM_A8
    assert B.moe_resolve_mode(4096, B.MOE_W_E4M3_B128) == B.MOE_MODE_GEMM_A8
