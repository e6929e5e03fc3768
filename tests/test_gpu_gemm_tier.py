"""GPU parity of the grouped-GEMM tier for E4M3 banks (wide M) against the
FP64 oracle, which quantizes x and h per 1x128 group as the tier does:

- the activation codes and scales bit for bit, on every token;
- the layer output END TO END against the oracle's own layer (its own h
  codes), within max|err| <= 2e-3 * max|ref| and relative L2 <= 1e-3, and
  every packed y row against the oracle's y of the same slot;
- per stage, every h code the kernel wrote against the exact h, within the
  rounding the kernel's gate/up sums allow (bf16 matrix cores: exact
  products, FP32 sums), and the flip rate;

on reduced shapes with the full oracle and at the full prefill size on a
set of tokens that covers the first and last row of every row chunk of the
heaviest experts, the last chunk of lighter ones, and random tokens."""
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

# rows per chunk of the tier's schedule: an expert with n rows runs in
# ceil(n / 128) chunks of ceil(n / chunks) rows (the last one shorter)
CHUNK = 128

_cache = {}


def get_case(wl):
    key = (wl.name, wl.hidden, wl.inter, wl.experts, wl.top_k, wl.seed, wl.M)
    if key not in _cache:
        _cache.clear()
        gc.collect()
        torch.cuda.empty_cache()
        _cache[key] = GpuCase(wl)
    return _cache[key]


def chunks_of(n):
    """(first, last) packed-row offsets of the chunks of an expert with n rows."""
    nch = -(-n // CHUNK)
    cs = -(-n // nch)
    return [(c * cs, min((c + 1) * cs, n) - 1) for c in range(nch) if c * cs < n]


def run_gemm(case, ids, w, tokens=None, label="", check_h=True):
    wl = case.wl
    out, y, tabs, L = case.run(ids, w, B.MOE_MODE_GEMM_A8)
    M, k = ids.shape
    S = M * k
    xq, xs, hq, hs = gemm_scratch_views(L.ws, M, S, wl.experts, wl.hidden, wl.inter)
    # activation codes and scales of EVERY token: bit-exact against the oracle's quantizer
    xf_all = torch.from_numpy(x_bits(case.x[:M]).view(np.int16)).view(torch.bfloat16).float().numpy()
    q_all, s_all = oracle.quant_1x128(xf_all)
    assert np.array_equal(xq.cpu().numpy(), q_all), f"{label}: x codes differ"
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), s_all.view(np.uint32)), f"{label}: x scales differ"

    rows = np.arange(M) if tokens is None else np.asarray(tokens)
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
    # end to end: the layer output against the oracle's own layer
    ref = oracle.combine(res["y"], w[rows], valid.astype(np.int32).ravel())
    r = check_fp(out[rows], ref, f"{label} out (end to end)")
    # every packed y row of the checked tokens against the oracle's y of its slot
    t2p = tabs["token_to_perm"].reshape(ids.shape)
    pairs = [(t2p[t, j], i * k + j) for i, t in enumerate(rows) for j in range(k) if t2p[t, j] >= 0]
    p, sl = np.array(pairs).T
    check_fp(y[p], res["y"][sl], f"{label} y rows (end to end)")
    flip_rate = float("nan")
    if check_h:
        # per stage: each h code the kernel wrote, against the exact h
        hq_g, hs_g = hq.cpu().numpy()[p], hs.cpu().numpy()[p]
        sw = np.vectorize(oracle.swiglu_clamp)
        g_ex, u_ex = res["g"][sl], res["u"][sl]
        h_exact = sw(g_ex, u_ex, wl.limit)
        tab = oracle.e4m3_table()
        xhat = np.abs(tab[q_all[rows]] * np.repeat(s_all[rows].astype(np.float64), 128, axis=1))
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
        assert flip_rate < 1e-3, f"{label}: h code flip rate {flip_rate:.2e}"
    print(f"  {label}: end to end max err frac {r[0]:.2e}, rel L2 {r[1]:.2e}; h code flips {flip_rate:.2e}",
          flush=True)
    return r


REDUCED = [
    # name, overrides, M: several full and partial row chunks per expert
    ("h512_i256_e8_k2", dict(hidden=512, inter=256, experts=8, top_k=2), 300),
    ("h256_i384_e5_k3", dict(hidden=256, inter=384, experts=5, top_k=3), 100),
    ("h1024_i128_e16_k4", dict(hidden=1024, inter=128, experts=16, top_k=4), 77),
    ("h384_i256_e3_k1", dict(hidden=384, inter=256, experts=3, top_k=1), 3),
    # K loops that are not a multiple of four steps (a tail of 1, 2 or 3 steps)
    ("h640_i384_e6_k2", dict(hidden=640, inter=384, experts=6, top_k=2), 150),
    ("h768_i640_e4_k2", dict(hidden=768, inter=640, experts=4, top_k=2), 90),
]


@pytest.mark.parametrize("name,over,M", REDUCED, ids=[r[0] for r in REDUCED])
def test_gemm_tier_reduced_shapes_full_oracle(name, over, M):
    base = workloads.WORKLOADS["prefill_e4m3_m4096"]
    wl = workloads.with_shape(base, name=name, M=M, **over)
    case = get_case(wl)
    ids, w, info = workloads.make_routes(wl, 0)
    print(f"gemm tier {name} M={M} max load {info['max_load']}", flush=True)
    run_gemm(case, ids, w, label=name)


def test_gemm_tier_skewed_and_invalid_ids():
    base = workloads.WORKLOADS["prefill_e4m3_m4096"]
    wl = workloads.with_shape(base, name="skew", hidden=256, inter=256, experts=6, top_k=2, M=400)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 0)
    ids[:, 0] = 2                      # one expert takes every token: 4 chunks
    ids[5, 1] = -1
    ids[9, 1] = 99
    ids[ids[:, 1] == 2, 1] = 3
    print("gemm tier skewed", flush=True)
    run_gemm(case, ids, w, label="skewed")


def test_gemm_tier_row_counts_at_every_chunk_size():
    """Experts with 1..33 rows and around the chunk size (127, 128, 129, 255,
    256, 257 rows): every specialization of the kernels (up to 32, 64, 96 and
    128 rows per chunk) and balanced splits."""
    base = workloads.WORKLOADS["prefill_e4m3_m4096"]
    counts = [1, 2, 15, 16, 17, 31, 32, 33, 63, 65, 96, 97, 127, 128, 129, 255, 256, 257]
    E = len(counts) + 1                # the last expert gets no rows
    M = sum(counts)
    # one slot per token: a single legitimate tie flip of an h code moves a
    # y row by about 1/8 of an E4M3 step of one of its inter terms, so a
    # wide inter keeps that inside the tolerance as at the full shape
    wl = workloads.with_shape(base, name="rowcounts", hidden=256, inter=2048, experts=E, top_k=1, M=M)
    case = get_case(wl)
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)[:, None]
    ids = ids[np.random.default_rng(5).permutation(M)]
    w = np.ones((M, 1), np.float32)
    print(f"gemm tier row counts M={M}", flush=True)
    run_gemm(case, ids, w, label="row counts")


def prefill_tokens(ids, tabs, E, rng):
    """Tokens whose rows are the first and last rows of every chunk of the
    five heaviest experts, all rows of the last chunk of five lighter ones
    (at most 24 each), and random tokens, at least 128 in all."""
    off = tabs["expert_offsets"]
    st = tabs["sorted_token"]
    counts = np.diff(off[:E + 1])
    order = np.argsort(-counts, kind="stable")
    toks = set()
    for e in order[:5]:
        for a, b in chunks_of(int(counts[e])):
            toks.add(int(st[off[e] + a]))
            toks.add(int(st[off[e] + b]))
    lighter = [e for e in order[5:] if counts[e] > 0]
    for e in rng.choice(lighter, 5, replace=False):
        a, b = chunks_of(int(counts[e]))[-1]
        for r in range(a, b + 1)[-24:]:
            toks.add(int(st[off[e] + r]))
    while len(toks) < 160:
        toks.add(int(rng.integers(0, ids.shape[0])))
    return np.array(sorted(toks))


def test_gemm_tier_prefill_full_size():
    wl = workloads.WORKLOADS["prefill_e4m3_m4096"]
    case = get_case(wl)
    ids, w, info = workloads.make_routes(wl, 0)
    # the route tables decide which tokens sit at chunk borders
    _, _, tabs, _ = case.run(ids, w, B.MOE_MODE_GEMM_A8)
    tokens = prefill_tokens(ids, tabs, wl.experts, np.random.default_rng(7))
    print(f"prefill M=4096: max load {info['max_load']}, mean {info['mean_load']:.1f}; "
          f"checking {len(tokens)} tokens end to end", flush=True)
    # the per-stage h check is costly at full size: the first 48 tokens
    run_gemm(case, ids, w, tokens=tokens, label="prefill", check_h=False)
    run_gemm(case, ids, w, tokens=tokens[:48], label="prefill h codes")


def test_auto_mode_picks_gemm_above_16_tokens():
    assert B.moe_resolve_mode(17, B.MOE_W_E4M3_B128) == B.MOE_MODE_GEMM_A8
    assert B.moe_resolve_mode(4096, B.MOE_W_E4M3_B128) == B.MOE_MODE_GEMM_A8
