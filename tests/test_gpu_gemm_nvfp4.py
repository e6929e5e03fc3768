"""GPU parity of the 16-bit MFMA grouped-GEMM tier for NVFP4 banks (wide M)
against the oracle.

x is bf16 as given, every weight (E2M1 code x E4M3 group scale) is exact in
bf16 and in FP16, scale_2 multiplies the FP32 sums, and h passes between
the projections as FP16, rounded once (relative error at most 2^-11) after
a power-of-two factor picked from the clamp limit.  The layer's tolerance
(max|err| <= 2e-3 * max|ref|, relative L2 <= 1e-3) is checked against the
oracle's plain FP64 layer, on the whole output and on every packed y row:
reduced shapes with several full and partial 128-row tiles per expert and K
loops of 4 to 20 steps, one expert taking every token, invalid ids, h past
FP16's largest value and below its smallest normal one, the tier forced at a handful of tokens
(against the GEMV tier too), and the prefill size M=4096 on at least 128
tokens (the first and last rows of every tile of the heaviest experts, ragged
last tiles of lighter ones, random tokens)."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads
from fp4_block_scaled_amd import binding as B
from moe_cases import GpuCase, check_fp, host_bank, oracle_layer, x_bits

pytestmark = pytest.mark.gpu

A16 = B.MOE_MODE_GEMM_A16
_cache = {}


def get_case(wl):
    key = (wl.name, wl.hidden, wl.inter, wl.experts, wl.top_k, wl.seed, wl.M)
    if key not in _cache:
        _cache.clear()
        gc.collect()
        torch.cuda.empty_cache()
        _cache[key] = GpuCase(wl)
    return _cache[key]


def run_a16(case, ids, w, tokens=None, label="", mode=A16):
    wl = case.wl
    assert B.moe_resolve_mode(ids.shape[0], wl.fmt, mode) == A16
    out, y, tabs, _ = case.run(ids, w, mode)
    ref_out, ref_y = oracle_layer(case.banks, case.x, ids, w, wl.limit, act_fp8=False, tokens=tokens)
    sel = np.arange(ids.shape[0]) if tokens is None else np.asarray(tokens)
    r = check_fp(out[sel], ref_out, f"{label} out")
    t2p = tabs["token_to_perm"].reshape(ids.shape)
    pairs = [(t2p[t, j], i * ids.shape[1] + j) for i, t in enumerate(sel)
             for j in range(ids.shape[1]) if t2p[t, j] >= 0]
    if pairs:
        p, s = np.array(pairs).T
        check_fp(y[p], ref_y[s], f"{label} y rows")
    print(f"  {label}: max err frac {r[0]:.2e}, rel L2 {r[1]:.2e}", flush=True)
    return out


REDUCED = [
    # name, overrides, M: K loops of 4..20 steps of 64, 1..5 tiles per expert
    ("nv_h512_i256_e8_k2", dict(hidden=512, inter=256, experts=8, top_k=2), 300),
    ("nv_h256_i768_e5_k3", dict(hidden=256, inter=768, experts=5, top_k=3), 100),
    ("nv_h1280_i512_e16_k4", dict(hidden=1280, inter=512, experts=16, top_k=4), 77),
    ("nv_h768_i256_e3_k1", dict(hidden=768, inter=256, experts=3, top_k=1), 20),
    ("nv_h2048_i1536_e12_k8", dict(hidden=2048, inter=1536, experts=12, top_k=8), 64),
]


@pytest.mark.parametrize("name,over,M", REDUCED, ids=[r[0] for r in REDUCED])
def test_a16_tier_reduced_shapes_full_oracle(name, over, M):
    base = workloads.WORKLOADS["nvfp4_m4096"]
    wl = workloads.with_shape(base, name=name, M=M, **over)
    case = get_case(wl)
    ids, w, info = workloads.make_routes(wl, 0)
    print(f"A16 tier {name} M={M} max load {info['max_load']}", flush=True)
    run_a16(case, ids, w, label=name, mode=B.MOE_MODE_AUTO)


def test_a16_tier_skewed_and_invalid_ids():
    base = workloads.WORKLOADS["nvfp4_m4096"]
    wl = workloads.with_shape(base, name="nv_skew", hidden=512, inter=512, experts=6, top_k=2, M=400)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 0)
    ids[:, 0] = 2                      # one expert takes every token: 4 tiles
    ids[5, 1] = -1
    ids[9, 1] = 99
    ids[ids[:, 1] == 2, 1] = 3
    print("A16 tier skewed", flush=True)
    run_a16(case, ids, w, label="skewed")


@pytest.mark.parametrize("limit,xmul", [(3000.0, 1024), (1e-5, 1)], ids=["past_fp16_max", "below_fp16_normal"])
def test_a16_tier_h_range_factor(limit, xmul):
    """h far outside FP16's normal range.  Clamp limit 3000 with x times 1024
    (exact in bf16): about 2.6 % of h lies past FP16's largest finite value
    65504 (max |h| about 3e5).  Clamp limit 1e-5: every |h| lies below FP16's
    smallest normal value 2^-14 (max |h| about 2.4e-6), where FP16 holds only a
    few significant bits.  The tier scales h by a power of two before the FP16
    rounding (2^-9 and 2^33 here) and the down GEMM undoes it, so the layer
    meets the tolerance either way."""
    base = workloads.WORKLOADS["nvfp4_m4096"]
    wl = workloads.with_shape(base, name=f"nv_h_range_{limit}", hidden=512, inter=256, experts=6,
                              top_k=2, M=64, limit=limit)
    case = get_case(wl)
    case.x.mul_(xmul)
    ids, w, _ = workloads.make_routes(wl, 0)
    used = np.unique(ids[ids >= 0])
    hb = [host_bank(b, used) for b in case.banks]
    h = oracle.expert_slots(hb[0], hb[1], hb[2], x_bits(case.x), np.searchsorted(used, ids).astype(np.int32),
                            wl.limit, False, want=("h",))["h"]
    hmax = float(np.abs(h).max())
    print(f"A16 tier h range, limit {limit}: max |h| {hmax:.3e}", flush=True)
    assert hmax > 65504.0 if limit > 1 else 0.0 < hmax < 2.0 ** -14
    run_a16(case, ids, w, label=f"h range {limit}")


@pytest.mark.parametrize("M", [1, 5, 16])
def test_a16_tier_forced_at_few_tokens_matches_gemv(M):
    base = workloads.WORKLOADS["nvfp4_m4096"]
    wl = workloads.with_shape(base, name="nv_few", hidden=1024, inter=768, experts=10, top_k=4, M=16)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 0, M=M)
    print(f"A16 tier forced M={M}", flush=True)
    out = run_a16(case, ids, w, label=f"forced M{M}")
    gemv, _, _, _ = case.run(ids, w, B.MOE_MODE_GEMV_A16)
    # the GEMV tier keeps h in FP32, this tier rounds it once to FP16 (relative
    # error at most 2^-11 per element, about 2^-11/sqrt(3) RMS): the two
    # agree to a few times that in relative L2, and the largest error stays
    # well under the layer's 2e-3 of max |ref|
    check_fp(out[:M], gemv[:M], f"A16 vs GEMV M{M}", max_frac=1e-3, rel_l2=5e-4)


def a16_prefill_tokens(ids, tabs, E, rng):
    """Tokens whose rows are the first and last rows of every 128-row tile of
    the five heaviest experts, the last rows of the ragged last tile of five
    lighter ones (at most 24 each), the first and last token, and random
    tokens, at least 128 in all."""
    off = tabs["expert_offsets"]
    st = tabs["sorted_token"]
    counts = np.diff(off[:E + 1])
    order = np.argsort(-counts, kind="stable")
    toks = {0, ids.shape[0] - 1}
    for e in order[:5]:
        n = int(counts[e])
        for a in range(0, n, 128):
            toks.add(int(st[off[e] + a]))
            toks.add(int(st[off[e] + min(a + 127, n - 1)]))
    lighter = [e for e in order[5:] if counts[e] % 128]
    for e in rng.choice(lighter, 5, replace=False):
        n = int(counts[e])
        for r in range(n - n % 128, n)[-24:]:
            toks.add(int(st[off[e] + r]))
    while len(toks) < 128:
        toks.add(int(rng.integers(0, ids.shape[0])))
    return np.array(sorted(toks))


def test_a16_tier_prefill_full_size_sampled_tokens():
    wl = workloads.WORKLOADS["nvfp4_m4096"]
    case = get_case(wl)
    ids, w, info = workloads.make_routes(wl, 0)
    # the route tables decide which tokens sit at tile borders
    _, _, tabs, _ = case.run(ids, w, B.MOE_MODE_AUTO)
    tokens = a16_prefill_tokens(ids, tabs, wl.experts, np.random.default_rng(11))
    print(f"NVFP4 prefill M=4096: max load {info['max_load']}, mean {info['mean_load']:.1f}; "
          f"checking {len(tokens)} tokens end to end", flush=True)
    out = run_a16(case, ids, w, tokens=tokens, label="nvfp4 prefill", mode=B.MOE_MODE_AUTO)
    # run to run bit identity
    out2, _, _, _ = case.run(ids, w, B.MOE_MODE_AUTO)
    assert np.array_equal(out, out2)
