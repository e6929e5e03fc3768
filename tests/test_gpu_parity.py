"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Route tables are compared bit for bit; layer outputs to
max|err| <= 2e-3 * max|ref| and relative L2 <= 1e-3 (whole [M, hidden]
output, and per packed y row as a diagnostic)."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads
from fp4_block_scaled_amd import binding as B
from moe_cases import GpuCase, check_fp, oracle_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    yield
    gc.collect()
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# route pack: bit-exact
# --------------------------------------------------------------------------

def gpu_pack(ids: np.ndarray, E: int):
    M, k = ids.shape
    nbytes = B.moe_workspace_bytes(M, k, E, 128, 128, B.MOE_W_E4M3_B128, B.MOE_MODE_GEMV_A16)
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    route = B.moe_route_pack(ids_d, M, k, E, ws)
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in B.route_tensors(route, ws).items()}


def assert_pack_equal(got, ref, S):
    nv = int(ref["expert_offsets"][-1])
    assert np.array_equal(got["expert_offsets"], ref["expert_offsets"])
    assert np.array_equal(got["sorted_slot"][:nv], ref["sorted_slot"])
    assert np.array_equal(got["sorted_token"][:nv], ref["sorted_token"])
    assert np.array_equal(got["token_to_perm"], ref["token_to_perm"])
    assert int(got["num_active"][0]) == ref["num_active"]
    assert np.array_equal(got["active_experts"][:ref["num_active"]], ref["active_experts"])
    assert np.all(got["active_experts"][ref["num_active"]:] == -1)
    assert int(got["status"][0]) == ref["invalid"]


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
@pytest.mark.parametrize("route_set", [0, 1, 2])
def test_route_pack_bit_exact_on_workloads(name, route_set):
    wl = workloads.WORKLOADS[name]
    ids, _, _ = workloads.make_routes(wl, route_set)
    print(f"route_pack {name} set {route_set} M={wl.M}", flush=True)
    assert_pack_equal(gpu_pack(ids, wl.experts), oracle.route_pack(ids, wl.experts), ids.size)


@pytest.mark.parametrize("case", ["one_expert", "E1", "E2", "k_eq_E", "invalid", "all_invalid",
                                  "dups", "max_experts", "ragged_chunks", "big", "split_ragged",
                                  "split_max_experts", "split_threshold", "below_split"])
def test_route_pack_bit_exact_adversarial(case):
    rng = np.random.default_rng(17)
    if case == "one_expert":
        ids, E = np.full((600, 4), 5, np.int32), 9
    elif case == "E1":
        ids, E = np.zeros((1500, 1), np.int32), 1
    elif case == "E2":
        ids, E = rng.integers(0, 2, (777, 2)).astype(np.int32), 2
    elif case == "k_eq_E":
        E = 6
        ids = np.stack([rng.permutation(E) for _ in range(300)]).astype(np.int32)
    elif case == "invalid":
        E = 64
        ids = rng.integers(0, E, (300, 6)).astype(np.int32)
        flat = ids.ravel()
        pos = rng.choice(flat.size, 100, replace=False)
        flat[pos[:40]] = -1
        flat[pos[40:70]] = E + rng.integers(0, 1000, 30)
        flat[pos[70:]] = -rng.integers(2, 1 << 30, 30)
    elif case == "all_invalid":
        ids, E = np.full((5, 3), -1, np.int32), 4
        ids[2, 2] = 4
    elif case == "dups":
        ids, E = rng.integers(0, 5, (2000, 4)).astype(np.int32), 5
    elif case == "max_experts":
        E = B.MOE_MAX_EXPERTS
        ids = np.stack([rng.choice(E, 8, replace=False) for _ in range(700)]).astype(np.int32)
    elif case == "ragged_chunks":
        E = 37
        ids = rng.integers(0, E, (1025, 3)).astype(np.int32)
    elif case == "split_ragged":
        # large enough for the split pack (count / place / token launches),
        # a ragged last group, and invalid ids of every kind
        E = 100
        ids = rng.integers(0, E, (2743, 3)).astype(np.int32)
        flat = ids.ravel()
        pos = rng.choice(flat.size, 300, replace=False)
        flat[pos[:100]] = -1
        flat[pos[100:200]] = E + rng.integers(0, 50, 100)
        flat[pos[200:]] = -rng.integers(2, 1000, 100)
    elif case == "split_max_experts":
        E = B.MOE_MAX_EXPERTS
        ids = np.stack([rng.choice(E, 8, replace=False) for _ in range(2100)]).astype(np.int32)
    elif case == "split_threshold":
        # the smallest split pack: 8192 slots, 16 runs of 512 experts' counters
        E = B.MOE_MAX_EXPERTS
        ids = np.stack([rng.choice(E, 8, replace=False) for _ in range(1024)]).astype(np.int32)
    elif case == "below_split":
        # one slot short of the split: the one-workgroup pack with a ragged last group
        E = 77
        ids = rng.integers(-1, E, (8191, 1)).astype(np.int32)
    else:
        E = 256
        bias = rng.normal(0, 0.5, E)
        ids, _ = workloads.topk_softmax(rng.standard_normal((8192, E)) + bias, 8)
    print(f"route_pack adversarial {case} S={ids.size} E={E}", flush=True)
    assert_pack_equal(gpu_pack(ids, E), oracle.route_pack(ids, E), ids.size)


@pytest.mark.parametrize("case", ["s1", "s8_invalid", "s63_dups", "s64_e512", "e1", "all_invalid",
                                  "k_eq_E", "one_expert", "neg_ids"])
def test_route_pack_bit_exact_small_routes(case):
    """Routes of at most 64 slots run a one-wave kernel of their own."""
    rng = np.random.default_rng(29)
    if case == "s1":
        ids, E = np.array([[5]], np.int32), 16
    elif case == "s8_invalid":
        ids, E = np.array([[3, -1, 17, 3, 200, 0, -1, 16]], np.int32), 17
    elif case == "s63_dups":
        ids, E = rng.integers(0, 4, (21, 3)).astype(np.int32), 4
    elif case == "s64_e512":
        E = 512
        ids = np.stack([rng.choice(E, 8, replace=False) for _ in range(8)]).astype(np.int32)
    elif case == "e1":
        ids, E = np.zeros((7, 1), np.int32), 1
    elif case == "all_invalid":
        ids, E = np.full((4, 4), -1, np.int32), 8
        ids[1, 2] = 8
    elif case == "k_eq_E":
        E = 8
        ids = np.stack([rng.permutation(E) for _ in range(8)]).astype(np.int32)
    elif case == "one_expert":
        ids, E = np.full((16, 4), 9, np.int32), 10
    else:
        ids, E = rng.integers(-3, 40, (5, 12)).astype(np.int32), 37
    assert ids.size <= 64
    print(f"route_pack small {case} S={ids.size} E={E}", flush=True)
    assert_pack_equal(gpu_pack(ids, E), oracle.route_pack(ids, E), ids.size)


@pytest.mark.parametrize("case", ["s65", "s128_e160", "s200_invalid", "s256_e512", "s256_one_expert",
                                  "s129_dups", "s96_k12"])
def test_route_pack_bit_exact_mid_routes(case):
    """Routes of 65 to 256 slots: up to 128 a one-wave kernel with two slots
    per lane, above that the one-workgroup one."""
    rng = np.random.default_rng(31)
    if case == "s65":
        ids, E = rng.integers(0, 20, (65, 1)).astype(np.int32), 20
    elif case == "s128_e160":
        E = 160
        ids = np.stack([rng.choice(E, 8, replace=False) for _ in range(16)]).astype(np.int32)
    elif case == "s200_invalid":
        E = 50
        ids = rng.integers(0, E, (25, 8)).astype(np.int32)
        flat = ids.ravel()
        pos = rng.choice(flat.size, 30, replace=False)
        flat[pos[:10]] = -1
        flat[pos[10:20]] = E + rng.integers(0, 9, 10)
        flat[pos[20:]] = -rng.integers(2, 99, 10)
    elif case == "s256_e512":
        E = 512
        ids = np.stack([rng.choice(E, 8, replace=False) for _ in range(32)]).astype(np.int32)
    elif case == "s256_one_expert":
        ids, E = np.full((32, 8), 3, np.int32), 9
    elif case == "s129_dups":
        ids, E = rng.integers(0, 3, (43, 3)).astype(np.int32), 3
    else:
        ids, E = rng.integers(-1, 24, (8, 12)).astype(np.int32), 24
    assert 64 < ids.size <= 256
    print(f"route_pack mid {case} S={ids.size} E={E}", flush=True)
    assert_pack_equal(gpu_pack(ids, E), oracle.route_pack(ids, E), ids.size)


def test_route_pack_bit_exact_random_65_to_128_slots():
    """60 random routes of 65 to 128 slots (the two-slots-per-lane one-wave
    kernel): random top_k dividing S, expert counts from 1 to 512, invalid
    ids of every kind in a third of them, a handful of experts in others."""
    rng = np.random.default_rng(37)
    n = 0
    while n < 60:
        S = int(rng.integers(65, 129))
        k = int(rng.choice([d for d in range(1, 13) if S % d == 0]))
        E = int(rng.choice([1, 2, 3, 7, 20, 64, 100, 160, 256, 257, 511, 512]))
        if k > E:
            continue
        ids = rng.integers(0, E, S).astype(np.int32)
        if n % 3 == 0:
            pos = rng.choice(S, int(rng.integers(1, 20)), replace=False)
            ids[pos] = rng.choice([-1, E, E + 5, -7], pos.size)
        if n % 7 == 0:
            ids[:] = rng.integers(0, min(E, 3), S)
        ids = ids.reshape(S // k, k)
        assert_pack_equal(gpu_pack(ids, E), oracle.route_pack(ids, E), ids.size)
        n += 1
    print(f"route_pack random mid: {n} routes", flush=True)


# --------------------------------------------------------------------------
# layer parity
# --------------------------------------------------------------------------

def run_and_check(case: GpuCase, ids, w, mode=B.MOE_MODE_AUTO, tokens=None, label=""):
    wl = case.wl
    resolved = B.moe_resolve_mode(ids.shape[0], wl.fmt, mode)
    act_fp8 = resolved == B.MOE_MODE_GEMM_A8
    out, y, tabs, _ = case.run(ids, w, mode)
    ref_out, ref_y = oracle_layer(case.banks, case.x, ids, w, wl.limit, act_fp8, tokens)
    sel = np.arange(ids.shape[0]) if tokens is None else np.asarray(tokens)
    r = check_fp(out[sel], ref_out, f"{label} out")
    # per packed row diagnostics (valid slots of the checked tokens)
    t2p = tabs["token_to_perm"].reshape(ids.shape)
    rows = []
    for i, t in enumerate(sel):
        for j in range(ids.shape[1]):
            if t2p[t, j] >= 0:
                rows.append((t2p[t, j], i * ids.shape[1] + j))
    if rows:
        p, s = np.array(rows).T
        check_fp(y[p], ref_y[s], f"{label} y rows")
    return r


_cache = {}


def get_case(name_or_wl):
    wl = workloads.WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    key = (wl.name, wl.hidden, wl.inter, wl.experts, wl.top_k, wl.fmt, wl.seed, wl.M)
    if key not in _cache:
        _cache.clear()
        gc.collect()
        torch.cuda.empty_cache()
        _cache[key] = GpuCase(wl)
    return _cache[key]


# Every route set of the tiny, verify and NVFP4 workloads (different expert
# overlap and duplication patterns per set), the first four of decode M=1.
GEMV_ROUTE_SETS = ([("tiny_e4m3_m1", r) for r in range(16)] +
                   [("decode_e4m3_m1", r) for r in range(4)] +
                   [("verify_e4m3_m8", r) for r in range(16)] +
                   [("nvfp4_m1", r) for r in range(16)] +
                   [("nvfp4_m16", r) for r in range(16)])


@pytest.mark.parametrize("name,route_set", GEMV_ROUTE_SETS,
                         ids=[f"{n}-set{r}" for n, r in GEMV_ROUTE_SETS])
def test_layer_parity_gemv_tier_full_workloads(name, route_set):
    wl = workloads.WORKLOADS[name]
    print(f"layer parity {name} route set {route_set}", flush=True)
    case = get_case(wl)
    ids, w, info = workloads.make_routes(wl, route_set)
    r = run_and_check(case, ids, w, label=f"{name} set {route_set}")
    print(f"  {name} set {route_set}: max err frac {r[0]:.2e}, rel L2 {r[1]:.2e}, routes {info}", flush=True)


REDUCED = [
    # (name, base, overrides, M list)
    ("e4m3_h384_i256", "tiny_e4m3_m1", dict(hidden=384, inter=256, experts=8, top_k=3), [1, 3, 16]),
    ("e4m3_h1152_i384", "tiny_e4m3_m1", dict(hidden=1152, inter=384, experts=6, top_k=2), [1, 7]),
    ("e4m3_h256_i2304", "tiny_e4m3_m1", dict(hidden=256, inter=2304, experts=4, top_k=2), [1, 5]),
    ("nvfp4_h2304_i512", "nvfp4_m1", dict(hidden=2304, inter=512, experts=8, top_k=3), [1, 16]),
    ("nvfp4_h256_i2560", "nvfp4_m1", dict(hidden=256, inter=2560, experts=4, top_k=2), [2]),
    # one token: the down launch also does the combine, one K unrolling per
    # inter of 512..2560 (E4M3) or 512..2048 (NVFP4)
    ("e4m3_h384_i512", "tiny_e4m3_m1", dict(hidden=384, inter=512, experts=8, top_k=3), [1, 3]),
    ("e4m3_h1024_i1536", "tiny_e4m3_m1", dict(hidden=1024, inter=1536, experts=12, top_k=8), [1]),
    ("e4m3_h768_i2560", "tiny_e4m3_m1", dict(hidden=768, inter=2560, experts=4, top_k=2), [1]),
    ("nvfp4_h512_i1024", "nvfp4_m1", dict(hidden=512, inter=1024, experts=6, top_k=5), [1, 2]),
    ("nvfp4_h1024_i2048", "nvfp4_m1", dict(hidden=1024, inter=2048, experts=10, top_k=8), [1]),
    # several tokens: the down GEMVs' four-slot passes over two row groups per wave
    ("nvfp4_h512_i2048", "nvfp4_m1", dict(hidden=512, inter=2048, experts=6, top_k=4), [3, 5]),
    # one token, hidden a multiple of 24 with more 16-row blocks than the 256
    # CUs: the combining down kernel takes 24-row blocks
    ("nvfp4_h4608_i1536", "nvfp4_m1", dict(hidden=4608, inter=1536, experts=8, top_k=8), [1]),
    ("nvfp4_h6144_i512", "nvfp4_m1", dict(hidden=6144, inter=512, experts=6, top_k=5), [1]),
    ("nvfp4_h6144_i2048", "nvfp4_m1", dict(hidden=6144, inter=2048, experts=5, top_k=3), [1]),
    ("e4m3_h640_i1280", "tiny_e4m3_m1", dict(hidden=640, inter=1280, experts=5, top_k=3), [4, 6]),
    # one token, hidden a multiple of 28 with more 16-row blocks than the 256
    # CUs: the combining down kernel takes 28-row blocks, two waves per slot
    ("e4m3_h4480_i1024", "tiny_e4m3_m1", dict(hidden=4480, inter=1024, experts=10, top_k=8), [1]),
    ("e4m3_h7168_i512", "tiny_e4m3_m1", dict(hidden=7168, inter=512, experts=6, top_k=5), [1]),
    ("e4m3_h4480_i1536", "tiny_e4m3_m1", dict(hidden=4480, inter=1536, experts=5, top_k=3), [1]),
    # the same forms with one slot: every other wave of the block has none
    ("e4m3_h7168_i1024_k1", "tiny_e4m3_m1", dict(hidden=7168, inter=1024, experts=3, top_k=1), [1]),
    ("nvfp4_h6144_i1536_k1", "nvfp4_m1", dict(hidden=6144, inter=1536, experts=3, top_k=1), [1]),
]


@pytest.mark.parametrize("name,base,over,Ms", REDUCED, ids=[r[0] for r in REDUCED])
def test_layer_parity_reduced_shapes_ragged(name, base, over, Ms):
    wl = workloads.with_shape(workloads.WORKLOADS[base], name=name, M=max(Ms), **over)
    case = get_case(wl)
    for M in Ms:
        ids, w, _ = workloads.make_routes(wl, 0, M=M)
        print(f"layer parity {name} M={M}", flush=True)
        run_and_check(case, ids, w, label=f"{name} M={M}")


def test_layer_parity_many_slots_per_expert_gemv():
    # 40 tokens on 3 experts: slot tiles of the GEMV kernels loop several times
    wl = workloads.with_shape(workloads.WORKLOADS["tiny_e4m3_m1"], name="e4m3_crowded",
                              hidden=512, inter=256, experts=3, top_k=2, M=40)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 0)
    run_and_check(case, ids, w, mode=B.MOE_MODE_GEMV_A16, label="crowded e4m3")


def test_layer_parity_many_slots_per_expert_gemv_nvfp4():
    wl = workloads.with_shape(workloads.WORKLOADS["nvfp4_m1"], name="nvfp4_crowded",
                              hidden=512, inter=512, experts=3, top_k=2, M=40)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 0)
    run_and_check(case, ids, w, mode=B.MOE_MODE_GEMV_A16, label="crowded nvfp4")


@pytest.mark.parametrize("name", ["decode_e4m3_m1", "nvfp4_m1"])
def test_layer_parity_full_shape_repeated_expert(name):
    """One token whose top-k repeats experts, at the full decode shape: the
    repeated expert holds two or three slots, so the unrolled GEMV kernels
    (one slot per pass at this hidden size) run several passes over its
    weights, restaging x, h and the group scales each pass."""
    wl = workloads.WORKLOADS[name]
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 0)
    ids[0, 3] = ids[0, 1]
    ids[0, 6] = ids[0, 1]
    ids[0, 7] = ids[0, 2]
    print(f"layer parity repeated experts {name}", flush=True)
    run_and_check(case, ids, w, label=f"{name} repeated experts")


def test_invalid_and_unfilled_ids_contribute_zero():
    wl = workloads.with_shape(workloads.WORKLOADS["tiny_e4m3_m1"], name="e4m3_invalid", M=6)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 0)
    ids[1, 2] = -1
    ids[3, 0] = wl.experts + 3
    ids[4, 1] = -9
    out, y, tabs, _ = case.run(ids, w)
    assert int(tabs["status"][0]) == 2
    ref_out, _ = oracle_layer(case.banks, case.x, ids, w, wl.limit, False)
    check_fp(out, ref_out, "invalid ids out")


def test_repeat_runs_bit_identical_and_canaries_survive():
    wl = workloads.WORKLOADS["nvfp4_m16"]
    wl = workloads.with_shape(wl, name="nvfp4_canary", hidden=1024, inter=512, experts=20)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 0)
    L = case.layer(max_M=wl.M + 4)
    # NaN canaries in every row the layer must not write
    L.y.fill_(float("nan"))
    L.out.fill_(float("nan"))
    out1, y1, tabs, _ = case.run(ids, w, layer=L)
    nv = int(tabs["expert_offsets"][-1])
    assert np.all(np.isnan(y1[nv:])), "rows past the valid slots were written"
    assert np.all(np.isnan(L.out[wl.M:].cpu().numpy())), "output rows past M were written"
    out2, y2, _, _ = case.run(ids, w, layer=L)
    assert np.array_equal(out1.view(np.uint32), out2.view(np.uint32))
    assert np.array_equal(y1[:nv].view(np.uint32), y2[:nv].view(np.uint32))


def test_grouping_rows_never_changes_a_row():
    # a token's output does not depend on which other tokens share the sweep
    wl = workloads.with_shape(workloads.WORKLOADS["tiny_e4m3_m1"], name="e4m3_group", M=12,
                              hidden=512, inter=256, experts=16, top_k=4)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 0)
    full, _, _, _ = case.run(ids, w)
    for t in (0, 5, 11):
        x1 = case.x[t:t + 1].contiguous()
        one, _, _, _ = case.run(ids[t:t + 1], w[t:t + 1], x=x1)
        assert np.array_equal(one[0].view(np.uint32), full[t].view(np.uint32)), t


@pytest.mark.parametrize("name,M,mode,invalid", [
    ("decode_e4m3_m1", 1, B.MOE_MODE_AUTO, "some"), ("verify_e4m3_m8", 8, B.MOE_MODE_AUTO, "some"),
    ("verify_e4m3_m8", 16, B.MOE_MODE_AUTO, "some"), ("nvfp4_m1", 1, B.MOE_MODE_AUTO, "some"),
    ("tiny_e4m3_m1", 1, B.MOE_MODE_AUTO, "some"), ("tiny_e4m3_m1", 40, B.MOE_MODE_GEMV_A16, "some"),
    ("tiny_e4m3_m1", 20, B.MOE_MODE_AUTO, "some"), ("tiny_e4m3_m1", 6, B.MOE_MODE_AUTO, "all"),
    ("tiny_e4m3_m1", 5, B.MOE_MODE_AUTO, "token"), ("nvfp4_m16", 8, B.MOE_MODE_AUTO, "some"),
    ("nvfp4_m16", 16, B.MOE_MODE_AUTO, "some"),
    ("decode_e4m3_m1", 1, B.MOE_MODE_AUTO, "slots"), ("nvfp4_m1", 1, B.MOE_MODE_AUTO, "slots"),
    ("decode_e4m3_m1", 1, B.MOE_MODE_AUTO, "all"), ("nvfp4_m1", 1, B.MOE_MODE_AUTO, "all"),
])
def test_single_call_layer_matches_three_calls(name, M, mode, invalid):
    """moe_layer (route pack inside the gate/up launch for small routes)
    gives the route tables, y rows and outputs of the three calls bit for bit,
    also with invalid ids, a token with no valid slot, and no valid slot at
    all (zero outputs)."""
    from fp4_block_scaled_amd.layer import MoeLayer
    wl = workloads.with_shape(workloads.WORKLOADS[name], M=max(M, workloads.WORKLOADS[name].M))
    print(f"single call {name} M={M} mode={mode}", flush=True)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 1, M=M)
    if invalid == "all":
        ids[:] = -1
        ids[0, 0] = wl.experts
    elif invalid == "token":
        ids[2, :] = -1
    elif invalid == "slots":
        ids[0, 2] = -1
        ids[0, -1] = wl.experts + 3
    elif M > 1:
        ids[1, 0] = -1
        ids[M - 1, -1] = wl.experts + 3
    res = []
    for single in (True, False):
        L = MoeLayer(*case.cbanks, wl.hidden, wl.inter, wl.top_k, M, wl.limit, mode, single_call=single)
        L.ws.fill_(0x5A)
        L.y.fill_(float("nan"))
        L.out.fill_(float("nan"))
        ids_d = torch.from_numpy(np.ascontiguousarray(ids)).cuda()
        w_d = torch.from_numpy(np.ascontiguousarray(w)).cuda()
        assert case.x.shape[0] >= M
        out = L(case.x[:M], ids_d, w_d).clone()
        torch.cuda.synchronize()
        tabs = {k: v.cpu().numpy() for k, v in L.route_tables().items()}
        nv = int(tabs["expert_offsets"][-1])
        res.append((out.cpu().numpy(), L.y[:nv].cpu().numpy(), tabs))
    (o1, y1, t1), (o2, y2, t2) = res
    for key in t1:
        a, b = t1[key], t2[key]
        if key in ("sorted_slot", "sorted_token"):
            a, b = a[:int(t1["expert_offsets"][-1])], b[:int(t2["expert_offsets"][-1])]
        assert np.array_equal(a, b), f"route table {key} differs"
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.all(np.isfinite(o1))
    if invalid == "all":
        assert np.all(o1 == 0.0)
    if invalid == "token":
        assert np.all(o1[2] == 0.0)
