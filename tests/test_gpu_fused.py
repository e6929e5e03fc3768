"""GPU tests of moe_layer_fused, the one-launch decode layer: route tables bit
for bit against the oracle's route pack, layer outputs against the oracle
(max|err| <= 2e-3 * max|ref|, relative L2 <= 1e-3), and comparison with the
three-call path (moe_route_pack, moe_expert_ffn, moe_combine).  The general
kernel runs the three-call path's items, so out and y are bit-identical to
it.  The one-token kernel (M = 1, hidden a multiple of 1024 up to 8192) sums
gate/up products in another order (per lane over its K segments, then over
64 lanes), so there y and out agree with the three-call path to the same
tolerance as with the oracle."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads
from fp4_block_scaled_amd import binding as B
from moe_cases import GpuCase, check_fp, oracle_layer

pytestmark = pytest.mark.gpu

_cache = {}


def get_case(wl):
    key = (wl.name, wl.hidden, wl.inter, wl.experts, wl.top_k, wl.fmt, wl.seed, wl.M)
    if key not in _cache:
        _cache.clear()
        gc.collect()
        torch.cuda.empty_cache()
        _cache[key] = GpuCase(wl)
    return _cache[key]


def assert_route_equal(tabs, ids, E):
    ref = oracle.route_pack(ids, E)
    nv = int(ref["expert_offsets"][-1])
    assert np.array_equal(tabs["expert_offsets"], ref["expert_offsets"])
    assert np.array_equal(tabs["sorted_slot"][:nv], ref["sorted_slot"])
    assert np.array_equal(tabs["sorted_token"][:nv], ref["sorted_token"])
    assert np.array_equal(tabs["token_to_perm"], ref["token_to_perm"])
    assert int(tabs["num_active"][0]) == ref["num_active"]
    assert np.array_equal(tabs["active_experts"][:ref["num_active"]], ref["active_experts"])
    assert np.all(tabs["active_experts"][ref["num_active"]:] == -1)
    return ref


def one_token_kernel(M, hidden, fmt=workloads.E4M3_B128):
    if fmt == workloads.NVFP4_B16:
        return True                      # the only NVFP4 fused path (M = 1, hidden % 2048 == 0)
    return M == 1 and hidden % 1024 == 0 and hidden <= 8192


def fused_vs_three_call(case, ids, w, label, x=None):
    """Run the fused layer and the three-call path on the same inputs; check the
    route, the oracle parity, and out and the valid y rows against the
    three-call path (bit for bit where the fused kernel runs its items)."""
    wl = case.wl
    M = ids.shape[0]
    Lf = case.layer(max_M=M, mode=B.MOE_MODE_FUSED)
    Lf.y.fill_(float("nan"))
    out_f, y_f, tabs, _ = case.run(ids, w, x=x, layer=Lf)
    ref = assert_route_equal(tabs, ids, wl.experts)
    assert int(tabs["status"][0]) == ref["invalid"], "status (a timed-out wait adds 2^30)"
    nv = int(ref["expert_offsets"][-1])
    assert np.all(np.isnan(y_f[nv:])), f"{label}: fused layer wrote y rows past the valid slots"
    out_3, y_3, _, _ = case.run(ids, w, B.MOE_MODE_GEMV_A16, x=x)
    if one_token_kernel(M, wl.hidden, wl.fmt):
        check_fp(out_f, out_3, f"{label} out vs three-call")
        check_fp(y_f[:nv], y_3[:nv], f"{label} y vs three-call")
    else:
        assert np.array_equal(out_f.view(np.uint32), out_3.view(np.uint32)), f"{label}: out differs"
        assert np.array_equal(y_f[:nv].view(np.uint32), y_3[:nv].view(np.uint32)), \
            f"{label}: y differs"
    xx = case.x if x is None else x
    ref_out, _ = oracle_layer(case.banks, xx, ids, w, wl.limit, False)
    return check_fp(out_f, ref_out, f"{label} out")


@pytest.mark.parametrize("name", ["tiny_e4m3_m1", "decode_e4m3_m1", "verify_e4m3_m8", "nvfp4_m1"])
@pytest.mark.parametrize("route_set", [0, 1])
def test_fused_layer_workloads(name, route_set):
    wl = workloads.WORKLOADS[name]
    print(f"fused {name} set {route_set}", flush=True)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, route_set)
    r = fused_vs_three_call(case, ids, w, f"{name}/{route_set}")
    print(f"  max err frac {r[0]:.2e}, rel L2 {r[1]:.2e}", flush=True)


REDUCED = [
    # one-token kernel: hidden 1024 and 2048 (1 and 2 loads per row), the generic down item
    ("f_h2048_i384", dict(hidden=2048, inter=384, experts=12, top_k=4), [1]),
    ("f_h1024_i128_k8", dict(hidden=1024, inter=128, experts=40, top_k=8), [1, 2]),
    ("f_h384_i256", dict(hidden=384, inter=256, experts=8, top_k=3), [1, 3, 16]),
    ("f_h1152_i384", dict(hidden=1152, inter=384, experts=6, top_k=2), [1, 7]),
    ("f_h256_i2304", dict(hidden=256, inter=2304, experts=4, top_k=2), [1, 5]),
    ("f_h1024_i512_k16", dict(hidden=1024, inter=512, experts=64, top_k=16), [16]),
]


@pytest.mark.parametrize("name,over,Ms", REDUCED, ids=[r[0] for r in REDUCED])
def test_fused_layer_reduced_shapes(name, over, Ms):
    wl = workloads.with_shape(workloads.WORKLOADS["tiny_e4m3_m1"], name=name, M=max(Ms), **over)
    case = get_case(wl)
    for M in Ms:
        ids, w, _ = workloads.make_routes(wl, 0, M=M)
        print(f"fused {name} M={M} S={ids.size}", flush=True)
        fused_vs_three_call(case, ids, w, f"{name} M={M}")


def test_fused_crowded_expert_and_invalid_ids():
    # 16 tokens, 12 of them on one expert (several weight passes), plus
    # unfilled and out-of-range ids
    wl = workloads.with_shape(workloads.WORKLOADS["tiny_e4m3_m1"], name="f_crowded",
                              hidden=512, inter=256, experts=5, top_k=2, M=16)
    case = get_case(wl)
    ids, w, _ = workloads.make_routes(wl, 0)
    ids[:12, 0] = 3
    ids[ids[:, 1] == 3, 1] = 1
    ids[2, 1] = -1
    ids[5, 1] = wl.experts + 4
    ids[7, 1] = -3
    print("fused crowded/invalid", flush=True)
    fused_vs_three_call(case, ids, w, "crowded")


def test_fused_all_ids_invalid_gives_zero_rows():
    wl = workloads.with_shape(workloads.WORKLOADS["tiny_e4m3_m1"], name="f_none", M=3)
    case = get_case(wl)
    ids = np.full((3, wl.top_k), -1, np.int32)
    ids[1, 2] = wl.experts
    w = np.ones(ids.shape, np.float32)
    L = case.layer(max_M=3, mode=B.MOE_MODE_FUSED)
    L.out.fill_(float("nan"))
    out, _, tabs, _ = case.run(ids, w, layer=L)
    assert np.all(out == 0.0)
    assert int(tabs["num_active"][0]) == 0 and int(tabs["status"][0]) == 1


def test_fused_back_to_back_calls_on_one_workspace():
    # the epoch counters need no clearing: successive calls with different
    # routes (and stale counter words in between) stay exact
    wl = workloads.WORKLOADS["tiny_e4m3_m1"]
    wl = workloads.with_shape(wl, name="f_epochs", M=4, experts=16, top_k=4)
    case = get_case(wl)
    L = case.layer(max_M=4, mode=B.MOE_MODE_FUSED)
    L.ws.fill_(0xFF)                                  # garbage counters
    for r in range(4):
        ids, w, _ = workloads.make_routes(wl, r)
        out_f, _, tabs, _ = case.run(ids, w, layer=L)
        assert int(tabs["status"][0]) == 0
        out_3, _, _, _ = case.run(ids, w, B.MOE_MODE_GEMV_A16)
        assert np.array_equal(out_f.view(np.uint32), out_3.view(np.uint32)), r
    # and the same call twice gives the same bits
    again, _, _, _ = case.run(ids, w, layer=L)
    assert np.array_equal(again.view(np.uint32), out_f.view(np.uint32))


def test_one_token_kernel_edge_routes():
    # M = 1 with hidden 1024: the one-token kernel.  Back-to-back calls on one
    # workspace filled with garbage, an expert chosen twice by the token (two
    # packed rows with the same h), unfilled and out-of-range ids, and a token
    # with no valid id at all.
    wl = workloads.with_shape(workloads.WORKLOADS["tiny_e4m3_m1"], name="f1_edge",
                              hidden=1024, inter=256, experts=16, top_k=6, M=1)
    case = get_case(wl)
    L = case.layer(max_M=1, mode=B.MOE_MODE_FUSED)
    L.ws.fill_(0xFF)
    for r in range(3):
        ids, w, _ = workloads.make_routes(wl, r)
        print(f"one-token back-to-back {r}", flush=True)
        out_f, _, tabs, _ = case.run(ids, w, layer=L)
        assert_route_equal(tabs, ids, wl.experts)
        assert int(tabs["status"][0]) == 0
        ref, _ = oracle_layer(case.banks, case.x, ids, w, wl.limit, False)
        check_fp(out_f, ref, f"one-token epoch {r}")
    ids = np.array([[3, 3, 7, -1, wl.experts + 2, 5]], np.int32)
    w = np.array([[0.25, 0.125, 0.2, 0.1, 0.15, 0.175]], np.float32)
    print("one-token duplicates/invalid", flush=True)
    fused_vs_three_call(case, ids, w, "one-token duplicates")
    ids = np.array([[-1, wl.experts, -1, -5, -1, -1]], np.int32)
    L.out.fill_(float("nan"))
    out, _, tabs, _ = case.run(ids, w, layer=L)
    assert np.all(out == 0.0)
    assert int(tabs["num_active"][0]) == 0 and int(tabs["status"][0]) == 2


NVFP4_REDUCED = [
    ("nf_h2048_i256", dict(hidden=2048, inter=256, experts=12, top_k=4)),    # 1 load per row
    ("nf_h4096_i512", dict(hidden=4096, inter=512, experts=20, top_k=8)),    # 2 loads per row
]


@pytest.mark.parametrize("name,over", NVFP4_REDUCED, ids=[r[0] for r in NVFP4_REDUCED])
def test_fused_nvfp4_reduced_shapes(name, over):
    wl = workloads.with_shape(workloads.WORKLOADS["nvfp4_m1"], name=name, M=1, **over)
    case = get_case(wl)
    for r in range(2):
        ids, w, _ = workloads.make_routes(wl, r)
        print(f"fused nvfp4 {name} set {r}", flush=True)
        fused_vs_three_call(case, ids, w, f"{name}/{r}")


def test_fused_nvfp4_edge_routes():
    wl = workloads.with_shape(workloads.WORKLOADS["nvfp4_m1"], name="nf_edge", hidden=2048,
                              inter=512, experts=16, top_k=6, M=1)
    case = get_case(wl)
    L = case.layer(max_M=1, mode=B.MOE_MODE_FUSED)
    L.ws.fill_(0xFF)
    for r in range(3):
        ids, w, _ = workloads.make_routes(wl, r)
        print(f"nvfp4 one-token back-to-back {r}", flush=True)
        out_f, _, tabs, _ = case.run(ids, w, layer=L)
        assert_route_equal(tabs, ids, wl.experts)
        assert int(tabs["status"][0]) == 0
        ref, _ = oracle_layer(case.banks, case.x, ids, w, wl.limit, False)
        check_fp(out_f, ref, f"nvfp4 one-token epoch {r}")
    ids = np.array([[3, 3, 7, -1, wl.experts + 2, 5]], np.int32)
    w = np.array([[0.25, 0.125, 0.2, 0.1, 0.15, 0.175]], np.float32)
    print("nvfp4 one-token duplicates/invalid", flush=True)
    fused_vs_three_call(case, ids, w, "nvfp4 duplicates")
    ids = np.array([[-1, wl.experts, -1, -5, -1, -1]], np.int32)
    L.out.fill_(float("nan"))
    out, _, tabs, _ = case.run(ids, w, layer=L)
    assert np.all(out == 0.0)
    assert int(tabs["num_active"][0]) == 0 and int(tabs["status"][0]) == 2
