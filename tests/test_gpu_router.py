"""GPU tests of moe_router_topk against the oracle's router.

The expert ids are compared bit for bit: they are integers decided from
binary32 keys that both sides form the same way (the softmax on the logits
themselves; the sigmoid in double, rounded once, plus the bias in one binary32
addition).  The weights are double arithmetic rounded once to binary32 on
both sides, so they are expected to be bit-identical too; the test allows 2
units in the last place, which only a one-ulp difference between the two
sides' double exp could cause, and reports the bit-exact share.  The end of
the file feeds the device router's output through the layer."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fp4_block_scaled_amd import binding as B
from moe_cases import GpuCase, check_fp, oracle_layer

pytestmark = pytest.mark.gpu

SOFTMAX, SIGMOID = B.MOE_ROUTER_SOFTMAX, B.MOE_ROUTER_SIGMOID


def run_router(logits, k, kind, bias=None, scale=1.0, renorm=1):
    M, E = logits.shape
    l_d = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    b_d = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias, np.float32)).cuda()
    ids = torch.full((M, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((M, k), float("nan"), dtype=torch.float32, device="cuda")
    B.moe_router_topk(l_d, M, E, k, kind, b_d, scale, renorm, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def compare(logits, k, kind, bias=None, scale=1.0, renorm=1, label=""):
    ids_g, w_g = run_router(logits, k, kind, bias, scale, renorm)
    ids_o, w_o = oracle.router_topk(logits, k, kind, bias, scale, bool(renorm))
    assert np.array_equal(ids_g, ids_o), f"{label}: expert ids differ at " \
        f"{np.argwhere(ids_g != ids_o)[:5].tolist()}"
    assert np.all(np.isfinite(w_g))
    ulp = np.abs(w_g.view(np.int32).astype(np.int64) - w_o.view(np.int32).astype(np.int64))
    assert ulp.max() <= 2, f"{label}: weights differ by {ulp.max()} ulp"
    exact = float((ulp == 0).mean())
    print(f"  {label}: ids exact, weights bit-exact share {exact:.6f}", flush=True)
    return ids_g, w_g


SHAPES = [  # (M, E, k)
    (1, 256, 8), (8, 256, 8), (4096, 256, 8), (16, 160, 8), (1, 16, 4),
    (37, 512, 16), (5, 7, 7), (3, 100, 1), (64, 64, 64), (2, 512, 512), (130, 65, 9),
]


@pytest.mark.parametrize("M,E,k", SHAPES)
@pytest.mark.parametrize("kind,renorm,scale,with_bias", [
    (SOFTMAX, 1, 1.0, False), (SOFTMAX, 0, 1.0, False), (SOFTMAX, 1, 2.5, False),
    (SIGMOID, 1, 2.5, True), (SIGMOID, 0, 1.0, True), (SIGMOID, 1, 1.0, False),
])
def test_router_matches_oracle(M, E, k, kind, renorm, scale, with_bias):
    label = f"M{M} E{E} k{k} kind{kind} renorm{renorm} scale{scale} bias{int(with_bias)}"
    print(label, flush=True)
    rng = np.random.default_rng(M * 7919 + E * 31 + k + 1000 * kind)
    logits = rng.standard_normal((M, E)).astype(np.float32)
    bias = rng.normal(0.0, 0.1, E).astype(np.float32) if with_bias else None
    compare(logits, k, kind, bias, scale, renorm, label)


@pytest.mark.parametrize("kind", [SOFTMAX, SIGMOID])
def test_router_ties_and_signed_zeros(kind):
    print(f"ties kind {kind}", flush=True)
    rng = np.random.default_rng(21)
    logits = (np.round(rng.standard_normal((300, 96)) * 2) / 2).astype(np.float32)
    logits[0] = 0.0
    logits[1, ::2] = -0.0
    logits[1, 1::2] = 0.0
    bias = (np.round(rng.normal(0, 0.2, 96) * 4) / 4).astype(np.float32) if kind == SIGMOID else None
    ids, _ = compare(logits, 8, kind, bias, label="ties")
    if kind == SOFTMAX:                      # an all-zero row: the lowest ids (with a bias the
        assert ids[0].tolist() == list(range(8))   # sigmoid router follows the bias instead)


@pytest.mark.parametrize("kind", [SOFTMAX, SIGMOID])
def test_router_non_finite_logits(kind):
    print(f"non-finite kind {kind}", flush=True)
    rng = np.random.default_rng(33)
    logits = rng.standard_normal((40, 48)).astype(np.float32)
    logits[rng.random((40, 48)) < 0.1] = np.nan
    logits[rng.random((40, 48)) < 0.05] = np.inf
    logits[rng.random((40, 48)) < 0.05] = -np.inf
    logits[0] = np.nan
    compare(logits, 6, kind, label="non-finite")


@pytest.mark.parametrize("name", ["decode_e4m3_m1", "verify_e4m3_m8", "prefill_e4m3_m4096",
                                  "nvfp4_m16"])
def test_router_on_the_workload_logits(name):
    wl = workloads.WORKLOADS[name]
    print(f"workload logits {name}", flush=True)
    for r in range(3):
        logits, _ = workloads.make_logits(wl, r)
        compare(logits.astype(np.float32), wl.top_k, SOFTMAX, label=f"{name}/{r}")


@pytest.mark.parametrize("name", ["tiny_e4m3_m1", "decode_e4m3_m1", "verify_e4m3_m8"])
def test_router_feeds_the_layer(name):
    """Logits -> moe_router_topk -> moe_route_pack -> moe_expert_ffn ->
    moe_combine, all on the device with no host hop, against the oracle's
    router and layer."""
    wl = workloads.WORKLOADS[name]
    print(f"router + layer {name}", flush=True)
    case = GpuCase(wl)
    logits = workloads.make_logits(wl, 0)[0].astype(np.float32)
    L = case.layer()
    l_d = torch.from_numpy(logits).cuda()
    ids_d = torch.empty((wl.M, wl.top_k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((wl.M, wl.top_k), dtype=torch.float32, device="cuda")
    B.moe_router_topk(l_d, wl.M, wl.experts, wl.top_k, SOFTMAX, None, 1.0, 1, ids_d, w_d)
    out = L(case.x[: wl.M], ids_d, w_d)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.router_topk(logits, wl.top_k, SOFTMAX)
    assert np.array_equal(ids_d.cpu().numpy(), ids_o)
    ref, _ = oracle_layer(case.banks, case.x, ids_o, w_o, wl.limit, False)
    check_fp(out.cpu().numpy(), ref, f"{name} router + layer")
