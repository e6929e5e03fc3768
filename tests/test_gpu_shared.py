"""GPU tests of the shared expert (moe_shared_expert) and of the final add
routed-plus-shared-then-residual (moe_combine_residual) against the oracle.

The shared expert's products are exact in FP32 (bf16 x bf16 in the gate/up
projections, bf16 x FP32 rounded once in the down projection), so only the
order of the FP32 sums differs from the FP64 definition: the layer's
tolerance (max |err| <= 2e-3 max |ref|, rel L2 <= 1e-3) holds with a wide
margin.  moe_combine_residual adds the shared row and then the residual to
the routed sum in one rounded FP32 addition each, which the test checks bit
for bit against moe_combine's output plus the two rows added in numpy
float32, besides the tolerance check against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fp4_block_scaled_amd import binding as B
from moe_cases import GpuCase, check_fp, oracle_layer

pytestmark = pytest.mark.gpu

LIMIT = 7.0


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_shared(gate, up, down, x, limit=LIMIT, ws=None):
    M, H = x.shape
    W = gate.shape[0]
    out = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = torch.empty(B.moe_shared_workspace_bytes(M, H, W), dtype=torch.uint8, device="cuda")
    B.moe_shared_expert(gate, up, down, x, M, H, W, limit, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def shared_case(M, H, W, seed, gate_std=2.5):
    gate, up, down = workloads.make_shared_expert(H, W, seed, "cuda", gate_std)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    x = torch.randn((M, H), generator=g, device="cuda").to(torch.bfloat16).contiguous()
    return gate, up, down, x


SHAPES = [  # (M, H, W): the decode workload's width, the NVFP4 one's, max sizes, ragged M
    (1, 7168, 2048), (8, 7168, 2048), (16, 7168, 2048), (1, 6144, 1536), (16, 6144, 1536),
    (1, 512, 512), (3, 1024, 1536), (7, 2560, 512), (13, 512, 4096), (2, 8192, 8192),
    (16, 8192, 512), (5, 4608, 7680),
]


@pytest.mark.parametrize("M,H,W", SHAPES)
def test_shared_expert_matches_oracle(M, H, W):
    print(f"shared M{M} H{H} W{W}", flush=True)
    gate, up, down, x = shared_case(M, H, W, seed=M * 131 + H + W)
    got = run_shared(gate, up, down, x)
    ref = oracle.shared_expert(bits(gate), bits(up), bits(down), bits(x), LIMIT)
    frac, l2 = check_fp(got, ref, f"shared M{M} H{H} W{W}")
    print(f"  max err {frac:.2e} of max |ref|, rel L2 {l2:.2e}", flush=True)


def test_shared_expert_clamp_is_reached():
    """A draw with large gate/up pre-activations, where most of h is clamped:
    a sign or bound mistake in the clamp shows here."""
    print("shared clamp", flush=True)
    gate, up, down, x = shared_case(4, 2048, 1024, seed=77, gate_std=12.0)
    got = run_shared(gate, up, down, x)
    ref = oracle.shared_expert(bits(gate), bits(up), bits(down), bits(x), LIMIT)
    check_fp(got, ref, "shared clamp")
    got_small = run_shared(gate, up, down, x, limit=0.5)
    ref_small = oracle.shared_expert(bits(gate), bits(up), bits(down), bits(x), 0.5)
    check_fp(got_small, ref_small, "shared clamp 0.5")
    assert not np.allclose(ref, ref_small)


def test_shared_expert_workspace_reuse_and_zero_token():
    """Two calls in a row on one workspace, the second with fewer tokens; a
    token of zeros gives a zero row."""
    print("shared reuse", flush=True)
    H, W = 2048, 1536
    gate, up, down, x = shared_case(16, H, W, seed=5)
    x[3].zero_()
    ws = torch.empty(B.moe_shared_workspace_bytes(16, H, W), dtype=torch.uint8, device="cuda")
    a = run_shared(gate, up, down, x, ws=ws)
    b = run_shared(gate, up, down, x[:5].contiguous(), ws=ws)
    assert np.array_equal(a[:5], b)
    assert np.all(a[3] == 0.0)
    ref = oracle.shared_expert(bits(gate), bits(up), bits(down), bits(x), LIMIT)
    check_fp(a, ref, "shared reuse")


@pytest.mark.parametrize("H,W", [(7168, 2048), (6144, 1536), (1024, 4096)])
def test_shared_expert_token_alone_matches_batch(H, W):
    """A token's shared-expert row is the same bits alone (M = 1) as inside a
    batch of 16: the rows per wave differ between the two calls (at H7168
    W2048 the down launch holds 1 row per wave alone and 4 in the batch; at
    H6144 W1536 gate/up 1 against 2 and down 2 against 4), while each output's
    sum keeps its order."""
    print(f"shared alone-vs-batch H{H} W{W}", flush=True)
    gate, up, down, x = shared_case(16, H, W, seed=H + W + 3)
    batch = run_shared(gate, up, down, x)
    for t in (0, 7, 15):
        alone = run_shared(gate, up, down, x[t:t + 1].contiguous())
        assert np.array_equal(alone[0], batch[t]), t


def test_shared_expert_rejects_on_device():
    gate, up, down, x = shared_case(17, 512, 512, seed=3)
    out = torch.empty((17, 512), dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.MoeError) as e:
        B.moe_shared_expert(gate, up, down, x, 17, 512, 512, LIMIT, out, ws)
    assert e.value.status == B.MOE_ERR_UNSUPPORTED
    with pytest.raises(B.MoeError) as e:
        B.moe_shared_expert(gate, up, down, x, 4, 512, 512, LIMIT, out, ws, ws_bytes=64)
    assert e.value.status == B.MOE_ERR_WORKSPACE


def f32_add(a, b):
    return (np.asarray(a, np.float32) + np.asarray(b, np.float32)).astype(np.float32)


@pytest.mark.parametrize("name,M", [("decode_e4m3_m1", 1), ("verify_e4m3_m8", 8),
                                    ("nvfp4_m16", 16)])
def test_layer_with_shared_expert_and_residual(name, M):
    """Routed layer (route pack, expert FFN), the shared expert on the same
    x, then moe_combine_residual, against the oracle end to end."""
    print(f"layer+shared {name} M{M}", flush=True)
    wl = workloads.WORKLOADS[name]
    case = GpuCase(wl)
    ids, w, _ = workloads.make_routes(wl, M=M)
    out_routed, _, _, L = case.run(ids, w)
    H = wl.hidden
    W = wl.inter                                  # one shared expert as wide as a routed one
    gate, up, down = workloads.make_shared_expert(H, W, wl.seed * 10 + 11, "cuda")
    x = case.x[:M].contiguous()
    sh = torch.empty((M, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.moe_shared_workspace_bytes(M, H, W), dtype=torch.uint8, device="cuda")
    B.moe_shared_expert(gate, up, down, x, M, H, W, LIMIT, sh, ws)
    res = workloads.make_residual(M, H, wl.seed + 5, "cuda")
    w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    out = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
    B.moe_combine_residual(L.y, L.route, w_d, sh, res, H, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    sh_h, res_h = sh.cpu().numpy(), res.cpu().numpy()
    # exactly two rounded FP32 additions after the routed combine
    assert np.array_equal(got, f32_add(f32_add(out_routed[:M], sh_h), res_h))
    ref_routed, y_ref = oracle_layer(case.banks, x, ids, w, wl.limit, act_fp8=False)
    ref_sh = oracle.shared_expert(bits(gate), bits(up), bits(down), bits(x), LIMIT)
    valid = ((ids >= 0) & (ids < wl.experts)).astype(np.int32).ravel()
    ref = oracle.combine_residual(y_ref, w, valid, ref_sh, res_h)
    check_fp(sh_h, ref_sh, f"{name} shared")
    check_fp(got, ref, f"{name} routed+shared+residual")
    np.testing.assert_allclose(ref, ref_routed + ref_sh + res_h.astype(np.float64), rtol=1e-12,
                               atol=1e-9)


@pytest.mark.parametrize("with_shared,with_res", [(False, False), (True, False), (False, True)])
def test_combine_residual_optional_terms(with_shared, with_res):
    print(f"combine_residual shared{int(with_shared)} res{int(with_res)}", flush=True)
    wl = workloads.with_shape(workloads.WORKLOADS["tiny_e4m3_m1"], M=37)
    case = GpuCase(wl)
    ids, w, _ = workloads.make_routes(wl, M=37)
    ids[2, 1] = -1                                 # an empty slot
    w[2, 1] = 0.0
    out_routed, _, _, L = case.run(ids, w)
    H = wl.hidden
    sh = workloads.make_residual(37, H, 91, "cuda") if with_shared else None
    res = workloads.make_residual(37, H, 92, "cuda") if with_res else None
    w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    out = torch.full((37, H), float("nan"), dtype=torch.float32, device="cuda")
    B.moe_combine_residual(L.y, L.route, w_d, sh, res, H, out)
    torch.cuda.synchronize()
    want = out_routed[:37]
    if sh is not None:
        want = f32_add(want, sh.cpu().numpy())
    if res is not None:
        want = f32_add(want, res.cpu().numpy())
    assert np.array_equal(out.cpu().numpy(), want)
