"""moe_layer_static (the entry point for callers that cannot allocate: its
workspace is the library's static device array) against moe_layer with a
caller workspace, through the C ABI: route tables, packed y rows and
outputs bit for bit, on two calls in a row, the second with a smaller
input, for the GEMV tier at the decode shape and for the GEMM tier."""
import ctypes as C

import numpy as np
import pytest
import torch

import workloads
from fp4_block_scaled_amd import binding as B
from fp4_block_scaled_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu

_hip = C.CDLL("libamdhip64.so")
_hip.hipMemcpy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int]
_hip.hipMemcpy.restype = C.c_int


def d2h_i32(ptr, n):
    a = np.empty(max(n, 1), np.int32)
    assert _hip.hipMemcpy(a.ctypes.data, ptr, 4 * n, 2) == 0     # hipMemcpyDeviceToHost
    return a[:n]


def tables(route):
    S, E = route.num_slots, route.num_experts
    A = min(S, E)
    t = dict(expert_offsets=d2h_i32(route.expert_offsets, E + 1),
             token_to_perm=d2h_i32(route.token_to_perm, S),
             active_experts=d2h_i32(route.active_experts, A),
             num_active=d2h_i32(route.num_active, 1), status=d2h_i32(route.status, 1))
    nv = int(t["expert_offsets"][-1])
    t["sorted_slot"] = d2h_i32(route.sorted_slot, S)[:nv]
    t["sorted_token"] = d2h_i32(route.sorted_token, S)[:nv]
    return t


def run_pair(case_banks, x, wl, M, route_set, mode):
    ids, w, _ = workloads.make_routes(wl, route_set, M=M)
    ids_d = torch.from_numpy(np.ascontiguousarray(ids)).cuda()
    w_d = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    cb = [B.Bank.from_device_bank(b) for b in case_banks]
    ref = MoeLayer(*cb, wl.hidden, wl.inter, wl.top_k, M, wl.limit, mode)
    out_ref = ref(x[:M], ids_d, w_d).clone()
    y = torch.full((M * wl.top_k, wl.hidden), float("nan"), device="cuda")
    out = torch.full((M, wl.hidden), float("nan"), device="cuda")
    route = B.moe_layer_static(*cb, x[:M], ids_d, w_d, M, wl.top_k, wl.hidden, wl.inter, wl.limit,
                               mode, y, out)
    torch.cuda.synchronize()
    t_ref = {k: v.cpu().numpy() for k, v in ref.route_tables().items()}
    t_got = tables(route)
    nv = int(t_ref["expert_offsets"][-1])
    for k in t_got:
        a = t_ref[k][:nv] if k in ("sorted_slot", "sorted_token") else t_ref[k]
        assert np.array_equal(a, t_got[k]), f"route table {k} differs"
    assert np.array_equal(ref.y[:nv].cpu().numpy().view(np.uint32), y[:nv].cpu().numpy().view(np.uint32))
    assert np.array_equal(out_ref.cpu().numpy().view(np.uint32), out.cpu().numpy().view(np.uint32))
    assert np.all(np.isfinite(out.cpu().numpy()))


@pytest.mark.parametrize("name,Ms,mode", [
    ("verify_e4m3_m8", (16, 1), B.MOE_MODE_AUTO),          # GEMV tier, decode shape
    ("nvfp4_m16", (16, 3), B.MOE_MODE_AUTO),               # GEMV tier, NVFP4
    ("tiny_e4m3_m1", (40, 20), B.MOE_MODE_GEMM_A8),        # GEMM tier, small
])
def test_static_scratch_layer_matches_moe_layer(name, Ms, mode):
    base = workloads.WORKLOADS[name]
    wl = workloads.with_shape(base, M=max(Ms))
    banks = workloads.make_banks(wl, "cuda")
    x = workloads.make_x(wl, "cuda")
    for i, M in enumerate(Ms):
        print(f"moe_layer_static {name} M={M} mode={mode}", flush=True)
        run_pair(banks, x, wl, M, i + 1, mode)


def test_static_scratch_rejects_a_layer_too_large_for_it():
    wl = workloads.WORKLOADS["prefill_e4m3_m4096"]
    small = workloads.with_shape(wl, experts=8)
    banks = workloads.make_banks(small, "cuda")
    cb = [B.Bank.from_device_bank(b) for b in banks]
    need = B.moe_workspace_bytes(4096, 8, 8, wl.hidden, wl.inter, B.MOE_W_E4M3_B128, B.MOE_MODE_AUTO)
    assert need > B.MOE_STATIC_SCRATCH_BYTES
    p = torch.empty(16, device="cuda")
    r = B.moe_route_t()
    st = B.lib.moe_layer_static(C.byref(cb[0].c), C.byref(cb[1].c), C.byref(cb[2].c), p.data_ptr(),
                                p.data_ptr(), p.data_ptr(), 4096, 8, wl.hidden, wl.inter, 7.0,
                                B.MOE_MODE_AUTO, p.data_ptr(), p.data_ptr(), C.byref(r), None)
    assert st == B.MOE_ERR_WORKSPACE
    assert "static" in B.moe_last_error()
