"""GPU tests of HIP-graph capture.

The three calls (moe_route_pack, moe_expert_ffn, moe_combine) of several
layers, one per route set and each with its own buffers, are captured once
into a graph.  The graph is replayed several times, with eager layer calls and
synchronizations between the replays, and every layer's output after every
replay is compared bit for bit with the same layer run eagerly.  The library
records no memset and allocates nothing, so the captured calls are exactly the
eager ones.  moe_layer_fused takes a fresh epoch per call on the host and
must refuse capture with MOE_ERR_UNSUPPORTED, launching nothing."""
import gc

import numpy as np
import pytest
import torch

import workloads
from fp4_block_scaled_amd import binding as B
from moe_cases import GpuCase

pytestmark = pytest.mark.gpu

ROUTE_SETS = 4

CASES = [
    # (label, workload, reduced shape or None)
    ("gemv_decode", "decode_e4m3_m1", None),
    ("gemv_nvfp4_m16", "nvfp4_m16", None),
    ("gemm_m96", "prefill_e4m3_m4096", dict(hidden=1024, inter=512, experts=16, top_k=4, M=96)),
]


def _workload(name, shape):
    wl = workloads.WORKLOADS[name]
    return wl if shape is None else workloads.with_shape(wl, name=f"{name}_reduced", **shape)


@pytest.mark.parametrize("label,name,shape", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(label, name, shape):
    gc.collect()
    torch.cuda.empty_cache()
    wl = _workload(name, shape)
    print(f"graph {label}: M={wl.M} H={wl.hidden} I={wl.inter} E={wl.experts}", flush=True)
    case = GpuCase(wl)
    routes = [workloads.make_routes(wl, r) for r in range(ROUTE_SETS)]
    ids_d = [torch.from_numpy(np.ascontiguousarray(r[0], np.int32)).cuda() for r in routes]
    w_d = [torch.from_numpy(np.ascontiguousarray(r[1], np.float32)).cuda() for r in routes]
    layers = [case.layer() for _ in range(ROUTE_SETS)]
    x = case.x[: wl.M]

    eager = []
    for i, L in enumerate(layers):
        eager.append(L(x, ids_d[i], w_d[i]).clone())
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i, L in enumerate(layers):
            L(x, ids_d[i], w_d[i])
    torch.cuda.synchronize()

    side = case.layer()
    for rep in range(3):
        for L in layers:                      # clobber the outputs between replays
            L.out.fill_(float("nan"))
        side(x, ids_d[rep % ROUTE_SETS], w_d[rep % ROUTE_SETS])   # eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, L in enumerate(layers):
            got = L.out[: wl.M]
            assert torch.equal(got.view(torch.int32), eager[i].view(torch.int32)), \
                f"{label}: replay {rep}, route set {i} differs from the eager layer"
    del g


def test_fused_layer_refuses_capture():
    wl = workloads.WORKLOADS["tiny_e4m3_m1"]
    print("fused capture refusal", flush=True)
    case = GpuCase(wl)
    ids, w, _ = workloads.make_routes(wl, 0)
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    L = case.layer(mode=B.MOE_MODE_FUSED)
    want = L(case.x[: wl.M], ids_d, w_d).clone()
    torch.cuda.synchronize()
    L.out.fill_(float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(B.MoeError) as ei:
        with torch.cuda.graph(g):
            L(case.x[: wl.M], ids_d, w_d)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED
    assert "graph" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.isnan(L.out).all(), "a refused capture must launch nothing"
    del g
    # the eager call still works afterwards
    got = L(case.x[: wl.M], ids_d, w_d)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))
