#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN layer on one MI355X.

A step is one full layer: moe_route_pack -> moe_expert_ffn -> moe_combine on
one stream, inputs resident in HBM.  The headline workload is single-token
decode (H7168, I2048, 256 block-scaled E4M3 experts, top-8, M=1); the value is
microseconds per layer.  16 route sets are rotated across steps so that
consecutive steps read different experts and the 256 MB last-level cache
cannot serve a repeated working set.

Printed: ONE JSON line with the contract fields, the dominant kernel's
roofline (algorithmic bytes / its average duration from HIP events recorded
on its own stream during a stage-timing pass), and the CPU oracle timed on a
bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense FP8 MFMA (no sparsity)
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA (no sparsity)
METRIC = "µs/MoE layer + weight-read GB/s (% HBM peak) at M=1; tokens/s at M=4096"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_e4m3_m1")
    ap.add_argument("--route-sets", type=int, default=16)
    ap.add_argument("--also", default="verify_e4m3_m8,nvfp4_m1,nvfp4_m16,prefill_e4m3_m4096,nvfp4_m4096",
                    help="comma-separated extra workloads reported under 'also' ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-also-seconds", type=float, default=6.0,
                    help="CPU budget of the oracle beside each 'also' workload (at least one layer)")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the one-launch fused layer rows")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="first run 3 device copies of this many MB (a plain copy kernel of known "
                         "size, to scale HBM byte counters)")
    return ap.parse_args()


# --------------------------------------------------------------------------
# HIP events on the stream the kernels run on (ctypes, no torch wrapper)
# --------------------------------------------------------------------------
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000     # hipEventDisableSystemFence


class Hip:
    def __init__(self):
        self.h = C.CDLL("libamdhip64.so")
        self.h.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.h.hipEventSynchronize.argtypes = [C.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.h.hipEventDestroy.argtypes = [C.c_void_p]

    def events(self, n):
        arr = (C.c_void_p * n)()
        for i in range(n):
            p = C.c_void_p()
            # timing events without the system-scope release a default
            # event adds: nothing on the host reads the layer's output through
            # an event, and torch's synchronize precedes every host read
            assert self.h.hipEventCreateWithFlags(C.byref(p), HIP_EVENT_DISABLE_SYSTEM_FENCE) == 0
            arr[i] = p.value
        return arr

    def record(self, ev, stream):
        assert self.h.hipEventRecord(ev, stream) == 0

    def ms(self, a, b):
        f = C.c_float()
        assert self.h.hipEventSynchronize(b) == 0
        assert self.h.hipEventElapsedTime(C.byref(f), a, b) == 0
        return f.value


def algorithmic_bytes(wl, banks, ids):
    """Bytes a layer must move at least: codes + scales of every expert the
    routes select (each once), x read, out written, ids and weights read."""
    import numpy as np
    E = wl.experts
    used = np.unique(ids[(ids >= 0) & (ids < E)])
    per_expert = sum(b.nbytes_per_expert() for b in banks)
    gu_per_expert = banks[0].nbytes_per_expert() + banks[1].nbytes_per_expert()
    M = ids.shape[0]
    io = M * wl.hidden * 2 + M * wl.hidden * 4 + ids.size * 8
    return len(used) * per_expert + io, len(used) * gu_per_expert + M * wl.hidden * 2, len(used)


def nearest_rank(v, q):
    """q-th percentile of v by nearest rank (1-based rank ceil(q/100 * n))."""
    import math
    v = sorted(v)
    return v[max(1, math.ceil(q / 100.0 * len(v))) - 1]


def percentiles(us):
    return {"mean": round(sum(us) / len(us), 3), "min": round(min(us), 3),
            "p50": round(nearest_rank(us, 50), 3), "p90": round(nearest_rank(us, 90), 3),
            "p99": round(nearest_rank(us, 99), 3)}


def graph_replay(layer, x, ids_d, w_d, steps, hip):
    """One HIP graph of len(ids_d) layers (one per route set), replayed until
    at least `steps` layers ran.  Every replay's output is checked bit for bit
    against the eager layer of the last route set, with eager work and a
    synchronization between replays."""
    import torch
    R = len(ids_d)
    want = layer(x, ids_d[R - 1], w_d[R - 1]).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(R):
            layer(x, ids_d[i], w_d[i])
    torch.cuda.synchronize()
    ok = True
    for _ in range(3):                       # checked replays, eager work in between
        layer(x, ids_d[0], w_d[0])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ok &= bool(torch.equal(layer.out.view(torch.int32), want.view(torch.int32)))
    reps = max(1, (steps + R - 1) // R)
    sh = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.events(2)
    torch.cuda.synchronize()
    hip.record(e0, sh)
    for _ in range(reps):
        g.replay()
    hip.record(e1, sh)
    torch.cuda.synchronize()
    us = hip.ms(e0, e1) * 1000.0 / (reps * R)
    ok &= bool(torch.equal(layer.out.view(torch.int32), want.view(torch.int32)))
    del g
    return {"us_layer": round(us, 3), "layers": reps * R, "replays_match_eager": ok}


def cold_layers(layer, x, ids_d, w_d, steps, hip):
    """Each layer timed on its own after a 1 GiB device write (outside the
    events) that evicts the last-level cache."""
    import torch
    R = len(ids_d)
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    evs = [hip.events(2) for _ in range(steps)]
    for i in range(steps):
        flush.fill_(float(i))
        hip.record(evs[i][0], sh)
        layer(x, ids_d[i % R], w_d[i % R])
        hip.record(evs[i][1], sh)
    torch.cuda.synchronize()
    us = [hip.ms(a, b) * 1000.0 for a, b in evs]
    del flush
    torch.cuda.empty_cache()
    return percentiles(us)


def measure(wl, banks, steps, warmup, route_sets, hip, want_stages=True, fused=False,
            graph=True, cold=False):
    import numpy as np
    import torch

    import workloads
    from fp4_block_scaled_amd import binding as B
    from fp4_block_scaled_amd.layer import MoeLayer

    x = workloads.make_x(wl, "cuda")
    sets = [workloads.make_routes(wl, r) for r in range(route_sets)]
    ids_d = [torch.from_numpy(s[0]).cuda() for s in sets]
    w_d = [torch.from_numpy(s[1]).cuda() for s in sets]
    cb = [B.Bank.from_device_bank(b) for b in banks]
    mode = B.MOE_MODE_FUSED if fused else B.moe_resolve_mode(wl.M, wl.fmt)
    layer = MoeLayer(*cb, wl.hidden, wl.inter, wl.top_k, wl.M, wl.limit,
                     mode=B.MOE_MODE_FUSED if fused else B.MOE_MODE_AUTO)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    for i in range(warmup):
        layer(x, ids_d[i % route_sets], w_d[i % route_sets])
    torch.cuda.synchronize()
    ref = layer(x, ids_d[0], w_d[0]).clone()
    torch.cuda.synchronize()

    # timed region: exactly `steps` layers, events on the layer's stream
    e0, e1 = hip.events(2)
    torch.cuda.synchronize()
    hip.record(e0, sh)
    for i in range(steps):
        layer(x, ids_d[i % route_sets], w_d[i % route_sets])
    hip.record(e1, sh)
    torch.cuda.synchronize()
    total_ms = hip.ms(e0, e1)
    us_layer = total_ms * 1000.0 / steps

    # per-layer times: two events around each layer, nothing else in between
    pev = [hip.events(2) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        hip.record(pev[i][0], sh)
        layer(x, ids_d[i % route_sets], w_d[i % route_sets])
        hip.record(pev[i][1], sh)
    torch.cuda.synchronize()
    pct = percentiles([hip.ms(a, b) * 1000.0 for a, b in pev])

    # output must not drift across runs (deterministic kernels)
    again = layer(x, ids_d[0], w_d[0])
    torch.cuda.synchronize()
    stable = bool(torch.equal(again.view(torch.int32), ref.view(torch.int32)))

    stages = None
    sums_stable = None
    host_ahead = None
    if want_stages:
        nst = B.moe_set_stage_events(None, wl.fmt, wl.hidden, wl.inter, mode)
        per = nst + 3       # route start, ffn stage marks (nst+1), combine end
        evs = [hip.events(per) for _ in range(steps)]
        sums = []
        # The stage events time the GPU only if the host has queued a step's
        # launches before the GPU reaches them: otherwise a host gap between
        # an event and the next launch counts as kernel time.  So the steps
        # go in batches, each queued behind a spin kernel that outlasts the
        # host's queueing of the batch (checked below).
        batch = 16
        c0, c1 = hip.events(2)
        torch.cuda.synchronize()
        hip.record(c0, sh)
        torch.cuda._sleep(1 << 20)
        hip.record(c1, sh)
        torch.cuda.synchronize()
        us_per_cycle = hip.ms(c0, c1) * 1000.0 / (1 << 20)
        hold_us = 4000.0
        cycles = int(hold_us / max(us_per_cycle, 1e-6))
        host_us = []
        ref.view(torch.int32).to(torch.int64).sum()     # the checksum's kernels loaded once
        torch.cuda.synchronize()
        for i in range(steps):
            if i % batch == 0:
                if i:
                    host_us.append((time.perf_counter() - t_b) * 1e6)
                torch.cuda._sleep(cycles)
                t_b = time.perf_counter()
            ev = evs[i]
            sub = (C.c_void_p * (nst + 1))(*[ev[1 + j] for j in range(nst + 1)])
            evs[i] = (ev, sub)
            hip.record(ev[0], sh)
            B.moe_set_stage_events(sub, wl.fmt, wl.hidden, wl.inter, mode)
            out = layer(x, ids_d[i % route_sets], w_d[i % route_sets])
            hip.record(ev[per - 1], sh)
            # checksum of the output bits, outside the events
            sums.append(out.view(torch.int32).to(torch.int64).sum())
        host_us.append((time.perf_counter() - t_b) * 1e6)
        B.moe_set_stage_events(None, wl.fmt, wl.hidden, wl.inter, mode)
        torch.cuda.synchronize()
        host_ahead = max(host_us) < hold_us
        print(f"# {wl.name}: stage batches queued in {min(host_us):.0f}-{max(host_us):.0f} us "
              f"behind a {hold_us:.0f} us spin", file=sys.stderr, flush=True)
        sums = [int(v) for v in sums]
        sums_stable = all(sums[i] == sums[i % route_sets] for i in range(steps))
        if mode == B.MOE_MODE_GEMM_A8:
            names = ["route_pack", "act_quant_tiles", "gateup_gemm", "down_gemm", "combine"]
        elif mode == B.MOE_MODE_GEMM_A16:
            names = ["route_pack", "tiles", "gateup_gemm", "down_gemm", "combine"]
        elif mode == B.MOE_MODE_FUSED:
            names = ["host", "fused_layer", "tail"]
        else:
            names = ["route_pack", "gateup_gemv", "down_gemv", "combine"]
        acc = np.zeros(per - 1)
        for ev, _ in evs:
            for j in range(per - 1):
                acc[j] += hip.ms(ev[j], ev[j + 1])
        stages = {names[j]: float(acc[j] * 1000.0 / steps) for j in range(per - 1)}

    alg = [algorithmic_bytes(wl, banks, s[0]) for s in sets]
    alg_layer = float(np.mean([a[0] for a in alg]))
    alg_gateup = float(np.mean([a[1] for a in alg]))
    uniq = float(np.mean([a[2] for a in alg]))
    # dense-equivalent FLOPs of the valid slots: 2 (gate, up) + 1 (down) products of I*H
    flops = float(np.mean([6.0 * int(((s[0] >= 0) & (s[0] < wl.experts)).sum()) * wl.hidden * wl.inter
                           for s in sets]))
    if fused:       # the one-launch layer refuses graph capture (a fresh epoch per call)
        gr = {"unsupported": "moe_layer_fused takes a fresh epoch per call and refuses capture"}
    else:
        gr = graph_replay(layer, x, ids_d, w_d, steps, hip) if graph else None
    cl = cold_layers(layer, x, ids_d, w_d, steps, hip) if cold else None
    return dict(name=wl.name, us_layer=us_layer, ms_total=total_ms, stable=stable, stages=stages,
                percentiles=pct, checksums_stable=sums_stable, host_ahead=host_ahead, graph=gr, cold=cl,
                alg_layer_bytes=alg_layer, alg_gateup_bytes=alg_gateup, unique_experts=uniq,
                flops=flops, mode=mode, layer=layer, x=x, sets=sets)


def cpu_baseline(wl, banks, x, sets, budget_s, stride=1, act_fp8=False):
    """The oracle, as it stands, on whole layers of the same workload; with
    stride > 1 on the deterministic subset of tokens t = 0, stride, 2*stride,
    ... of each layer (its routes, weights and x rows as they are), the time
    scaled by stride to a whole layer.  act_fp8: the oracle of the FP8 GEMM
    tier (x and h quantized per 1x128 group)."""
    import numpy as np

    import oracle  # CPU baseline leg only
    import torch
    E = wl.experts
    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)[::stride]
    sets = [(ids[::stride], w[::stride], extra) for ids, w, extra in sets]
    # the route sets' selected experts, copied to the host once (outside the
    # timing), as many sets as fit about 2 GB of host memory (at least one)
    host, held = [], 0
    for ids, w, _ in sets:
        if host and held >= (2 << 30):
            break
        used = np.unique(ids[(ids >= 0) & (ids < E)])
        hb = []
        for b in banks:
            sub = b.select(used)
            hb.append(oracle.Bank(sub.fmt, sub.codes.cpu().numpy(), sub.scales.cpu().numpy(),
                                  None if sub.scale2 is None else sub.scale2.cpu().numpy()))
        host.append((hb, np.searchsorted(used, ids).astype(np.int32), w))
        held += sum(h.codes.nbytes + h.scales.nbytes for h in hb)
    # whole layers, cycling over the route sets, until the budget of CPU time
    times = []
    while sum(times) < budget_s and len(times) < 100000:
        hb, remap, w = host[len(times) % len(host)]
        t0 = time.perf_counter()
        oracle.moe_layer(*hb, xb, remap, w, wl.limit, act_fp8)
        times.append(time.perf_counter() - t0)
    n = len(times)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    what = (f"{n} whole layers of {wl.name}" if stride == 1 else
            f"{n} layers of {wl.name} on the 1/{stride} token subset t % {stride} == 0 "
            f"({len(xb)} of {wl.M} tokens), time x {stride} per whole layer")
    return dict(value=float(np.mean(times) * stride * 1e6), unit="us/layer", cores=threads,
                kind="oracle",
                sample=f"{what} ({sum(times):.1f} s), cycling over route sets 0..{len(host) - 1}, "
                       f"FP64{', x and h quantized per 1x128 as the FP8 GEMM tier' if act_fp8 else ''}, "
                       f"selected experts copied to host before timing")


# HBM bytes per launch of the roofline kernel, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
# counter reads for a plain 256 MB device copy in the same run: FETCH_SIZE
# reads 131,088 KiB for it (x 2.0), WRITE_SIZE 262,144 KiB (x 1.0).  The
# entry holds only while the kernel sources hash to `src` (first 16 hex
# digits of the sha256 of the listed files, concatenated); otherwise the
# traffic is reported as null.
COUNTER_SCALE = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
TRAFFIC = {
    "decode_e4m3_m1": {"kernel": "gemv_gateup", "files": ["gemv_e4m3.hip", "fused_common.h", "moe_device.h"],
        "src": "cde11db9bf57e724d7277bb1a4b625a5e0174e2455c8b818", "fetch_kib": 115083, "write_kib": 65},
    "decode_e4m3_m1/fused": {"kernel": "moe_fused_decode", "files": ["gemv_e4m3.hip", "fused_common.h", "moe_device.h"],
        "src": "cde11db9bf57e724d7277bb1a4b625a5e0174e2455c8b818", "fetch_kib": 173074, "write_kib": 1070},
    "nvfp4_m1": {"kernel": "gemv_gateup", "files": ["gemv_nvfp4.hip", "fused_common.h", "moe_device.h"],
        "src": "9a1dcecde0b5c179d7277bb1a4b625a5e0174e2455c8b818", "fetch_kib": 41626, "write_kib": 49},
    "nvfp4_m1/fused": {"kernel": "moe_fused_decode", "files": ["gemv_nvfp4.hip", "fused_common.h", "moe_device.h"],
        "src": "9a1dcecde0b5c179d7277bb1a4b625a5e0174e2455c8b818", "fetch_kib": 64883, "write_kib": 835},
    "prefill_e4m3_m4096": {"kernel": "gemm_gateup", "files": ["gemm_fp8.hip", "gemm_common.h", "moe_device.h"],
        "src": "e7bd3c69fc01c3df46ff9d1401442f7fe0174e2455c8b818", "fetch_kib": 4022574, "write_kib": 68917},
    "nvfp4_m4096": {"kernel": "gemm_gateup_nvfp4", "files": ["gemm_nvfp4.hip", "gemm_common.h", "moe_device.h"],
        "src": "268b195ef0d0f1e646ff9d1401442f7fe0174e2455c8b818", "fetch_kib": 2153835, "write_kib": 98304},
    "verify_e4m3_m8": {"kernel": "gemv_gateup", "files": ["gemv_e4m3.hip", "fused_common.h", "moe_device.h"],
        "src": "cde11db9bf57e724d7277bb1a4b625a5e0174e2455c8b818", "fetch_kib": 646018, "write_kib": 514},
    "nvfp4_m16": {"kernel": "gemv_gateup", "files": ["gemv_nvfp4.hip", "fused_common.h", "moe_device.h"],
        "src": "9a1dcecde0b5c179d7277bb1a4b625a5e0174e2455c8b818", "fetch_kib": 444742, "write_kib": 768},
}


def measured_traffic(name):
    import hashlib
    t = TRAFFIC.get(name)
    if t is None:
        return None
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp4_block_scaled_amd", "csrc")
    src = "".join(hashlib.sha256(open(os.path.join(d, f), "rb").read()).hexdigest()[:16]
                  for f in t["files"])
    if src != t["src"]:
        return None
    return round((t["fetch_kib"] * COUNTER_SCALE["FETCH_SIZE"] +
                  t["write_kib"] * COUNTER_SCALE["WRITE_SIZE"]) * 1024)


def roofline(r):
    """Roofline of the dominant kernel of the tier that ran: the gate/up GEMV
    against HBM bandwidth, the gate/up FP8 GEMM against the FP8 MFMA peak, or
    the one-launch fused layer (all of the layer's bytes) against HBM."""
    if r["mode"] == 3:
        us = r["stages"]["fused_layer"]
        gbps = r["alg_layer_bytes"] / (us * 1e-6) / 1e9
        return {"kernel": "moe_fused_decode", "bound": "hbm", "achieved": round(gbps, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(r["name"] + "/fused"),
                "alg_bytes_per_launch": round(r["alg_layer_bytes"]), "avg_launch_us": round(us, 3)}
    if r["mode"] == 2:
        # the E4M3 tier's gate/up contracts on the bf16 MFMA (E4M3 codes are
        # bf16 values exactly): its peak is the bf16 one
        us = r["stages"]["gateup_gemm"]
        flop = r["flops"] * 2.0 / 3.0
        tf = flop / (us * 1e-6) / 1e12
        return {"kernel": "gemm_gateup", "bound": "mfma", "achieved": round(tf, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(r["name"]), "alg_flop_per_launch": round(flop),
                "avg_launch_us": round(us, 3)}
    if r["mode"] == 4:
        us = r["stages"]["gateup_gemm"]
        flop = r["flops"] * 2.0 / 3.0
        tf = flop / (us * 1e-6) / 1e12
        return {"kernel": "gemm_gateup_nvfp4", "bound": "mfma", "achieved": round(tf, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(r["name"]), "alg_flop_per_launch": round(flop),
                "avg_launch_us": round(us, 3)}
    us = r["stages"]["gateup_gemv"]
    gbps = r["alg_gateup_bytes"] / (us * 1e-6) / 1e9
    return {"kernel": "gemv_gateup", "bound": "hbm", "achieved": round(gbps, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(r["name"]),
            "alg_bytes_per_launch": round(r["alg_gateup_bytes"]), "avg_launch_us": round(us, 3)}


def router_rows(wl, banks, steps, route_sets, hip, M=None):
    """moe_router_topk (softmax, renormalized) alone on [M, E] logits, and, at
    the workload's own M, router + the three layer calls with no host hop."""
    import numpy as np
    import torch

    import workloads
    from fp4_block_scaled_amd import binding as B
    from fp4_block_scaled_amd.layer import MoeLayer

    M = wl.M if M is None else M
    logits = [torch.from_numpy(workloads.make_logits(wl, r, M)[0].astype(np.float32)).cuda()
              for r in range(route_sets)]
    ids = torch.empty((M, wl.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, wl.top_k), dtype=torch.float32, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream

    def router(i):
        B.moe_router_topk(logits[i % route_sets], M, wl.experts, wl.top_k, B.MOE_ROUTER_SOFTMAX,
                          None, 1.0, 1, ids, w)

    for i in range(3):
        router(i)
    e0, e1 = hip.events(2)
    torch.cuda.synchronize()
    hip.record(e0, sh)
    for i in range(steps):
        router(i)
    hip.record(e1, sh)
    torch.cuda.synchronize()
    out = {"rows": M, "experts": wl.experts, "top_k": wl.top_k,
           "router_us": round(hip.ms(e0, e1) * 1000.0 / steps, 3)}
    if M == wl.M:
        cb = [B.Bank.from_device_bank(b) for b in banks]
        layer = MoeLayer(*cb, wl.hidden, wl.inter, wl.top_k, wl.M, wl.limit)
        x = workloads.make_x(wl, "cuda")
        for i in range(3):
            router(i)
            layer(x, ids, w)
        torch.cuda.synchronize()
        hip.record(e0, sh)
        for i in range(steps):
            router(i)
            layer(x, ids, w)
        hip.record(e1, sh)
        torch.cuda.synchronize()
        out["router_plus_layer_us"] = round(hip.ms(e0, e1) * 1000.0 / steps, 3)
        del layer
    del logits
    torch.cuda.empty_cache()
    return out


def shared_rows(wl, banks, steps, hip):
    """The shared expert (bf16 SwiGLU MLP as wide as one routed expert) on the
    workload's M tokens alone, and the whole layer with it: route pack, expert
    FFN, shared expert, then the combine with the shared row and a residual."""
    import numpy as np
    import torch

    import workloads
    from fp4_block_scaled_amd import binding as B
    from fp4_block_scaled_amd.layer import MoeLayer

    M, H, W = wl.M, wl.hidden, wl.inter
    gate, up, down = workloads.make_shared_expert(H, W, wl.seed * 10 + 11, "cuda")
    x = workloads.make_x(wl, "cuda")
    sh = torch.empty((M, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.moe_shared_workspace_bytes(M, H, W), dtype=torch.uint8, device="cuda")
    res = workloads.make_residual(M, H, wl.seed + 5, "cuda")
    st = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.events(2)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        hip.record(e0, st)
        for _ in range(steps):
            fn()
        hip.record(e1, st)
        torch.cuda.synchronize()
        return hip.ms(e0, e1) * 1000.0 / steps

    def shared():
        B.moe_shared_expert(gate, up, down, x, M, H, W, wl.limit, sh, ws)

    us_sh = timed(shared)
    nbytes = 3 * W * H * 2 + M * H * 2 + M * H * 4
    cb = [B.Bank.from_device_bank(b) for b in banks]
    layer = MoeLayer(*cb, H, W, wl.top_k, M, wl.limit)
    ids, w, _ = workloads.make_routes(wl)
    ids_d = torch.from_numpy(ids).cuda()
    w_d = torch.from_numpy(w).cuda()
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    layer(x, ids_d, w_d)

    def combine_res():
        B.moe_combine_residual(layer.y, layer.route, w_d, sh, res, H, out)

    us_cr = timed(combine_res)

    def full():
        r = B.moe_route_pack(ids_d, M, wl.top_k, layer.E, layer.ws)
        B.moe_expert_ffn(layer.gate, layer.up, layer.down, x, r, H, W, wl.limit, B.MOE_MODE_AUTO,
                         layer.y, layer.ws)
        shared()
        B.moe_combine_residual(layer.y, r, w_d, sh, res, H, out)

    us_full = timed(full)
    del layer
    torch.cuda.empty_cache()
    return {"shared_width": W, "shared_us": round(us_sh, 3),
            "shared_hbm_frac": round(nbytes / (us_sh * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "combine_residual_us": round(us_cr, 3),
            "layer_with_shared_and_residual_us": round(us_full, 3)}


def extra_rows(r):
    """Per-layer percentiles, the output checksum check, the routing's
    statistics (expert loads over the route sets, rho of correlated
    routing), HIP-graph replay and the cold-cache row of one measured
    workload."""
    infos = [s[2] for s in r["sets"]]
    routing = {"max_expert_load": max(i["max_load"] for i in infos),
               "mean_expert_load": round(float(sum(i["mean_load"] for i in infos) / len(infos)), 3)}
    if "rho" in infos[0]:
        routing["rho"] = [round(float(i["rho"]), 4) for i in infos]
    out = {"layer_us_percentiles": r["percentiles"], "checksums_stable": r["checksums_stable"],
           "routing": routing}
    if r["graph"] is not None:
        out["graph"] = r["graph"]
    if r["cold"] is not None:
        out["cold_us_percentiles"] = r["cold"]
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer keeps every "
              f"expert resident on a single MI355X and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import numpy as np
    import torch

    import workloads
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    hip = Hip()

    if args.copy_calib_mb > 0:
        src = torch.empty(args.copy_calib_mb << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"# copy calibration: 3 copies of {args.copy_calib_mb} MB", file=sys.stderr, flush=True)

    wl = workloads.WORKLOADS[args.workload]
    t0 = time.time()
    banks = workloads.make_banks(wl, "cuda")
    torch.cuda.synchronize()
    print(f"# banks for {wl.name} ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    r = measure(wl, banks, args.steps, args.warmup, args.route_sets, hip, cold=wl.M <= 16)
    print(f"# {wl.name}: {r['us_layer']:.2f} us/layer, stages {r['stages']}", file=sys.stderr,
          flush=True)

    gbps = r["alg_layer_bytes"] / (r["us_layer"] * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(r["us_layer"], 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_total"] / args.steps, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3*bf16->f32" if wl.fmt == 1 else "e2m1*bf16->f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "hidden": wl.hidden, "inter": wl.inter,
                   "experts": wl.experts, "top_k": wl.top_k, "M": wl.M,
                   "route_sets": args.route_sets, "unique_experts": r["unique_experts"]},
        "weight_read_GBps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(wl.M / (r["us_layer"] * 1e-6), 1),
        "stages_us": {k: round(v, 3) for k, v in r["stages"].items()},
        "stages_host_ahead": r["host_ahead"],
        "output_stable": r["stable"],
        "roofline": roofline(r),
    }
    line.update(extra_rows(r))
    if r["mode"] == 2:
        line["alg_TFLOPs"] = round(r["flops"] / (r["us_layer"] * 1e-6) / 1e12, 1)

    def fused_row(w2, b2):
        rf = measure(w2, b2, args.steps, args.warmup, args.route_sets, hip, fused=True,
                     cold=w2.M <= 16)
        gf = rf["alg_layer_bytes"] / (rf["us_layer"] * 1e-6) / 1e9
        print(f"# {w2.name} fused: {rf['us_layer']:.2f} us/layer", file=sys.stderr, flush=True)
        return {"us_layer": round(rf["us_layer"], 3), "weight_read_GBps": round(gf, 1),
                "hbm_frac": round(gf / HBM_PEAK_GBPS, 4),
                "tokens_per_s": round(w2.M / (rf["us_layer"] * 1e-6), 1),
                "stages_us": {k: round(v, 3) for k, v in rf["stages"].items()},
                "stages_host_ahead": rf["host_ahead"],
                "output_stable": rf["stable"], "roofline": roofline(rf), **extra_rows(rf)}

    def fused_ok(w2):
        if args.no_fused or w2.M * w2.top_k > 256:
            return False
        return w2.fmt == 1 or (w2.M == 1 and w2.hidden % 2048 == 0 and w2.hidden <= 16384)

    if fused_ok(wl):
        line["fused"] = fused_row(wl, banks)
    line["router"] = router_rows(wl, banks, args.steps, args.route_sets, hip)
    if wl.M <= 16:
        line["shared_expert"] = shared_rows(wl, banks, args.steps, hip)
    also = {}
    for name in [a for a in args.also.split(",") if a]:
        w2 = workloads.WORKLOADS[name]
        same = (w2.hidden, w2.inter, w2.experts, w2.fmt) == (wl.hidden, wl.inter, wl.experts, wl.fmt)
        b2 = banks if same else workloads.make_banks(w2, "cuda")
        r2 = measure(w2, b2, max(20, args.steps // 2), args.warmup, args.route_sets, hip,
                     cold=w2.M <= 16)
        g2 = r2["alg_layer_bytes"] / (r2["us_layer"] * 1e-6) / 1e9
        tf = r2["flops"] / (r2["us_layer"] * 1e-6) / 1e12
        also[name] = {"us_layer": round(r2["us_layer"], 3), "weight_read_GBps": round(g2, 1),
                      "hbm_frac": round(g2 / HBM_PEAK_GBPS, 4),
                      "tokens_per_s": round(w2.M / (r2["us_layer"] * 1e-6), 1),
                      "unique_experts": r2["unique_experts"],
                      "stages_us": {k: round(v, 3) for k, v in r2["stages"].items()},
                      "stages_host_ahead": r2["host_ahead"],
                      "output_stable": r2["stable"]}
        also[name]["roofline"] = roofline(r2)
        also[name].update(extra_rows(r2))
        if fused_ok(w2):
            also[name]["fused"] = fused_row(w2, b2)
        if w2.M <= 16:
            also[name]["shared_expert"] = shared_rows(w2, b2, max(20, args.steps // 2), hip)
        if w2.M > 16:
            also[name]["router"] = router_rows(w2, b2, max(20, args.steps // 2), args.route_sets,
                                               hip)
        if r2["mode"] == 2:
            also[name].update({"tier": "grouped_gemm_bf16_gateup_fp8_down", "alg_TFLOPs": round(tf, 1),
                               "mfma_frac_bf16": round(tf / BF16_PEAK_TFLOPS, 4)})
            line["prefill_tokens_per_s"] = also[name]["tokens_per_s"]
        elif r2["mode"] == 4:
            also[name].update({"tier": "bf16_mfma_grouped_gemm_w4a16", "alg_TFLOPs": round(tf, 1),
                               "mfma_frac_bf16": round(tf / BF16_PEAK_TFLOPS, 4)})
            line["nvfp4_prefill_tokens_per_s"] = also[name]["tokens_per_s"]
        print(f"# {name}: {r2['us_layer']:.2f} us/layer", file=sys.stderr, flush=True)
        if not args.no_cpu_baseline:
            # the oracle beside this config: whole layers at decode sizes, a
            # 1/8 token subset of the prefill layers
            cb = cpu_baseline(w2, b2, r2["x"], r2["sets"], args.cpu_also_seconds,
                              stride=8 if w2.M > 16 else 1, act_fp8=r2["mode"] == 2)
            also[name]["cpu_baseline"] = cb
            print(f"# {name}: oracle {cb['value']:.0f} us/layer on {cb['cores']} threads",
                  file=sys.stderr, flush=True)
        if not same:
            del b2
        del r2
        torch.cuda.empty_cache()
    if also:
        line["also"] = also
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, banks, r["x"], r["sets"], args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
