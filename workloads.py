"""Seeded synthetic inputs for the routed MoE FFN layer.

Both sides of every comparison (the HIP library and the CPU oracle) take their
inputs from here; this module holds none of the layer's arithmetic (no
dequantization, projection, activation or combine).  It draws:

* expert banks: block-scaled E4M3 (codes from clamp(64 * N(0,1), +-448) cast to
  float8_e4m3fn by torch, one FP32 scale exp(-6 + 0.5 N(0,1)) per 128x128
  block) or NVFP4 (uniform E2M1 nibbles, one E4M3 scale per 16 from |N(0,1)|,
  scale_2 = 1/448 per expert);
* activations x in bf16 (N(0,1) or U[-2, 2]);
* routes: ids and weights from a softmax over FP64 logits on the host, top-k
  by descending probability with ties to the lower expert id, renormalised
  over the k picks and rounded to FP32.

Bank tensors are drawn with torch's generator on the requested device in fixed
chunks of experts, so a given (seed, device) always yields the same bytes.
Routing uses numpy's PCG64 on the host.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

E4M3_B128 = 1
NVFP4_B16 = 2

_CHUNK_EXPERTS = 8


@dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    inter: int
    experts: int
    top_k: int
    M: int
    fmt: int
    x_dist: str          # "normal" or "uniform2"
    route: str           # "softmax", "correlated", "biased"
    limit: float = 7.0
    seed: int = 1000
    note: str = ""

    @property
    def slots(self) -> int:
        return self.M * self.top_k


WORKLOADS = {
    "tiny_e4m3_m1": Workload(
        "tiny_e4m3_m1", 256, 128, 16, 4, 1, E4M3_B128, "uniform2", "softmax",
        seed=1000, note="1 layer, H256 I128, 16 experts top-4, M=1"),
    "decode_e4m3_m1": Workload(
        "decode_e4m3_m1", 7168, 2048, 256, 8, 1, E4M3_B128, "normal", "softmax",
        seed=1001, note="decode, H7168 I2048, 256 experts top-8, M=1"),
    "verify_e4m3_m8": Workload(
        "verify_e4m3_m8", 7168, 2048, 256, 8, 8, E4M3_B128, "normal", "correlated",
        seed=1002, note="speculative verify, M=8, ~30% of slots share experts"),
    "prefill_e4m3_m4096": Workload(
        "prefill_e4m3_m4096", 7168, 2048, 256, 8, 4096, E4M3_B128, "normal", "biased",
        seed=1003, note="grouped prefill, M=4096, logits + per-expert bias N(0,0.5)"),
    "nvfp4_m1": Workload(
        "nvfp4_m1", 6144, 1536, 160, 8, 1, NVFP4_B16, "uniform2", "softmax",
        seed=1004, note="NVFP4 experts, H6144 I1536, 160 experts top-8, M=1"),
    "nvfp4_m16": Workload(
        "nvfp4_m16", 6144, 1536, 160, 8, 16, NVFP4_B16, "uniform2", "softmax",
        seed=1004, note="NVFP4 experts, M=16"),
    "nvfp4_m4096": Workload(
        "nvfp4_m4096", 6144, 1536, 160, 8, 4096, NVFP4_B16, "uniform2", "softmax",
        seed=1004, note="NVFP4 experts, prefill M=4096 (the M=1/16 draws at prefill width)"),
}


def with_shape(base: Workload, **kw) -> Workload:
    """A reduced copy of a workload (same distributions, other sizes)."""
    d = dict(base.__dict__)
    d.update(kw)
    return Workload(**d)


# --------------------------------------------------------------------------
# banks
# --------------------------------------------------------------------------

@dataclass
class DeviceBank:
    fmt: int
    codes: torch.Tensor            # uint8
    scales: torch.Tensor           # float32 (E4M3) or uint8 (NVFP4)
    scale2: Optional[torch.Tensor] = None  # float32 [E] (NVFP4)

    @property
    def num_experts(self):
        return int(self.codes.shape[0])

    @property
    def n_out(self):
        return int(self.codes.shape[1])

    @property
    def k_in(self):
        k = int(self.codes.shape[2])
        return 2 * k if self.fmt == NVFP4_B16 else k

    def nbytes_per_expert(self) -> int:
        b = self.codes[0].numel() + self.scales[0].numel() * self.scales.element_size()
        if self.scale2 is not None:
            b += 4
        return int(b)

    def select(self, experts) -> "DeviceBank":
        idx = torch.as_tensor(np.asarray(experts, dtype=np.int64), device=self.codes.device)
        return DeviceBank(self.fmt, self.codes.index_select(0, idx).contiguous(),
                          self.scales.index_select(0, idx).contiguous(),
                          None if self.scale2 is None else
                          self.scale2.index_select(0, idx).contiguous())


def make_e4m3_bank(E: int, n: int, k: int, seed: int, device) -> DeviceBank:
    """E4M3 codes from clamp(64 * N(0,1), +-448); FP32 scales exp(-6 + 0.5 N(0,1))
    per 128x128 block."""
    assert n % 128 == 0 and k % 128 == 0
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    codes = torch.empty((E, n, k), dtype=torch.uint8, device=device)
    for e0 in range(0, E, _CHUNK_EXPERTS):
        e1 = min(E, e0 + _CHUNK_EXPERTS)
        z = torch.randn((e1 - e0, n, k), generator=g, device=device, dtype=torch.float32)
        z.mul_(64.0).clamp_(-448.0, 448.0)
        codes[e0:e1] = z.to(torch.float8_e4m3fn).view(torch.uint8)
        del z
    zs = torch.randn((E, n // 128, k // 128), generator=g, device=device, dtype=torch.float32)
    scales = torch.exp(zs * 0.5 - 6.0)
    return DeviceBank(E4M3_B128, codes, scales.contiguous())


def make_nvfp4_bank(E: int, n: int, k: int, seed: int, device) -> DeviceBank:
    """Uniform E2M1 nibbles; E4M3 scales from |N(0,1)| per 16; scale_2 = 1/448."""
    assert n % 128 == 0 and k % 128 == 0
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    codes = torch.empty((E, n, k // 2), dtype=torch.uint8, device=device)
    for e0 in range(0, E, _CHUNK_EXPERTS):
        e1 = min(E, e0 + _CHUNK_EXPERTS)
        codes[e0:e1] = torch.randint(0, 256, (e1 - e0, n, k // 2), generator=g,
                                     device=device, dtype=torch.int32).to(torch.uint8)
    zs = torch.randn((E, n, k // 16), generator=g, device=device, dtype=torch.float32)
    scales = zs.abs_().to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    scale2 = torch.full((E,), 1.0 / 448.0, dtype=torch.float32, device=device)
    return DeviceBank(NVFP4_B16, codes, scales, scale2)


def make_banks(wl: Workload, device):
    """(gate [E, I, H], up [E, I, H], down [E, H, I]) for a workload."""
    mk = make_e4m3_bank if wl.fmt == E4M3_B128 else make_nvfp4_bank
    s = wl.seed * 10
    gate = mk(wl.experts, wl.inter, wl.hidden, s + 1, device)
    up = mk(wl.experts, wl.inter, wl.hidden, s + 2, device)
    down = mk(wl.experts, wl.hidden, wl.inter, s + 3, device)
    return gate, up, down


# --------------------------------------------------------------------------
# activations
# --------------------------------------------------------------------------

def make_x(wl: Workload, device, seed: Optional[int] = None, M: Optional[int] = None) -> torch.Tensor:
    M = wl.M if M is None else M
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 10 + 7 if seed is None else seed)
    if wl.x_dist == "normal":
        x = torch.randn((M, wl.hidden), generator=g, device=device, dtype=torch.float32)
    else:
        x = torch.rand((M, wl.hidden), generator=g, device=device, dtype=torch.float32) * 4.0 - 2.0
    return x.to(torch.bfloat16).contiguous()


# --------------------------------------------------------------------------
# shared expert and residual
# --------------------------------------------------------------------------

def make_shared_expert(hidden: int, width: int, seed: int, device, gate_std: float = 2.5):
    """bf16 (gate [W, H], up [W, H], down [H, W]) of a shared expert.

    Entries N(0, s^2) rounded to bf16, s = gate_std / sqrt(H) for gate and up
    (so with N(0,1) activations g and u are about N(0, gate_std^2) and the
    clamp at 7 is reached now and then) and 1 / sqrt(W) for down."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    sg = gate_std / hidden ** 0.5
    gate = (torch.randn((width, hidden), generator=g, device=device) * sg).to(torch.bfloat16)
    up = (torch.randn((width, hidden), generator=g, device=device) * sg).to(torch.bfloat16)
    down = (torch.randn((hidden, width), generator=g, device=device) / width ** 0.5) \
        .to(torch.bfloat16)
    return gate.contiguous(), up.contiguous(), down.contiguous()


def make_residual(M: int, hidden: int, seed: int, device) -> torch.Tensor:
    """FP32 residual rows N(0, 1)."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((M, hidden), generator=g, device=device, dtype=torch.float32)


# --------------------------------------------------------------------------
# routes (host, FP64)
# --------------------------------------------------------------------------

def topk_softmax(logits: np.ndarray, k: int):
    """Top-k of softmax(logits) per row, ties to the lower expert id;
    weights renormalised over the picks, rounded to FP32."""
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]
    pk = np.take_along_axis(p, order, axis=1)
    w = pk / pk.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def _correlated_logits(rng, M, E, rho):
    zc = rng.standard_normal(E)
    zt = rng.standard_normal((M, E))
    return np.sqrt(rho) * zc[None, :] + np.sqrt(1.0 - rho) * zt


def calibrate_rho(seed: int, M: int, E: int, k: int, shared: float = 0.30) -> float:
    """rho in [0, 1] such that 1 - U/(M k) is closest to `shared` for this seed
    (U = number of distinct experts over the M tokens), by bisection."""
    target_u = (1.0 - shared) * M * k

    def union(rho):
        rng = np.random.default_rng(seed)
        ids, _ = topk_softmax(_correlated_logits(rng, M, E, rho), k)
        return len(np.unique(ids))

    lo, hi = 0.0, 1.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if union(mid) > target_u:
            lo = mid
        else:
            hi = mid
    best = min((lo, hi), key=lambda r: abs(union(r) - target_u))
    return float(best)


def make_logits(wl: Workload, route_set: int = 0, M: Optional[int] = None):
    """(router logits float64 [M, E], info dict) of one route set."""
    M = wl.M if M is None else M
    seed = wl.seed * 100 + route_set
    rng = np.random.default_rng(seed)
    info = {"seed": seed}
    if wl.route == "softmax":
        logits = rng.standard_normal((M, wl.experts))
    elif wl.route == "biased":
        bias = np.random.default_rng(wl.seed).normal(0.0, 0.5, wl.experts)
        logits = rng.standard_normal((M, wl.experts)) + bias[None, :]
    elif wl.route == "correlated":
        rho = calibrate_rho(seed, M, wl.experts, wl.top_k)
        logits = _correlated_logits(np.random.default_rng(seed), M, wl.experts, rho)
        info["rho"] = rho
    else:
        raise ValueError(wl.route)
    return logits, info


def make_routes(wl: Workload, route_set: int = 0, M: Optional[int] = None):
    """(ids int32 [M, k], weights float32 [M, k], info dict)."""
    logits, info = make_logits(wl, route_set, M)
    ids, w = topk_softmax(logits, wl.top_k)
    info["unique_experts"] = int(len(np.unique(ids)))
    counts = np.bincount(ids.ravel(), minlength=wl.experts)
    info["max_load"] = int(counts.max())
    info["mean_load"] = float(counts[counts > 0].mean())
    return ids, w, info
