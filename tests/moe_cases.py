"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads
from fp4_block_scaled_amd import binding as B
from fp4_block_scaled_amd.layer import MoeLayer

MAX_ERR_FRAC = 2e-3     # max |gpu - ref| <= 2e-3 * max |ref|
REL_L2 = 1e-3           # ||gpu - ref||_2 / ||ref||_2 <= 1e-3


def check_fp(gpu: np.ndarray, ref: np.ndarray, what: str, max_frac=MAX_ERR_FRAC, rel_l2=REL_L2):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    scale = np.abs(ref).max()
    err = np.abs(gpu - ref)
    l2 = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300)
    assert err.max() <= max_frac * scale, f"{what}: max err {err.max():.3e} > {max_frac} * {scale:.3e}"
    assert l2 <= rel_l2, f"{what}: rel L2 {l2:.3e} > {rel_l2}"
    return float(err.max() / max(scale, 1e-300)), float(l2)


def host_bank(dev_bank: workloads.DeviceBank, experts) -> oracle.Bank:
    """Copy the listed experts of a device bank to the host (oracle input)."""
    sub = dev_bank.select(experts)
    return oracle.Bank(sub.fmt, sub.codes.cpu().numpy(), sub.scales.cpu().numpy(),
                       None if sub.scale2 is None else sub.scale2.cpu().numpy())


def x_bits(x: torch.Tensor) -> np.ndarray:
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_layer(banks, x: torch.Tensor, ids: np.ndarray, w: np.ndarray, limit: float,
                 act_fp8: bool, tokens=None):
    """Oracle out rows (FP64) for `tokens` (default all) and y per flat slot
    of those tokens.  Only the experts those tokens select are copied."""
    M, k = ids.shape
    E = banks[0].num_experts
    tokens = np.arange(M) if tokens is None else np.asarray(tokens)
    sel = ids[tokens]
    valid = (sel >= 0) & (sel < E)
    used = np.unique(sel[valid])
    hb = [host_bank(b, used) for b in banks]
    remap = np.full(sel.shape, -1, np.int32)
    remap[valid] = np.searchsorted(used, sel[valid]).astype(np.int32)
    remap[~valid] = np.where(sel[~valid] == -1, -1, len(used) + 7)  # keep invalid invalid
    xb = x_bits(x)[tokens]
    res = oracle.expert_slots(hb[0], hb[1], hb[2], xb, remap, limit, act_fp8)
    out = oracle.combine(res["y"], w[tokens], valid.astype(np.int32).ravel())
    return out, res["y"]


class GpuCase:
    """Banks, x and routes of one workload on the GPU."""

    def __init__(self, wl: workloads.Workload, device="cuda"):
        self.wl = wl
        self.banks = workloads.make_banks(wl, device)
        self.x = workloads.make_x(wl, device)
        self.cbanks = [B.Bank.from_device_bank(b) for b in self.banks]

    def layer(self, max_M=None, mode=B.MOE_MODE_AUTO):
        wl = self.wl
        return MoeLayer(*self.cbanks, wl.hidden, wl.inter, wl.top_k, max_M or wl.M,
                        wl.limit, mode)

    def run(self, ids: np.ndarray, w: np.ndarray, mode=B.MOE_MODE_AUTO, x=None, layer=None):
        x = self.x if x is None else x
        L = layer or self.layer(max_M=ids.shape[0], mode=mode)
        ids_d = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
        w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
        out = L(x[: ids.shape[0]], ids_d, w_d)
        torch.cuda.synchronize()
        tabs = {k: v.cpu().numpy() for k, v in L.route_tables().items()}
        return out.cpu().numpy(), L.y.cpu().numpy(), tabs, L
