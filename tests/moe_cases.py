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
        # the kernels read x rows of every token: never hand them fewer rows
        assert x.shape[0] >= ids.shape[0], (x.shape, ids.shape)
        L = layer or self.layer(max_M=ids.shape[0], mode=mode)
        ids_d = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
        w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
        out = L(x[: ids.shape[0]], ids_d, w_d)
        torch.cuda.synchronize()
        tabs = {k: v.cpu().numpy() for k, v in L.route_tables().items()}
        return out.cpu().numpy(), L.y.cpu().numpy(), tabs, L


def _a256(n):
    return (n + 255) // 256 * 256


def route_region_bytes(S, E):
    A = min(S, E)
    return _a256(4 * (E + 1)) + 3 * _a256(4 * S) + _a256(4 * max(A, 1)) + _a256(8)


def gemm_scratch_views(ws: torch.Tensor, M, S, E, hidden, inter):
    """xq, xs, hq, hs of the FP8 GEMM tier inside the workspace (the carving
    order of the library's GEMM scratch: xq, xs, hq, hs, tiles, count)."""
    o = route_region_bytes(S, E)
    xq = ws[o:o + M * hidden].view(M, hidden)
    o += _a256(M * hidden)
    xs = ws[o:o + 4 * M * (hidden // 128)].view(torch.float32).view(M, hidden // 128)
    o += _a256(4 * M * (hidden // 128))
    hq = ws[o:o + S * inter].view(S, inter)
    o += _a256(S * inter)
    hs = ws[o:o + 4 * S * (inter // 128)].view(torch.float32).view(S, inter // 128)
    return xq, xs, hq, hs


# Accuracy of the gate/up sums of the E4M3 GEMM tier, per 128-wide K block,
# relative to the block's largest |w x| term.  The products of E4M3 codes are
# exact on the bf16 MFMA and a block's 128 terms are summed in FP32 (measured
# on MI355X against FP64: at most 3e-6 of the largest term; FP32 rounding of
# 128 terms bounds it by 128 * 2^-24 = 7.6e-6), then promoted with one FP32
# multiply-add.  2e-5 per block is the bound used here.
MFMA_DOT_EPS = 2e-5


def blockmax_sum(w_abs: np.ndarray, x_abs: np.ndarray) -> np.ndarray:
    """For rows x (n, K) and a matrix |W| (N, K): sum over 128-wide K blocks
    of the largest |w_k x_k| in the block -> (n, N)."""
    N, K = w_abs.shape
    Wr = w_abs.reshape(N, K // 128, 128)
    out = np.empty((x_abs.shape[0], N))
    for i in range(x_abs.shape[0]):
        out[i] = (Wr * x_abs[i].reshape(K // 128, 128)[None]).max(axis=2).sum(axis=1)
    return out


def h_error_bound(g, u, g_blk, u_blk, limit, eps=MFMA_DOT_EPS):
    """Bound on |h_gpu - h_exact| when g and u carry absolute errors up to
    dg = eps * g_blk, du = eps * u_blk (g_blk, u_blk from blockmax_sum).
    |silu'| <= 1.1 everywhere; the gate term vanishes once g is surely above
    the cap, the up term once |u| is surely above it."""
    dg, du = eps * g_blk, eps * u_blk
    gc = np.minimum(g, limit)
    silu = gc / (1.0 + np.exp(-gc))
    gate = np.where(g - dg < limit, 1.1 * dg, 0.0) * np.minimum(np.abs(u) + du, limit)
    up = np.where(np.abs(u) - du < limit, (np.abs(silu) + 1.1 * dg) * du, 0.0)
    return gate + up + 1e-6 * np.abs(silu * np.clip(u, -limit, limit))


def check_h_codes(hq_gpu, hs_gpu, h_exact, dh_bound, label):
    """h is re-quantized per 1x128 group from g and u that the GPU accumulates
    on FP8 MFMA, so its rounding decisions are taken on values the oracle
    knows only to within dh_bound (a decision the oracle cannot take in the
    kernel's precision).  Valid: a code between the roundings of v - d and
    v + d, with v = h_exact / scale and d = dh_bound / scale + |v| * (scale
    tolerance) in code units (rounding is monotone).  The group scale must
    agree to the bound of the group's largest element."""
    tab = oracle.e4m3_table()
    hf = h_exact.astype(np.float32)
    q_ref, s_ref = oracle.quant_1x128(hf)
    amax = np.abs(hf.reshape(hf.shape[0], -1, 128)).max(axis=2).astype(np.float64)
    gb = dh_bound.reshape(hf.shape[0], -1, 128).max(axis=2)
    rel = np.abs(hs_gpu.astype(np.float64) / s_ref - 1.0)
    tol = gb / np.maximum(amax, 1e-30) + 1e-6
    assert np.all(rel <= tol), f"{label}: h scales differ by {rel.max():.2e}"
    sc = np.repeat(s_ref.astype(np.float64), 128, axis=1)
    v = hf.astype(np.float64) / sc
    d = dh_bound / sc + np.abs(v) * np.repeat(tol, 128, axis=1) + 1e-9
    diff = hq_gpu != q_ref
    idx = np.nonzero(diff)
    if idx[0].size:
        lo = oracle.e4m3_encode((v[idx] - d[idx]).astype(np.float32))
        hi = oracle.e4m3_encode((v[idx] + d[idx]).astype(np.float32))
        gv = tab[hq_gpu[idx]]
        ok = (gv >= tab[lo]) & (gv <= tab[hi])
        assert ok.all(), f"{label}: {int((~ok).sum())} h codes outside the kernel's error bound"
    return float(diff.mean())
