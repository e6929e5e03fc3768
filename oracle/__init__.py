"""CPU oracle for the routed MoE FFN layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, loads or calls it, and the two share no
code.  The arithmetic lives in ``moe_oracle.c`` (plain C, FP64, OpenMP over
output rows); this module compiles it with gcc, loads it with ctypes and
marshals numpy arrays.

Every function is pinned by a ``-m "not gpu"`` test to something other than
itself (the pins are listed in each docstring).  No function is "parity
unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

E4M3_B128 = 1
NVFP4_B16 = 2


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", _SRC,
           "-o", _LIB + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB)
        u8, i32, i64, f32, f64 = C.c_uint8, C.c_int32, C.c_int64, C.c_float, C.c_double
        P = C.c_void_p
        L.oracle_e4m3_value.argtypes = [u8]
        L.oracle_e4m3_value.restype = f64
        L.oracle_e2m1_value.argtypes = [u8]
        L.oracle_e2m1_value.restype = f64
        L.oracle_bf16_value.argtypes = [C.c_uint16]
        L.oracle_bf16_value.restype = f64
        L.oracle_e4m3_encode.argtypes = [f32]
        L.oracle_e4m3_encode.restype = u8
        L.oracle_quant_1x128.argtypes = [P, i64, i64, P, P]
        L.oracle_quant_1x128.restype = None
        L.oracle_route_pack.argtypes = [P, i32, i32, i32, P, P, P, P, P, P]
        L.oracle_route_pack.restype = C.c_int
        L.oracle_dequant_expert.argtypes = [C.POINTER(_Bank), i32, P]
        L.oracle_dequant_expert.restype = None
        L.oracle_swiglu_clamp.argtypes = [f64, f64, f64]
        L.oracle_swiglu_clamp.restype = f64
        L.oracle_expert_slots.argtypes = [C.POINTER(_Bank)] * 3 + [
            P, P, i32, i32, i32, i32, f32, i32, P, i32, P, P, P, P]
        L.oracle_expert_slots.restype = None
        L.oracle_combine.argtypes = [P, P, P, i32, i32, i32, P]
        L.oracle_router_topk.argtypes = [P, i32, i32, i32, i32, P, f32, i32, P, P]
        L.oracle_router_topk.restype = i32
        L.oracle_shared_expert.argtypes = [P, P, P, P, i32, i32, i32, f32, P]
        L.oracle_shared_expert.restype = None
        L.oracle_combine_residual.argtypes = [P, P, P, P, P, i32, i32, i32, P]
        L.oracle_combine_residual.restype = None
        L.oracle_combine.restype = None
        _lib = L
    return _lib


class _Bank(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("num_experts", C.c_int32),
                ("n_out", C.c_int32), ("k_in", C.c_int32),
                ("codes", C.c_void_p), ("scales", C.c_void_p),
                ("scale2", C.c_void_p)]


@dataclass
class Bank:
    """Host copy of one projection bank for all experts (expert-major).

    E4M3: codes uint8 [E, n, k]; scales float32 [E, n/128, k/128]; scale2 None.
    NVFP4: codes uint8 [E, n, k/2] (low nibble = even k); scales uint8 E4M3
    [E, n, k/16]; scale2 float32 [E].
    """
    fmt: int
    codes: np.ndarray
    scales: np.ndarray
    scale2: Optional[np.ndarray] = None

    @property
    def num_experts(self) -> int:
        return int(self.codes.shape[0])

    @property
    def n_out(self) -> int:
        return int(self.codes.shape[1])

    @property
    def k_in(self) -> int:
        k = int(self.codes.shape[2])
        return k * 2 if self.fmt == NVFP4_B16 else k

    def _c(self) -> _Bank:
        self.codes = np.ascontiguousarray(self.codes, dtype=np.uint8)
        if self.fmt == E4M3_B128:
            self.scales = np.ascontiguousarray(self.scales, dtype=np.float32)
        else:
            self.scales = np.ascontiguousarray(self.scales, dtype=np.uint8)
            self.scale2 = np.ascontiguousarray(self.scale2, dtype=np.float32)
        return _Bank(self.fmt, self.num_experts, self.n_out, self.k_in,
                     self.codes.ctypes.data, self.scales.ctypes.data,
                     None if self.scale2 is None else self.scale2.ctypes.data)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# --------------------------------------------------------------------------
# code tables
# --------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """E4M3FN decode.  Pinned: table invariants and torch.float8_e4m3fn."""
    return lib().oracle_e4m3_value(int(code))


def e2m1_value(nib: int) -> float:
    """E2M1 decode.  Pinned: the 16 OCP values and torch's FP4 packing."""
    return lib().oracle_e2m1_value(int(nib))


def e4m3_table() -> np.ndarray:
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e2m1_table() -> np.ndarray:
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def bf16_value(bits: int) -> float:
    return lib().oracle_bf16_value(int(bits))


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """binary32 -> E4M3FN, RNE, saturating.  Pinned: torch's float8 cast."""
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    f = lib().oracle_e4m3_encode
    return np.array([f(float(x)) for x in v], dtype=np.uint8)


def quant_1x128(x: np.ndarray):
    """Per 1x128 group E4M3 quantization.  Returns (codes uint8, scales f32).

    Pinned: exhaustive bf16 sweep against the half-ulp bound and against
    torch's float8 cast of x / scale."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((rows, cols // 128), dtype=np.float32)
    lib().oracle_quant_1x128(_ptr(x), rows, cols, _ptr(q), _ptr(s))
    return q, s


# --------------------------------------------------------------------------
# route pack
# --------------------------------------------------------------------------

def route_pack(ids: np.ndarray, num_experts: int) -> dict:
    """Stable counting sort of route slots by expert.

    Pinned: brute-force sort by (id, slot) and the pages' route fixtures."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    M, k = ids.shape
    S = M * k
    E = num_experts
    offsets = np.zeros(E + 1, np.int32)
    sorted_slot = np.full(S, -1, np.int32)
    sorted_token = np.full(S, -1, np.int32)
    token_to_perm = np.full(S, -1, np.int32)
    active = np.full(max(1, min(E, S)), -1, np.int32)
    num_active = np.zeros(1, np.int32)
    invalid = lib().oracle_route_pack(_ptr(ids), M, k, E, _ptr(offsets),
                                      _ptr(sorted_slot), _ptr(sorted_token),
                                      _ptr(token_to_perm), _ptr(active),
                                      _ptr(num_active))
    nv = int(offsets[E])
    na = int(num_active[0])
    return dict(expert_offsets=offsets, sorted_slot=sorted_slot[:nv],
                sorted_token=sorted_token[:nv], token_to_perm=token_to_perm,
                active_experts=active[:na], num_active=na, invalid=invalid)


# --------------------------------------------------------------------------
# FFN
# --------------------------------------------------------------------------

def dequant_expert(bank: Bank, e: int) -> np.ndarray:
    """Dense FP64 copy of one expert matrix [n, k].

    Pinned: torch float8/float4 decode + numpy scale broadcast."""
    out = np.empty((bank.n_out, bank.k_in), np.float64)
    cb = bank._c()
    lib().oracle_dequant_expert(C.byref(cb), int(e), _ptr(out))
    return out


def swiglu_clamp(g: float, u: float, limit: float) -> float:
    """silu(min(g, L)) * clamp(u, -L, L).  Pinned: closed forms."""
    return lib().oracle_swiglu_clamp(float(g), float(u), float(limit))


def expert_slots(gate: Bank, up: Bank, down: Bank, x_bf16: np.ndarray,
                 ids: np.ndarray, limit: float, act_fp8: bool,
                 slot_list=None, want=("y",)):
    """g, u, h [n, inter] and y [n, hidden] (FP64) for the listed flat slots.

    Pinned: hand-worked diagonal 2x2 experts, numpy FP64 matmul of the
    dequantized experts, integer special case, dense top-1 reduction."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    M, k = ids.shape
    hidden = x_bf16.shape[1]
    inter = gate.n_out
    if slot_list is None:
        slot_list = np.arange(M * k, dtype=np.int32)
    slot_list = np.ascontiguousarray(slot_list, dtype=np.int32)
    n = len(slot_list)
    outs = {}
    ptrs = []
    for name, width in (("g", inter), ("u", inter), ("h", inter), ("y", hidden)):
        if name in want:
            outs[name] = np.empty((n, width), np.float64)
            ptrs.append(_ptr(outs[name]))
        else:
            ptrs.append(None)
    cg, cu, cd = gate._c(), up._c(), down._c()
    lib().oracle_expert_slots(C.byref(cg), C.byref(cu), C.byref(cd),
                              _ptr(x_bf16), _ptr(ids), M, k, hidden, inter,
                              float(limit), int(bool(act_fp8)), _ptr(slot_list),
                              n, *ptrs)
    return outs


def combine(y_by_slot: np.ndarray, w: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """out[t] = sum_j w[t, j] * y[t*k + j] in slot order.

    Pinned: the pages' worked combine example and linearity."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    M, k = w.shape
    y_by_slot = np.ascontiguousarray(y_by_slot, dtype=np.float64)
    hidden = y_by_slot.shape[1]
    valid = np.ascontiguousarray(valid, dtype=np.int32)
    out = np.empty((M, hidden), np.float64)
    lib().oracle_combine(_ptr(y_by_slot), _ptr(w), _ptr(valid), M, k, hidden,
                         _ptr(out))
    return out


def moe_layer(gate: Bank, up: Bank, down: Bank, x_bf16: np.ndarray,
              ids: np.ndarray, w: np.ndarray, limit: float, act_fp8: bool):
    """The whole layer for every token: returns (out [M, hidden] FP64, y)."""
    M, k = ids.shape
    E = gate.num_experts
    res = expert_slots(gate, up, down, x_bf16, ids, limit, act_fp8)
    valid = ((ids >= 0) & (ids < E)).astype(np.int32).ravel()
    return combine(res["y"], w, valid), res["y"]


# --------------------------------------------------------------------------
# router
# --------------------------------------------------------------------------

ROUTER_SOFTMAX = 0
ROUTER_SIGMOID = 1


def router_topk(logits: np.ndarray, top_k: int, kind: int = ROUTER_SOFTMAX,
                bias: Optional[np.ndarray] = None, routed_scale: float = 1.0,
                renormalize: bool = True):
    """(ids int32 [M, k], weights float32 [M, k]) of the softmax or sigmoid
    top-k router on binary32 logits [M, E].

    Pinned: a brute-force ranking of the keys in numpy, scipy's softmax and
    logistic functions on the chosen experts, hand-worked rows where the
    selection bias changes the choice, ties, and non-finite logits."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    M, E = logits.shape
    ids = np.empty((M, top_k), np.int32)
    w = np.empty((M, top_k), np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    rc = lib().oracle_router_topk(_ptr(logits), M, E, top_k, kind,
                                  None if b is None else _ptr(b), float(routed_scale),
                                  int(bool(renormalize)), _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_router_topk: bad arguments")
    return ids, w


# --------------------------------------------------------------------------
# shared expert and residual
# --------------------------------------------------------------------------

def shared_expert(gate_bf16: np.ndarray, up_bf16: np.ndarray, down_bf16: np.ndarray,
                  x_bf16: np.ndarray, limit: float) -> np.ndarray:
    """The shared expert's output [M, H] (FP64) for bf16 bit arrays gate, up
    [W, H], down [H, W] and x [M, H].

    Pinned: numpy FP64 matmuls of the bf16-decoded weights, a diagonal MLP
    with a closed form, and zero rows."""
    gate_bf16 = np.ascontiguousarray(gate_bf16, np.uint16)
    up_bf16 = np.ascontiguousarray(up_bf16, np.uint16)
    down_bf16 = np.ascontiguousarray(down_bf16, np.uint16)
    x_bf16 = np.ascontiguousarray(x_bf16, np.uint16)
    W, H = gate_bf16.shape
    M = x_bf16.shape[0]
    assert up_bf16.shape == (W, H) and down_bf16.shape == (H, W) and x_bf16.shape[1] == H
    out = np.empty((M, H), np.float64)
    lib().oracle_shared_expert(_ptr(gate_bf16), _ptr(up_bf16), _ptr(down_bf16), _ptr(x_bf16),
                               M, H, W, float(limit), _ptr(out))
    return out


def combine_residual(y_by_slot: np.ndarray, w: np.ndarray, valid: np.ndarray,
                     shared: Optional[np.ndarray], residual: Optional[np.ndarray]) -> np.ndarray:
    """((sum_j w[t, j] * y[t*k + j]) + shared[t]) + residual[t] (FP64).

    Pinned: the pages' worked combine example extended by hand, reduction
    to the plain combine, and linearity."""
    w = np.ascontiguousarray(w, np.float32)
    M, k = w.shape
    y_by_slot = np.ascontiguousarray(y_by_slot, np.float64)
    hidden = y_by_slot.shape[1]
    valid = np.ascontiguousarray(valid, np.int32).reshape(-1)
    sh = None if shared is None else np.ascontiguousarray(shared, np.float64)
    rs = None if residual is None else np.ascontiguousarray(residual, np.float32)
    out = np.empty((M, hidden), np.float64)
    lib().oracle_combine_residual(_ptr(y_by_slot), _ptr(w), _ptr(valid),
                                  None if sh is None else _ptr(sh),
                                  None if rs is None else _ptr(rs), M, k, hidden, _ptr(out))
    return out
