"""Thin ctypes binding of libmoe (include/moe.h), same names as the C ABI.

Argument marshalling only: torch tensors are passed as device pointers and
the current HIP stream; every step of the layer runs in libmoe's kernels.
Importing this module loads ``libmoe.so`` and fails loudly if it is missing
or cannot be loaded -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
MOE_ERR_ARG = 1
MOE_ERR_SHAPE = 2
MOE_ERR_FORMAT = 3
MOE_ERR_WORKSPACE = 4
MOE_ERR_HIP = 5
MOE_ERR_UNSUPPORTED = 6

MOE_W_E4M3_B128 = 1
MOE_W_NVFP4_B16 = 2

MOE_MODE_AUTO = 0
MOE_MODE_GEMV_A16 = 1
MOE_MODE_GEMM_A8 = 2
MOE_MODE_FUSED = 3
MOE_MODE_GEMM_A16 = 4

MOE_ROUTER_SOFTMAX = 0
MOE_ROUTER_SIGMOID = 1

MOE_GEMV_MAX_M = 16
MOE_STATIC_SCRATCH_BYTES = 8 << 20
MOE_MAX_EXPERTS = 512
MOE_MAX_DIM = 16384
MOE_FUSED_MAX_SLOTS = 256

EXPORTS = ("moe_workspace_bytes", "moe_resolve_mode", "moe_router_topk", "moe_route_pack",
           "moe_expert_ffn", "moe_layer", "moe_layer_static", "moe_layer_fused", "moe_combine",
           "moe_shared_workspace_bytes",
           "moe_shared_expert", "moe_combine_residual", "moe_set_stage_events", "moe_last_error")


class moe_bank_t(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("num_experts", C.c_int32), ("n_out", C.c_int32),
                ("k_in", C.c_int32), ("codes", C.c_void_p), ("scales", C.c_void_p),
                ("scale2", C.c_void_p)]


class moe_route_t(C.Structure):
    _fields_ = [("M", C.c_int32), ("top_k", C.c_int32), ("num_experts", C.c_int32),
                ("num_slots", C.c_int32),
                ("expert_offsets", C.c_void_p), ("sorted_slot", C.c_void_p),
                ("sorted_token", C.c_void_p), ("token_to_perm", C.c_void_p),
                ("active_experts", C.c_void_p), ("num_active", C.c_void_p),
                ("status", C.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libmoe status {status}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libmoe.so not built at {_LIB_PATH}; run __graft_entry__.build()")
    L = C.CDLL(_LIB_PATH)
    P, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    L.moe_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.moe_workspace_bytes.restype = sz
    L.moe_resolve_mode.argtypes = [i32, i32, i32]
    L.moe_resolve_mode.restype = i32
    L.moe_router_topk.argtypes = [P, i32, i32, i32, i32, P, C.c_float, i32, P, P, P]
    L.moe_router_topk.restype = i32
    L.moe_route_pack.argtypes = [P, i32, i32, i32, P, sz, C.POINTER(moe_route_t), P]
    L.moe_route_pack.restype = i32
    L.moe_expert_ffn.argtypes = [C.POINTER(moe_bank_t)] * 3 + [
        P, C.POINTER(moe_route_t), i32, i32, C.c_float, i32, P, P, sz, P]
    L.moe_expert_ffn.restype = i32
    L.moe_layer_fused.argtypes = [C.POINTER(moe_bank_t)] * 3 + [
        P, P, P, i32, i32, i32, i32, C.c_float, P, P, P, sz, C.POINTER(moe_route_t), P]
    L.moe_layer_fused.restype = i32
    L.moe_layer.argtypes = [C.POINTER(moe_bank_t)] * 3 + [P, P, P, i32, i32, i32, i32, C.c_float,
                                                         i32, P, P, P, sz, C.POINTER(moe_route_t), P]
    L.moe_layer.restype = i32
    L.moe_layer_static.argtypes = [C.POINTER(moe_bank_t)] * 3 + [P, P, P, i32, i32, i32, i32,
                                                                C.c_float, i32, P, P,
                                                                C.POINTER(moe_route_t), P]
    L.moe_layer_static.restype = i32
    L.moe_combine.argtypes = [P, C.POINTER(moe_route_t), P, i32, P, P]
    L.moe_combine.restype = i32
    L.moe_combine_residual.argtypes = [P, C.POINTER(moe_route_t), P, P, P, i32, P, P]
    L.moe_combine_residual.restype = i32
    L.moe_shared_workspace_bytes.argtypes = [i32, i32, i32]
    L.moe_shared_workspace_bytes.restype = sz
    L.moe_shared_expert.argtypes = [P, P, P, P, i32, i32, i32, C.c_float, P, P, sz, P]
    L.moe_shared_expert.restype = i32
    L.moe_set_stage_events.argtypes = [P, i32, i32, i32, i32, i32]
    L.moe_set_stage_events.restype = i32
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = C.c_char_p
    return L


lib = _load()


def _ptr(t) -> int:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, moe_last_error())


def moe_last_error() -> str:
    return lib.moe_last_error().decode()


def moe_workspace_bytes(max_M, top_k, num_experts, hidden, inter, fmt, mode=MOE_MODE_AUTO) -> int:
    return int(lib.moe_workspace_bytes(max_M, top_k, num_experts, hidden, inter, fmt, mode))


def moe_resolve_mode(M, fmt, requested=MOE_MODE_AUTO) -> int:
    return int(lib.moe_resolve_mode(M, fmt, requested))


class Bank:
    """A moe_bank_t plus references to the tensors it points into."""

    def __init__(self, fmt, codes, scales, scale2=None):
        self.tensors = (codes, scales, scale2)
        E, n = int(codes.shape[0]), int(codes.shape[1])
        k = int(codes.shape[2]) * (2 if fmt == MOE_W_NVFP4_B16 else 1)
        self.c = moe_bank_t(fmt, E, n, k, _ptr(codes), _ptr(scales), _ptr(scale2))

    @classmethod
    def from_device_bank(cls, b):
        return cls(b.fmt, b.codes, b.scales, b.scale2)


def moe_router_topk(logits, M, num_experts, top_k, kind, bias, routed_scale, renormalize,
                    topk_ids, topk_weights, stream=None) -> None:
    _check(lib.moe_router_topk(_ptr(logits), M, num_experts, top_k, kind, _ptr(bias),
                               float(routed_scale), int(renormalize), _ptr(topk_ids),
                               _ptr(topk_weights), _stream(stream)))


def moe_route_pack(topk_ids, M, top_k, num_experts, ws, ws_bytes=None, stream=None) -> moe_route_t:
    route = moe_route_t()
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib.moe_route_pack(_ptr(topk_ids), M, top_k, num_experts, _ptr(ws), nbytes,
                              C.byref(route), _stream(stream)))
    return route


def moe_expert_ffn(gate: Bank, up: Bank, down: Bank, x_bf16, route: moe_route_t, hidden, inter,
                   limit, mode, y_packed, ws, ws_bytes=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib.moe_expert_ffn(C.byref(gate.c), C.byref(up.c), C.byref(down.c), _ptr(x_bf16),
                              C.byref(route), hidden, inter, float(limit), mode, _ptr(y_packed),
                              _ptr(ws), nbytes, _stream(stream)))


def moe_layer(gate: Bank, up: Bank, down: Bank, x_bf16, topk_ids, topk_weights, M, top_k, hidden,
              inter, limit, mode, y_packed, out, ws, ws_bytes=None, stream=None) -> moe_route_t:
    route = moe_route_t()
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib.moe_layer(C.byref(gate.c), C.byref(up.c), C.byref(down.c), _ptr(x_bf16),
                         _ptr(topk_ids), _ptr(topk_weights), M, top_k, hidden, inter, float(limit),
                         mode, _ptr(y_packed), _ptr(out), _ptr(ws), nbytes, C.byref(route),
                         _stream(stream)))
    return route


def moe_layer_static(gate: Bank, up: Bank, down: Bank, x_bf16, topk_ids, topk_weights, M, top_k,
                     hidden, inter, limit, mode, y_packed, out, stream=None) -> moe_route_t:
    route = moe_route_t()
    _check(lib.moe_layer_static(C.byref(gate.c), C.byref(up.c), C.byref(down.c), _ptr(x_bf16),
                                _ptr(topk_ids), _ptr(topk_weights), M, top_k, hidden, inter,
                                float(limit), mode, _ptr(y_packed), _ptr(out), C.byref(route),
                                _stream(stream)))
    return route


def moe_layer_fused(gate: Bank, up: Bank, down: Bank, x_bf16, topk_ids, topk_weights, M, top_k,
                    hidden, inter, limit, y_packed, out, ws, ws_bytes=None,
                    stream=None) -> moe_route_t:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    route = moe_route_t()
    _check(lib.moe_layer_fused(C.byref(gate.c), C.byref(up.c), C.byref(down.c), _ptr(x_bf16),
                               _ptr(topk_ids), _ptr(topk_weights), M, top_k, hidden, inter,
                               float(limit), _ptr(y_packed), _ptr(out), _ptr(ws), nbytes,
                               C.byref(route), _stream(stream)))
    return route


def moe_combine(y_packed, route: moe_route_t, topk_weights, hidden, out, stream=None) -> None:
    _check(lib.moe_combine(_ptr(y_packed), C.byref(route), _ptr(topk_weights), hidden, _ptr(out),
                           _stream(stream)))


def moe_combine_residual(y_packed, route: moe_route_t, topk_weights, shared_out, residual, hidden,
                         out, stream=None) -> None:
    _check(lib.moe_combine_residual(_ptr(y_packed), C.byref(route), _ptr(topk_weights),
                                    _ptr(shared_out), _ptr(residual), hidden, _ptr(out),
                                    _stream(stream)))


def moe_shared_workspace_bytes(max_M, hidden, shared_width) -> int:
    return int(lib.moe_shared_workspace_bytes(max_M, hidden, shared_width))


def moe_shared_expert(gate_bf16, up_bf16, down_bf16, x_bf16, M, hidden, shared_width, limit,
                      shared_out, ws, ws_bytes=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib.moe_shared_expert(_ptr(gate_bf16), _ptr(up_bf16), _ptr(down_bf16), _ptr(x_bf16), M,
                                 hidden, shared_width, float(limit), _ptr(shared_out), _ptr(ws),
                                 nbytes, _stream(stream)))


def moe_set_stage_events(events, fmt, hidden, inter, mode) -> int:
    """events: a ctypes array of hipEvent_t handles (or None to turn off)."""
    if events is None:
        return int(lib.moe_set_stage_events(None, 0, fmt, hidden, inter, mode))
    return int(lib.moe_set_stage_events(C.cast(events, C.c_void_p), len(events), fmt, hidden,
                                        inter, mode))


def route_tensors(route: moe_route_t, ws) -> dict:
    """int32 views of the route tables inside the workspace tensor `ws`."""
    base = ws.data_ptr()
    w32 = ws.view(torch.int32)
    S, E = route.num_slots, route.num_experts
    A = min(S, E)

    def view(ptr, n):
        off = ptr - base
        assert off % 4 == 0 and off >= 0
        return w32[off // 4: off // 4 + n]
    return dict(expert_offsets=view(route.expert_offsets, E + 1),
                sorted_slot=view(route.sorted_slot, S), sorted_token=view(route.sorted_token, S),
                token_to_perm=view(route.token_to_perm, S),
                active_experts=view(route.active_experts, A),
                num_active=view(route.num_active, 1), status=view(route.status, 1))
