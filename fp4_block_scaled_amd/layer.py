"""Device buffers for one routed-MoE layer call sequence (plumbing only).

Allocates the workspace, packed-y and output tensors once for a maximum M and
runs the layer on the current stream: moe_layer (route pack, expert FFN and
combine in one call), or moe_route_pack -> moe_expert_ffn -> moe_combine as
three calls with single_call=False, or moe_layer_fused (one launch) when
built with mode MOE_MODE_FUSED.  No arithmetic happens here."""
from __future__ import annotations

import torch

from . import binding as B


class MoeLayer:
    def __init__(self, gate: B.Bank, up: B.Bank, down: B.Bank, hidden: int, inter: int,
                 top_k: int, max_M: int, limit: float = 7.0, mode: int = B.MOE_MODE_AUTO,
                 device="cuda", single_call: bool = True):
        self.gate, self.up, self.down = gate, up, down
        self.hidden, self.inter, self.top_k = hidden, inter, top_k
        self.E = gate.c.num_experts
        self.fmt = gate.c.fmt
        self.limit, self.mode = limit, mode
        self.max_M = max_M
        self.single_call = single_call
        nbytes = B.moe_workspace_bytes(max_M, top_k, self.E, hidden, inter, self.fmt, mode)
        if nbytes == 0:
            raise B.MoeError(B.MOE_ERR_SHAPE, "moe_workspace_bytes rejected the sizes")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.y = torch.empty((max_M * top_k, hidden), dtype=torch.float32, device=device)
        self.out = torch.empty((max_M, hidden), dtype=torch.float32, device=device)
        self.route = None

    def __call__(self, x_bf16, ids, weights, stream=None):
        M = int(ids.shape[0])
        assert M <= self.max_M and int(ids.shape[1]) == self.top_k
        if self.mode == B.MOE_MODE_FUSED:
            self.route = B.moe_layer_fused(self.gate, self.up, self.down, x_bf16, ids, weights, M,
                                           self.top_k, self.hidden, self.inter, self.limit, self.y,
                                           self.out, self.ws, stream=stream)
            return self.out[:M]
        if self.single_call:
            self.route = B.moe_layer(self.gate, self.up, self.down, x_bf16, ids, weights, M,
                                     self.top_k, self.hidden, self.inter, self.limit, self.mode,
                                     self.y, self.out, self.ws, stream=stream)
            return self.out[:M]
        self.route = B.moe_route_pack(ids, M, self.top_k, self.E, self.ws, stream=stream)
        B.moe_expert_ffn(self.gate, self.up, self.down, x_bf16, self.route, self.hidden,
                         self.inter, self.limit, self.mode, self.y, self.ws, stream=stream)
        B.moe_combine(self.y, self.route, weights, self.hidden, self.out, stream=stream)
        return self.out[:M]

    def route_tables(self):
        return B.route_tensors(self.route, self.ws)
