"""MI355X-native routed MoE FFN layer with block-scaled E4M3 / NVFP4 experts.

The computation lives in ``libmoe.so`` (hand-written HIP for gfx950, C ABI in
``include/moe.h``); ``binding`` is its ctypes wrapper and ``layer`` a small
convenience that owns the device buffers one layer call sequence needs."""
from . import binding  # noqa: F401  (loads libmoe.so; raises if it is missing)
from .binding import (MOE_MODE_AUTO, MOE_MODE_GEMM_A8, MOE_MODE_GEMV_A16,  # noqa: F401
                      MOE_W_E4M3_B128, MOE_W_NVFP4_B16, MoeError, moe_combine,
                      moe_expert_ffn, moe_last_error, moe_resolve_mode, moe_route_pack,
                      moe_workspace_bytes)
