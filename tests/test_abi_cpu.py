"""The C ABI without a GPU: the library loads, exports every function that
include/moe.h declares, sizes its workspace as documented, resolves tiers,
and rejects bad arguments on the host before launching anything."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    from fp4_block_scaled_amd import binding as B
    names = header_functions()
    assert set(names) == set(B.EXPORTS)
    lib = C.CDLL(os.path.join(ROOT, "fp4_block_scaled_amd", "libmoe.so"))
    for n in names:
        assert hasattr(lib, n), n


def a256(n):
    return (n + 255) // 256 * 256


def test_workspace_bytes_hand_computed():
    from fp4_block_scaled_amd import binding as B
    # decode: H7168 I2048 E256 k8 M=1, E4M3, GEMV tier
    S, E, H, I = 8, 256, 7168, 2048
    route = a256(4 * (E + 1)) + 3 * a256(4 * S) + a256(4 * min(S, E)) + a256(8)
    # h only: both GEMVs cover the whole of K per block
    gemv = a256(4 * S * I)
    assert B.moe_workspace_bytes(1, 8, E, H, I, B.MOE_W_E4M3_B128, B.MOE_MODE_GEMV_A16) == route + gemv
    # NVFP4 M=16: H6144 I1536 E160
    S, E, H, I = 128, 160, 6144, 1536
    route = a256(4 * (E + 1)) + 3 * a256(4 * S) + a256(4 * min(S, E)) + a256(8)
    gemv = a256(4 * S * I)
    assert B.moe_workspace_bytes(16, 8, E, H, I, B.MOE_W_NVFP4_B16, B.MOE_MODE_AUTO) == route + gemv
    # odd shapes need no extra scratch: both GEMVs cover the whole of K
    S, E, H, I = 2, 4, 256, 2304
    route = a256(4 * (E + 1)) + 3 * a256(4 * S) + a256(4 * min(S, E)) + a256(8)
    gemv = a256(4 * S * I)
    assert B.moe_workspace_bytes(1, 2, E, H, I, B.MOE_W_E4M3_B128, B.MOE_MODE_GEMV_A16) == route + gemv
    # prefill, GEMM tier: H7168 I2048 E256 k8 M=4096 -> S=32768 slots; x codes
    # + scales, h codes + scales, at most min(S,E) + S/128 tiles of 16 bytes,
    # and the tile count
    M, S, E, H, I = 4096, 32768, 256, 7168, 2048
    route = a256(4 * (E + 1)) + 3 * a256(4 * S) + a256(4 * min(S, E)) + a256(8)
    tmax = min(S, E) + S // 128
    gemm = (a256(M * H) + a256(4 * M * (H // 128)) + a256(S * I) + a256(4 * S * (I // 128))
            + a256(16 * tmax) + 256)
    assert B.moe_workspace_bytes(M, 8, E, H, I, B.MOE_W_E4M3_B128, B.MOE_MODE_GEMM_A8) == route + gemm
    # monotone in max_M
    sizes = [B.moe_workspace_bytes(m, 8, 256, 7168, 2048, B.MOE_W_E4M3_B128, B.MOE_MODE_GEMV_A16)
             for m in (1, 2, 4, 8, 16)]
    assert sizes == sorted(sizes)


@pytest.mark.parametrize("args", [
    (0, 8, 256, 7168, 2048, 1, 0),      # M = 0
    (1, 0, 256, 7168, 2048, 1, 0),      # top_k = 0
    (1, 9, 8, 7168, 2048, 1, 0),        # top_k > E
    (1, 8, 513, 7168, 2048, 1, 0),      # E > max
    (1, 8, 256, 7100, 2048, 1, 0),      # hidden % 128
    (1, 8, 256, 7168, 2000, 1, 0),      # inter % 128
    (1, 8, 256, 6144, 1664, 2, 0),      # NVFP4 needs % 256
    (1, 8, 256, 7168, 2048, 3, 0),      # unknown format
    (1, 8, 256, 7168, 2048, 1, 7),      # unknown mode
    (64, 8, 256, 16512, 2048, 1, 2),    # hidden > MOE_MAX_DIM
    (1, 8, 256, 7168, 16512, 1, 1),     # inter > MOE_MAX_DIM
    (131072, 8, 256, 16384, 2048, 1, 2),  # GEMM tier: M * hidden = 2^31
    (32768, 8, 256, 7168, 8192, 1, 2),  # GEMM tier: M * top_k * inter = 2^31
])
def test_workspace_bytes_rejects_bad_sizes(args):
    from fp4_block_scaled_amd import binding as B
    assert B.lib.moe_workspace_bytes(*args) == 0


def test_auto_workspace_sizes_the_tier_each_format_runs():
    from fp4_block_scaled_amd import binding as B
    L = B.lib
    # NVFP4 above MOE_GEMV_MAX_M tokens runs the bf16 GEMM tier: route region
    # + max(GEMV scratch for 16 tokens, h FP16 [S][I] + tiles + count)
    M, k, E, H, I = 20, 8, 20, 1024, 512
    S = M * k
    tmax = min(S, E) + (S + 127) // 128
    route = a256(4 * (E + 1)) + 3 * a256(4 * S) + a256(4 * min(S, E)) + a256(8)
    a16 = a256(2 * S * I) + a256(16 * tmax) + 256
    assert L.moe_workspace_bytes(M, k, E, H, I, B.MOE_W_NVFP4_B16, B.MOE_MODE_GEMM_A16) == route + a16
    gemv16 = a256(4 * 16 * k * I)
    assert L.moe_workspace_bytes(M, k, E, H, I, B.MOE_W_NVFP4_B16, B.MOE_MODE_AUTO) == \
        route + max(a16, gemv16)
    # each GEMM tier serves one format
    assert L.moe_workspace_bytes(M, k, E, H, I, B.MOE_W_E4M3_B128, B.MOE_MODE_GEMM_A16) == 0
    assert L.moe_workspace_bytes(M, k, E, H, I, B.MOE_W_NVFP4_B16, B.MOE_MODE_GEMM_A8) == 0
    assert L.moe_workspace_bytes(M, k, E, H, I, B.MOE_W_NVFP4_B16, 5) == 0
    # E4M3 past the FP8 GEMM tier's 32-bit row offsets (M * hidden = 2^31):
    # AUTO sizes the GEMV scratch only
    assert L.moe_workspace_bytes(131072, 1, 256, 16384, 128, B.MOE_W_E4M3_B128, B.MOE_MODE_AUTO) > 0
    assert L.moe_workspace_bytes(131072, 1, 256, 16384, 128, B.MOE_W_E4M3_B128, B.MOE_MODE_GEMM_A8) == 0
    # the bf16 tier's rows are 2 bytes an element: 2^30 elements is the limit
    assert L.moe_workspace_bytes(65536, 1, 256, 16384, 256, B.MOE_W_NVFP4_B16, B.MOE_MODE_GEMM_A16) == 0
    assert L.moe_workspace_bytes(65535, 1, 256, 16384, 256, B.MOE_W_NVFP4_B16, B.MOE_MODE_GEMM_A16) > 0


def test_resolve_mode():
    from fp4_block_scaled_amd import binding as B
    assert B.moe_resolve_mode(1, B.MOE_W_E4M3_B128) == B.MOE_MODE_GEMV_A16
    assert B.moe_resolve_mode(16, B.MOE_W_NVFP4_B16) == B.MOE_MODE_GEMV_A16
    assert B.moe_resolve_mode(17, B.MOE_W_E4M3_B128) == B.MOE_MODE_GEMM_A8
    assert B.moe_resolve_mode(17, B.MOE_W_NVFP4_B16) == B.MOE_MODE_GEMM_A16
    assert B.moe_resolve_mode(4096, B.MOE_W_NVFP4_B16) == B.MOE_MODE_GEMM_A16
    assert B.moe_resolve_mode(8, B.MOE_W_NVFP4_B16, B.MOE_MODE_GEMM_A16) == B.MOE_MODE_GEMM_A16
    assert B.moe_resolve_mode(4096, B.MOE_W_E4M3_B128, B.MOE_MODE_GEMV_A16) == B.MOE_MODE_GEMV_A16


# Fake device addresses: the checks below fail before anything is launched or
# dereferenced, so no GPU is needed.
FAKE = 0x7F0000000000


def _bank(B, fmt=1, E=16, n=128, k=256, scale2=None, codes=FAKE):
    return B.moe_bank_t(fmt, E, n, k, codes, FAKE + 0x1000, scale2)


def _route(B, ws, M=1, k=4, E=16):
    r = B.moe_route_t()
    r.M, r.top_k, r.num_experts, r.num_slots = M, k, E, M * k
    r.expert_offsets = ws
    r.token_to_perm = ws + 0x400
    return r


def _ffn(B, gate, up, down, route, ws, hidden=256, inter=128, mode=0, limit=7.0,
         ws_bytes=1 << 30, x=FAKE + 0x2000, y=FAKE + 0x3000):
    return B.lib.moe_expert_ffn(C.byref(gate), C.byref(up), C.byref(down), x, C.byref(route),
                                hidden, inter, limit, mode, y, ws, ws_bytes, None)


def test_ffn_error_contract_on_host():
    from fp4_block_scaled_amd import binding as B
    ws = FAKE + 0x100000
    g, u, d = _bank(B), _bank(B), _bank(B, n=256, k=128)
    r = _route(B, ws)
    # null pointers
    assert B.lib.moe_expert_ffn(None, C.byref(u), C.byref(d), FAKE, C.byref(r), 256, 128, 7.0, 0,
                                FAKE, ws, 1 << 30, None) == B.MOE_ERR_ARG
    assert _ffn(B, g, u, d, r, ws, x=None) == B.MOE_ERR_ARG
    assert "null" in B.moe_last_error()
    # shapes
    assert _ffn(B, g, u, d, r, ws, hidden=200) == B.MOE_ERR_SHAPE
    assert _ffn(B, g, u, _bank(B, n=128, k=128), r, ws) == B.MOE_ERR_SHAPE
    assert _ffn(B, _bank(B, E=8), u, d, r, ws) == B.MOE_ERR_SHAPE
    # formats
    assert _ffn(B, g, _bank(B, fmt=2, scale2=FAKE), d, r, ws) == B.MOE_ERR_FORMAT
    assert _ffn(B, _bank(B, scale2=FAKE), u, d, r, ws) == B.MOE_ERR_FORMAT
    assert _ffn(B, _bank(B, fmt=9), u, d, r, ws) == B.MOE_ERR_FORMAT
    assert _ffn(B, _bank(B, fmt=2, k=256, n=256), _bank(B, fmt=2, k=256, n=256),
                _bank(B, fmt=2, n=256, k=256), r, ws, hidden=256, inter=256) == B.MOE_ERR_FORMAT
    # workspace too small
    assert _ffn(B, g, u, d, r, ws, ws_bytes=512) == B.MOE_ERR_WORKSPACE
    # route not from this workspace
    assert _ffn(B, g, u, d, _route(B, ws + 256), ws) == B.MOE_ERR_ARG
    # misaligned codes
    assert _ffn(B, _bank(B, codes=FAKE + 3), u, d, r, ws) == B.MOE_ERR_ARG
    # bad limit, unknown mode
    assert _ffn(B, g, u, d, r, ws, limit=0.0) == B.MOE_ERR_ARG
    assert _ffn(B, g, u, d, r, ws, mode=5) == B.MOE_ERR_ARG
    # each GEMM tier serves one format; the bf16 tier reads scales as dwords
    assert _ffn(B, g, u, d, r, ws, mode=B.MOE_MODE_GEMM_A16) == B.MOE_ERR_UNSUPPORTED
    nv = _bank(B, fmt=2, k=256, n=256, scale2=FAKE)
    assert _ffn(B, nv, nv, nv, r, ws, hidden=256, inter=256,
                mode=B.MOE_MODE_GEMM_A8) == B.MOE_ERR_UNSUPPORTED
    odd = B.moe_bank_t(2, 16, 256, 256, FAKE, FAKE + 0x1002, FAKE)
    assert _ffn(B, nv, odd, nv, r, ws, hidden=256, inter=256,
                mode=B.MOE_MODE_GEMM_A16) == B.MOE_ERR_ARG
    assert "4-byte" in B.moe_last_error()
    # hidden beyond MOE_MAX_DIM, any tier
    big = 16512
    rg = _route(B, ws, M=32)
    assert _ffn(B, _bank(B, n=128, k=big), _bank(B, n=128, k=big), _bank(B, n=big, k=128), rg, ws,
                hidden=big, inter=128, mode=2) == B.MOE_ERR_SHAPE
    assert "at most 16384" in B.moe_last_error()


def test_route_pack_and_combine_error_contract_on_host():
    from fp4_block_scaled_amd import binding as B
    ws = FAKE + 0x100000
    r = B.moe_route_t()
    L = B.lib
    assert L.moe_route_pack(None, 1, 4, 16, ws, 1 << 20, C.byref(r), None) == B.MOE_ERR_ARG
    assert L.moe_route_pack(FAKE, 0, 4, 16, ws, 1 << 20, C.byref(r), None) == B.MOE_ERR_SHAPE
    assert L.moe_route_pack(FAKE, 1, 17, 16, ws, 1 << 20, C.byref(r), None) == B.MOE_ERR_SHAPE
    assert L.moe_route_pack(FAKE, 1, 4, 600, ws, 1 << 20, C.byref(r), None) == B.MOE_ERR_SHAPE
    assert L.moe_route_pack(FAKE, 1, 4, 16, ws, 64, C.byref(r), None) == B.MOE_ERR_WORKSPACE
    assert L.moe_route_pack(FAKE, 1, 4, 16, ws + 8, 1 << 20, C.byref(r), None) == B.MOE_ERR_ARG
    rr = _route(B, ws)
    assert L.moe_combine(None, C.byref(rr), FAKE, 256, FAKE, None) == B.MOE_ERR_ARG
    assert L.moe_combine(FAKE, C.byref(rr), FAKE, 258, FAKE, None) == B.MOE_ERR_SHAPE
    assert L.moe_combine(FAKE + 4, C.byref(rr), FAKE, 256, FAKE, None) == B.MOE_ERR_ARG
    empty = B.moe_route_t()
    empty.token_to_perm = FAKE
    assert L.moe_combine(FAKE, C.byref(empty), FAKE, 256, FAKE, None) == B.MOE_ERR_ARG


def test_fused_workspace_and_error_contract_on_host():
    from fp4_block_scaled_amd import binding as B
    L = B.lib
    # workspace: route region + h [S][I] FP32 + one 32-bit flag per gate/up
    # item (A x I/2, the one-token kernel's 2-row items) and per down item
    # (H/32 x A), A = min(S, E)
    M, k, E, H, I = 1, 8, 256, 7168, 2048
    S = M * k
    route = a256(4 * (E + 1)) + 3 * a256(4 * S) + a256(4 * min(S, E)) + a256(8)
    want = route + a256(4 * S * I) + a256(4 * min(S, E) * (I // 2 + H // 32))
    assert L.moe_workspace_bytes(M, k, E, H, I, B.MOE_W_E4M3_B128, B.MOE_MODE_FUSED) == want
    # NVFP4: one token with hidden a multiple of 2048 (7168 is not)
    assert L.moe_workspace_bytes(M, k, E, H, I, B.MOE_W_NVFP4_B16, B.MOE_MODE_FUSED) == 0
    assert L.moe_workspace_bytes(1, k, E, 6144, 1536, B.MOE_W_NVFP4_B16, B.MOE_MODE_FUSED) == \
        route + a256(4 * S * 1536) + a256(4 * min(S, E) * (1536 // 2 + 6144 // 32))
    assert L.moe_workspace_bytes(2, k, E, 6144, 1536, B.MOE_W_NVFP4_B16, B.MOE_MODE_FUSED) == 0
    assert L.moe_workspace_bytes(33, 8, E, H, I, B.MOE_W_E4M3_B128, B.MOE_MODE_FUSED) == 0
    assert L.moe_workspace_bytes(M, k, E, H, I, B.MOE_W_E4M3_B128, 4) == 0
    assert B.moe_resolve_mode(1, B.MOE_W_E4M3_B128, B.MOE_MODE_FUSED) == B.MOE_MODE_FUSED

    ws = FAKE + 0x100000
    g, u, d = _bank(B), _bank(B), _bank(B, n=256, k=128)
    r = B.moe_route_t()

    def fused(gate=g, up=u, down=d, M=1, k=4, hidden=256, inter=128, ws_=ws, nbytes=1 << 30,
              x=FAKE + 0x2000, limit=7.0):
        return L.moe_layer_fused(C.byref(gate), C.byref(up), C.byref(down), x, FAKE + 0x4000,
                                 FAKE + 0x5000, M, k, hidden, inter, limit, FAKE + 0x3000,
                                 FAKE + 0x6000, ws_, nbytes, C.byref(r), None)

    assert fused(x=None) == B.MOE_ERR_ARG
    assert fused(M=80, k=4) == B.MOE_ERR_SHAPE                 # S = 320 > 256
    assert "256" in B.moe_last_error()
    assert fused(hidden=200) == B.MOE_ERR_SHAPE
    assert fused(gate=_bank(B, E=8)) == B.MOE_ERR_SHAPE
    nv = _bank(B, fmt=2, k=256, n=256, scale2=FAKE)
    assert fused(gate=nv, up=nv, down=_bank(B, fmt=2, n=256, k=256, scale2=FAKE), hidden=256,
                 inter=256) == B.MOE_ERR_UNSUPPORTED
    nv2 = _bank(B, fmt=2, k=2048, n=256, scale2=FAKE)      # hidden 2048 fits, but M = 2 does not
    assert fused(gate=nv2, up=nv2, down=_bank(B, fmt=2, n=2048, k=256, scale2=FAKE), hidden=2048,
                 inter=256, M=2, k=4) == B.MOE_ERR_UNSUPPORTED
    assert "M = 1" in B.moe_last_error()
    assert fused(nbytes=512) == B.MOE_ERR_WORKSPACE
    assert fused(ws_=ws + 64) == B.MOE_ERR_ARG
    assert fused(limit=-1.0) == B.MOE_ERR_ARG
    # moe_expert_ffn points the fused mode at moe_layer_fused
    rr = _route(B, ws)
    assert _ffn(B, g, u, d, rr, ws, mode=B.MOE_MODE_FUSED) == B.MOE_ERR_ARG
    assert "moe_layer_fused" in B.moe_last_error()


def test_router_error_contract_on_host():
    from fp4_block_scaled_amd import binding as B
    L = B.lib
    FAKE = 0x7F0000000000

    def router(logits=FAKE, M=4, E=16, k=4, kind=B.MOE_ROUTER_SOFTMAX, bias=None, scale=1.0,
               renorm=1, ids=FAKE + 0x1000, w=FAKE + 0x2000):
        return L.moe_router_topk(logits, M, E, k, kind, bias, scale, renorm, ids, w, None)

    assert router(logits=None) == B.MOE_ERR_ARG
    assert router(ids=None) == B.MOE_ERR_ARG
    assert router(w=None) == B.MOE_ERR_ARG
    assert router(M=0) == B.MOE_ERR_SHAPE
    assert router(k=0) == B.MOE_ERR_SHAPE
    assert router(k=17) == B.MOE_ERR_SHAPE
    assert router(E=B.MOE_MAX_EXPERTS + 1, k=2) == B.MOE_ERR_SHAPE
    assert router(kind=2) == B.MOE_ERR_ARG
    assert router(bias=FAKE) == B.MOE_ERR_ARG              # softmax takes no bias
    assert "bias" in B.moe_last_error()
    assert router(scale=0.0) == B.MOE_ERR_ARG
    assert router(scale=float("inf")) == B.MOE_ERR_ARG
    assert router(scale=float("nan")) == B.MOE_ERR_ARG
    assert router(renorm=2) == B.MOE_ERR_ARG


def test_shared_expert_workspace_and_error_contract_on_host():
    from fp4_block_scaled_amd import binding as B
    L = B.lib
    # h [M][W] FP32, rounded up to 256 bytes
    assert L.moe_shared_workspace_bytes(1, 7168, 2048) == 4 * 2048
    assert L.moe_shared_workspace_bytes(3, 512, 1536) == a256(4 * 3 * 1536)
    assert L.moe_shared_workspace_bytes(16, 8192, 8192) == 4 * 16 * 8192
    for args in [(0, 512, 512), (17, 512, 512), (1, 500, 512), (1, 512, 1000), (1, 8704, 512),
                 (1, 512, 8704), (1, 0, 512)]:
        assert L.moe_shared_workspace_bytes(*args) == 0, args

    def shared(M=2, H=512, W=512, limit=7.0, ws=FAKE + 0x100000, nbytes=1 << 20, x=FAKE + 0x1000,
               out=FAKE + 0x2000, gate=FAKE + 0x3000):
        return L.moe_shared_expert(gate, FAKE + 0x4000, FAKE + 0x5000, x, M, H, W, limit, out, ws,
                                   nbytes, None)

    assert shared(x=None) == B.MOE_ERR_ARG
    assert shared(out=None) == B.MOE_ERR_ARG
    assert shared(ws=None) == B.MOE_ERR_ARG
    assert shared(M=0) == B.MOE_ERR_SHAPE
    assert shared(M=17) == B.MOE_ERR_UNSUPPORTED
    assert shared(H=640) == B.MOE_ERR_SHAPE
    assert shared(W=8704) == B.MOE_ERR_SHAPE
    assert shared(limit=0.0) == B.MOE_ERR_ARG
    assert shared(limit=float("nan")) == B.MOE_ERR_ARG
    assert shared(gate=FAKE + 0x3008) == B.MOE_ERR_ARG
    assert shared(ws=FAKE + 0x100040) == B.MOE_ERR_ARG
    assert shared(nbytes=4 * 2 * 512 - 4) == B.MOE_ERR_WORKSPACE


def test_combine_residual_error_contract_on_host():
    from fp4_block_scaled_amd import binding as B
    L = B.lib
    rr = _route(B, FAKE + 0x100000)

    def cr(y=FAKE, w=FAKE + 0x1000, sh=None, res=None, H=256, out=FAKE + 0x2000, route=rr):
        return L.moe_combine_residual(y, C.byref(route), w, sh, res, H, out, None)

    assert cr(y=None) == B.MOE_ERR_ARG
    assert cr(w=None) == B.MOE_ERR_ARG
    assert cr(out=None) == B.MOE_ERR_ARG
    assert cr(H=258) == B.MOE_ERR_SHAPE
    assert cr(sh=FAKE + 0x3004) == B.MOE_ERR_ARG
    assert cr(res=FAKE + 0x3008) == B.MOE_ERR_ARG
    empty = B.moe_route_t()
    empty.token_to_perm = FAKE
    assert cr(route=empty) == B.MOE_ERR_ARG


def test_single_call_layer_error_contract_on_host():
    from fp4_block_scaled_amd import binding as B
    L = B.lib
    ws = FAKE + 0x100000
    g, u, d = _bank(B), _bank(B), _bank(B, n=256, k=128)
    r = B.moe_route_t()

    def layer(gate=g, up=u, down=d, M=1, k=4, hidden=256, inter=128, mode=0, ws_=ws,
              nbytes=1 << 30, ids=FAKE + 0x4000, limit=7.0):
        return L.moe_layer(C.byref(gate), C.byref(up), C.byref(down), FAKE + 0x2000, ids,
                           FAKE + 0x5000, M, k, hidden, inter, limit, mode, FAKE + 0x3000,
                           FAKE + 0x6000, ws_, nbytes, C.byref(r), None)

    assert layer(ids=None) == B.MOE_ERR_ARG
    assert layer(k=17) == B.MOE_ERR_SHAPE
    assert layer(mode=B.MOE_MODE_FUSED) == B.MOE_ERR_ARG
    assert layer(mode=7) == B.MOE_ERR_ARG
    assert layer(nbytes=256) == B.MOE_ERR_WORKSPACE            # route region alone is larger
    assert layer(ws_=ws + 64) == B.MOE_ERR_ARG
    assert layer(hidden=200) == B.MOE_ERR_SHAPE                # the FFN's checks apply
    assert layer(limit=0.0) == B.MOE_ERR_ARG
    assert layer(gate=_bank(B, E=8)) == B.MOE_ERR_SHAPE
    # up to 128 slots the route is built in the gate/up launch (its route
    # region is checked first); more take the three calls' path, where the
    # route pack's and FFN's own checks still apply
    assert layer(M=20, k=4, mode=B.MOE_MODE_GEMV_A16, nbytes=600) == B.MOE_ERR_WORKSPACE
    assert layer(M=40, k=4, mode=B.MOE_MODE_GEMV_A16, nbytes=600) == B.MOE_ERR_WORKSPACE
