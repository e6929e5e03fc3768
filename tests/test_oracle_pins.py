"""Pins for the oracle's layer arithmetic (CPU only).

Each test ties an oracle function to something other than itself: values the
pages print, closed forms, exact integer arithmetic, library routines
(torch's float8 decode, numpy's FP64 matmul, scipy's logistic function), or
invariants that a dropped term, a wrong sign, a wrong index or a transposed
operand would break."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from oracle import Bank, E4M3_B128, NVFP4_B16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
L = 7.0


# --------------------------------------------------------------------------
# independent dequantization (torch float8 decode, numpy broadcast)
# --------------------------------------------------------------------------

def _torch_e4m3(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _e2m1_list():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt"))
            if l.strip() and not l.startswith("#")]
    return np.array([float(v) for _, v in rows], np.float64)


def indep_dense(bank: Bank, e: int) -> np.ndarray:
    if bank.fmt == E4M3_B128:
        w = _torch_e4m3(bank.codes[e])
        s = np.kron(bank.scales[e].astype(np.float64), np.ones((128, 128)))
        return w * s
    byte = bank.codes[e]
    lo, hi = byte & 15, byte >> 4
    nib = np.empty((byte.shape[0], byte.shape[1] * 2), np.uint8)
    nib[:, 0::2] = lo
    nib[:, 1::2] = hi
    vals = _e2m1_list()[nib]
    sc = np.repeat(_torch_e4m3(bank.scales[e]), 16, axis=1)
    return vals * sc * float(bank.scale2[e])


def rand_e4m3_bank(rng, E, n, k):
    z = np.clip(rng.standard_normal((E, n, k)) * 64, -448, 448).astype(np.float32)
    codes = torch.from_numpy(z).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scales = np.exp(-6 + 0.5 * rng.standard_normal((E, n // 128, k // 128))).astype(np.float32)
    return Bank(E4M3_B128, codes, scales)


def rand_nvfp4_bank(rng, E, n, k):
    codes = rng.integers(0, 256, (E, n, k // 2), dtype=np.uint8)
    sc = np.abs(rng.standard_normal((E, n, k // 16))).astype(np.float32)
    scales = torch.from_numpy(sc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return Bank(NVFP4_B16, codes, scales, np.full(E, 1.0 / 448.0, np.float32))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_vals(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def silu_ref(z):
    return z * expit(z)


# --------------------------------------------------------------------------
# dequantization and projections
# --------------------------------------------------------------------------

def test_dequant_e4m3_matches_torch_decode_and_block_broadcast():
    rng = np.random.default_rng(1)
    b = rand_e4m3_bank(rng, 3, 256, 384)
    for e in range(3):
        assert np.array_equal(oracle.dequant_expert(b, e), indep_dense(b, e))


def test_dequant_nvfp4_matches_ocp_values_and_low_nibble_first():
    rng = np.random.default_rng(2)
    b = rand_nvfp4_bank(rng, 2, 128, 256)
    for e in range(2):
        assert np.array_equal(oracle.dequant_expert(b, e), indep_dense(b, e))


def test_nvfp4_nibble_order_hand_case():
    # one row: byte 0 = 0x72 -> element 0 = code 2 (1.0), element 1 = code 7 (6.0)
    codes = np.zeros((1, 128, 64), np.uint8)
    codes[0, 0, 0] = 0x72
    codes[0, 0, 1] = 0x9C  # element 2 = code 12 (-2.0), element 3 = code 9 (-0.5)
    scales = np.full((1, 128, 8), 0x38, np.uint8)  # E4M3 1.0
    b = Bank(NVFP4_B16, codes, scales, np.array([0.5], np.float32))
    w = oracle.dequant_expert(b, 0)
    assert list(w[0, :4]) == [0.5, 3.0, -1.0, -0.25]
    assert np.all(w[0, 4:] == 0) and np.all(w[1:] == 0)


@pytest.mark.parametrize("fmt", [E4M3_B128, NVFP4_B16])
def test_projections_match_numpy_fp64_matmul(fmt):
    rng = np.random.default_rng(3 + fmt)
    E, H, I, M, k = 4, 384, 256, 3, 2
    mk = rand_e4m3_bank if fmt == E4M3_B128 else rand_nvfp4_bank
    gate, up, down = mk(rng, E, I, H), mk(rng, E, I, H), mk(rng, E, H, I)
    x = bf16_bits(rng.uniform(-2, 2, (M, H)))
    ids = np.array([[0, 3], [2, 0], [1, 2]], np.int32)
    res = oracle.expert_slots(gate, up, down, x, ids, L, False, want=("g", "u", "h", "y"))
    xv = bf16_vals(x)
    for s in range(M * k):
        t, e = s // k, ids.flat[s]
        g = indep_dense(gate, e) @ xv[t]
        u = indep_dense(up, e) @ xv[t]
        h = silu_ref(np.minimum(g, L)) * np.clip(u, -L, L)
        y = indep_dense(down, e) @ h
        np.testing.assert_allclose(res["g"][s], g, rtol=1e-12, atol=1e-12 * np.abs(g).max())
        np.testing.assert_allclose(res["u"][s], u, rtol=1e-12, atol=1e-12 * np.abs(u).max())
        np.testing.assert_allclose(res["h"][s], h, rtol=1e-12, atol=1e-12 * np.abs(h).max())
        np.testing.assert_allclose(res["y"][s], y, rtol=1e-11, atol=1e-11 * np.abs(y).max())


def test_projection_integer_case_is_exact():
    # integer-valued E4M3 codes, power-of-two block scales, small-integer x:
    # every product and sum is a dyadic rational far inside FP64, so the
    # oracle must equal exact rational arithmetic bit for bit.
    rng = np.random.default_rng(7)
    E, H, I = 2, 256, 128
    ints = np.array([-8, -6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 5, 6, 7, 8], np.float32)

    def bank(n, k):
        vals = rng.choice(ints, (E, n, k))
        codes = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        exps = rng.integers(-3, 4, (E, n // 128, k // 128))
        return Bank(E4M3_B128, codes, (2.0 ** exps).astype(np.float32)), vals, exps

    (gate, gv, ge), (up, uv, ue) = bank(I, H), bank(I, H)
    down, dv, de = bank(H, I)
    xi = rng.integers(-3, 4, (1, H)).astype(np.float32)
    ids = np.array([[1, 0]], np.int32)
    res = oracle.expert_slots(gate, up, down, bf16_bits(xi), ids, 1e30, False, want=("g", "u"))
    for s, e in enumerate(ids[0]):
        for n in range(0, I, 17):
            exact_g = sum(Fraction(int(gv[e, n, kk])) * Fraction(2) ** int(ge[e, n // 128, kk // 128])
                          * int(xi[0, kk]) for kk in range(H))
            exact_u = sum(Fraction(int(uv[e, n, kk])) * Fraction(2) ** int(ue[e, n // 128, kk // 128])
                          * int(xi[0, kk]) for kk in range(H))
            assert res["g"][s, n] == float(exact_g)
            assert res["u"][s, n] == float(exact_u)


# --------------------------------------------------------------------------
# SwiGLU closed forms
# --------------------------------------------------------------------------

def test_swiglu_closed_forms():
    f = oracle.swiglu_clamp
    # gate saturates at L: h = L * sigmoid(L) * clamp(u)
    for g in (7.0, 7.5, 100.0, 1e300):
        assert f(g, 1.0, L) == pytest.approx(7.0 * expit(7.0), rel=1e-15)
    assert 7.0 * expit(7.0) == pytest.approx(6.993622641639196, rel=1e-14)
    # up clamps symmetrically
    assert f(7.0, 50.0, L) == pytest.approx(7.0 * expit(7.0) * 7.0, rel=1e-15)
    assert f(7.0, -50.0, L) == pytest.approx(-7.0 * expit(7.0) * 7.0, rel=1e-15)
    # zeros
    assert f(0.0, 3.0, L) == 0.0
    assert f(2.0, 0.0, L) == 0.0
    # gate is NOT clamped from below (the clamp is asymmetric)
    assert f(-20.0, 1.0, L) == pytest.approx(silu_ref(-20.0), rel=1e-12)
    # odd in u, and plain silu(g) * u when the limit is out of reach
    rng = np.random.default_rng(0)
    for g, u in rng.uniform(-6, 6, (200, 2)):
        assert f(g, u, L) == -f(g, -u, L)
        assert f(g, u, 1e9) == pytest.approx(silu_ref(g) * u, rel=1e-14, abs=1e-300)
        assert f(g, u, L) == pytest.approx(silu_ref(min(g, L)) * np.clip(u, -L, L), rel=1e-14, abs=1e-300)
    assert f(1.0, 1.0, L) == pytest.approx(0.7310585786300049, rel=1e-15)  # sigmoid(1)


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

def _read_combine_golden():
    sec, data = None, {}
    for line in open(os.path.join(GOLDEN, "combine_worked_example.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        if parts[0] in ("top_k", "width"):
            data[parts[0]] = int(parts[1])
        elif len(parts) == 1:
            sec = parts[0]
            data[sec] = []
        else:
            data[sec].append([float(p) for p in parts])
    return data


def test_combine_worked_example_from_the_page():
    d = _read_combine_golden()
    k, width = d["top_k"], d["width"]
    y = np.array(d["down_rows"], np.float64)
    w = np.array(d["weights"], np.float32).reshape(1, k)
    out = oracle.combine(y, w, np.ones(k, np.int32))
    assert out.shape == (1, width)
    assert list(out[0]) == d["expected"][0]


def test_combine_linearity_and_partition_of_unity():
    rng = np.random.default_rng(4)
    M, k, H = 5, 4, 33
    y1, y2 = rng.standard_normal((M * k, H)), rng.standard_normal((M * k, H))
    w = rng.uniform(0, 1, (M, k)).astype(np.float32)
    v = np.ones(M * k, np.int32)
    a = 0.375
    lhs = oracle.combine(a * y1 + y2, w, v)
    rhs = a * oracle.combine(y1, w, v) + oracle.combine(y2, w, v)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13, atol=1e-13)
    # equal rows and weights summing to one give the row back
    row = rng.standard_normal(H)
    yy = np.tile(row, (M * k, 1))
    ww = np.tile(np.array([0.5, 0.25, 0.125, 0.125], np.float32), (M, 1))
    np.testing.assert_allclose(oracle.combine(yy, ww, v), np.tile(row, (M, 1)), rtol=1e-15)
    # invalid slots drop out
    v2 = v.copy()
    v2[1] = 0
    ref = oracle.combine(y1, w, v) - (w[0, 1].astype(np.float64) * y1[1])[None, :] * (np.arange(M) == 0)[:, None]
    np.testing.assert_allclose(oracle.combine(y1, w, v2), ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------

def _diag_bank(E, coeff_codes, exps):
    codes = np.zeros((E, 128, 128), np.uint8)
    for e in range(E):
        np.fill_diagonal(codes[e], coeff_codes[e])
    scales = np.array([[[2.0 ** exps[e]]] for e in range(E)], np.float32)
    return Bank(E4M3_B128, codes, scales)


def test_hand_worked_two_experts_two_tokens():
    # Diagonal experts W[n][K] = c * 2^p * delta(n, K), so every projection is
    # elementwise and each output can be written down by hand:
    #   expert 0: gate 2.0 (code 0x40) * 2^0, up 1.0 (0x38) * 2^1, down -1.5 (0xBC) * 2^-1
    #   expert 1: gate 0.5 (0x30) * 2^2, up -1.0 (0xB8) * 2^0, down 1.0 (0x38) * 2^-2
    gate = _diag_bank(2, [0x40, 0x30], [0, 2])
    up = _diag_bank(2, [0x38, 0xB8], [1, 0])
    down = _diag_bank(2, [0xBC, 0x38], [-1, -2])
    x = np.zeros((2, 128), np.float32)
    x[0, :4] = [1.0, 4.0, -0.5, 0.0]
    x[1, :4] = [3.0, -8.0, 0.25, 2.0]
    ids = np.array([[0, 1], [1, 0]], np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5]], np.float32)
    out, y = oracle.moe_layer(gate, up, down, bf16_bits(x), ids, w, L, False)
    s = expit
    # token 0 (x = [1, 4, -0.5, 0]), expert 0: g = 2x = [2, 8, -1, 0], u = 2x
    #   h = [silu(2)*2, silu(7)*7, silu(-1)*(-1), 0]  (g = 8 clamps to 7, u = 8 to 7)
    h00 = np.array([4 * s(2), 49 * s(7), s(-1), 0.0])
    # token 0, expert 1: g = 2x = [2, 8, -1, 0], u = -x = [-1, -4, 0.5, 0]
    h01 = np.array([-2 * s(2), -28 * s(7), -0.5 * s(-1), 0.0])
    # token 1 (x = [3, -8, 0.25, 2]), expert 1: g = [6, -16, 0.5, 4], u = [-3, 8 -> 7, -0.25, -2]
    h11 = np.array([-18 * s(6), -112 * s(-16), -0.125 * s(0.5), -8 * s(4)])
    # token 1, expert 0: g = [6, -16, 0.5, 4], u = [6, -16 -> -7, 0.5, 4]
    h10 = np.array([36 * s(6), 112 * s(-16), 0.25 * s(0.5), 16 * s(4)])
    exp_y = {0: -0.75 * h00, 1: 0.25 * h01, 2: 0.25 * h11, 3: -0.75 * h10}
    for slot, yy in exp_y.items():
        np.testing.assert_allclose(y[slot, :4], yy, rtol=1e-14, atol=1e-15)
        assert np.all(y[slot, 4:] == 0)
    np.testing.assert_allclose(out[0, :4], 0.75 * exp_y[0] + 0.25 * exp_y[1], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(out[1, :4], 0.5 * exp_y[2] + 0.5 * exp_y[3], rtol=1e-14, atol=1e-15)


def test_top1_weight1_is_one_dense_ffn_and_invariances():
    rng = np.random.default_rng(11)
    E, H, I, M = 5, 256, 128, 4
    gate, up, down = rand_e4m3_bank(rng, E, I, H), rand_e4m3_bank(rng, E, I, H), rand_e4m3_bank(rng, E, H, I)
    x = bf16_bits(rng.standard_normal((M, H)))
    xv = bf16_vals(x)
    ids1 = np.array([[2], [0], [4], [2]], np.int32)
    out, _ = oracle.moe_layer(gate, up, down, x, ids1, np.ones((M, 1), np.float32), L, False)
    for t in range(M):
        e = ids1[t, 0]
        g = indep_dense(gate, e) @ xv[t]
        u = indep_dense(up, e) @ xv[t]
        ref = indep_dense(down, e) @ (silu_ref(np.minimum(g, L)) * np.clip(u, -L, L))
        np.testing.assert_allclose(out[t], ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())
    # top-2 layer: relabelling experts, permuting tokens, duplicating tokens
    ids = np.array([[2, 0], [1, 4], [3, 2], [0, 1]], np.int32)
    w = rng.uniform(0.1, 1, (M, 2)).astype(np.float32)
    base, _ = oracle.moe_layer(gate, up, down, x, ids, w, L, False)
    perm = np.array([3, 0, 4, 1, 2])  # new expert p holds old expert perm[p]
    inv = np.argsort(perm)

    def relabel(b):
        return Bank(b.fmt, b.codes[perm], b.scales[perm])
    out2, _ = oracle.moe_layer(relabel(gate), relabel(up), relabel(down), x, inv[ids].astype(np.int32), w, L, False)
    assert np.array_equal(out2, base)
    tp = np.array([2, 0, 3, 1])
    out3, _ = oracle.moe_layer(gate, up, down, x[tp], ids[tp], w[tp], L, False)
    assert np.array_equal(out3, base[tp])
    xd = np.stack([x[1], x[1]])
    out4, _ = oracle.moe_layer(gate, up, down, xd, np.stack([ids[1], ids[1]]), np.stack([w[1], w[1]]), L, False)
    assert np.array_equal(out4[0], out4[1]) and np.array_equal(out4[0], base[1])


# --------------------------------------------------------------------------
# 1x128 activation quantization (FP8 tier)
# --------------------------------------------------------------------------

def _e4m3_half_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * 2.0 ** (e - 3)


def test_quant_1x128_exhaustive_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_vals(bits)
    finite = bits[np.isfinite(vals)]
    n = (len(finite) // 128) * 128
    x = bf16_vals(finite[:n]).astype(np.float32).reshape(-1, 128)
    q, s = oracle.quant_1x128(x)
    amax = np.abs(x).max(axis=1)
    exp_s = np.where(amax == 0, np.float32(1.0), (amax / np.float32(448.0)).astype(np.float32))
    assert np.array_equal(s[:, 0], exp_s)
    ratio = (x / s).astype(np.float32)   # IEEE binary32 division
    ref = torch.from_numpy(ratio).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    deq = _torch_e4m3(q)
    err = np.abs(deq - ratio.astype(np.float64))
    assert np.all(err <= _e4m3_half_ulp(ratio.astype(np.float64)) * (1 + 1e-12))


def test_quant_1x128_exact_multiples_and_zero_group():
    t = _torch_e4m3(np.arange(0x7F, dtype=np.uint8))
    rng = np.random.default_rng(9)
    codes = rng.choice(t, (4, 256))
    codes[:, 0] = 448.0  # every group holds the top magnitude -> scale exactly s
    codes[:, 128] = -448.0
    s = np.float32(2.0 ** -5)
    x = (codes * float(s)).astype(np.float32)
    q, sc = oracle.quant_1x128(x)
    assert np.all(sc == s)
    assert np.array_equal(_torch_e4m3(q) * float(s), x.astype(np.float64))
    z = np.zeros((1, 128), np.float32)
    qz, sz = oracle.quant_1x128(z)
    assert sz[0, 0] == 1.0 and np.all(qz == 0)


def test_fp8_tier_layer_uses_quantized_x_and_h():
    rng = np.random.default_rng(12)
    E, H, I = 3, 256, 256
    gate, up, down = rand_e4m3_bank(rng, E, I, H), rand_e4m3_bank(rng, E, I, H), rand_e4m3_bank(rng, E, H, I)
    x = bf16_bits(rng.standard_normal((2, H)))
    ids = np.array([[0, 2], [1, 0]], np.int32)
    res = oracle.expert_slots(gate, up, down, x, ids, L, True, want=("g", "u", "h", "y"))
    q, s = oracle.quant_1x128(bf16_vals(x).astype(np.float32))
    xq = _torch_e4m3(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    for slot in range(4):
        t, e = slot // 2, ids.flat[slot]
        g = indep_dense(gate, e) @ xq[t]
        u = indep_dense(up, e) @ xq[t]
        h = silu_ref(np.minimum(g, L)) * np.clip(u, -L, L)
        hq, hs = oracle.quant_1x128(h.astype(np.float32)[None, :])
        hh = _torch_e4m3(hq[0]) * np.repeat(hs[0].astype(np.float64), 128)
        np.testing.assert_allclose(res["g"][slot], g, rtol=1e-12, atol=1e-12 * np.abs(g).max())
        np.testing.assert_allclose(res["h"][slot], hh, rtol=0, atol=1e-9 * np.abs(hh).max())
        y = indep_dense(down, e) @ hh
        np.testing.assert_allclose(res["y"][slot], y, rtol=1e-9, atol=1e-9 * np.abs(y).max())
