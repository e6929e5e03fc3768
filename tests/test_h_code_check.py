"""CPU checks of the rule the GEMM-tier parity test applies to re-quantized h
codes: planted mistakes (a two-step code, a flip far from a midpoint, a wrong
scale) must be rejected; a one-step flip at a midpoint must be accepted."""
import numpy as np
import pytest

import oracle
from moe_cases import blockmax_sum, check_h_codes, h_error_bound


def _case():
    rng = np.random.default_rng(3)
    h = rng.standard_normal((4, 256)) * 10
    q, s = oracle.quant_1x128(h.astype(np.float32))
    return h, q, s


def test_identical_codes_pass():
    h, q, s = _case()
    assert check_h_codes(q.copy(), s.copy(), h, np.zeros_like(h), "same") == 0.0


def test_flip_at_midpoint_passes():
    h, q, s = _case()
    # put element (0, 5) exactly on the midpoint between two codes
    tab = oracle.e4m3_table()
    c = int(q[0, 5]) & 0x7F
    c = min(max(c, 0x20), 0x70)
    lo, hi = tab[c], tab[c + 1]
    h[0, 5] = 0.5 * (lo + hi) * float(s[0, 0])
    q2, s2 = oracle.quant_1x128(h.astype(np.float32))
    g = q2.copy()
    g[0, 5] = c if q2[0, 5] == c + 1 else c + 1     # the other neighbour
    assert check_h_codes(g, s2, h, np.zeros_like(h), "midpoint") > 0


def test_two_step_or_far_flip_or_bad_scale_fail():
    h, q, s = _case()
    g = q.copy()
    g[1, 7] = (int(g[1, 7]) & 0x80) | min((int(g[1, 7]) & 0x7F) + 2, 0x7E)
    with pytest.raises(AssertionError):
        check_h_codes(g, s, h, np.zeros_like(h), "two steps")
    g = q.copy()
    # one step away but the value is not near a midpoint: pick an element sitting on a code
    tab = oracle.e4m3_table()
    h2 = h.copy()
    h2[2, 9] = tab[0x40] * float(s[2, 0])
    q2, s2 = oracle.quant_1x128(h2.astype(np.float32))
    g = q2.copy()
    g[2, 9] = 0x41
    with pytest.raises(AssertionError):
        check_h_codes(g, s2, h2, np.zeros_like(h2), "far flip")
    with pytest.raises(AssertionError):
        check_h_codes(q.copy(), s * np.float32(1.001), h, np.zeros_like(h), "scale")


def test_error_bound_closed_forms():
    L = 7.0
    # g far above the cap, |u| far above it: h is constant, no error
    assert h_error_bound(np.array([50.0]), np.array([30.0]), np.array([10.0]), np.array([10.0]), L,
                         eps=1e-3)[0] <= 1e-4
    # up inside the range: the up error passes through silu(min(g, L))
    b = h_error_bound(np.array([50.0]), np.array([1.0]), np.array([0.0]), np.array([100.0]), L, eps=1e-3)[0]
    assert abs(b - 7.0 / (1 + np.exp(-7.0)) * 0.1) < 1e-3
    # a flip admitted only through the bound: v just off a midpoint
    h, q, s = _case()
    tab = oracle.e4m3_table()
    c = 0x40
    v = 0.5 * (tab[c] + tab[c + 1]) + 0.01
    h[3, 3] = v * float(s[3, 0])
    q2, s2 = oracle.quant_1x128(h.astype(np.float32))
    g = q2.copy()
    g[3, 3] = c
    with pytest.raises(AssertionError):
        check_h_codes(g, s2, h, np.zeros_like(h), "no bound")
    bound = np.zeros_like(h)
    bound[3, 3] = 0.02 * float(s2[3, 0])
    assert check_h_codes(g, s2, h, bound, "bound") > 0


def test_blockmax_sum_by_hand():
    w = np.zeros((2, 256))
    x = np.ones((1, 256))
    w[0, 3], w[0, 7], w[0, 200] = 2.0, -5.0, 1.5     # block 0 max 5, block 1 max 1.5
    w[1, 130] = 4.0
    assert blockmax_sum(np.abs(w), x).tolist() == [[6.5, 4.0]]
