"""Pins of the oracle's shared expert (oracle.shared_expert) and of the final
add order routed, then shared, then residual (oracle.combine_residual), to
things other than the oracle itself: numpy FP64 matrix products of the
decoded bf16 weights, a diagonal MLP with an elementwise closed form, the
pages' worked combine example extended by hand, and reductions to the plain
combine."""
import numpy as np
import torch

import oracle


def bf16_bits(a) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def swiglu_ref(g, u, L):
    gc = np.minimum(g, L)
    return gc / (1.0 + np.exp(-gc)) * np.clip(u, -L, L)


def test_shared_expert_matches_numpy_matmuls_of_decoded_weights():
    rng = np.random.default_rng(21)
    M, H, W, L = 3, 96, 40, 7.0
    g = bf16_bits(rng.standard_normal((W, H)) * 0.3)
    u = bf16_bits(rng.standard_normal((W, H)) * 0.3)
    d = bf16_bits(rng.standard_normal((H, W)) * 0.3)
    x = bf16_bits(rng.standard_normal((M, H)))
    out = oracle.shared_expert(g, u, d, x, L)
    xv = bf16_values(x)
    gv, uv = xv @ bf16_values(g).T, xv @ bf16_values(u).T          # [M, W]
    ref = swiglu_ref(gv, uv, L) @ bf16_values(d).T                   # [M, H]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # the clamp is active somewhere in this draw, and with a huge limit the
    # result is the plain SiLU MLP
    assert np.any(gv > L) or np.any(np.abs(uv) > L)
    out_big = oracle.shared_expert(g, u, d, x, 1e30)
    plain = (gv / (1.0 + np.exp(-gv)) * uv) @ bf16_values(d).T
    np.testing.assert_allclose(out_big, plain, rtol=1e-12, atol=1e-12)


def test_diagonal_shared_expert_closed_form():
    # W = H, diagonal gate/up/down with power-of-two entries: each output is
    # c_i * silu(min(a_i x_i, L)) * clamp(b_i x_i, -L, L)
    H, L = 16, 7.0
    a = 2.0 ** np.arange(-3, 13 - 3).repeat(2)[:H]
    b = np.where(np.arange(H) % 2 == 0, 0.5, -4.0)
    c = np.where(np.arange(H) % 3 == 0, 0.25, 2.0)
    x = bf16_bits(np.linspace(-3, 3, H)[None, :])
    out = oracle.shared_expert(bf16_bits(np.diag(a)), bf16_bits(np.diag(b)), bf16_bits(np.diag(c)),
                               x, L)
    xv = bf16_values(x)[0]
    g, u = a * xv, b * xv
    want = c * (np.minimum(g, L) / (1 + np.exp(-np.minimum(g, L)))) * np.clip(u, -L, L)
    np.testing.assert_allclose(out[0], want, rtol=1e-14, atol=1e-14)
    # a token of zeros gives a zero row
    z = oracle.shared_expert(bf16_bits(np.diag(a)), bf16_bits(np.diag(b)), bf16_bits(np.diag(c)),
                             bf16_bits(np.zeros((1, H))), L)
    assert np.all(z == 0.0)


def test_combine_residual_worked_example_extended():
    # the pages' example: slots [1,10], [2,20], [-4,8] with weights 0.5,
    # 0.25, 0.125 combine to [0.5, 11.0]; then + shared [0.25, -1] = [0.75, 10]
    # and + residual [-0.5, 2] = [0.25, 12]
    k = 8
    y = np.zeros((k, 2))
    y[0], y[1], y[2] = [1, 10], [2, 20], [-4, 8]
    w = np.array([[0.5, 0.25, 0.125, 0, 0, 0, 0, 0]], np.float32)
    v = np.ones(k, np.int32)
    shared = np.array([[0.25, -1.0]])
    res = np.array([[-0.5, 2.0]], np.float32)
    assert oracle.combine_residual(y, w, v, None, None).tolist() == [[0.5, 11.0]]
    assert oracle.combine_residual(y, w, v, shared, None).tolist() == [[0.75, 10.0]]
    assert oracle.combine_residual(y, w, v, shared, res).tolist() == [[0.25, 12.0]]
    assert oracle.combine_residual(y, w, v, None, res).tolist() == [[0.0, 13.0]]


def test_combine_residual_reduces_to_the_combine_and_is_linear():
    rng = np.random.default_rng(9)
    M, k, H = 4, 3, 21
    y = rng.standard_normal((M * k, H))
    w = rng.uniform(0, 1, (M, k)).astype(np.float32)
    v = (rng.random(M * k) > 0.2).astype(np.int32)
    base = oracle.combine(y, w, v)
    np.testing.assert_array_equal(oracle.combine_residual(y, w, v, None, None), base)
    sh = rng.standard_normal((M, H))
    res = rng.standard_normal((M, H)).astype(np.float32)
    got = oracle.combine_residual(y, w, v, sh, res)
    np.testing.assert_allclose(got, base + sh + res.astype(np.float64), rtol=1e-14, atol=1e-14)
