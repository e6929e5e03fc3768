"""Pins of the oracle's router (oracle.router_topk) to things other than
itself: what a top-k choice must satisfy (checked by brute force over every
expert pair), scipy's softmax and logistic functions on the special cases
where the weights reduce to them, hand-worked rows in which the selection
bias changes the choice, ties, and non-finite logits."""
import itertools

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
from oracle import ROUTER_SIGMOID, ROUTER_SOFTMAX


def _keys(logits, kind, bias):
    """Selection keys as the definition states them, for the brute-force check."""
    l = np.nan_to_num(logits.astype(np.float32), nan=-np.finfo(np.float32).max,
                      posinf=np.finfo(np.float32).max, neginf=-np.finfo(np.float32).max)
    if kind == ROUTER_SOFTMAX:
        return l
    s = expit(l.astype(np.float64)).astype(np.float32)
    b = np.zeros_like(s) if bias is None else bias.astype(np.float32)
    return (s + b).astype(np.float32)


def _check_choice(ids, keys, k):
    """Every chosen key beats every unchosen one (ties: the lower id is
    chosen); ranks are in non-increasing key order, ties by ascending id."""
    M, E = keys.shape
    for t in range(M):
        chosen = list(ids[t])
        assert len(set(chosen)) == k
        rest = [e for e in range(E) if e not in chosen]
        for c, r in itertools.product(chosen, rest):
            assert keys[t, c] > keys[t, r] or (keys[t, c] == keys[t, r] and c < r), (t, c, r)
        for a, b in zip(chosen, chosen[1:]):
            assert keys[t, a] > keys[t, b] or (keys[t, a] == keys[t, b] and a < b), (t, a, b)


@pytest.mark.parametrize("kind", [ROUTER_SOFTMAX, ROUTER_SIGMOID])
@pytest.mark.parametrize("E,k", [(6, 1), (6, 3), (16, 4), (40, 8), (7, 7)])
def test_choice_satisfies_the_top_k_order(kind, E, k):
    rng = np.random.default_rng(E * 10 + k + kind)
    logits = rng.standard_normal((20, E)).astype(np.float32)
    logits[:5] = np.round(logits[:5] * 2) / 2          # many exact ties
    bias = rng.normal(0, 0.3, E).astype(np.float32) if kind == ROUTER_SIGMOID else None
    ids, _ = oracle.router_topk(logits, k, kind, bias)
    _check_choice(ids, _keys(logits, kind, bias), k)


def test_softmax_weights_reduce_to_scipy_softmax():
    rng = np.random.default_rng(7)
    logits = (rng.standard_normal((8, 12)) * 3).astype(np.float32)
    # k = E, renormalized: the full softmax in rank order
    ids, w = oracle.router_topk(logits, 12, ROUTER_SOFTMAX, renormalize=True)
    p = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids, 1), rtol=2e-7, atol=0)
    # any k, not renormalized: the chosen entries of the full softmax
    ids, w = oracle.router_topk(logits, 3, ROUTER_SOFTMAX, renormalize=False)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids, 1), rtol=2e-7, atol=0)
    # any k, renormalized: softmax over the chosen logits only
    ids, w = oracle.router_topk(logits, 3, ROUTER_SOFTMAX, renormalize=True, routed_scale=2.5)
    sub = softmax(np.take_along_axis(logits, ids, 1).astype(np.float64), axis=1)
    np.testing.assert_allclose(w, 2.5 * sub, rtol=2e-7, atol=0)


def test_two_expert_renormalized_softmax_is_the_logistic_of_the_gap():
    logits = np.array([[1.25, -0.5, 3.0, 0.0]], np.float32)
    ids, w = oracle.router_topk(logits, 2, ROUTER_SOFTMAX)
    assert ids.tolist() == [[2, 0]]
    np.testing.assert_allclose(w[0], [expit(1.75), expit(-1.75)], rtol=2e-7)


def test_sigmoid_weights_reduce_to_scipy_expit():
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((6, 20)).astype(np.float32)
    bias = rng.normal(0, 0.5, 20).astype(np.float32)
    ids, w = oracle.router_topk(logits, 5, ROUTER_SIGMOID, bias, routed_scale=1.0, renormalize=False)
    s = expit(np.take_along_axis(logits, ids, 1).astype(np.float64))
    np.testing.assert_allclose(w, s, rtol=2e-7, atol=0)         # the bias never enters a weight
    ids2, w2 = oracle.router_topk(logits, 5, ROUTER_SIGMOID, bias, routed_scale=2.5, renormalize=True)
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w2, 2.5 * s / s.sum(1, keepdims=True), rtol=3e-7, atol=0)
    np.testing.assert_allclose(w2.sum(1), 2.5, rtol=1e-6)


def test_hand_worked_bias_changes_the_choice():
    # s = sigmoid(l) = [0.622, 0.881, 0.269, 0.881]; a bias of 1 on expert 2
    # lifts it to the top; experts 1 and 3 tie and the lower id wins
    l = np.array([[0.5, 2.0, -1.0, 2.0]], np.float32)
    ids, w = oracle.router_topk(l, 2, ROUTER_SIGMOID, np.array([0, 0, 1, 0], np.float32))
    assert ids.tolist() == [[2, 1]]
    s2, s1 = expit(-1.0), expit(2.0)
    np.testing.assert_allclose(w[0], [s2 / (s1 + s2), s1 / (s1 + s2)], rtol=2e-7)
    # without the bias, the two largest sigmoids win, lower id first
    ids, _ = oracle.router_topk(l, 2, ROUTER_SIGMOID, None)
    assert ids.tolist() == [[1, 3]]
    # a negative bias can push the largest logit out
    ids, _ = oracle.router_topk(l, 1, ROUTER_SIGMOID, np.array([0, -0.5, 0, 0], np.float32))
    assert ids.tolist() == [[3]]


def test_ties_go_to_the_lower_expert_id():
    l = np.zeros((1, 9), np.float32)
    ids, w = oracle.router_topk(l, 4, ROUTER_SOFTMAX)
    assert ids.tolist() == [[0, 1, 2, 3]]
    assert np.all(w == np.float32(0.25))
    l = np.array([[-0.0, 0.0, -0.0, 0.0]], np.float32)           # -0 and +0 are equal keys
    ids, _ = oracle.router_topk(l, 2, ROUTER_SOFTMAX)
    assert ids.tolist() == [[0, 1]]


def test_non_finite_logits():
    inf, nan = np.float32(np.inf), np.float32(np.nan)
    l = np.array([[nan, 1.0, inf, -inf, 0.5]], np.float32)
    ids, w = oracle.router_topk(l, 5, ROUTER_SOFTMAX)
    # +inf ranks first (as FLT_MAX); NaN and -inf are both -FLT_MAX, lower id first
    assert ids.tolist() == [[2, 1, 4, 0, 3]]
    assert np.all(np.isfinite(w))
    assert w[0, 0] == np.float32(1.0) and np.all(w[0, 1:] == 0)
    ids, w = oracle.router_topk(l, 2, ROUTER_SIGMOID)
    assert ids.tolist() == [[2, 1]] and np.all(np.isfinite(w))
    # every chosen sigmoid is 0: nothing to renormalize, the weights are 0
    ids, w = oracle.router_topk(np.full((1, 4), nan, np.float32), 2, ROUTER_SIGMOID)
    assert ids.tolist() == [[0, 1]] and np.all(w == 0)
    ids, w = oracle.router_topk(np.full((1, 4), -1000.0, np.float32), 2, ROUTER_SIGMOID)
    assert np.all(w == 0)


def test_shift_invariance_of_the_softmax():
    rng = np.random.default_rng(3)
    logits = np.round(rng.standard_normal((10, 32)) * 64) / 64          # exact on a 1/64 grid
    a = logits.astype(np.float32)
    b = (logits + 5.0).astype(np.float32)
    ia, wa = oracle.router_topk(a, 6, ROUTER_SOFTMAX)
    ib, wb = oracle.router_topk(b, 6, ROUTER_SOFTMAX)
    assert np.array_equal(ia, ib)
    np.testing.assert_array_equal(wa, wb)        # the differences l[j] - l[0] are the same doubles


def test_relabelling_experts_relabels_the_choice():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((12, 24)).astype(np.float32)
    perm = rng.permutation(24)
    ids, w = oracle.router_topk(logits, 4, ROUTER_SOFTMAX)
    ids_p, w_p = oracle.router_topk(logits[:, perm], 4, ROUTER_SOFTMAX)
    assert np.array_equal(perm[ids_p], ids)                      # no ties in continuous draws
    np.testing.assert_array_equal(w_p, w)


def test_bad_arguments():
    l = np.zeros((2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.router_topk(l, 5)
    with pytest.raises(ValueError):
        oracle.router_topk(l, 0)
