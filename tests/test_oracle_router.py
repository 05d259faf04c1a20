"""Pins of the oracle's sigmoid router top-k.

Module glm5next_mlp: "The stack this layer runs" (fp32 router logits, then a
top-k that emits K ids and K weights); "Traps this module exists to hold" (the
bias changes only the choice, weights from the plain sigmoid scores,
routed_scaling_factor on the weights, renormalised over the chosen experts of
the full count); Constants, KERNEL_MAX_TOP_K (K <= 16).
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special

import oracle as O


def test_logits_brute_force_loops():
    g = np.random.default_rng(2)
    x = g.standard_normal((3, 5))
    Wr = g.standard_normal((4, 5))
    want = [[sum(x[t, h] * Wr[e, h] for h in range(5)) for e in range(4)] for t in range(3)]
    np.testing.assert_allclose(O.router_logits(x, Wr), want, rtol=1e-14, atol=1e-14)


def test_sigmoid_special_values_and_library():
    assert O.sigmoid(0.0) == 0.5
    assert abs(O.sigmoid(math.log(3.0)) - 0.75) < 1e-15
    z = np.linspace(-40, 40, 2001)
    np.testing.assert_allclose(O.sigmoid(z), scipy.special.expit(z), rtol=1e-14, atol=0)
    np.testing.assert_allclose(O.sigmoid(-z), 1.0 - O.sigmoid(z), atol=1e-15)


@pytest.mark.parametrize("E,K", [(16, 4), (12, 1), (10, 5), (8, 8), (16, 2), (9, 7)])
def test_topk_brute_force_all_subsets(E, K):
    g = np.random.default_rng(E * 100 + K)
    for _ in range(20):
        sel = g.standard_normal(E)
        best = max(itertools.combinations(range(E), K), key=lambda c: sum(sel[i] for i in c))
        ids = O.select_topk(sel[None, :], K)[0]
        assert set(ids.tolist()) == set(best)
        # descending order, by a different routine (Python's sorted)
        assert ids.tolist() == sorted(best, key=lambda i: -sel[i])


def test_topk_tie_goes_to_lower_index():
    sel = np.array([[0.5, 0.9, 0.5, 0.9, 0.1]])
    assert O.select_topk(sel, 3)[0].tolist() == [1, 3, 0]


def test_zero_bias_selects_largest_logits():
    """sigmoid is monotone, so with no bias the chosen set is the top-K logits."""
    g = np.random.default_rng(3)
    x = g.standard_normal((50, 32))
    Wr = g.standard_normal((20, 32)) * 0.1
    ids, w, l, _ = O.route(x, Wr, np.zeros(20), 6, 2.5)
    for t in range(50):
        want = sorted(range(20), key=lambda e: -l[t, e])[:6]
        assert ids[t].tolist() == want


def _setup(seed=4, T=64, E=24, H=48):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, H))
    Wr = g.standard_normal((E, H)) * 0.2
    b = g.uniform(-0.2, 0.2, E)
    return x, Wr, b


def test_weights_sum_to_rsf_and_follow_score_ratios():
    x, Wr, b = _setup()
    rsf = 2.5
    ids, w, l, _ = O.route(x, Wr, b, 5, rsf)
    np.testing.assert_allclose(w.sum(-1), rsf, rtol=1e-14)
    # w_i / w_j = s_i / s_j = (1 + e^-l_j) / (1 + e^-l_i)
    for t in range(x.shape[0]):
        i, j = ids[t, 0], ids[t, 1]
        ratio = (1 + math.exp(-l[t, j])) / (1 + math.exp(-l[t, i]))
        assert abs(w[t, 0] / w[t, 1] - ratio) < 1e-13 * ratio


def test_equal_logits_give_equal_weights():
    """All logits 0 -> every score 0.5 -> weights rsf/K regardless of bias."""
    x = np.zeros((3, 8))
    Wr = np.ones((10, 8))
    b = np.linspace(-0.1, 0.1, 10)
    ids, w, _, _ = O.route(x, Wr, b, 4, 2.5)
    np.testing.assert_allclose(w, 2.5 / 4, rtol=0, atol=1e-15)
    assert ids[0].tolist() == [9, 8, 7, 6]          # the bias alone decides the order


def test_bias_steers_selection_only():
    """Weights of the chosen set are the unbiased scores; gathering biased
    scores (the trap) gives different weights."""
    x, Wr, b = _setup(5)
    ids, w, l, sel = O.route(x, Wr, b, 5, 1.0)
    s = O.sigmoid(l)
    assert not np.array_equal(ids, O.select_topk(s, 5))      # the bias changes some choices
    biased = np.take_along_axis(sel, ids, -1)
    biased = biased / biased.sum(-1, keepdims=True)
    assert np.max(np.abs(biased - w)) > 1e-3
    # a bias that keeps the chosen set keeps the weights (as a map id -> weight)
    b2 = b.copy()
    b2[ids[0]] += 0.01
    ids2, w2, _, _ = O.route(x[:1], Wr, b2, 5, 1.0)
    assert dict(zip(ids2[0].tolist(), w2[0].tolist())) == pytest.approx(dict(zip(ids[0].tolist(), w[0].tolist())), rel=1e-15)


def test_k_equals_e_ignores_bias():
    x, Wr, b = _setup(6, E=10)
    ids1, w1, _, _ = O.route(x, Wr, b, 10, 2.5)
    ids2, w2, _, _ = O.route(x, Wr, -3 * b, 10, 2.5)
    for t in range(x.shape[0]):
        m1 = dict(zip(ids1[t].tolist(), w1[t].tolist()))
        m2 = dict(zip(ids2[t].tolist(), w2[t].tolist()))
        assert m1 == pytest.approx(m2, rel=1e-15)


def test_renormalises_over_full_count():
    """Ranking a subset of the experts (the local-count trap) changes the weights."""
    x, Wr, b = _setup(7, E=24)
    ids, w, _, _ = O.route(x, Wr, b, 6, 2.5)
    ids_h, w_h, _, _ = O.route(x, Wr[:12], b[:12], 6, 2.5)
    differs = [t for t in range(x.shape[0]) if not set(ids[t]) <= set(range(12))]
    assert differs
    t = differs[0]
    assert set(ids[t].tolist()) != set(ids_h[t].tolist())
