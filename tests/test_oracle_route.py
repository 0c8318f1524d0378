"""Pins of the oracle's route step (CPU only).

Route = FarSkip-Collective section 2.1 (gate G(A) = s(A W_R^T)) with the router of Expert
Coupling in MoE Pretraining, Appendix A-A1 Table II (softmax over all experts, then top-k).
"""
import itertools
import math

import numpy as np
import pytest

from oracle import moe_oracle as O


def test_hand_built_order_and_ties():
    # expert 3 and 1 tie at the top, 0 and 4 tie below: ties go to the lower index
    l = np.array([[0.5, 2.0, -1.0, 2.0, 0.5]], np.float32)
    idx, w = O.route(l, None, 4, "softmax")
    assert idx.tolist() == [[1, 3, 0, 4]]
    # equal logits give equal weights; the pair of weights follows exp of the logit gap
    assert w[0, 0] == w[0, 1] and w[0, 2] == w[0, 3]
    assert math.isclose(w[0, 0] / w[0, 2], math.exp(1.5), rel_tol=1e-6)


def test_descending_not_ascending():
    l = np.array([[-3.0, 5.0, 1.0, 4.0]], np.float32)
    idx, _ = O.route(l, None, 2, "softmax")
    assert idx.tolist() == [[1, 3]]


def test_bias_changes_selection_and_weight():
    l = np.array([[1.0, 0.9, 0.0]], np.float32)
    b = np.array([0.0, 0.2, 0.0], np.float32)
    idx, w = O.route(l, b, 1, "sigmoid")
    assert idx.tolist() == [[1]]
    biased = np.float32(np.float32(0.9) + np.float32(0.2))
    assert math.isclose(float(w[0, 0]), 1.0 / (1.0 + math.exp(-float(biased))), rel_tol=1e-7)


def test_brute_force_selection_small():
    """Against exhaustive search: the selected set maximises the sum of logits over all
    k-subsets, and no unselected logit beats a selected one."""
    rng = np.random.default_rng(0)
    for E, k in [(5, 2), (6, 3), (7, 1), (4, 4)]:
        l = rng.integers(-3, 4, size=(40, E)).astype(np.float32)   # many ties
        idx, _ = O.route(l, None, k, "softmax")
        for t in range(l.shape[0]):
            best = max(itertools.combinations(range(E), k),
                       key=lambda s: (sum(l[t, list(s)]), [-e for e in s]))
            # among subsets of maximal sum, the tie rule picks lower indices first
            assert sorted(idx[t].tolist()) == sorted(best)
            vals = l[t, idx[t]]
            assert np.all(np.diff(vals) <= 0)
            rest = np.setdiff1d(np.arange(E), idx[t])
            if rest.size:
                assert l[t, rest].max() <= vals.min()


def test_k_equals_e_lists_all_experts():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((20, 8)).astype(np.float32)
    idx, w = O.route(l, None, 8, "softmax")
    assert all(sorted(r) == list(range(8)) for r in idx.tolist())
    # renormalised over all experts = the full softmax
    full = np.exp(l.astype(np.float64) - l.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    np.testing.assert_allclose(w, np.take_along_axis(full, idx.astype(np.int64), 1), rtol=1e-6)


def test_softmax_weights_sum_to_one_and_k1():
    rng = np.random.default_rng(2)
    l = (rng.standard_normal((500, 64)) * 3).astype(np.float32)
    _, w = O.route(l, None, 6, "softmax")
    assert np.abs(w.astype(np.float64).sum(1) - 1).max() < 4 * np.finfo(np.float32).eps
    _, w1 = O.route(l, None, 1, "softmax")
    assert np.all(w1 == 1.0)


def test_sigmoid_closed_form():
    l = np.array([[0.0, -9.0], [math.log(3.0), -9.0]], np.float32)
    _, w = O.route(l, None, 1, "sigmoid")
    assert w[0, 0] == np.float32(0.5)
    assert math.isclose(float(w[1, 0]), 0.75, rel_tol=1e-6)


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        O.route(np.zeros((2, 3), np.float32), None, 4, "softmax")
