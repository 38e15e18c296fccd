"""Pins for the oracle's router (softmax over E, top-k, renormalised weights).

* closed forms: logits ln(1..n) give weights proportional to the picked
  integers; k = 1 gives weight 1 on the argmax; k = E gives the full softmax
  (in fp64 by numpy on the exactly representable probabilities);
* brute force on tiny E: the picked set maximises the summed probability over
  all k-subsets, and its order is descending;
* invariants: adding a constant to a row changes nothing; permuting the
  experts permutes the ids; ties go to the lower expert; -inf logits are
  picked only when fewer than k logits are finite, and then with weight 0.
"""
import itertools

import numpy as np
import pytest

import oracle


def test_log_integers_closed_form():
    l = np.log(np.arange(1, 9, dtype=np.float64)).astype(np.float32)[None, :]
    idx, w = oracle.router_topk(l, 3)
    assert idx.tolist() == [[7, 6, 5]]
    # softmax of ln(j) is j / sum, renormalised over {8, 7, 6}: 8/21, 7/21, 6/21
    # (up to the fp32 rounding of ln j)
    assert np.allclose(w[0], np.array([8, 7, 6]) / 21.0, rtol=1e-6, atol=0)


def test_k1_is_argmax_with_weight_one():
    rng = np.random.default_rng(0)
    l = rng.standard_normal((50, 33)).astype(np.float32)
    idx, w = oracle.router_topk(l, 1)
    assert np.array_equal(idx[:, 0], np.argmax(l, axis=1))
    assert (w == 1.0).all()


def test_k_equals_e_is_full_softmax():
    rng = np.random.default_rng(1)
    l = (rng.standard_normal((20, 16)) * 3).astype(np.float32)
    idx, w = oracle.router_topk(l, 16)
    p = np.exp(l.astype(np.float64) - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    order = np.argsort(-l, axis=1, kind="stable")
    assert np.array_equal(idx, order)
    assert np.allclose(w, np.take_along_axis(p, order, 1), rtol=1e-6, atol=1e-30)
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, rtol=1e-6)


@pytest.mark.parametrize("E,k", [(5, 2), (6, 3), (7, 4)])
def test_bruteforce_subset_maximises_probability(E, k):
    rng = np.random.default_rng(E * 10 + k)
    l = rng.standard_normal((40, E)).astype(np.float32)
    idx, w = oracle.router_topk(l, k)
    for t in range(40):
        best = max(itertools.combinations(range(E), k), key=lambda c: (sum(np.exp(float(l[t, e])) for e in c), -sum(c)))
        assert sorted(idx[t].tolist()) == sorted(best)
        assert all(l[t, idx[t, j]] >= l[t, idx[t, j + 1]] for j in range(k - 1))
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) < 1e-6


def test_shift_and_permutation_invariance():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((30, 64)).astype(np.float32)
    idx, w = oracle.router_topk(l, 8)
    idx2, w2 = oracle.router_topk(l + np.float32(0.5), 8)  # the shift rounds each logit: same ids, weights to rounding
    assert np.array_equal(idx, idx2)
    assert np.allclose(w, w2, rtol=1e-6)
    perm = rng.permutation(64)
    idx3, w3 = oracle.router_topk(l[:, perm], 8)
    assert np.array_equal(perm[idx3], idx) and np.array_equal(w3, w)


def test_ties_go_to_the_lower_expert():
    l = np.zeros((3, 10), np.float32)
    l[1, [2, 5, 7]] = 1.0
    l[2, :] = -1.0
    l[2, 9] = 2.0
    idx, w = oracle.router_topk(l, 4)
    assert idx[0].tolist() == [0, 1, 2, 3] and np.allclose(w[0], 0.25)
    assert idx[1].tolist() == [2, 5, 7, 0]
    assert idx[2].tolist() == [9, 0, 1, 2]


def test_masked_experts():
    l = np.full((2, 12), -np.inf, np.float32)
    l[0, [3, 8, 10]] = [0.0, 1.0, -1.0]
    l[1, :] = np.arange(12, dtype=np.float32)
    l[1, [11, 4]] = -np.inf
    idx, w = oracle.router_topk(l, 5)
    # row 0: three finite logits, then the two lowest-index masked experts with weight 0
    assert idx[0].tolist() == [8, 3, 10, 0, 1]
    assert w[0, 3] == 0 and w[0, 4] == 0 and abs(float(w[0, :3].astype(np.float64).sum()) - 1) < 1e-6
    assert idx[1].tolist() == [10, 9, 8, 7, 6]
