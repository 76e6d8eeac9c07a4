"""Pins for the oracle's router (softmax + top-k): a hand-worked example,
brute force over expert subsets, scipy's softmax, and invariants."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def test_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "route_example.json")))
    lg = np.array([g["logits"]], np.float32)
    w, ids = oracle.route(lg, g["topk"], renormalize=True)
    assert ids[0].tolist() == g["ids"]
    np.testing.assert_allclose(w[0], g["weights_renorm"], rtol=2 ** -23)
    w0, ids0 = oracle.route(lg, g["topk"], renormalize=False)
    assert ids0[0].tolist() == g["ids"]
    np.testing.assert_allclose(w0[0], g["weights_full_softmax"], rtol=2 ** -23)


def test_ties_go_to_lower_expert_index():
    lg = np.array([[1.0, 3.0, 3.0, 1.0, 3.0]], np.float32)
    w, ids = oracle.route(lg, 4)
    assert ids[0].tolist() == [1, 2, 4, 0]
    # equal logits -> equal weights
    assert w[0, 0] == w[0, 1] == w[0, 2]


@pytest.mark.parametrize("E,topk", [(4, 1), (4, 2), (6, 3), (8, 2), (7, 7)])
def test_brute_force_subsets(E, topk):
    rng = np.random.default_rng(10 + E * 10 + topk)
    lg = rng.standard_normal((50, E)).astype(np.float32)
    w, ids = oracle.route(lg, topk, renormalize=True)
    wf, idsf = oracle.route(lg, topk, renormalize=False)
    assert (ids == idsf).all()
    for m in range(lg.shape[0]):
        # the chosen set maximises the logit sum over all k-subsets
        best = max(itertools.combinations(range(E), topk), key=lambda s: sum(float(lg[m, e]) for e in s))
        assert set(ids[m].tolist()) == set(best)
        # ordering: descending logit
        assert all(lg[m, ids[m, j]] >= lg[m, ids[m, j + 1]] for j in range(topk - 1))
        sel = lg[m, ids[m]].astype(np.float64)
        np.testing.assert_allclose(w[m], softmax(sel), rtol=2 ** -23, atol=0)
        np.testing.assert_allclose(wf[m], softmax(lg[m].astype(np.float64))[ids[m]], rtol=2 ** -23, atol=0)


def test_invariants_large():
    rng = np.random.default_rng(3)
    E, topk = 160, 6
    lg = (rng.standard_normal((2000, E)) * 3).astype(np.float32)
    w, ids = oracle.route(lg, topk)
    assert ids.min() >= 0 and ids.max() < E
    for row in ids:
        assert len(set(row.tolist())) == topk
    assert (np.diff(w, axis=1) <= 0).all()                   # non-increasing weights
    np.testing.assert_allclose(w.sum(1, dtype=np.float64), 1.0, atol=topk * 2 ** -24)


def test_shift_invariance():
    """softmax(l + c) = softmax(l): adding a constant to a row changes nothing
    beyond float32 rounding of the shifted logits."""
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((100, 8)).astype(np.float32)
    w1, i1 = oracle.route(lg, 2)
    w2, i2 = oracle.route((lg + np.float32(0.5)).astype(np.float32), 2)
    assert (i1 == i2).all()
    np.testing.assert_allclose(w1, w2, rtol=1e-6)
