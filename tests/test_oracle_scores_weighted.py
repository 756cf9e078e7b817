"""Pins for the oracle's weighted, activated indexer heads (CPU only).

score[q, s] = sum_h w[q,h] * max(0, q_idx[q,h,:] . k_idx[seq(q),s,:]).  Pins:
a hand-worked example (tests/golden/index_weighted_worked.json); with unit
weights and every dot product positive it equals the already pinned
unit-weight indexer; every dot product negative gives 0; a head pair v, -v
with unit weights gives |v . k| (one-head matrix-vector product, absolute
value); the score is linear in the weights (a scale of one head's weight
scales only that head's term); routing and candidate masking as in the
unit-weight indexer.  A dropped ReLU, a weight applied to the wrong head or
query, or the ReLU applied after the weighting fails one of them.
"""
import json
import os

import numpy as np

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "index_weighted_worked.json")


def test_hand_worked_example(oracle):
    g = json.load(open(GOLD))
    q = np.array(g["q"])[None]
    k = np.array(g["k"])[None]
    w = np.array(g["w"], np.float32)[None]
    out = oracle.index_scores_weighted(q, w, k, [k.shape[1]])
    np.testing.assert_array_equal(out[0], g["expected"])


def test_unit_weights_and_positive_dots_equal_the_unit_indexer(oracle):
    rng = np.random.default_rng(1)
    q = np.abs(rng.standard_normal((2, 5, 8)))
    K = np.abs(rng.standard_normal((2, 30, 8)))
    w = np.ones((2, 5), np.float32)
    np.testing.assert_allclose(oracle.index_scores_weighted(q, w, K, [30, 30]),
                               oracle.index_scores(q, K, [30, 30]), rtol=1e-14, atol=1e-14)


def test_negative_dots_give_zero_and_opposite_heads_give_abs(oracle):
    rng = np.random.default_rng(2)
    v = rng.standard_normal(8)
    K = rng.standard_normal((1, 40, 8))
    # every dot negative: q = -|.|, K = +|.|
    qn = -np.abs(rng.standard_normal((1, 3, 8)))
    out = oracle.index_scores_weighted(qn, np.ones((1, 3), np.float32), np.abs(K), [40])
    assert (out == 0).all()
    # heads v and -v: relu(x) + relu(-x) = |x|, with x the one-head product
    q2 = np.stack([v, -v])[None]
    got = oracle.index_scores_weighted(q2, np.ones((1, 2), np.float32), K, [40])
    one = oracle.index_scores(v[None, None], K, [40])
    np.testing.assert_allclose(got, np.abs(one), rtol=1e-14, atol=1e-14)


def test_linear_in_each_heads_weight(oracle):
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 4, 8))
    K = rng.standard_normal((1, 25, 8))
    w = rng.standard_normal((1, 4)).astype(np.float32)
    base = oracle.index_scores_weighted(q, w, K, [25])
    for h in range(4):
        w2 = w.copy()
        w2[0, h] *= 4.0  # a power of two: the fp32 weight stays exact
        only = np.zeros_like(w)
        only[0, h] = w[0, h]
        term = oracle.index_scores_weighted(q, only, K, [25])
        np.testing.assert_allclose(oracle.index_scores_weighted(q, w2, K, [25]), base + 3.0 * term,
                                   rtol=1e-12, atol=1e-12)


def test_routing_and_masking(oracle):
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 2, 4))
    K = rng.standard_normal((2, 10, 4))
    w = rng.standard_normal((3, 2)).astype(np.float32)
    out = oracle.index_scores_weighted(q, w, K, [10, 4, 0], q_seq=[1, 0, 1])
    ref1 = oracle.index_scores_weighted(q[:1], w[:1], K[1:2], [10])
    np.testing.assert_array_equal(out[0], ref1[0])
    assert np.isnan(out[1, 4:]).all() and not np.isnan(out[1, :4]).any()
    assert np.isnan(out[2]).all()
