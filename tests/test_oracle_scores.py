"""Pins for the oracle's indexer scores (CPU only).

The oracle computes score[q, s] = sum_h sum_e q_idx[q,h,e] * k_idx[seq(q),s,e].
Pins: one head reduces to a matrix-vector product (numpy), each single head
alone reduces to the same product with that head (so a dropped or misplaced
head fails), the head sum equals the product with the summed query (a
different order of the same sum), unit key rows pick out one channel, and
the sequence routing and candidate masking behave as stated.
"""
import numpy as np


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_one_head_is_a_matrix_vector_product(oracle):
    q = _rand((3, 1, 16), 1)
    K = _rand((3, 50, 16), 2)
    out = oracle.index_scores(q, K, n_cand=[50, 50, 50])
    for i in range(3):
        np.testing.assert_allclose(out[i], K[i] @ q[i, 0], rtol=1e-13, atol=1e-13)


def test_each_head_alone(oracle):
    H, d = 6, 8
    K = _rand((1, 40, d), 3)
    base = _rand((1, H, d), 4)
    for h in range(H):
        q = np.zeros((1, H, d))
        q[0, h] = base[0, h]
        out = oracle.index_scores(q, K, n_cand=[40])
        np.testing.assert_allclose(out[0], K[0] @ base[0, h], rtol=1e-13, atol=1e-13)


def test_head_sum_equals_summed_query(oracle):
    q = _rand((2, 64, 128), 5)
    K = _rand((2, 300, 128), 6)
    out = oracle.index_scores(q, K, n_cand=[300, 300])
    for i in range(2):
        np.testing.assert_allclose(out[i], K[i] @ q[i].sum(axis=0), rtol=1e-10, atol=1e-10)


def test_unit_key_rows_pick_one_channel(oracle):
    H, d = 4, 10
    q = _rand((1, H, d), 7)
    K = np.eye(d)[None]  # row s is the unit vector e_s
    out = oracle.index_scores(q, K, n_cand=[d])
    np.testing.assert_allclose(out[0], q[0].sum(axis=0), rtol=0, atol=1e-14)


def test_sequence_routing_and_candidate_mask(oracle):
    q = _rand((4, 2, 8), 8)
    K = _rand((2, 20, 8), 9)
    q_seq = [1, 0, 1, 0]
    n_cand = [20, 5, 0, 13]
    out = oracle.index_scores(q, K, n_cand=n_cand, q_seq=q_seq)
    for i in range(4):
        n = n_cand[i]
        want = K[q_seq[i]][:n] @ q[i].sum(axis=0)
        np.testing.assert_allclose(out[i, :n], want, rtol=1e-12, atol=1e-12)
        assert np.all(np.isnan(out[i, n:]))


def test_bf16_inputs_widen_exactly(oracle):
    import torch

    g = torch.Generator().manual_seed(3)
    q = torch.randn(2, 4, 16, generator=g).to(torch.bfloat16)
    K = torch.randn(2, 30, 16, generator=g).to(torch.bfloat16)
    a = oracle.index_scores(q, K, n_cand=[30, 30])
    b = oracle.index_scores(q.double().numpy(), K.double().numpy(), n_cand=[30, 30])
    np.testing.assert_array_equal(a, b)
