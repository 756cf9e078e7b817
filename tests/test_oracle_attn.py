"""Pins for the oracle's decode and prefill attention (CPU only).

The oracle loops over an explicit row list per query.  The pins compare it
with full dense attention over every slot/row with an explicit validity mask
(numpy), and with closed forms: a hand-worked two-row example, q = 0 giving
the plain mean of the value rows, a single row giving that row, k >= the
number of candidates giving the dense mode, invariance to the order of the
index list, and a causal-window mask for prefill.
"""
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(v):
    if isinstance(v, str):
        return math.log(float(v[2:])) if v.startswith("ln") else float(v)
    return float(v)


def _arr(nested):
    return np.vectorize(_num, otypes=[np.float64])(np.array(nested, dtype=object))


def _masked_softmax(q, rows, mult, scale, d_v):
    """Dense attention of q [H, d] over rows [R, d] with integer multiplicities mult [R]."""
    logits = scale * (q @ rows.T)  # [H, R]
    logits = np.where(mult[None, :] > 0, logits, -np.inf)
    mx = logits.max(axis=1, keepdims=True)
    w = mult[None, :] * np.exp(logits - mx)
    z = w.sum(axis=1, keepdims=True)
    return (w / z) @ rows[:, :d_v], (mx + np.log(z))[:, 0]


def test_golden_worked_example(oracle):
    g = json.load(open(os.path.join(GOLDEN, "attn_worked.json")))
    q, swa, comp = _arr(g["q"]), _arr(g["swa_kv"]), _arr(g["comp_kv"])
    o, lse = oracle.attn_decode(q, swa, g["swa_len"], comp, g["comp_len_sparse"], 1.0, 1,
                                comp_idx=g["comp_idx"])
    assert abs(o[0, 0, 0] - g["expected_o"]) < g["tolerance_abs"]
    assert abs(lse[0, 0] - _num(g["expected_lse"])) < g["tolerance_abs"]
    o2, lse2 = oracle.attn_decode(q, swa, g["swa_len"], comp, g["comp_len_dense"], 1.0, 1)
    assert abs(o2[0, 0, 0] - g["expected_o"]) < g["tolerance_abs"]
    assert abs(lse2[0, 0] - _num(g["expected_lse"])) < g["tolerance_abs"]


def _decode_case(seed, B=3, H=4, d_qk=12, d_v=8, W=6, S=20, k=7):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, d_qk))
    swa = rng.standard_normal((B, W, d_qk))
    comp = rng.standard_normal((B, S, d_qk))
    swa_len = rng.integers(1, W + 1, size=B)
    comp_len = rng.integers(0, S + 1, size=B)
    idx = np.full((B, k), -1, dtype=np.int32)
    for b in range(B):
        # some valid rows, a duplicate, an out-of-range row and -1 padding
        cand = rng.permutation(S)[: k - 2]
        idx[b, : k - 2] = cand
        if k - 2 > 0:
            idx[b, k - 2] = cand[0]
    return q, swa, comp, swa_len, comp_len, idx


def test_decode_matches_dense_masked_attention(oracle):
    for seed in range(5):
        q, swa, comp, swa_len, comp_len, idx = _decode_case(seed)
        B, H, d_qk = q.shape
        W, S, d_v, scale = swa.shape[1], comp.shape[1], 8, 0.37
        o, lse = oracle.attn_decode(q, swa, swa_len, comp, comp_len, scale, d_v, comp_idx=idx)
        od, lsed = oracle.attn_decode(q, swa, swa_len, comp, comp_len, scale, d_v)
        for b in range(B):
            rows = np.concatenate([swa[b], comp[b]])
            mult = np.zeros(W + S)
            mult[: swa_len[b]] = 1
            for i in idx[b]:
                if 0 <= i < comp_len[b]:
                    mult[W + i] += 1
            wo, wl = _masked_softmax(q[b], rows, mult, scale, d_v)
            np.testing.assert_allclose(o[b], wo, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b], wl, rtol=0, atol=1e-12)
            dense = np.zeros(W + S)
            dense[: swa_len[b]] = 1
            dense[W: W + comp_len[b]] = 1
            wo, wl = _masked_softmax(q[b], rows, dense, scale, d_v)
            np.testing.assert_allclose(od[b], wo, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lsed[b], wl, rtol=0, atol=1e-12)


def test_k_at_least_candidates_equals_dense_and_order_invariance(oracle):
    q, swa, comp, swa_len, _, _ = _decode_case(9, k=4)
    B, S = q.shape[0], comp.shape[1]
    comp_len = np.full(B, S)
    rng = np.random.default_rng(9)
    idx = np.stack([rng.permutation(S) for _ in range(B)]).astype(np.int32)
    idx = np.concatenate([idx, np.full((B, 5), -1, np.int32)], axis=1)  # k > n
    o, lse = oracle.attn_decode(q, swa, swa_len, comp, comp_len, 0.5, 8, comp_idx=idx)
    od, lsed = oracle.attn_decode(q, swa, swa_len, comp, comp_len, 0.5, 8)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, rtol=0, atol=1e-12)
    o2, _ = oracle.attn_decode(q, swa, swa_len, comp, comp_len, 0.5, 8, comp_idx=idx[:, ::-1].copy())
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)


def test_zero_query_is_mean_and_single_row_is_that_row(oracle):
    q, swa, comp, swa_len, comp_len, idx = _decode_case(4)
    o, lse = oracle.attn_decode(np.zeros_like(q), swa, swa_len, comp, comp_len, 1.0, 8)
    for b in range(q.shape[0]):
        rows = np.concatenate([swa[b, : swa_len[b]], comp[b, : comp_len[b]]])
        np.testing.assert_allclose(o[b], np.tile(rows[:, :8].mean(axis=0), (q.shape[1], 1)),
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], math.log(len(rows)), rtol=0, atol=1e-12)
    one = np.ones(q.shape[0], dtype=np.int32)
    o, lse = oracle.attn_decode(q, swa, one, comp, np.zeros_like(one), 0.3, 8)
    for b in range(q.shape[0]):
        np.testing.assert_allclose(o[b], np.tile(swa[b, 0, :8], (q.shape[1], 1)), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], 0.3 * (q[b] @ swa[b, 0]), rtol=0, atol=1e-12)


def test_unused_slots_are_never_read(oracle):
    q, swa, comp, swa_len, comp_len, idx = _decode_case(6)
    swa2, comp2 = swa.copy(), comp.copy()
    for b in range(q.shape[0]):
        swa2[b, swa_len[b]:] = np.nan
        comp2[b, comp_len[b]:] = np.nan
    a = oracle.attn_decode(q, swa, swa_len, comp, comp_len, 0.2, 8, comp_idx=idx)
    c = oracle.attn_decode(q, swa2, swa_len, comp2, comp_len, 0.2, 8, comp_idx=idx)
    np.testing.assert_array_equal(a[0], c[0])
    np.testing.assert_array_equal(a[1], c[1])


def test_prefill_matches_causal_dense_masked_attention(oracle):
    rng = np.random.default_rng(21)
    n_seq, T, H, d_qk, d_v, W, m = 2, 40, 3, 10, 6, 5, 4
    q_start, n_q = 25, 15
    S = T // m
    k = 6
    q = rng.standard_normal((n_seq, n_q, H, d_qk))
    kv = rng.standard_normal((n_seq, T, d_qk))
    comp = rng.standard_normal((n_seq, S, d_qk))
    idx = np.stack([rng.permutation(S)[:k] for _ in range(n_seq * n_q)]).astype(np.int32)
    idx[::3, -1] = -1
    scale = 0.41
    o, lse = oracle.attn_prefill(q, kv, comp, q_start, W, m, scale, d_v, comp_idx=idx)
    od, lsed = oracle.attn_prefill(q, kv, comp, q_start, W, m, scale, d_v)
    for b in range(n_seq):
        for i in range(n_q):
            p, fid = q_start + i, b * n_q + i
            rows = np.concatenate([kv[b], comp[b]])
            t = np.arange(T)
            mult = np.concatenate([((t <= p) & (t > p - W)).astype(float), np.zeros(S)])
            dense = mult.copy()
            vis = (p + 1) // m
            dense[T: T + vis] = 1
            for r in idx[fid]:
                if 0 <= r < vis:
                    mult[T + r] += 1
            wo, wl = _masked_softmax(q[b, i], rows, mult, scale, d_v)
            np.testing.assert_allclose(o[fid], wo, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[fid], wl, rtol=0, atol=1e-12)
            wo, wl = _masked_softmax(q[b, i], rows, dense, scale, d_v)
            np.testing.assert_allclose(od[fid], wo, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lsed[fid], wl, rtol=0, atol=1e-12)
    # a subset of queries gives the same rows of the result
    sel = [3, 17, 29]
    o3, _ = oracle.attn_prefill(q, kv, comp, q_start, W, m, scale, d_v, comp_idx=idx, sel=sel)
    np.testing.assert_array_equal(o3, o[sel])


def test_prefill_is_causal(oracle):
    rng = np.random.default_rng(22)
    n_seq, T, H, d, W, m = 1, 32, 2, 8, 4, 4
    q = rng.standard_normal((n_seq, 8, H, d))
    kv = rng.standard_normal((n_seq, T, d))
    comp = rng.standard_normal((n_seq, T // m, d))
    a = oracle.attn_prefill(q, kv, comp, 16, W, m, 0.3, d)
    kv2, comp2 = kv.copy(), comp.copy()
    kv2[:, 24:] = 1e3  # tokens after the last query position
    comp2[:, 6:] = 1e3  # blocks that complete after position 23
    b = oracle.attn_prefill(q, kv2, comp2, 16, W, m, 0.3, d)
    np.testing.assert_array_equal(a[0], b[0])
