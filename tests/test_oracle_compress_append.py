"""Pins for the oracle's decode-time compression state (CPU only).

Appending tokens one at a time must, for every completed block, give the
entry the block compressor gives for the whole sequence at once; a block that
is still open must leave its pool row alone and keep its tokens in ring slots
position mod m.  Each test checks one of these facts, or a closed form
(m = 1 identity, uniform gates -> mean of the block's tokens), against
values formed without the append path.  A wrong slot, an off-by-one on block
completion, a wrong pool row or a token taken by an idle sequence fails one
of them.
"""
import numpy as np
import pytest
import torch


def _state(B, m, D, dtype=np.float64):
    return np.zeros((B, m, D), dtype), np.zeros((B, m, D), dtype)


@pytest.mark.parametrize("m", [1, 3, 4, 16])
def test_streaming_matches_whole_sequence(oracle, m):
    """Token-by-token appends, started at ragged offsets, reproduce the
    block compressor's entries over the whole sequence."""
    rng = np.random.default_rng(100 + m)
    B, D, T = 3, 6, 5 * m + 2
    x = rng.standard_normal((B, T, D))
    g = rng.standard_normal((B, T, D)) * 2.0
    bias = rng.standard_normal((m, D))
    S = T // m
    want = oracle.compress(x, g, bias, m)
    rx, rg = _state(B, m, D)
    pool = np.full((B, S, D), np.nan)
    start = [0, 1, m + 1]  # sequence b joins the stream after start[b] steps
    for step in range(T + max(start)):
        xt = np.full((B, D), np.nan)  # idle sequences' tokens must not be read
        gt = np.full((B, D), np.nan)
        pos = np.full(B, -1, np.int32)
        for b in range(B):
            if start[b] <= step < start[b] + T:
                pos[b] = step - start[b]
                xt[b] = x[b, pos[b]]
                gt[b] = g[b, pos[b]]
        oracle.compress_append(xt, gt, bias, rx, rg, pos, pool, m)
    np.testing.assert_allclose(pool, want, rtol=0, atol=1e-13)


def test_open_block_keeps_tokens_in_ring_and_pool_untouched(oracle):
    rng = np.random.default_rng(7)
    B, m, D, S = 2, 4, 5, 3
    rx, rg = _state(B, m, D)
    pool = np.full((B, S, D), np.nan)
    bias = rng.standard_normal((m, D))
    toks = rng.standard_normal((6, B, D))
    gates = rng.standard_normal((6, B, D))
    for t in range(6):
        pos = np.full(B, t, np.int32)
        wrote = oracle.compress_append(toks[t], gates[t], bias, rx, rg, pos, pool, m)
        assert wrote == ([(0, 0), (1, 0)] if t == 3 else [])
    # Tokens 4 and 5 sit in slots 0 and 1 of the new block; slots 2 and 3 still
    # hold tokens 2 and 3 of the completed block.
    for b in range(B):
        np.testing.assert_array_equal(rx[b, 0], toks[4, b])
        np.testing.assert_array_equal(rx[b, 1], toks[5, b])
        np.testing.assert_array_equal(rx[b, 2], toks[2, b])
        np.testing.assert_array_equal(rg[b, 3], gates[3, b])
    assert np.isfinite(pool[:, 0]).all()
    assert np.isnan(pool[:, 1:]).all()


def test_m1_every_token_is_its_own_entry(oracle):
    rng = np.random.default_rng(3)
    B, D, S = 2, 4, 5
    rx, rg = _state(B, 1, D)
    pool = np.full((B, S, D), np.nan)
    bias = rng.standard_normal((1, D))
    toks = rng.standard_normal((S, B, D))
    for t in range(S):
        oracle.compress_append(toks[t], rng.standard_normal((B, D)) * 9, bias, rx, rg,
                               np.full(B, t, np.int32), pool, 1)
    np.testing.assert_allclose(pool, toks.transpose(1, 0, 2), rtol=0, atol=1e-15)


def test_uniform_gates_give_mean_of_block(oracle):
    rng = np.random.default_rng(5)
    B, m, D, S = 1, 8, 3, 2
    rx, rg = _state(B, m, D)
    pool = np.full((B, S, D), np.nan)
    bias = np.tile(rng.standard_normal((1, D)), (m, 1))
    toks = rng.standard_normal((2 * m, B, D))
    for t in range(2 * m):
        level = np.full((B, D), 0.7 if t < m else -3.0)
        oracle.compress_append(toks[t], level, bias, rx, rg, np.full(B, t, np.int32), pool, m)
    want = toks.transpose(1, 0, 2).reshape(B, 2, m, D).mean(axis=2)
    np.testing.assert_allclose(pool, want, rtol=0, atol=1e-14)


def test_block_past_pool_end_is_dropped(oracle):
    rng = np.random.default_rng(9)
    B, m, D, S = 1, 2, 3, 1
    rx, rg = _state(B, m, D)
    pool = np.full((B, S, D), np.nan)
    bias = rng.standard_normal((m, D))
    wrote = []
    for t in range(4):
        wrote += oracle.compress_append(rng.standard_normal((B, D)), rng.standard_normal((B, D)),
                                        bias, rx, rg, np.full(B, t, np.int32), pool, m)
    assert wrote == [(0, 0)]


def test_bf16_tokens_match_whole_sequence(oracle):
    torch.manual_seed(0)
    B, m, D, T = 2, 4, 8, 12
    x = torch.randn(B, T, D).to(torch.bfloat16)
    g = torch.randn(B, T, D).to(torch.bfloat16)
    bias = torch.randn(m, D).to(torch.bfloat16)
    want = oracle.compress(x, g, bias, m)
    rx = torch.zeros(B, m, D, dtype=torch.bfloat16)
    rg = torch.zeros(B, m, D, dtype=torch.bfloat16)
    pool = np.full((B, T // m, D), np.nan)
    for t in range(T):
        oracle.compress_append(x[:, t], g[:, t], bias, rx, rg, np.full(B, t, np.int32), pool, m)
    np.testing.assert_allclose(pool, want, rtol=0, atol=0)
