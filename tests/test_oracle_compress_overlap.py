"""Pins for the oracle's overlapping-block compressor (CPU only).

Entry i covers the 2m tokens m(i-1) .. m(i+1)-1 that exist, bias [2m, D].
Pins: entry 0 (no earlier block) equals the plain compressor of block 0 with
bias rows m..2m-1; a bias of -200 on the earlier half reduces every entry to
the plain compressor (to within exp(-200)); uniform gates give the mean of
the window's tokens; m = 1 gives the two-token logistic weights in closed
form; every entry lies between the window's smallest and largest token; and
streaming tokens through the ring of 2m reproduces the whole-sequence result.
A window shifted by one token, a dropped or doubled half, a bias row taken
for the wrong token or a ring slot off by one fails one of them.
"""
import numpy as np
import pytest


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("m", [1, 2, 4])
def test_first_entry_and_dominated_earlier_half_reduce_to_plain(oracle, m):
    B, T, D = 2, 6 * m + 1, 5
    x, g = _rand((B, T, D), 1), _rand((B, T, D), 2, 2.0)
    bias = _rand((2 * m, D), 3, 0.5)
    out = oracle.compress_overlap(x, g, bias, m)
    plain = oracle.compress(x, g, bias[m:], m)
    np.testing.assert_allclose(out[:, 0], plain[:, 0], rtol=1e-14, atol=1e-14)
    b2 = bias.copy()
    b2[:m] = -200.0
    np.testing.assert_allclose(oracle.compress_overlap(x, g, b2, m), plain, rtol=0, atol=1e-60)
    # and the earlier half does matter when it is not dominated
    assert np.abs(out[:, 1:] - plain[:, 1:]).max() > 1e-3


def test_uniform_gates_give_the_window_mean(oracle):
    m, B, T, D = 4, 1, 20, 3
    x = _rand((B, T, D), 4)
    g = np.full((B, T, D), 0.7)
    bias = np.zeros((2 * m, D))
    out = oracle.compress_overlap(x, g, bias, m)
    np.testing.assert_allclose(out[0, 0], x[0, 0:4].mean(0), rtol=1e-14)
    for i in range(1, T // m):
        np.testing.assert_allclose(out[0, i], x[0, 4 * i - 4:4 * i + 4].mean(0), rtol=1e-14)


def test_m1_two_token_logistic(oracle):
    B, T, D = 1, 7, 2
    x, g = _rand((B, T, D), 5), _rand((B, T, D), 6)
    bias = _rand((2, D), 7)
    out = oracle.compress_overlap(x, g, bias, 1)
    np.testing.assert_allclose(out[0, 0], x[0, 0], rtol=1e-15)
    for i in range(1, T):
        z0, z1 = g[0, i - 1] + bias[0], g[0, i] + bias[1]
        w1 = 1.0 / (1.0 + np.exp(z0 - z1))
        np.testing.assert_allclose(out[0, i], w1 * x[0, i] + (1 - w1) * x[0, i - 1], rtol=1e-13)


def test_entries_are_convex_combinations_of_their_window(oracle):
    m, B, T, D = 4, 2, 33, 6
    x, g = _rand((B, T, D), 8), _rand((B, T, D), 9, 3.0)
    out = oracle.compress_overlap(x, g, _rand((8, D), 10), m)
    for b in range(B):
        for i in range(T // m):
            win = x[b, max(0, 4 * i - 4):4 * i + 4]
            assert (out[b, i] >= win.min(0) - 1e-12).all() and (out[b, i] <= win.max(0) + 1e-12).all()


@pytest.mark.parametrize("m", [1, 3, 4])
def test_streaming_ring_matches_whole_sequence(oracle, m):
    rng = np.random.default_rng(20 + m)
    B, D, T = 3, 4, 6 * m + 1
    x = rng.standard_normal((B, T, D))
    g = rng.standard_normal((B, T, D)) * 2
    bias = rng.standard_normal((2 * m, D))
    want = oracle.compress_overlap(x, g, bias, m)
    rx, rg = np.zeros((B, 2 * m, D)), np.zeros((B, 2 * m, D))
    pool = np.full((B, T // m, D), np.nan)
    start = [0, 1, m + 2]
    for step in range(T + max(start)):
        pos = np.full(B, -1, np.int32)
        xt, gt = np.full((B, D), np.nan), np.full((B, D), np.nan)
        for b in range(B):
            if start[b] <= step < start[b] + T:
                pos[b] = step - start[b]
                xt[b], gt[b] = x[b, pos[b]], g[b, pos[b]]
        oracle.compress_append_overlap(xt, gt, bias, rx, rg, pos, pool, m)
    np.testing.assert_allclose(pool, want, rtol=0, atol=1e-13)
