"""Pins for the oracle's compressor (CPU only).

The oracle computes, per block i of m tokens and channel d,
    c = sum_j softmax_j(gate[m*i+j, d] + bias[j, d]) * x[m*i+j, d].
Each test below checks it against something other than that formula: a
hand-worked example, closed forms (m=1 identity, m=2 logistic weights,
uniform gates -> block mean, one dominant gate -> that token), invariances
and bounds.  A dropped term, a wrong block offset, a transposed bias or a
sign slip in the softmax fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(v):
    if isinstance(v, str):
        if v.startswith("ln"):
            return math.log(float(v[2:]))
        return float(v)
    return float(v)


def test_golden_worked_example(oracle):
    g = json.load(open(os.path.join(GOLDEN, "compress_worked.json")))
    x = np.array([[_num(v) for v in row] for row in g["x"]])[None]
    gate = np.array([[_num(v) for v in row] for row in g["gate"]])[None]
    bias = np.array([[_num(v) for v in row] for row in g["bias"]])
    out = oracle.compress(x, gate, bias, g["m"])
    assert out.shape == (1, 2, 2)
    np.testing.assert_allclose(out[0], np.array(g["expected"]), rtol=0, atol=g["tolerance_abs"])


@pytest.mark.parametrize("m", [1, 4, 128])
def test_uniform_gates_give_block_mean(oracle, m):
    rng = np.random.default_rng(11 + m)
    B, nblk, D = 2, 3, 5
    T = m * nblk + (m - 1)  # plus an incomplete trailing block
    x = rng.standard_normal((B, T, D))
    level = rng.standard_normal((B, nblk + 1, D)) * 3.0
    gate = np.repeat(level, m, axis=1)[:, :T, :]  # constant inside each block
    bias = np.tile(rng.standard_normal((1, D)), (m, 1))  # constant over positions
    out = oracle.compress(x, gate, bias, m)
    want = x[:, : m * nblk, :].reshape(B, nblk, m, D).mean(axis=2)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)


def test_m1_is_identity(oracle):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 7, 3))
    gate = rng.standard_normal((2, 7, 3)) * 10
    bias = rng.standard_normal((1, 3))
    np.testing.assert_allclose(oracle.compress(x, gate, bias, 1), x, rtol=0, atol=1e-15)


def test_m2_logistic_closed_form(oracle):
    # softmax of two logits is the logistic function of their difference.
    rng = np.random.default_rng(2)
    B, T, D = 3, 10, 6
    x = rng.standard_normal((B, T, D))
    gate = rng.standard_normal((B, T, D)) * 2
    bias = rng.standard_normal((2, D))
    z = gate.reshape(B, T // 2, 2, D) + bias[None, None]
    xx = x.reshape(B, T // 2, 2, D)
    sig = lambda t: 1.0 / (1.0 + np.exp(-t))
    want = xx[:, :, 0] * sig(z[:, :, 0] - z[:, :, 1]) + xx[:, :, 1] * sig(z[:, :, 1] - z[:, :, 0])
    np.testing.assert_allclose(oracle.compress(x, gate, bias, 2), want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("m", [4, 128])
def test_dominant_gate_selects_its_token(oracle, m):
    rng = np.random.default_rng(3 + m)
    B, nblk, D = 2, 2, 4
    x = rng.standard_normal((B, m * nblk, D))
    gate = rng.standard_normal((B, m * nblk, D))
    bias = rng.standard_normal((m, D)) * 0.1
    j0 = rng.integers(0, m, size=(B, nblk, D))
    want = np.empty((B, nblk, D))
    for b in range(B):
        for i in range(nblk):
            for d in range(D):
                gate[b, m * i + j0[b, i, d], d] += 80.0
                want[b, i, d] = x[b, m * i + j0[b, i, d], d]
    np.testing.assert_allclose(oracle.compress(x, gate, bias, m), want, rtol=0, atol=1e-12)


def test_bias_is_indexed_by_position_then_channel(oracle):
    # gate 0, bias[j, d] = ln(w[j, d]) -> weights w[:, d] / sum; distinct per channel,
    # so reading bias as [d, j] (or ignoring it) fails.
    m, D = 4, 3
    w = np.array([[1.0, 5.0, 2.0], [2.0, 1.0, 2.0], [3.0, 1.0, 2.0], [4.0, 1.0, 2.0]])
    x = np.arange(m * D, dtype=np.float64).reshape(1, m, D) + 1.0
    out = oracle.compress(x, np.zeros((1, m, D)), np.log(w), m)
    want = (w * x[0]).sum(axis=0) / w.sum(axis=0)
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-12)


def test_block_offsets_and_trailing_block(oracle):
    # x[t] = t with uniform gates: block i averages tokens m*i .. m*i+m-1.
    m, T = 4, 18
    x = np.tile(np.arange(T, dtype=np.float64)[:, None], (1, 2))[None]
    out = oracle.compress(x, np.zeros_like(x), np.zeros((m, 2)), m)
    assert out.shape == (1, T // m, 2)
    want = np.array([m * i + (m - 1) / 2 for i in range(T // m)])
    np.testing.assert_allclose(out[0, :, 0], want, rtol=0, atol=1e-12)
    # tokens 16, 17 (incomplete block) change nothing
    x2, g2 = x.copy(), np.zeros_like(x)
    x2[0, 16:] = 1e6
    g2[0, 16:] = 40.0
    np.testing.assert_array_equal(oracle.compress(x2, g2, np.zeros((m, 2)), m), out)


def test_shift_invariance_linearity_and_bounds(oracle):
    rng = np.random.default_rng(5)
    B, m, nblk, D = 2, 4, 6, 8
    x1 = rng.standard_normal((B, m * nblk, D))
    x2 = rng.standard_normal((B, m * nblk, D))
    gate = rng.standard_normal((B, m * nblk, D))
    bias = rng.standard_normal((m, D)) * 0.1
    c1 = oracle.compress(x1, gate, bias, m)
    # a constant added to all logits of a block leaves the softmax unchanged
    shift = np.repeat(rng.standard_normal((B, nblk, D)) * 30, m, axis=1)
    np.testing.assert_allclose(oracle.compress(x1, gate + shift, bias, m), c1, rtol=0, atol=1e-12)
    # linear in x
    c2 = oracle.compress(x2, gate, bias, m)
    c12 = oracle.compress(2.5 * x1 - x2, gate, bias, m)
    np.testing.assert_allclose(c12, 2.5 * c1 - c2, rtol=0, atol=1e-12)
    # a convex combination of the block's tokens
    xb = x1.reshape(B, nblk, m, D)
    assert np.all(c1 <= xb.max(axis=2) + 1e-12) and np.all(c1 >= xb.min(axis=2) - 1e-12)


def test_bf16_inputs_widen_exactly(oracle):
    import torch

    g = torch.Generator().manual_seed(7)
    x = torch.randn(2, 8, 16, generator=g).to(torch.bfloat16)
    gate = torch.randn(2, 8, 16, generator=g).to(torch.bfloat16)
    bias = (torch.randn(4, 16, generator=g) * 0.1).to(torch.bfloat16)
    a = oracle.compress(x, gate, bias, 4)
    b = oracle.compress(x.double().numpy(), gate.double().numpy(), bias.double().numpy(), 4)
    np.testing.assert_array_equal(a, b)
