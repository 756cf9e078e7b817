"""GPU parity: hsa_compress against the oracle compressor.

fp32 cases must agree to 1e-5 (max-abs and max-abs / max|ref|), bf16 cases
to 2e-2 / 1e-2 (the bf16 output rounding alone is up to 2^-9 relative)."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, TOL_FP32, compare, note

pytestmark = pytest.mark.gpu


def _inputs(B, T, D, m, dt, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, T, D, generator=g).to(dt)
    gate = torch.randn(B, T, D, generator=g).to(dt)
    bias = (torch.randn(m, D, generator=g) * 0.1).to(dt)
    return x, gate, bias


CASES = [
    # (m, T, B, D, dtype) -- ragged T, one-thread and split-block paths
    (1, 5, 2, 16, torch.float32),
    (2, 9, 3, 8, torch.float32),
    (3, 20, 2, 24, torch.float32),
    (4, 1030, 2, 128, torch.float32),
    (5, 40, 2, 24, torch.float32),   # four threads per unit: one part of the block empty
    (7, 50, 1, 16, torch.float32),   # parts of 2, 2, 2 and 1 rows
    (16, 100, 1, 64, torch.float32),
    (17, 70, 2, 32, torch.float32),
    (64, 300, 2, 16, torch.float32),
    (200, 450, 1, 40, torch.float32),
    (1024, 2048, 1, 8, torch.float32),
    (4, 1027, 3, 576, torch.bfloat16),
    (128, 700, 2, 576, torch.bfloat16),
    (128, 1024, 1, 8, torch.bfloat16),
]


@pytest.mark.parametrize("m,T,B,D,dt", CASES)
def test_compress_matches_oracle(oracle, m, T, B, D, dt):
    import hybrid_sparse_compressed_amd as hsa

    x, gate, bias = _inputs(B, T, D, m, dt, seed=100 + m + T)
    note("compress m=%d T=%d B=%d D=%d %s" % (m, T, B, D, dt))
    got = hsa.hsa_compress(x.cuda(), gate.cuda(), bias.cuda(), m)
    torch.cuda.synchronize()
    ref = oracle.compress(x, gate, bias, m)
    compare(got, ref, TOL_FP32 if dt == torch.float32 else TOL_BF16, "compress m=%d" % m)


def test_tiny_fp32_workload(oracle):
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.tiny_fp32_decode("cpu")
    note("compress tiny_fp32_decode")
    got = hsa.hsa_compress(w["x"].cuda(), w["gate"].cuda(), w["bias"].cuda(), 4)
    ref = oracle.compress(w["x"], w["gate"], w["bias"], 4)
    assert got.shape == (1, 256, 128)
    compare(got, ref, TOL_FP32, "tiny compress")


def test_prefill_full_size_compress(oracle):
    """8 x 32768 x 576 bf16, C4 and C128 calls; two sequences checked against the oracle."""
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.prefill("cuda")
    note("compress prefill_32k full size")
    c4 = hsa.hsa_compress(w["x"], w["gate4"], w["bias4"], 4)
    c128 = hsa.hsa_compress(w["x"], w["gate128"], w["bias128"], 128)
    torch.cuda.synchronize()
    assert c4.shape == (8, 8192, 576) and c128.shape == (8, 256, 576)
    for b in (0, 7):
        xs = w["x"][b: b + 1].cpu()
        ref4 = oracle.compress(xs, w["gate4"][b: b + 1].cpu(), w["bias4"].cpu(), 4)
        compare(c4[b: b + 1], ref4, TOL_BF16, "prefill C4 seq %d" % b)
        ref128 = oracle.compress(xs, w["gate128"][b: b + 1].cpu(), w["bias128"].cpu(), 128)
        compare(c128[b: b + 1], ref128, TOL_BF16, "prefill C128 seq %d" % b)


def test_compress_is_deterministic():
    import hybrid_sparse_compressed_amd as hsa

    x, gate, bias = _inputs(2, 4096, 576, 128, torch.bfloat16, seed=5)
    x, gate, bias = x.cuda(), gate.cuda(), bias.cuda()
    note("compress determinism")
    a = hsa.hsa_compress(x, gate, bias, 128)
    b = hsa.hsa_compress(x, gate, bias, 128)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_uniform_gates_give_block_mean_on_gpu():
    import hybrid_sparse_compressed_amd as hsa

    B, T, D, m = 2, 512, 64, 4
    x = torch.randn(B, T, D, generator=torch.Generator().manual_seed(3))
    gate = torch.zeros(B, T, D)
    bias = torch.zeros(m, D)
    note("compress uniform gates")
    got = hsa.hsa_compress(x.cuda(), gate.cuda(), bias.cuda(), m).cpu().double().numpy()
    want = x.double().numpy().reshape(B, T // m, m, D).mean(axis=2)
    assert np.abs(got - want).max() <= 1e-6
