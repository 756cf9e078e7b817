"""GPU parity: the overlapping-block compressor (hsa_compress_overlap) and its
decode-time ring (hsa_compress_append_overlap), a method variant: entry i over
blocks i-1 and i with a bias of 2m rows, entry 0 over its own block.

Against the oracle: every entry, fp32 at 1e-5 and bf16 at the bf16 bound, for
m = 1..4, ragged T, and the full prefill_32k C4 shape.  Streaming tokens one
call at a time through the ring of 2m reproduces the whole-sequence kernel's
entries bit for bit (same arithmetic in the same order) and the oracle's."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, TOL_FP32, compare, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_small_against_oracle(oracle, m, dtype):
    import hybrid_sparse_compressed_amd as hsa

    g = torch.Generator().manual_seed(40 + m)
    B, T, D = 2, 23 * m + (m - 1), 576 if dtype == torch.bfloat16 else 128
    x = torch.randn(B, T, D, generator=g).to(dtype)
    gt = (torch.randn(B, T, D, generator=g) * 2).to(dtype)
    bias = (torch.randn(2 * m, D, generator=g) * 0.5).to(dtype)
    note("compress_overlap m=%d %s" % (m, dtype))
    out = hsa.hsa_compress_overlap(x.cuda(), gt.cuda(), bias.cuda(), m)
    torch.cuda.synchronize()
    ref = oracle.compress_overlap(x, gt, bias, m)
    print(compare(out, ref, TOL_FP32 if dtype == torch.float32 else TOL_BF16, "overlap m=%d" % m))


def test_prefill_32k_c4_overlap(oracle):
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.prefill("cuda")
    x, g4 = w["x"], w["gate4"]
    D = x.shape[2]
    gen = torch.Generator(device="cuda").manual_seed(8)
    bias = (torch.randn(8, D, device="cuda", generator=gen) * 0.1).to(torch.bfloat16)
    note("compress_overlap prefill_32k C4")
    out = hsa.hsa_compress_overlap(x, g4, bias, 4)
    torch.cuda.synchronize()
    # two sequences in full (every entry of them), against the oracle
    for b in (0, 7):
        ref = oracle.compress_overlap(x[b:b + 1].cpu(), g4[b:b + 1].cpu(), bias.cpu(), 4)
        print(compare(out[b:b + 1], ref, TOL_BF16, "prefill_32k overlap seq %d" % b))


@pytest.mark.parametrize("m", [1, 4])
def test_streaming_equals_whole_sequence(oracle, m):
    import hybrid_sparse_compressed_amd as hsa

    g = torch.Generator().manual_seed(70 + m)
    B, D, T, S = 3, 576, 9 * m + 2, 64
    bf = torch.bfloat16
    x = torch.randn(B, T, D, generator=g).to(bf).cuda()
    gt = (torch.randn(B, T, D, generator=g) * 2).to(bf).cuda()
    bias = (torch.randn(2 * m, D, generator=g) * 0.5).to(bf).cuda()
    rx = torch.randn(B, 2 * m, D, generator=g).to(bf).cuda()  # garbage the ring must overwrite first
    rg = torch.randn(B, 2 * m, D, generator=g).to(bf).cuda()
    pool = torch.zeros(B, S, D, dtype=bf, device="cuda")
    start = [0, 1, m + 2]
    note("compress_append_overlap streaming m=%d" % m)
    for step in range(T + max(start)):
        pos = torch.tensor([step - start[b] if start[b] <= step < start[b] + T else -1 for b in range(B)],
                           dtype=torch.int32)
        xt = torch.stack([x[b, max(0, min(T - 1, int(pos[b])))] for b in range(B)])
        gg = torch.stack([gt[b, max(0, min(T - 1, int(pos[b])))] for b in range(B)])
        hsa.hsa_compress_append_overlap(xt.contiguous(), gg.contiguous(), bias, rx, rg, pos.cuda(), pool)
    torch.cuda.synchronize()
    whole = hsa.hsa_compress_overlap(x, gt, bias, m)
    torch.cuda.synchronize()
    nblk = T // m
    assert torch.equal(pool[:, :nblk], whole)
    assert not pool[:, nblk:].any()
    ref = oracle.compress_overlap(x.cpu(), gt.cpu(), bias.cpu(), m)
    print(compare(pool[:, :nblk], ref, TOL_BF16, "streamed overlap m=%d" % m))
