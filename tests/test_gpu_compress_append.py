"""GPU parity: hsa_compress_append (decode-time compression state) against the
oracle, streamed token by token.

Ring contents are byte copies of the tokens and must match the oracle's ring
exactly; pool rows of completed blocks meet the compressor's tolerances (fp32
1e-5, bf16 2e-2 / 1e-2); pool rows of open blocks must keep their sentinel."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, TOL_FP32, compare, note

pytestmark = pytest.mark.gpu


def _tokens(B, T, D, m, dt, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, T, D, generator=g).to(dt)
    gate = torch.randn(B, T, D, generator=g).to(dt)
    bias = (torch.randn(m, D, generator=g) * 0.1).to(dt)
    return x, gate, bias


def _stream(oracle, m, T, B, D, dt, S_max, seed):
    """Feed T tokens per sequence, sequence b starting after b steps (so blocks
    complete at different calls) and sitting idle (pos = -1) on every
    third call after it started; returns GPU and oracle states."""
    import hybrid_sparse_compressed_amd as hsa

    x, gate, bias = _tokens(B, T, D, m, dt, seed)
    dev = "cuda"
    ring_x = torch.zeros(B, m, D, dtype=dt, device=dev)
    ring_g = torch.zeros(B, m, D, dtype=dt, device=dev)
    pool = torch.full((B, S_max, D), float("nan"), dtype=dt, device=dev)
    o_rx = torch.zeros(B, m, D, dtype=dt)
    o_rg = torch.zeros(B, m, D, dtype=dt)
    o_pool = np.full((B, S_max, D), np.nan)
    bias_d = bias.to(dev)
    nxt = [0] * B
    call = 0
    while min(nxt) < T:
        pos = np.full(B, -1, np.int32)
        xt = torch.full((B, D), float("nan"), dtype=dt)
        gt = torch.full((B, D), float("nan"), dtype=dt)
        for b in range(B):
            if call >= b and nxt[b] < T and (call - b) % 3 != 2:
                pos[b] = nxt[b]
                xt[b] = x[b, nxt[b]]
                gt[b] = gate[b, nxt[b]]
                nxt[b] += 1
        hsa.hsa_compress_append(xt.to(dev), gt.to(dev), bias_d, ring_x, ring_g,
                                torch.from_numpy(pos).to(dev), pool)
        oracle.compress_append(xt, gt, bias, o_rx, o_rg, pos, o_pool, m)
        call += 1
    torch.cuda.synchronize()
    return ring_x.cpu(), ring_g.cpu(), pool.cpu(), o_rx, o_rg, o_pool, x, gate, bias


CASES = [
    # (m, T, B, D, dtype, S_max)
    (1, 6, 2, 16, torch.float32, 6),
    (3, 20, 3, 24, torch.float32, 6),
    (4, 23, 5, 576, torch.bfloat16, 5),
    (4, 9, 2, 4096, torch.bfloat16, 2),        # more chunks than one workgroup holds
    (16, 40, 2, 64, torch.float32, 2),         # third block falls past the pool
    (100, 205, 2, 40, torch.float32, 2),       # rows not a multiple of the parts
    (128, 263, 3, 576, torch.bfloat16, 2),
    (1024, 1027, 1, 8, torch.float32, 1),
]


@pytest.mark.parametrize("m,T,B,D,dt,S_max", CASES)
def test_streamed_append_matches_oracle(oracle, m, T, B, D, dt, S_max):
    note("compress_append m=%d T=%d B=%d D=%d %s S_max=%d" % (m, T, B, D, dt, S_max))
    rx, rg, pool, o_rx, o_rg, o_pool, x, gate, bias = _stream(oracle, m, T, B, D, dt, S_max,
                                                             seed=7 * m + T)
    assert torch.equal(rx.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       o_rx.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
    assert torch.equal(rg.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       o_rg.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
    done = min(T // m, S_max)
    tol = TOL_FP32 if dt == torch.float32 else TOL_BF16
    compare(pool[:, :done], o_pool[:, :done], tol, "append pool m=%d" % m)
    assert torch.isnan(pool[:, done:].float()).all(), "rows of open blocks were written"
    # the whole-sequence compressor gives the same entries
    whole = oracle.compress(x, gate, bias, m)
    compare(pool[:, :done], whole[:, :done], tol, "append vs whole m=%d" % m)


@pytest.mark.parametrize("name,B,m,n_blocks", [("c4_decode_1m", 4, 4, 262144),
                                                ("c128_dense_decode", 32, 128, 1024)])
def test_completing_call_at_decode_batch(oracle, name, B, m, n_blocks):
    """Every sequence of a decode batch completes a block in the same call, at
    positions spread over the whole context (4 x 1M tokens at C4, 32 x 128K
    at C128), into a pool of the full size; rings pre-filled with random tokens."""
    import hybrid_sparse_compressed_amd as hsa

    D, dt = 576, torch.bfloat16
    g = torch.Generator().manual_seed(B * 1000 + m)
    ring_x = torch.randn(B, m, D, generator=g).to(dt)
    ring_g = torch.randn(B, m, D, generator=g).to(dt)
    xt = torch.randn(B, D, generator=g).to(dt)
    gt = torch.randn(B, D, generator=g).to(dt)
    bias = (torch.randn(m, D, generator=g) * 0.1).to(dt)
    blocks = torch.randint(0, n_blocks, (B,), generator=g)
    blocks[0] = n_blocks - 1  # the pool's last row
    pos = (blocks * m + m - 1).to(torch.int32)
    S_max = n_blocks
    note("compress_append completing call %s B=%d m=%d S_max=%d" % (name, B, m, S_max))
    pool = torch.zeros(B, S_max, D, dtype=dt, device="cuda")
    rx_d, rg_d = ring_x.cuda(), ring_g.cuda()
    hsa.hsa_compress_append(xt.cuda(), gt.cuda(), bias.cuda(), rx_d, rg_d, pos.cuda(), pool)
    torch.cuda.synchronize()
    o_pool = np.zeros((B, S_max, D))  # zero pages: only the written rows get memory
    o_rx, o_rg = ring_x.clone(), ring_g.clone()
    wrote = oracle.compress_append(xt, gt, bias, o_rx, o_rg, pos.numpy(), o_pool, m)
    assert len(wrote) == B
    rows = torch.tensor([r for _, r in wrote])
    got = pool[torch.arange(B), rows.cuda()].cpu()
    compare(got, o_pool[np.arange(B), rows.numpy()], TOL_BF16, name)
    assert torch.equal(rx_d.cpu().view(torch.int16), o_rx.view(torch.int16))
    assert torch.equal(rg_d.cpu().view(torch.int16), o_rg.view(torch.int16))
    # nothing else in the pool was written
    assert torch.count_nonzero(pool).item() == torch.count_nonzero(got).item()


def test_rejects_bad_arguments():
    import hybrid_sparse_compressed_amd as hsa

    lib = hsa.lib
    dev = "cuda"
    a = torch.zeros(2, 4, 16, dtype=torch.float32, device=dev)
    pos = torch.zeros(2, dtype=torch.int32, device=dev)
    p = a.data_ptr()
    note("compress_append argument checks")
    # m out of range, S_max < 1, D not a multiple of 16 bytes, null pointer
    assert lib.hsa_compress_append(0, p, p, p, p, p, pos.data_ptr(), p, 2, 16, 0, 1, None) == 1
    assert lib.hsa_compress_append(0, p, p, p, p, p, pos.data_ptr(), p, 2, 16, 4, 0, None) == 1
    assert lib.hsa_compress_append(0, p, p, p, p, p, pos.data_ptr(), p, 2, 3, 4, 1, None) == 2
    assert lib.hsa_compress_append(0, p, p, p, p, p, None, p, 2, 16, 4, 1, None) == 1
