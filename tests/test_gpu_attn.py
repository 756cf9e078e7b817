"""GPU parity: hsa_attn_decode / hsa_attn_prefill against the oracle on the same
inputs (index lists come from the oracle or from a seeded draw, never from
the GPU path).  fp32: 1e-5; bf16: 2e-2 max-abs and 1e-2 of max|ref|."""
import math

import numpy as np
import pytest
import torch

from helpers import TOL_BF16, TOL_FP32, compare, note

pytestmark = pytest.mark.gpu


def _tol(dt):
    return TOL_FP32 if dt == torch.float32 else TOL_BF16


def _decode(q, swa, swa_len, comp, comp_len, scale, d_v, idx=None):
    import hybrid_sparse_compressed_amd as hsa

    o, lse = hsa.hsa_attn_decode(q.cuda(), swa.cuda(), swa_len, comp.cuda(), comp_len, scale, d_v,
                                 comp_idx=idx)
    torch.cuda.synchronize()
    return o, lse


def _check_decode(oracle, q, swa, swa_len, comp, comp_len, scale, d_v, idx, what):
    note("decode " + what)
    o, lse = _decode(q, swa, swa_len, comp, comp_len, scale, d_v, idx)
    ro, rl = oracle.attn_decode(q, swa, np.asarray(swa_len), comp, np.asarray(comp_len), scale,
                                d_v, comp_idx=None if idx is None else np.asarray(idx))
    st = compare(o, ro, _tol(q.dtype), what + " out")
    compare(lse, rl, TOL_FP32 if q.dtype == torch.float32 else (1e-3, 1e-4), what + " lse")
    return st


def _rand(shape, dt, g):
    return torch.randn(*shape, generator=g).to(dt)


@pytest.mark.parametrize("dt,d_qk,d_v,H", [(torch.bfloat16, 576, 512, 64),
                                           (torch.bfloat16, 576, 512, 40),
                                           (torch.bfloat16, 128, 128, 16),
                                           (torch.float32, 128, 128, 8)])
def test_decode_ragged_sparse_and_dense(oracle, dt, d_qk, d_v, H):
    g = torch.Generator().manual_seed(d_qk + H)
    B, W, S, k = 3, 128, 200, 64
    q = _rand((B, H, d_qk), dt, g)
    swa = _rand((B, W, d_qk), dt, g)
    comp = _rand((B, S, d_qk), dt, g)
    swa_len = torch.tensor([128, 5, 1], dtype=torch.int32)
    comp_len = torch.tensor([150, 0, 37], dtype=torch.int32)
    idx = torch.full((B, k), -1, dtype=torch.int32)
    for b in range(B):
        r = torch.randperm(S, generator=g)[: k - 8].to(torch.int32)
        idx[b, : k - 8] = r          # some beyond comp_len (skipped), -1 padding at the end
        idx[b, k - 8] = r[0]         # a duplicate (counted twice)
    # poison everything the row sets exclude
    for b in range(B):
        swa[b, int(swa_len[b]):] = float("nan")
        comp[b, int(comp_len[b]):] = float("nan")
    scale = 1.0 / math.sqrt(d_qk)
    _check_decode(oracle, q, swa, swa_len, comp, comp_len, scale, d_v, idx, "sparse %s H=%d" % (dt, H))
    _check_decode(oracle, q, swa, swa_len, comp, comp_len, scale, d_v, None, "dense %s H=%d" % (dt, H))


def test_decode_empty_row_set():
    g = torch.Generator().manual_seed(1)
    q = _rand((2, 64, 576), torch.bfloat16, g)
    swa = _rand((2, 128, 576), torch.bfloat16, g)
    comp = _rand((2, 10, 576), torch.bfloat16, g)
    z = torch.zeros(2, dtype=torch.int32)
    note("decode empty row set")
    o, lse = _decode(q, swa, z, comp, z, 0.04, 512)
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


def test_decode_tiny_fp32_workload(oracle):
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.tiny_fp32_decode("cpu")
    pool = torch.from_numpy(oracle.compress(w["x"], w["gate"], w["bias"], 4)).float()
    sc = oracle.index_scores(w["q_idx"], w["k_idx"], w["n_cand"].numpy())
    idx = torch.from_numpy(oracle.topk(sc.astype(np.float32), w["n_cand"].numpy(), 64))
    _check_decode(oracle, w["q"], w["swa_kv"], w["swa_len"], pool, w["comp_len"], w["scale"], 128,
                  idx, "tiny_fp32_decode")


@pytest.mark.parametrize("name", ["c4_decode_64k", "c4_decode_1m"])
def test_decode_full_size_c4(oracle, name):
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.c4_decode(name, "cuda")
    k = w["cfg"]["k"]
    ref = oracle.index_scores(w["q_idx"].cpu(), w["k_idx"].cpu(), w["n_cand"].cpu().numpy())
    idx = torch.from_numpy(oracle.topk(ref.astype(np.float32), w["n_cand"].cpu().numpy(), k))
    st = _check_decode(oracle, w["q"].cpu(), w["swa_kv"].cpu(), w["swa_len"].cpu(),
                       w["comp_kv"].cpu(), w["comp_len"].cpu(), w["scale"], 512, idx, name)
    print(name, st)


def test_decode_full_size_c128_dense(oracle):
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.c128_dense_decode("cuda")
    st = _check_decode(oracle, w["q"].cpu(), w["swa_kv"].cpu(), w["swa_len"].cpu(),
                       w["comp_kv"].cpu(), w["comp_len"].cpu(), w["scale"], 512, None,
                       "c128_dense_decode")
    print(st)


def test_decode_dense_64_heads_many_splits(oracle):
    """Dense decode with 64 heads and enough rows to use the 64-head workgroups
    (one per split and sequence): ragged window fill and compressed lengths,
    including empty ones, merged over 22 splits."""
    g = torch.Generator().manual_seed(321)
    B, W, S = 8, 128, 4096
    q = _rand((B, 64, 576), torch.bfloat16, g)
    swa = _rand((B, W, 576), torch.bfloat16, g)
    comp = _rand((B, S, 576), torch.bfloat16, g)
    swa_len = torch.tensor([128, 5, 128, 0, 64, 128, 1, 128], dtype=torch.int32)
    comp_len = torch.tensor([4096, 0, 1000, 4096, 17, 2048, 4095, 3000], dtype=torch.int32)
    _check_decode(oracle, q, swa, swa_len, comp, comp_len, 1.0 / 24.0, 512, None,
                  "dense 64-head splits")


def test_decode_dense_64_heads_one_split(oracle):
    """256 sequences of up to 160 rows: the device plan gives each one split of
    up to three tiles (the merge then only normalises)."""
    g = torch.Generator().manual_seed(654)
    B, W, S = 256, 128, 32
    q = _rand((B, 64, 576), torch.bfloat16, g)
    swa = _rand((B, W, 576), torch.bfloat16, g)
    comp = _rand((B, S, 576), torch.bfloat16, g)
    swa_len = torch.randint(1, W + 1, (B,), generator=g, dtype=torch.int32)
    comp_len = torch.randint(0, S + 1, (B,), generator=g, dtype=torch.int32)
    _check_decode(oracle, q, swa, swa_len, comp, comp_len, 1.0 / 24.0, 512, None,
                  "dense 64-head one split")


def test_decode_dense_64_heads_long_and_short(oracle):
    """Three sequences, one 16,384 rows long: the device plan's tiles per split
    are set by the split cap of the longest sequence (129 splits of two tiles
    would exceed 128), the short ones get one or a few splits."""
    g = torch.Generator().manual_seed(987)
    B, W, S = 3, 128, 16384
    q = _rand((B, 64, 576), torch.bfloat16, g)
    swa = _rand((B, W, 576), torch.bfloat16, g)
    comp = _rand((B, S, 576), torch.bfloat16, g)
    swa_len = torch.tensor([128, 7, 128], dtype=torch.int32)
    comp_len = torch.tensor([16384, 100, 9000], dtype=torch.int32)
    _check_decode(oracle, q, swa, swa_len, comp, comp_len, 1.0 / 24.0, 512, None,
                  "dense 64-head long and short")


@pytest.mark.parametrize("B", [64, 65])
def test_decode_dense_64_heads_plan_lane_boundary(oracle, B):
    """64 sequences: each lane of one wave reads one sequence's lengths and the
    split's own lengths come from the lanes; 65: the plan loops over the
    sequences and each split reads its lengths again.  Ragged lengths with
    empty windows and empty compressed pools at both ends of the batch."""
    g = torch.Generator().manual_seed(4100 + B)
    W, S = 128, 192
    q = _rand((B, 64, 576), torch.bfloat16, g)
    swa = _rand((B, W, 576), torch.bfloat16, g)
    comp = _rand((B, S, 576), torch.bfloat16, g)
    swa_len = torch.randint(0, W + 1, (B,), generator=g, dtype=torch.int32)
    comp_len = torch.randint(0, S + 1, (B,), generator=g, dtype=torch.int32)
    swa_len[0], comp_len[0] = 0, S
    swa_len[-1], comp_len[-1] = W, 0
    swa_len[B // 2], comp_len[B // 2] = 1, 1
    _check_decode(oracle, q, swa, swa_len, comp, comp_len, 1.0 / 24.0, 512, None,
                  "dense 64-head plan, %d sequences" % B)


def test_decode_is_deterministic():
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.c128_dense_decode("cuda", B=8)
    note("decode determinism")
    a = _decode(w["q"], w["swa_kv"], w["swa_len"], w["comp_kv"], w["comp_len"], w["scale"], 512)
    b = _decode(w["q"], w["swa_kv"], w["swa_len"], w["comp_kv"], w["comp_len"], w["scale"], 512)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


def _prefill(q, kv, comp, q_start, W, m, scale, d_v, idx):
    import hybrid_sparse_compressed_amd as hsa

    o, lse = hsa.hsa_attn_prefill(q.cuda(), kv.cuda(), comp.cuda(), q_start, W, m, scale, d_v,
                                  comp_idx=idx)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dt,d_qk,d_v,H", [(torch.bfloat16, 576, 512, 64),
                                           (torch.float32, 128, 128, 8)])
@pytest.mark.parametrize("sparse", [True, False])
def test_prefill_small(oracle, dt, d_qk, d_v, H, sparse):
    g = torch.Generator().manual_seed(7 + H)
    n_seq, T, n_q, W, m, k = 2, 300, 50, 128, 4, 16
    q_start = T - n_q
    S = T // m
    q = _rand((n_seq, n_q, H, d_qk), dt, g)
    kv = _rand((n_seq, T, d_qk), dt, g)
    comp = _rand((n_seq, S, d_qk), dt, g)
    idx = None
    if sparse:
        idx = torch.stack([torch.randperm(S, generator=g)[:k] for _ in range(n_seq * n_q)]).to(torch.int32)
        idx[::4, -3:] = -1
    scale = 1.0 / math.sqrt(d_qk)
    note("prefill small %s sparse=%s" % (dt, sparse))
    o, lse = _prefill(q, kv, comp, q_start, W, m, scale, d_v, idx)
    ro, rl = oracle.attn_prefill(q, kv, comp, q_start, W, m, scale, d_v,
                                 comp_idx=None if idx is None else idx.numpy())
    compare(o.reshape(n_seq * n_q, H, d_v), ro, _tol(dt), "prefill out")
    compare(lse, rl, TOL_FP32 if dt == torch.float32 else (1e-3, 1e-4), "prefill lse")


def test_prefill_dense_many_chunks(oracle):
    """Dense prefill with over a thousand visible compressed rows per query: the row
    list of a query is built in several chunks."""
    g = torch.Generator().manual_seed(123)
    n_seq, T, n_q, W, m, H = 1, 4400, 6, 128, 4, 64
    q_start = T - n_q
    q = _rand((n_seq, n_q, H, 576), torch.bfloat16, g)
    kv = _rand((n_seq, T, 576), torch.bfloat16, g)
    comp = _rand((n_seq, T // m, 576), torch.bfloat16, g)
    note("prefill dense many chunks")
    o, lse = _prefill(q, kv, comp, q_start, W, m, 0.04, 512, None)
    ro, rl = oracle.attn_prefill(q, kv, comp, q_start, W, m, 0.04, 512)
    compare(o.reshape(n_seq * n_q, H, 512), ro, TOL_BF16, "prefill dense chunks out")
    compare(lse, rl, (1e-3, 1e-4), "prefill dense chunks lse")


def test_prefill_sparse_long_lists_with_empty_tiles(oracle):
    """64-head prefill with k = 2048 (W + k = 2176 rows: three row-list chunks of
    1024 / 1024 / 128), an empty 64-row tile inside the first chunk, a second chunk
    with no row at all (the tile pipeline restarts after it) and the last chunk
    valid; the tile buffers alternate across all of it."""
    g = torch.Generator().manual_seed(321)
    n_seq, T, n_q, W, m, H, k = 1, 9000, 4, 128, 4, 64, 2048
    q_start = T - n_q
    S = T // m
    q = _rand((n_seq, n_q, H, 576), torch.bfloat16, g)
    kv = _rand((n_seq, T, 576), torch.bfloat16, g)
    comp = _rand((n_seq, S, 576), torch.bfloat16, g)
    idx = torch.stack([torch.randperm(S - 10, generator=g)[:k] for _ in range(n_q)]).to(torch.int32)
    idx[:, 256:320] = -1      # rows W + 256 .. W + 319: tile 6 of the first chunk
    idx[:, 896:1920] = -1     # every row of the second chunk
    idx[1, 1920:] = -1        # query 1: the last chunk empty as well
    note("prefill sparse k=2048 with empty tiles and chunks")
    o, lse = _prefill(q, kv, comp, q_start, W, m, 0.04, 512, idx)
    ro, rl = oracle.attn_prefill(q, kv, comp, q_start, W, m, 0.04, 512, comp_idx=idx.numpy())
    compare(o.reshape(n_q, H, 512), ro, TOL_BF16, "prefill long lists out")
    compare(lse, rl, (1e-3, 1e-4), "prefill long lists lse")


def test_prefill_window_start(oracle):
    """Queries at positions 0..39: windows shorter than W, few visible blocks."""
    g = torch.Generator().manual_seed(99)
    n_seq, T, n_q, W, m, H = 1, 64, 40, 128, 4, 64
    q = _rand((n_seq, n_q, H, 576), torch.bfloat16, g)
    kv = _rand((n_seq, T, 576), torch.bfloat16, g)
    comp = _rand((n_seq, T // m, 576), torch.bfloat16, g)
    note("prefill window start")
    o, lse = _prefill(q, kv, comp, 0, W, m, 0.04, 512, None)
    ro, rl = oracle.attn_prefill(q, kv, comp, 0, W, m, 0.04, 512)
    compare(o.reshape(n_q, H, 512), ro, TOL_BF16, "prefill start out")


def test_prefill_full_size_sampled(oracle):
    """8 x 2048 queries at the end of 32768-token sequences, seeded random visible
    top-512 lists; 64 sampled queries (first/last of each sequence included)."""
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.prefill("cuda")
    n_seq, n_q, T = 8, 2048, 32768
    S = T // 4
    comp = torch.from_numpy(oracle.compress(w["x"][:, :, :].cpu(), w["gate4"].cpu(),
                                            w["bias4"].cpu(), 4)).float().to(torch.bfloat16)
    pos = torch.arange(w["q_start"], T, device="cuda").repeat(n_seq)
    vis = (pos + 1) // 4
    gen = torch.Generator(device="cuda").manual_seed(5)
    r = torch.rand((n_seq * n_q, S), generator=gen, device="cuda")
    r[torch.arange(S, device="cuda")[None, :] >= vis[:, None]] = -1.0
    idx = torch.topk(r, 512, dim=1).indices.to(torch.int32).contiguous()
    note("prefill full size")
    o, lse = _prefill(w["q"], w["x"], comp, w["q_start"], 128, 4, w["scale"], 512, idx)
    rng = np.random.default_rng(0)
    sel = sorted(set([0, n_q - 1, n_q, 8 * n_q - 1] + rng.choice(8 * n_q, 60, replace=False).tolist()))
    ro, rl = oracle.attn_prefill(w["q"].cpu(), w["x"].cpu(), comp, w["q_start"], 128, 4,
                                 w["scale"], 512, comp_idx=idx.cpu().numpy(), sel=sel)
    st = compare(o.reshape(n_seq * n_q, 64, 512)[sel], ro, TOL_BF16, "prefill full out")
    compare(lse[sel], rl, (1e-3, 1e-4), "prefill full lse")
    print(st)
