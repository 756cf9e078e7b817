"""GPU parity: indexer scores and the selection they lead to.

Scores: each GPU score must lie within the fp32 error bound of the oracle's
fp64 score, |err_s| <= (H_I + d_I) * 2^-24 * A_s with
A_s = sum_e (sum_h |q_idx[h,e]|) * |k_idx[s,e]| (the heads are summed first,
then one dot product of length d_I, both in fp32).  Equal key rows must give
bitwise-equal scores.  Selection: the GPU set must overlap the oracle's set
(oracle scores rounded to fp32, oracle select) by >= 99.9 %."""
import numpy as np
import pytest
import torch

from helpers import note, to_np

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _check_scores(got, ref, q_idx, k_idx, q_seq, n_cand):
    g = got.detach().cpu().numpy().astype(np.float64)
    qa = np.abs(to_np(q_idx)).sum(axis=1)  # [Nq, d_I]
    ka = np.abs(to_np(k_idx))              # [B, S, d_I]
    H_I, d_I = q_idx.shape[1], q_idx.shape[2]
    worst = 0.0
    for i in range(g.shape[0]):
        n = int(n_cand[i])
        b = int(q_seq[i]) if q_seq is not None else i
        bound = (H_I + d_I) * U * (ka[b, :n] @ qa[i]) * 1.01 + 1e-30
        err = np.abs(g[i, :n] - ref[i, :n])
        assert np.all(err <= bound), "score %d: worst ratio %.3g" % (i, (err / bound).max())
        worst = max(worst, float((err / bound).max()) if n else 0.0)
    return worst


def _overlap(got_idx, want_idx):
    inter = tot = 0
    for g, w in zip(got_idx, want_idx):
        ws = set(int(v) for v in w if v >= 0)
        gs = set(int(v) for v in g if v >= 0)
        inter += len(ws & gs)
        tot += len(ws)
        assert len(gs) == len(ws)
    return inter / max(tot, 1)


def test_tiny_fp32_scores_and_selection(oracle):
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.tiny_fp32_decode("cpu")
    note("index tiny_fp32_decode")
    s, idx = hsa.hsa_index_topk(w["q_idx"].cuda(), w["k_idx"].cuda(), w["n_cand"], 64)
    torch.cuda.synchronize()
    ref = oracle.index_scores(w["q_idx"], w["k_idx"], w["n_cand"].numpy())
    _check_scores(s, ref, w["q_idx"], w["k_idx"], None, w["n_cand"].numpy())
    want = oracle.topk(ref.astype(np.float32), w["n_cand"].numpy(), 64)
    assert _overlap(idx.cpu().numpy(), want) == 1.0


@pytest.mark.parametrize("S_max,k", [(3000, 64), (20000, 100)])
def test_ragged_queries_and_sequence_routing(oracle, S_max, k):
    import hybrid_sparse_compressed_amd as hsa

    g = torch.Generator().manual_seed(S_max)
    B, Nq, H_I, d_I = 3, 12, 64, 128
    q_idx = torch.randn(Nq, H_I, d_I, generator=g).to(torch.bfloat16)
    k_idx = torch.randn(B, S_max, d_I, generator=g).to(torch.bfloat16)
    q_seq = torch.randint(0, B, (Nq,), generator=g, dtype=torch.int32)
    n_cand = torch.randint(0, S_max + 1, (Nq,), generator=g, dtype=torch.int32)
    n_cand[0], n_cand[1], n_cand[2] = 0, k, S_max
    note("index ragged S_max=%d k=%d" % (S_max, k))
    s, idx = hsa.hsa_index_topk(q_idx.cuda(), k_idx.cuda(), n_cand, k, q_seq=q_seq)
    torch.cuda.synchronize()
    ref = oracle.index_scores(q_idx, k_idx, n_cand.numpy(), q_seq=q_seq.numpy())
    _check_scores(s, ref, q_idx, k_idx, q_seq.numpy(), n_cand.numpy())
    want = oracle.topk(ref.astype(np.float32), n_cand.numpy(), k)
    assert _overlap(idx.cpu().numpy(), want) >= 0.999


@pytest.mark.parametrize("name", ["c4_decode_64k", "c4_decode_1m"])
def test_full_size_decode_selection(oracle, name):
    """Full-size indexer + select; the oracle's rank-512 row is copied to three more
    positions (one lower, two higher index) so a tie straddles the boundary."""
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.c4_decode(name, "cuda")
    k, S = w["cfg"]["k"], w["S"]
    q_idx_c, n_cand = w["q_idx"].cpu(), w["n_cand"].cpu().numpy()
    k_c = w["k_idx"].cpu()
    ref = oracle.index_scores(q_idx_c, k_c, n_cand)
    sel = oracle.topk(ref.astype(np.float32), n_cand, k)
    rng = np.random.default_rng(3)
    for b in range(w["cfg"]["B"]):
        chosen = sel[b]
        kth = chosen[np.argmin(ref[b, chosen])]
        lower = rng.integers(0, kth) if kth > 0 else kth
        higher = rng.integers(kth + 1, S, size=2)
        for p in [lower, *higher]:
            k_c[b, p] = k_c[b, kth]
    w["k_idx"].copy_(k_c)
    ref = oracle.index_scores(q_idx_c, k_c, n_cand)
    want = oracle.topk(ref.astype(np.float32), n_cand, k)
    note("index full size %s" % name)
    s, idx = hsa.hsa_index_topk(w["q_idx"], w["k_idx"], w["n_cand"], k)
    torch.cuda.synchronize()
    worst = _check_scores(s, ref, q_idx_c, k_c, None, n_cand)
    ov = _overlap(idx.cpu().numpy(), want)
    print("score error / bound (worst) = %.3g, selected-set overlap = %.6f" % (worst, ov))
    assert ov >= 0.999
    # planted duplicate rows score bitwise-equal on the GPU
    sg = s.cpu().numpy()
    for b in range(w["cfg"]["B"]):
        rows = k_c[b].view(torch.int16).numpy()
        _, first, inv = np.unique(rows, axis=0, return_index=True, return_inverse=True)
        dup = np.nonzero(first[inv.ravel()] != np.arange(S))[0]
        assert len(dup) > 0
        np.testing.assert_array_equal(sg[b, dup], sg[b, first[inv.ravel()][dup]])


@pytest.mark.parametrize("dt,d_I,S_max", [(torch.bfloat16, 64, 5000), (torch.bfloat16, 256, 14000),
                                          (torch.float32, 32, 3000), (torch.float32, 128, 13000),
                                          (torch.bfloat16, 128, 777)])
def test_scores_all_row_widths(oracle, dt, d_I, S_max):
    """128-, 256- and 512-byte key rows (8, 16 and 32 lanes per row), both select paths."""
    import hybrid_sparse_compressed_amd as hsa

    g = torch.Generator().manual_seed(d_I + S_max)
    B, Nq, H_I, k = 2, 5, 7, 96
    q_idx = torch.randn(Nq, H_I, d_I, generator=g).to(dt)
    k_idx = torch.randn(B, S_max, d_I, generator=g).to(dt)
    k_idx[1, 5:9] = k_idx[1, 100]  # equal rows at different positions of a batch
    q_seq = torch.tensor([0, 1, 1, 0, 1], dtype=torch.int32)
    n_cand = torch.tensor([S_max, S_max - 1, 33, 0, S_max // 2], dtype=torch.int32)
    note("index widths %s d_I=%d S=%d" % (dt, d_I, S_max))
    s, idx = hsa.hsa_index_topk(q_idx.cuda(), k_idx.cuda(), n_cand, k, q_seq=q_seq)
    torch.cuda.synchronize()
    ref = oracle.index_scores(q_idx, k_idx, n_cand.numpy(), q_seq=q_seq.numpy())
    _check_scores(s, ref, q_idx, k_idx, q_seq.numpy(), n_cand.numpy())
    sg = s.cpu().numpy()
    for i in (1, 4):  # queries of sequence 1 that see row 100
        assert np.all(sg[i, 5:9] == sg[i, 100])
    want = oracle.topk(ref.astype(np.float32), n_cand.numpy(), k)
    assert _overlap(idx.cpu().numpy(), want) >= 0.999


@pytest.mark.parametrize("d_I,S_max,routing", [(128, 3001, "mixed"), (64, 2048, "prefill"),
                                               (256, 1500, "prefill"), (128, 777, "mixed")])
def test_many_queries_per_sequence(oracle, d_I, S_max, routing):
    """Many queries per sequence (the matrix-product scoring path): workgroups of 32
    queries with one or several sequences, causal or random candidate counts, a key
    width of 64, 128 or 256, S_max not a multiple of the key block, equal key rows."""
    import hybrid_sparse_compressed_amd as hsa

    g = torch.Generator().manual_seed(d_I * 7 + S_max)
    B, Nq, H_I, k = 3, 100, 64, 64
    q_idx = torch.randn(Nq, H_I, d_I, generator=g).to(torch.bfloat16)
    k_idx = torch.randn(B, S_max, d_I, generator=g).to(torch.bfloat16)
    k_idx[2, 40:45] = k_idx[2, 300]
    if routing == "mixed":
        q_seq = torch.randint(0, B, (Nq,), generator=g, dtype=torch.int32)
        n_cand = torch.randint(0, S_max + 1, (Nq,), generator=g, dtype=torch.int32)
        n_cand[:4] = torch.tensor([0, 1, k, S_max], dtype=torch.int32)
    else:  # sequence-major, candidate count growing with the position
        q_seq = (torch.arange(Nq) * B // Nq).to(torch.int32)
        n_cand = torch.clamp((torch.arange(Nq) * 37) % (S_max + 1), max=S_max).to(torch.int32)
    note("index many queries d_I=%d S=%d %s" % (d_I, S_max, routing))
    s, idx = hsa.hsa_index_topk(q_idx.cuda(), k_idx.cuda(), n_cand, k, q_seq=q_seq)
    torch.cuda.synchronize()
    ref = oracle.index_scores(q_idx, k_idx, n_cand.numpy(), q_seq=q_seq.numpy())
    worst = _check_scores(s, ref, q_idx, k_idx, q_seq.numpy(), n_cand.numpy())
    want = oracle.topk(ref.astype(np.float32), n_cand.numpy(), k)
    ov = _overlap(idx.cpu().numpy(), want)
    print("score error / bound (worst) = %.3g, overlap = %.6f" % (worst, ov))
    assert ov >= 0.999
    sg = s.cpu().numpy()
    for i in range(Nq):  # equal key rows score bitwise-equal
        if int(q_seq[i]) == 2 and int(n_cand[i]) > 300:
            assert np.all(sg[i, 40:45] == sg[i, 300])


def test_prefill_32k_indexer_sampled(oracle):
    """Full-size prefill indexer: 8 x 2048 query positions over 8 x 8192 C4 keys
    (causal candidate counts); 24 sampled queries (first and last of sequences
    included) checked against the oracle's scores and selection."""
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.prefill("cuda")
    k = 512
    note("index prefill_32k full size")
    s, idx = hsa.hsa_index_topk(w["q_idx"], w["k_idx"], w["n_cand"], k, q_seq=w["q_seq"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    Nq = w["q_idx"].shape[0]
    sel = sorted(set([0, 2047, 2048, Nq - 1] + rng.choice(Nq, 20, replace=False).tolist()))
    qs = w["q_seq"].cpu()[sel]
    nc = w["n_cand"].cpu()[sel]
    q_sub = w["q_idx"][sel].cpu()
    ref = oracle.index_scores(q_sub, w["k_idx"].cpu(), nc.numpy(), q_seq=qs.numpy())
    worst = _check_scores(s[sel], ref, q_sub, w["k_idx"].cpu(), qs.numpy(), nc.numpy())
    want = oracle.topk(ref.astype(np.float32), nc.numpy(), k)
    ov = _overlap(idx[sel].cpu().numpy(), want)
    print("score error / bound (worst) = %.3g, overlap = %.6f" % (worst, ov))
    assert ov >= 0.999


@pytest.mark.parametrize("S_max,Nq", [(3000, 12), (20000, 12), (2048, 100)])
def test_query_routed_outside_the_batch_has_no_candidates(oracle, S_max, Nq):
    """A q_seq entry outside [0, B) (here -1 and B) gives that query no candidates:
    its top-k row is all -1 on every select path (one workgroup per row, the
    multi-workgroup select, and the matrix-product scoring with 100 queries), and
    the other queries are unaffected (exact against the oracle's select on the
    GPU's own scores)."""
    import hybrid_sparse_compressed_amd as hsa

    g = torch.Generator().manual_seed(S_max + Nq)
    B, H_I, d_I, k = 3, 64, 128, 64
    q_idx = torch.randn(Nq, H_I, d_I, generator=g).to(torch.bfloat16)
    k_idx = torch.randn(B, S_max, d_I, generator=g).to(torch.bfloat16)
    q_seq = torch.randint(0, B, (Nq,), generator=g, dtype=torch.int32)
    q_seq[1], q_seq[5] = -1, B
    n_cand = torch.full((Nq,), S_max, dtype=torch.int32)
    note("index bad q_seq S_max=%d Nq=%d" % (S_max, Nq))
    s, idx = hsa.hsa_index_topk(q_idx.cuda(), k_idx.cuda(), n_cand, k, q_seq=q_seq)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert (got[1] == -1).all() and (got[5] == -1).all()
    ok = [i for i in range(Nq) if i not in (1, 5)]
    nc = n_cand.numpy()[ok]
    np.testing.assert_array_equal(got[ok], oracle.topk(s.cpu().numpy()[ok], nc, k))
    ref = oracle.index_scores(q_idx[ok], k_idx, nc, q_seq=q_seq.numpy()[ok])
    _check_scores(s[ok], ref, q_idx[ok], k_idx, q_seq.numpy()[ok], nc)
