"""GPU parity: weighted, activated indexer heads (hsa_index_topk_weighted,
hsa_decode_sparse_weighted), score = sum_h w[q,h] * max(0, q_h . k) on MFMA.

Scores against the oracle's fp64 scores within the fp32 bound of the
arithmetic: each head's dot product of 128 exact bf16 products accumulated in
fp32 (error <= 128 u sum_e |q k|), then 64 weighted terms (error <= 64 u
sum_h |w relu|), u = 2^-24, with a factor 2 of slack.  Top-k bit-exact against
the oracle's select on the GPU's own scores; planted duplicate rows score
bitwise-equal; the fused decode equals the separate calls (scores, top-k) and
its attention meets the bf16 bound against the oracle over the selected rows.
Shapes: the LDS row select, the multi-workgroup select, the fused list path
with 256-row and 2048-row slots (the 1M-context workload), 16 / 48 / 64 heads,
negative weights, ragged candidate counts and query routing."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, compare, note

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
U = 2.0 ** -24


def _case(seed, Nq, B, S, H_I, dev="cuda", neg=True, dup=True):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(Nq, H_I, 128, generator=g).to(BF)
    k = torch.randn(B, S, 128, generator=g).to(BF)
    w = torch.rand(Nq, H_I, generator=g) * 2.0
    if neg:
        w[:, ::5] *= -1.0  # some heads weigh against
    if dup:
        for b in range(B):
            src = torch.randint(0, S, (max(1, S // 100),), generator=g)
            dst = torch.randint(0, S, (max(1, S // 100),), generator=g)
            k[b, dst] = k[b, src]
    return q.to(dev), w.float().to(dev), k.to(dev)


def _check_scores(oracle, q, w, k, n_cand, scores, q_seq=None, rows=None):
    """GPU scores against the oracle within the derived bound (rows: sample of columns)."""
    qc, wc, kc = q.cpu(), w.cpu(), k.cpu()
    nc = np.asarray(n_cand)
    sc = scores.cpu().numpy()
    Nq = qc.shape[0]
    seqs = np.arange(Nq) if q_seq is None else np.asarray(q_seq)
    cols = np.arange(kc.shape[1]) if rows is None else np.asarray(rows)
    ksub = kc[:, cols]
    ref = oracle.index_scores_weighted(qc, wc, ksub, np.minimum(nc, 0) + len(cols),
                                       q_seq=seqs if q_seq is not None else None)
    qa = np.abs(qc.double().numpy())
    wa = np.abs(wc.double().numpy())
    for i in range(Nq):
        kk = np.abs(ksub[seqs[i]].double().numpy())            # [cols, 128]
        a = (qa[i] @ kk.T)                                       # [H_I, cols]: sum_e |q k|
        dots = qc[i].double().numpy() @ ksub[seqs[i]].double().numpy().T
        c = np.maximum(dots, 0.0)
        bound = 2.0 * U * (128.0 * (wa[i] @ a) + 64.0 * (wa[i] @ c)) + 1e-30
        live = cols < nc[i]
        err = np.abs(sc[i, cols][live] - ref[i][live])
        assert (err <= bound[live]).all(), "row %d: max err/bound %.3g" % (i, (err / bound[live]).max())
    return sc


@pytest.mark.parametrize("S,H_I,k,Nq,B", [(4096, 64, 256, 3, 3), (20000, 48, 512, 2, 2),
                                           (9000, 16, 2048, 5, 2)])
def test_index_topk_weighted(oracle, S, H_I, k, Nq, B):
    import hybrid_sparse_compressed_amd as hsa

    q, w, kk = _case(S + H_I, Nq, B, S, H_I)
    n_cand = [S, S - 123, 77, S // 2, 0][:Nq]
    q_seq = [i % B for i in range(Nq)] if Nq > B else None
    note("index_topk_weighted S=%d H_I=%d k=%d" % (S, H_I, k))
    sc, idx = hsa.hsa_index_topk_weighted(q, w, kk, torch.tensor(n_cand, dtype=torch.int32), k,
                                          q_seq=None if q_seq is None else torch.tensor(q_seq, dtype=torch.int32))
    torch.cuda.synchronize()
    scn = _check_scores(oracle, q, w, kk, n_cand, sc, q_seq)
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk(scn, n_cand, k))
    # planted duplicates: equal rows score bitwise-equal
    kc = kk.cpu()
    for i in range(Nq):
        b = i % B if q_seq is not None else i
        rows = kc[b].view(torch.int16).numpy()
        _, first, inv = np.unique(rows, axis=0, return_index=True, return_inverse=True)
        inv = inv.reshape(-1)
        src = first[inv]
        live = (np.arange(S) < n_cand[i]) & (src < n_cand[i])
        np.testing.assert_array_equal(scn[i][live], scn[i][src][live])
        assert (src[live] != np.arange(S)[live]).sum() > 0 or n_cand[i] < 100


@pytest.mark.parametrize("name", ["c4_decode_64k", "c4_decode_1m"])
def test_decode_sparse_weighted_full_size(oracle, name):
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.c4_decode(name, "cuda")
    B, S, k = w["cfg"]["B"], w["S"], w["cfg"]["k"]
    g = torch.Generator().manual_seed(31)
    hw = (torch.rand(B, w["q_idx"].shape[1], generator=g) * 2.0 - 0.3).float().cuda()
    note("decode_sparse_weighted %s" % name)
    s1, i1, o1, l1 = hsa.hsa_decode_sparse_weighted(w["q_idx"], hw, w["k_idx"], w["n_cand"], k, w["q"],
                                                    w["swa_kv"], w["swa_len"], w["comp_kv"],
                                                    w["comp_len"], w["scale"], 512)
    s2, i2 = hsa.hsa_index_topk_weighted(w["q_idx"], hw, w["k_idx"], w["n_cand"], k)
    torch.cuda.synchronize()
    nc = w["n_cand"].cpu().numpy()
    for b in range(B):
        assert torch.equal(s1[b, :nc[b]], s2[b, :nc[b]])
    assert torch.equal(i1, i2)
    scn = s1.cpu().numpy()
    np.testing.assert_array_equal(i1.cpu().numpy(), oracle.topk(scn, nc, k))
    # scores on a sample of rows (first, last, and spread) against the oracle
    rows = np.unique(np.concatenate([np.arange(64), np.arange(S - 64, S),
                                     np.random.default_rng(5).integers(0, S, 4096)]))
    _check_scores(oracle, w["q_idx"], hw, w["k_idx"], nc, s1, rows=rows)
    ro, rl = oracle.attn_decode(w["q"].cpu(), w["swa_kv"].cpu(), w["swa_len"].cpu().numpy(),
                                w["comp_kv"].cpu(), w["comp_len"].cpu().numpy(), w["scale"], 512,
                                comp_idx=i1.cpu().numpy())
    print(compare(o1, ro, TOL_BF16, name + " weighted out vs oracle"))
    print(compare(l1, rl, TOL_BF16, name + " weighted lse vs oracle"))


def test_weighted_shape_limits():
    import hybrid_sparse_compressed_amd as hsa

    q, w, kk = _case(1, 2, 2, 1000, 64)
    for qq, ww, k2 in ((q[:, :40], w[:, :40], kk), (q.float(), w, kk.float())):
        with pytest.raises(hsa.HsaError) as e:
            hsa.hsa_index_topk_weighted(qq.contiguous(), ww.contiguous(), k2, [1000, 1000], 16)
        assert e.value.code == 2  # HSA_ERR_UNSUPPORTED, nothing launched
