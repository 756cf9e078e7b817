"""GPU end to end: the whole decode layer-step (compress -> score -> select ->
attend) on the GPU, against the same chain in the oracle.  The oracle rounds
the pool it stores to the storage dtype, as the GPU path does."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, TOL_FP32, compare, note

pytestmark = pytest.mark.gpu


def _overlap(a, b):
    inter = sum(len(set(x[x >= 0].tolist()) & set(y[y >= 0].tolist())) for x, y in zip(a, b))
    return inter / max(1, int((b >= 0).sum()))


def test_tiny_fp32_decode_chain(oracle):
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.tiny_fp32_decode("cpu")
    c = w["cfg"]
    note("e2e tiny_fp32_decode")
    pool = hsa.hsa_compress(w["x"].cuda(), w["gate"].cuda(), w["bias"].cuda(), 4)
    _, idx = hsa.hsa_index_topk(w["q_idx"].cuda(), w["k_idx"].cuda(), w["n_cand"], c["k"])
    o, lse = hsa.hsa_attn_decode(w["q"].cuda(), w["swa_kv"].cuda(), w["swa_len"], pool,
                                 w["comp_len"], w["scale"], 128, comp_idx=idx)
    torch.cuda.synchronize()

    rpool = oracle.compress(w["x"], w["gate"], w["bias"], 4).astype(np.float32)
    rs = oracle.index_scores(w["q_idx"], w["k_idx"], w["n_cand"].numpy())
    ridx = oracle.topk(rs.astype(np.float32), w["n_cand"].numpy(), c["k"])
    ro, rl = oracle.attn_decode(w["q"], w["swa_kv"], w["swa_len"].numpy(), rpool,
                                w["comp_len"].numpy(), w["scale"], 128, comp_idx=ridx)
    assert _overlap(idx.cpu().numpy(), ridx) == 1.0
    compare(o, ro, TOL_FP32, "e2e tiny out")
    compare(lse, rl, TOL_FP32, "e2e tiny lse")


def test_c4_1m_decode_chain(oracle):
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.c4_decode("c4_decode_1m", "cuda")
    k = w["cfg"]["k"]
    note("e2e c4_decode_1m")
    _, idx = hsa.hsa_index_topk(w["q_idx"], w["k_idx"], w["n_cand"], k)
    o, lse = hsa.hsa_attn_decode(w["q"], w["swa_kv"], w["swa_len"], w["comp_kv"], w["comp_len"],
                                 w["scale"], 512, comp_idx=idx)
    torch.cuda.synchronize()
    nc = w["n_cand"].cpu().numpy()
    rs = oracle.index_scores(w["q_idx"].cpu(), w["k_idx"].cpu(), nc)
    ridx = oracle.topk(rs.astype(np.float32), nc, k)
    ov = _overlap(idx.cpu().numpy(), ridx)
    print("selected-set overlap %.6f" % ov)
    assert ov >= 0.999
    ro, rl = oracle.attn_decode(w["q"].cpu(), w["swa_kv"].cpu(), w["swa_len"].cpu().numpy(),
                                w["comp_kv"].cpu(), w["comp_len"].cpu().numpy(), w["scale"], 512,
                                comp_idx=ridx)
    print(compare(o, ro, TOL_BF16, "e2e 1m out"))


def test_prefill_32k_chain_sampled(oracle):
    """The prefill workload as one chain on the GPU: C4 compression of the 8 x 32,768
    latents (hsa_compress), indexer scores and top-512 for all 16,384 query positions
    (hsa_index_topk, each query over the blocks complete by its position), then the
    prefill attention of every query over its window and its own selection
    (hsa_attn_prefill).  Against the oracle chain on 64 sampled queries, the first and
    last query of every sequence among them: the whole pool to the bf16 bound, the
    top-k bit-exact against the oracle's select on the GPU's own scores, the selected
    sets against the oracle's fp64 scores (overlap >= 0.999), the attention against
    the oracle's over the oracle's pool with the GPU's selection and, for queries whose
    selections agree, with the oracle's own selection."""
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads
    from helpers import round_bf16

    w = workloads.prefill("cuda")
    c = w["cfg"]
    n_seq, n_q, T, k, W = c["n_seq"], c["n_q"], c["T"], c["k"], c["W"]
    note("e2e prefill_32k chain")
    pool = hsa.hsa_compress(w["x"], w["gate4"], w["bias4"], 4)
    scores, idx = hsa.hsa_index_topk(w["q_idx"], w["k_idx"], w["n_cand"], k, q_seq=w["q_seq"])
    o, lse = hsa.hsa_attn_prefill(w["q"], w["x"], pool, w["q_start"], W, 4, w["scale"], 512,
                                  comp_idx=idx)
    torch.cuda.synchronize()

    rng = np.random.default_rng(7)
    ends = [b * n_q for b in range(n_seq)] + [b * n_q + n_q - 1 for b in range(n_seq)]
    rest = [int(x) for x in rng.choice(n_seq * n_q, 64, replace=False) if int(x) not in ends]
    sel = sorted(ends + rest[:64 - len(ends)])
    rpool = oracle.compress(w["x"].cpu(), w["gate4"].cpu(), w["bias4"].cpu(), 4)
    print(compare(pool, rpool, TOL_BF16, "chain pool"))
    rpool_bf = round_bf16(rpool)  # the pool as stored (bf16) feeds the attention
    nc = w["n_cand"].cpu().numpy()[sel]
    qs = w["q_seq"].cpu().numpy()[sel]
    rs = oracle.index_scores(w["q_idx"][sel].cpu(), w["k_idx"].cpu(), nc, q_seq=qs)
    ridx = oracle.topk(rs.astype(np.float32), nc, k)
    gidx = idx.cpu().numpy()
    np.testing.assert_array_equal(gidx[sel], oracle.topk(scores.cpu().numpy()[sel], nc, k))
    ov = _overlap(gidx[sel], ridx)
    print("selected-set overlap %.6f" % ov)
    assert ov >= 0.999
    ro, rl = oracle.attn_prefill(w["q"].cpu(), w["x"].cpu(), rpool_bf, w["q_start"], W, 4,
                                 w["scale"], 512, comp_idx=gidx, sel=sel)
    og = o.reshape(n_seq * n_q, c["H"], 512)
    print(compare(og[sel], ro, TOL_BF16, "chain out"))
    compare(lse[sel], rl, (1e-3, 1e-4), "chain lse")
    agree = [j for j, q in enumerate(sel) if set(gidx[q].tolist()) == set(ridx[j].tolist())]
    assert len(agree) >= len(sel) // 2
    full = gidx.copy()
    full[sel] = ridx
    ro2, _ = oracle.attn_prefill(w["q"].cpu(), w["x"].cpu(), rpool_bf, w["q_start"], W, 4,
                                 w["scale"], 512, comp_idx=full, sel=[sel[j] for j in agree])
    print(compare(og[[sel[j] for j in agree]], ro2, TOL_BF16, "chain out vs the oracle's own selection"))
