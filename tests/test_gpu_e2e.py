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
