"""GPU parity: hsa_decode_sparse, the C4 decode layer-step in one call.

Against the two separate calls (hsa_index_topk, then hsa_attn_decode with its
indices): scores bit-identical, top-k indices identical, out / lse within the
bf16 bound (the fused attention sums the selected rows in another order).
Against the oracle chain: selected-set overlap and out / lse as in the
separate-call end-to-end test.  The workspace is zero-filled once and then
reused: calls must be repeatable on it."""
import math

import numpy as np
import pytest
import torch

from helpers import TOL_BF16, compare, note

pytestmark = pytest.mark.gpu


def _separate(hsa, w, k, d_v=512):
    s, idx = hsa.hsa_index_topk(w["q_idx"], w["k_idx"], w["n_cand"], k)
    o, lse = hsa.hsa_attn_decode(w["q"], w["swa_kv"], w["swa_len"], w["comp_kv"], w["comp_len"],
                                 w["scale"], d_v, comp_idx=idx)
    return s, idx, o, lse


def _fused(hsa, w, k, d_v=512, workspace=None):
    return hsa.hsa_decode_sparse(w["q_idx"], w["k_idx"], w["n_cand"], k, w["q"], w["swa_kv"],
                                 w["swa_len"], w["comp_kv"], w["comp_len"], w["scale"], d_v,
                                 workspace=workspace)


def _workspace(hsa, w, k, d_v=512):
    B, H, _ = w["q"].shape
    W, S = w["swa_kv"].shape[1], w["comp_kv"].shape[1]
    need = hsa.lib.hsa_decode_sparse_workspace_size(B, H, d_v, W, S, k)
    sel = hsa.lib.hsa_index_topk_workspace_size(B, S, k)
    return torch.zeros(need, dtype=torch.uint8, device="cuda"), (sel + 255) // 256 * 256


def _check_against_separate(hsa, w, k, label):
    ws, sel_bytes = _workspace(hsa, w, k)
    s1, i1, o1, l1 = _separate(hsa, w, k)
    s2, i2, o2, l2 = _fused(hsa, w, k, workspace=ws)
    torch.cuda.synchronize()
    n = w["n_cand"].cpu().tolist()
    for b, nb in enumerate(n):  # scores past n_cand are not written
        assert torch.equal(s1[b, :nb], s2[b, :nb]), label + ": scores differ"
    np.testing.assert_array_equal(i2.cpu().numpy(), i1.cpu().numpy(), err_msg=label + ": top-k")
    print(compare(o2, o1.float(), TOL_BF16, label + " out vs separate"))
    print(compare(l2, l1, TOL_BF16, label + " lse vs separate"))
    # the same workspace again gives the same results
    s3, i3, o3, l3 = _fused(hsa, w, k, workspace=ws)
    assert torch.equal(i2, i3) and torch.equal(o2, o3) and torch.equal(l2, l3), label + ": not repeatable"
    return i2, o2, l2, s2


def _small_case(seed, B, S, H=64, W=128, k=512, dup=False, equal_keys=False):
    g = torch.Generator().manual_seed(seed)
    bf = torch.bfloat16
    w = dict(
        q=torch.randn(B, H, 576, generator=g).to(bf),
        swa_kv=torch.randn(B, W, 576, generator=g).to(bf),
        comp_kv=torch.randn(B, S, 576, generator=g).to(bf),
        q_idx=torch.randn(B, 64, 128, generator=g).to(bf),
        k_idx=torch.randn(B, S, 128, generator=g).to(bf),
        scale=1.0 / 24.0,
    )
    if equal_keys:
        w["k_idx"][:] = w["k_idx"][:, :1]  # every candidate scores the same
    if dup:
        for b in range(B):
            src = torch.randint(0, S, (S // 50,), generator=g)
            dst = torch.randint(0, S, (S // 50,), generator=g)
            w["k_idx"][b, dst] = w["k_idx"][b, src]
    return {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in w.items()}


@pytest.mark.parametrize("name", ["c4_decode_64k", "c4_decode_1m"])
def test_full_size_against_separate_and_oracle(oracle, name):
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.c4_decode(name, "cuda")
    k = w["cfg"]["k"]
    note("decode_sparse %s" % name)
    idx, o, lse, scores = _check_against_separate(hsa, w, k, name)
    nc = w["n_cand"].cpu().numpy()
    got = idx.cpu().numpy()
    # the fused select is bit-exact against the oracle's select on the GPU's own scores
    np.testing.assert_array_equal(got, oracle.topk(scores.cpu().numpy(), nc, k),
                                  err_msg=name + ": fused top-k vs oracle select on the same scores")
    rs = oracle.index_scores(w["q_idx"].cpu(), w["k_idx"].cpu(), nc)
    ridx = oracle.topk(rs.astype(np.float32), nc, k)
    inter = sum(len(set(a[a >= 0].tolist()) & set(b[b >= 0].tolist())) for a, b in zip(got, ridx))
    assert inter / int((ridx >= 0).sum()) >= 0.999
    ro, rl = oracle.attn_decode(w["q"].cpu(), w["swa_kv"].cpu(), w["swa_len"].cpu().numpy(),
                                w["comp_kv"].cpu(), w["comp_len"].cpu().numpy(), w["scale"], 512,
                                comp_idx=ridx)
    print(compare(o, ro, TOL_BF16, name + " out vs oracle"))
    print(compare(lse, rl, TOL_BF16, name + " lse vs oracle"))


def test_ragged_lengths_and_ties(oracle):
    """Ragged candidate counts (none, fewer than k, exactly k, all), ragged window
    fill and comp_len, duplicated key rows so ties straddle rank k."""
    import hybrid_sparse_compressed_amd as hsa

    B, S, k = 5, 20000, 512
    w = _small_case(11, B, S, dup=True)
    w["n_cand"] = torch.tensor([0, 300, k, S, S - 7], dtype=torch.int32, device="cuda")
    w["swa_len"] = torch.tensor([0, 5, 128, 128, 77], dtype=torch.int32, device="cuda")
    w["comp_len"] = torch.tensor([0, S, S, S - 1000, S], dtype=torch.int32, device="cuda")
    note("decode_sparse ragged")
    idx, o, lse, scores = _check_against_separate(hsa, w, k, "ragged")
    nc = w["n_cand"].cpu().numpy()
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk(scores.cpu().numpy(), nc, k))
    rs = oracle.index_scores(w["q_idx"].cpu(), w["k_idx"].cpu(), nc)
    ridx = oracle.topk(rs.astype(np.float32), nc, k)
    ro, rl = oracle.attn_decode(w["q"].cpu(), w["swa_kv"].cpu(), w["swa_len"].cpu().numpy(),
                                w["comp_kv"].cpu(), w["comp_len"].cpu().numpy(), w["scale"], 512,
                                comp_idx=idx.cpu().numpy())
    print(compare(o, ro, TOL_BF16, "ragged out vs oracle (same indices)"))
    print(compare(lse, rl, TOL_BF16, "ragged lse vs oracle (same indices)"))
    inter = sum(len(set(a[a >= 0].tolist()) & set(b[b >= 0].tolist())) for a, b in zip(idx.cpu().numpy(), ridx))
    assert inter / max(1, int((ridx >= 0).sum())) >= 0.999


def test_all_candidates_tie():
    """Every key row equal: the whole candidate list shares the threshold bin
    (short list far above the LDS capacity) and the lowest indices win."""
    import hybrid_sparse_compressed_amd as hsa

    B, S, k = 2, 30000, 512
    w = _small_case(12, B, S, equal_keys=True)
    w["n_cand"] = torch.tensor([S, S - 123], dtype=torch.int32, device="cuda")
    w["swa_len"] = torch.tensor([128, 64], dtype=torch.int32, device="cuda")
    w["comp_len"] = torch.tensor([S, S], dtype=torch.int32, device="cuda")
    note("decode_sparse all tie")
    idx, _, _, _ = _check_against_separate(hsa, w, k, "all-tie")
    np.testing.assert_array_equal(idx.cpu().numpy(), np.tile(np.arange(k, dtype=np.int32), (B, 1)))


def test_concentrated_top_rows_read_their_slot_from_the_score_row(oracle):
    """Most of the top-k inside one scoring workgroup's 2048 rows: that
    workgroup's candidate list cannot hold the threshold bin, so the select
    reads that slot's 2048 scores from the score row; results stay exact
    (against the separate calls and the oracle's top-k), with duplicated rows
    for ties, and the written top-k is sorted."""
    import hybrid_sparse_compressed_amd as hsa

    B, S, k = 2, 40000, 512
    w = _small_case(14, B, S, dup=True)
    w["k_idx"][0, 6144:6744] *= 8  # ~300 of sequence 0's top-k in rows 6144..8191
    w["k_idx"][1, 30000:30900] *= 8
    w["k_idx"][1, 30900:30910] = w["k_idx"][1, 30000:30010]  # exact ties among them
    w["n_cand"] = torch.tensor([S, S - 1111], dtype=torch.int32, device="cuda")
    w["swa_len"] = torch.tensor([128, 128], dtype=torch.int32, device="cuda")
    w["comp_len"] = torch.tensor([S, S], dtype=torch.int32, device="cuda")
    note("decode_sparse concentrated top rows")
    idx, o, lse, scores = _check_against_separate(hsa, w, k, "concentrated")
    nc = w["n_cand"].cpu().numpy()
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk(scores.cpu().numpy(), nc, k))
    rs = oracle.index_scores(w["q_idx"].cpu(), w["k_idx"].cpu(), nc)
    ridx = oracle.topk(rs.astype(np.float32), nc, k)
    inter = sum(len(set(a[a >= 0].tolist()) & set(b[b >= 0].tolist())) for a, b in zip(idx.cpu().numpy(), ridx))
    assert inter / int((ridx >= 0).sum()) >= 0.999


def test_fused_lists_fp32_and_large_k(oracle):
    """The list-based fused select at other shapes: fp32 with 128-wide latents
    and 8 heads (list capacity 64, select finished in the attention kernel),
    and bf16 576/512 with k = 2048 (selected list up to 2047 entries)."""
    import hybrid_sparse_compressed_amd as hsa

    g = torch.Generator().manual_seed(15)
    B, S, H, W, k = 3, 20000, 8, 128, 64
    w = dict(q=torch.randn(B, H, 128, generator=g), swa_kv=torch.randn(B, W, 128, generator=g),
             comp_kv=torch.randn(B, S, 128, generator=g), q_idx=torch.randn(B, 4, 64, generator=g),
             k_idx=torch.randn(B, S, 64, generator=g), scale=1.0 / math.sqrt(128))
    w = {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in w.items()}
    w["n_cand"] = torch.tensor([S, S - 5, 12345], dtype=torch.int32, device="cuda")
    w["swa_len"] = torch.tensor([128, 100, 1], dtype=torch.int32, device="cuda")
    w["comp_len"] = torch.tensor([S, S, S], dtype=torch.int32, device="cuda")
    note("decode_sparse fp32 lists")
    ws, _ = _workspace(hsa, w, k, d_v=128)
    s1, i1, o1, l1 = _separate(hsa, w, k, d_v=128)
    s2, i2, o2, l2 = _fused(hsa, w, k, d_v=128, workspace=ws)
    torch.cuda.synchronize()
    for b, nb in enumerate(w["n_cand"].cpu().tolist()):
        assert torch.equal(s1[b, :nb], s2[b, :nb])
    np.testing.assert_array_equal(i2.cpu().numpy(), i1.cpu().numpy())
    print(compare(o2, o1, (1e-5, 1e-5), "fp32 lists out vs separate"))
    print(compare(l2, l1, (1e-5, 1e-5), "fp32 lists lse vs separate"))
    nc = w["n_cand"].cpu().numpy()
    rs = oracle.index_scores(w["q_idx"].cpu(), w["k_idx"].cpu(), nc)
    ridx = oracle.topk(rs.astype(np.float32), nc, k)
    inter = sum(len(set(a[a >= 0].tolist()) & set(b[b >= 0].tolist())) for a, b in zip(i2.cpu().numpy(), ridx))
    assert inter / int((ridx >= 0).sum()) >= 0.999

    B, S, k = 2, 70000, 2048
    w = _small_case(16, B, S, k=k, dup=True)
    w["n_cand"] = torch.tensor([S, S - 3000], dtype=torch.int32, device="cuda")
    w["swa_len"] = torch.tensor([128, 77], dtype=torch.int32, device="cuda")
    w["comp_len"] = torch.tensor([S, S], dtype=torch.int32, device="cuda")
    note("decode_sparse k=2048 lists")
    idx, o, lse, scores = _check_against_separate(hsa, w, k, "k2048")
    nc = w["n_cand"].cpu().numpy()
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk(scores.cpu().numpy(), nc, k))
    rs = oracle.index_scores(w["q_idx"].cpu(), w["k_idx"].cpu(), nc)
    ridx = oracle.topk(rs.astype(np.float32), nc, k)
    inter = sum(len(set(a[a >= 0].tolist()) & set(b[b >= 0].tolist())) for a, b in zip(idx.cpu().numpy(), ridx))
    assert inter / int((ridx >= 0).sum()) >= 0.999


def test_every_slot_short_selects_from_the_score_row():
    """1.6M candidates with equal keys: all 782 slots' lists are cut above the
    threshold bin (more than the 768 the select reads one by one), so every
    workgroup selects from the whole score row; the lowest k indices win."""
    import hybrid_sparse_compressed_amd as hsa

    B, S, H, W, k = 1, 1600000, 64, 128, 512
    g = torch.Generator(device="cuda").manual_seed(17)
    bf = torch.bfloat16
    w = dict(q=torch.randn(B, H, 576, generator=g, device="cuda").to(bf),
             swa_kv=torch.randn(B, W, 576, generator=g, device="cuda").to(bf),
             comp_kv=torch.randn(B, S, 576, generator=g, device="cuda").to(bf),
             q_idx=torch.randn(B, 64, 128, generator=g, device="cuda").to(bf),
             scale=1.0 / 24.0)
    w["k_idx"] = torch.randn(B, 1, 128, generator=g, device="cuda").to(bf).expand(B, S, 128).contiguous()
    w["n_cand"] = torch.tensor([S], dtype=torch.int32, device="cuda")
    w["swa_len"] = torch.tensor([128], dtype=torch.int32, device="cuda")
    w["comp_len"] = torch.tensor([S], dtype=torch.int32, device="cuda")
    note("decode_sparse every slot short")
    idx, _, _, _ = _check_against_separate(hsa, w, k, "every-slot-short")
    np.testing.assert_array_equal(idx.cpu().numpy(), np.arange(k, dtype=np.int32)[None, :])


@pytest.mark.parametrize("k", [1, 3, 100])
def test_fused_lists_small_k(oracle, k):
    """Small k on the list path (one or a few selected rows, list capacity at
    its minimum), ragged candidate counts, against the separate calls and the
    oracle's top-k."""
    import hybrid_sparse_compressed_amd as hsa

    B, S = 3, 25000
    w = _small_case(18 + k, B, S, k=k, dup=True)
    w["n_cand"] = torch.tensor([S, S - 999, 2], dtype=torch.int32, device="cuda")
    w["swa_len"] = torch.tensor([128, 9, 128], dtype=torch.int32, device="cuda")
    w["comp_len"] = torch.tensor([S, S, S], dtype=torch.int32, device="cuda")
    note("decode_sparse small k=%d" % k)
    idx, _, _, _ = _check_against_separate(hsa, w, k, "k%d" % k)
    nc = w["n_cand"].cpu().numpy()
    rs = oracle.index_scores(w["q_idx"].cpu(), w["k_idx"].cpu(), nc)
    ridx = oracle.topk(rs.astype(np.float32), nc, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)


def test_small_pool_takes_the_separate_path():
    import hybrid_sparse_compressed_amd as hsa

    w = _small_case(13, 3, 9000, k=256)
    S = 9000
    w["n_cand"] = torch.tensor([S, 100, S - 1], dtype=torch.int32, device="cuda")
    w["swa_len"] = torch.tensor([128, 128, 3], dtype=torch.int32, device="cuda")
    w["comp_len"] = torch.tensor([S, S, S], dtype=torch.int32, device="cuda")
    note("decode_sparse small pool")
    ws, _ = _workspace(hsa, w, 256)
    s1, i1, o1, l1 = _separate(hsa, w, 256)
    s2, i2, o2, l2 = _fused(hsa, w, 256, workspace=ws)
    torch.cuda.synchronize()
    for b, nb in enumerate(w["n_cand"].cpu().tolist()):
        assert torch.equal(s1[b, :nb], s2[b, :nb])
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_repeatable_and_workspace_reusable():
    """Two calls on one workspace give bitwise-identical results; a call with
    other inputs in between changes nothing."""
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.c4_decode("c4_decode_64k", "cuda")
    k = w["cfg"]["k"]
    w2 = dict(w)
    w2["q_idx"] = torch.flip(w["q_idx"], dims=[0]).contiguous()
    w2["q"] = torch.flip(w["q"], dims=[0]).contiguous()
    ws, sel_bytes = _workspace(hsa, w, k)
    note("decode_sparse repeat")
    a = [t.clone() for t in _fused(hsa, w, k, workspace=ws)]
    _fused(hsa, w2, k, workspace=ws)
    b = [t.clone() for t in _fused(hsa, w, k, workspace=ws)]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
