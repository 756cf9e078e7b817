"""GPU parity: the radix-select top-k (select-only mode of hsa_index_topk) must
be bit-exact against the oracle on identical fp32 scores, on both the
LDS-resident path (n <= 12288) and the multi-workgroup path (ascending output
from the LDS bitmap up to 262,144 candidates, from the bucketed sort above)."""
import numpy as np
import pytest
import torch

from helpers import note

pytestmark = pytest.mark.gpu


def _select(scores, n_cand, k):
    import hybrid_sparse_compressed_amd as hsa

    _, idx = hsa.hsa_index_topk(None, None, n_cand, k, scores=scores.cuda())
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def _plant_boundary_ties(oracle, s, n_cand, k, rng):
    """Copy each row's rank-k value to positions on both sides of it, and place
    the float neighbours (+-1 ulp) of that value nearby."""
    s = s.copy()
    sel = oracle.topk(s, n_cand, k)
    for i in range(s.shape[0]):
        n = int(n_cand[i])
        if n <= k or n < 8:
            continue
        chosen = sel[i][sel[i] >= 0]
        vals = s[i, chosen]
        kth = chosen[np.argmin(vals)]
        v = s[i, kth]
        pos = rng.choice(n, size=min(6, n), replace=False)
        s[i, pos[:3]] = v
        s[i, pos[3:4]] = np.nextafter(v, np.float32(np.inf))
        s[i, pos[4:5]] = np.nextafter(v, np.float32(-np.inf))
        if len(pos) > 5:
            s[i, pos[5]] = -0.0 if v == 0 else v
    return s


@pytest.mark.parametrize(
    "Nq,S,k",
    [(3, 1, 1), (4, 7, 3), (5, 64, 64), (6, 1000, 64), (4, 5000, 2048), (3, 6140, 2048),
     (3, 6144, 2048), (3, 12288, 512), (3, 12289, 512), (4, 50000, 512), (2, 70000, 2048), (4, 262144, 512), (3, 300000, 1000)],
)
def test_select_bit_exact(oracle, Nq, S, k):
    from hybrid_sparse_compressed_amd import workloads

    rng = np.random.default_rng(S + k)
    scores = workloads.topk_scores(Nq, S, "cpu", seed=7 + S).numpy()
    n_cand = np.full(Nq, S, dtype=np.int32)
    if Nq >= 3:  # ragged candidate counts: fewer than k, exactly k, all
        n_cand[0] = max(0, min(S, k // 2))
        n_cand[1] = min(S, k)
        n_cand[2] = max(0, S - 3)
    scores = _plant_boundary_ties(oracle, scores, n_cand, k, rng)
    note("topk select Nq=%d S=%d k=%d" % (Nq, S, k))
    got = _select(torch.from_numpy(scores), torch.from_numpy(n_cand), k)
    want = oracle.topk(scores, n_cand, k)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("S", [3000, 20000])
def test_select_special_patterns(oracle, S):
    k = 256
    inc = np.arange(S, dtype=np.float32)
    pats = [
        np.full(S, 0.25, np.float32),                       # all equal
        inc,                                                 # ascending
        -inc,                                                # descending
        np.where(np.arange(S) % 2 == 0, -0.0, 0.0).astype(np.float32),  # signed zeros
        np.where(np.arange(S) % 97 == 0, np.inf, -np.inf).astype(np.float32),
        np.round(np.random.default_rng(1).standard_normal(S)).astype(np.float32),  # few levels
    ]
    scores = np.stack(pats)
    n_cand = np.full(len(pats), S, np.int32)
    note("topk special patterns S=%d" % S)
    got = _select(torch.from_numpy(scores), torch.from_numpy(n_cand), k)
    np.testing.assert_array_equal(got, oracle.topk(scores, n_cand, k))
    assert got[0].tolist() == list(range(k))
    assert got[1].tolist() == list(range(S - k, S))


@pytest.mark.parametrize("k", [64, 2048])
def test_row_select_crowded_boundary_bins(oracle, k):
    """Rows of the one-workgroup path (n <= 12288) whose boundary bin is crowded
    however the first digit is placed: a row of two levels (the short list
    exceeds 4096 entries at k = 2048), of 40 levels (hundreds of equal keys at
    the boundary), a tight cluster with one huge outlier (the row's key range
    is stretched so the cluster shares one first-digit bin) and a tight
    cluster alone."""
    S = 12000
    rng = np.random.default_rng(11)
    pats = [
        rng.integers(0, 2, S).astype(np.float32),
        rng.integers(0, 40, S).astype(np.float32),
        (1000.0 + 1e-3 * rng.standard_normal(S)).astype(np.float32),
        (1000.0 + 1e-3 * rng.standard_normal(S)).astype(np.float32),
    ]
    pats[2][rng.integers(0, S)] = 1e30
    scores = np.stack(pats)
    n_cand = np.array([S, S, S, S - 5], np.int32)
    note("topk row select crowded bins S=%d k=%d" % (S, k))
    got = _select(torch.from_numpy(scores), torch.from_numpy(n_cand), k)
    np.testing.assert_array_equal(got, oracle.topk(scores, n_cand, k))


def test_nan_ranks_below_numbers(oracle):
    S, k = 20000, 128
    rng = np.random.default_rng(4)
    s = rng.standard_normal((2, S)).astype(np.float32)
    s[:, rng.choice(S, 500, replace=False)] = np.nan
    n_cand = np.full(2, S, np.int32)
    note("topk NaN smoke")
    got = _select(torch.from_numpy(s), torch.from_numpy(n_cand), k)
    want = oracle.topk(np.nan_to_num(s, nan=-np.inf), n_cand, k)
    np.testing.assert_array_equal(got, want)


def test_workspace_is_reusable_and_results_deterministic(oracle):
    from hybrid_sparse_compressed_amd import workloads

    k, S = 512, 100000
    a = workloads.topk_scores(4, S, "cpu", seed=11).numpy()
    b = workloads.topk_scores(4, S, "cpu", seed=12).numpy()
    n_cand = np.full(4, S, np.int32)
    note("topk workspace reuse")
    r1 = _select(torch.from_numpy(a), torch.from_numpy(n_cand), k)
    r2 = _select(torch.from_numpy(b), torch.from_numpy(n_cand), k)
    r3 = _select(torch.from_numpy(a), torch.from_numpy(n_cand), k)
    np.testing.assert_array_equal(r1, oracle.topk(a, n_cand, k))
    np.testing.assert_array_equal(r2, oracle.topk(b, n_cand, k))
    np.testing.assert_array_equal(r1, r3)


def test_workspace_left_zero_across_layouts(oracle):
    """Calls with different (Nq, S, k) share one workspace; each is exact and the
    workspace is all-zero after every call."""
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    layouts = [(4, 100000, 512), (2, 30000, 64), (3, 13000, 2048), (4, 100000, 512)]
    need = max(hsa.lib.hsa_index_topk_workspace_size(n, s, k) for n, s, k in layouts)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for j, (Nq, S, k) in enumerate(layouts):
        s = workloads.topk_scores(Nq, S, "cpu", seed=40 + j).numpy()
        n_cand = np.full(Nq, S, np.int32)
        n_cand[0] = S - 17
        note("topk layout %d: Nq=%d S=%d k=%d" % (j, Nq, S, k))
        _, idx = hsa.hsa_index_topk(None, None, torch.from_numpy(n_cand), k,
                                    scores=torch.from_numpy(s).cuda(), workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk(s, n_cand, k))
        assert int(torch.count_nonzero(ws)) == 0


def test_default_workspace_not_shared_with_attention(oracle):
    """The binding's cached top-k workspace must stay zero-filled even after an
    attention call (whose split partials leave data in its own workspace)."""
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.c128_dense_decode("cuda", B=4)
    note("attention call before top-k")
    hsa.hsa_attn_decode(w["q"], w["swa_kv"], w["swa_len"], w["comp_kv"], w["comp_len"],
                        w["scale"], 512)
    S, k = 60000, 512
    s = workloads.topk_scores(4, S, "cpu", seed=77).numpy()
    n_cand = np.full(4, S, np.int32)
    got = _select(torch.from_numpy(s), torch.from_numpy(n_cand), k)
    np.testing.assert_array_equal(got, oracle.topk(s, n_cand, k))
