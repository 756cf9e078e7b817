"""GPU parity: hsa_decode_step_paged, the decode layer-step on paged pools.

Every pool is reached through its shadow (a per-sequence page map).  Against
the flat call: the same data laid out on shuffled physical pages (pages no
shadow names poisoned with NaN, SWA pages outside the window and the open
block not resident) must give hsa_decode_step's results bit for bit -- scores,
top-k, out, lse, the appended C4 entry and the stored token -- since only the
row addresses differ.  Cases cover the fused list path (2048- and 256-row list
slots, the append in the scoring launch), the separate path with the LDS row
select and with the multi-workgroup select.  Against the oracle: freed pages
(indexer and C4 rows, a window page) must drop exactly their rows: scores NaN,
top-k bit-exact against the oracle's select on the GPU's own scores, out and
lse against the oracle's paged attention."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, compare, note

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _nan_like(shape, dev):
    return torch.full(shape, float("nan"), dtype=BF, device=dev)


def _page_pool(flat, P, gen, spare=3):
    """flat [B, N, D] -> (pool [pages + spare, P, D], map [B, ceil(N/P)] int32):
    the logical pages on a random physical order, spare pages NaN."""
    B, N, D = flat.shape
    npg = (N + P - 1) // P
    if npg * P != N:
        flat = torch.cat([flat, flat.new_zeros(B, npg * P - N, D)], 1)
    perm = torch.randperm(B * npg + spare, generator=gen)
    pool = _nan_like((B * npg + spare, P, D), flat.device)
    pool[perm[:B * npg].to(flat.device)] = flat.reshape(B * npg, P, D)
    return pool, perm[:B * npg].reshape(B, npg).to(torch.int32).to(flat.device)


def _swa_paged(ring, rx, rg, pos, P, gen, W):
    """The window ring (slot j = token pos-n+1+j) and the open C4 block's ring
    slots as token-indexed paged pools: only pages holding the window or the open
    block are resident, on random physical pages; spare pages NaN."""
    B, _, D = ring.shape
    dev = ring.device
    need = []
    for b in range(B):
        p = int(pos[b])
        lo = max(0, min(p - W + 1, 4 * (p // 4)))
        need.append(list(range(lo // P, p // P + 1)) if p >= 0 else [])
    n_res = sum(len(x) for x in need)
    spare = 3
    perm = torch.randperm(n_res + spare, generator=gen).tolist()
    maxp = max(int(p) for p in pos) + 1
    smap = torch.full((B, max(1, (maxp + P - 1) // P)), -1, dtype=torch.int32)
    it = iter(perm)
    for b in range(B):
        for j in need[b]:
            smap[b, j] = next(it)
    pool, sx, sg = (_nan_like((n_res + spare, P, D), dev) for _ in range(3))
    return pool, sx, sg, smap.to(dev)


def _put(pool, smap, b, t, P, row):
    pg = int(smap[b, t // P])
    pool[pg, t % P] = row


def _case_from_flat(w, pos, swa_len, P_swa, P_c4, seed):
    """Paged copies of a flat decode-step case (w: flat tensors on the GPU)."""
    gen = torch.Generator().manual_seed(seed)
    W = w["swa_kv"].shape[1]
    d = {}
    d["kI_pool"], d["kI_map"] = _page_pool(w["k_idx"], P_c4, gen)
    d["c4_pool"], d["c4_map"] = _page_pool(w["comp_kv"], P_c4, gen)
    d["swa_pool"], d["state_x"], d["state_g"], d["swa_map"] = _swa_paged(
        w["swa_kv"], w["ring_x"], w["ring_g"], pos, P_swa, gen, W)
    for b in range(len(pos)):
        p = int(pos[b])
        if p < 0:
            continue
        n = min(int(swa_len[b]), W, p + 1)
        for j in range(n):
            _put(d["swa_pool"], d["swa_map"], b, p - n + 1 + j, P_swa, w["swa_kv"][b, j])
        bs = 4 * (p // 4)
        for j in range(p - bs):  # the open block's tokens before p: ring slots 0 .. p mod 4 - 1
            _put(d["state_x"], d["swa_map"], b, bs + j, P_swa, w["ring_x"][b, j])
            _put(d["state_g"], d["swa_map"], b, bs + j, P_swa, w["ring_g"][b, j])
    return d


def _flat_case(seed, B, S, H=64, W=128, D=576, dev="cuda"):
    g = torch.Generator().manual_seed(seed)
    w = dict(q=torch.randn(B, H, D, generator=g), swa_kv=torch.randn(B, W, D, generator=g),
             comp_kv=torch.randn(B, S, D, generator=g), q_idx=torch.randn(B, 64, 128, generator=g),
             k_idx=torch.randn(B, S, 128, generator=g), x_tok=torch.randn(B, D, generator=g),
             g_tok=torch.randn(B, D, generator=g), bias=torch.randn(4, D, generator=g) * 0.1,
             ring_x=torch.randn(B, 4, D, generator=g), ring_g=torch.randn(B, 4, D, generator=g))
    return {kk: v.to(BF).to(dev) for kk, v in w.items()}


def _run_both(hsa, w, pos, n_cand, swa_len, comp_len, k, P_swa, P_c4, seed, scale=1.0 / 24.0):
    B, S = w["k_idx"].shape[:2]
    W = w["swa_kv"].shape[1]
    dev = w["q"].device
    d = _case_from_flat(w, pos.tolist(), swa_len.tolist(), P_swa, P_c4, seed)
    pd, nd, cd = pos.to(dev), n_cand.to(dev), comp_len.to(dev)
    # the flat call: sequences without a query token see no window in the paged call
    sd_flat = torch.where(pos >= 0, swa_len, torch.zeros_like(swa_len)).to(dev)
    rx, rg, comp = w["ring_x"].clone(), w["ring_g"].clone(), w["comp_kv"].clone()
    note("paged step flat call B=%d S=%d k=%d" % (B, S, k))
    f = hsa.hsa_decode_step(w["x_tok"], w["g_tok"], w["bias"], rx, rg, pd, w["q_idx"], w["k_idx"],
                            nd, k, w["q"], w["swa_kv"], sd_flat, comp, cd, scale, 512)
    torch.cuda.synchronize()
    note("paged step paged call P_swa=%d P_c4=%d" % (P_swa, P_c4))
    p = hsa.hsa_decode_step_paged(w["x_tok"], w["g_tok"], w["bias"], d["state_x"], d["state_g"], pd,
                                  w["q_idx"], d["kI_pool"], d["kI_map"], nd, k, w["q"], d["swa_pool"],
                                  d["swa_map"], swa_len.to(dev), d["c4_pool"], d["c4_map"], cd, scale,
                                  512, W, S)
    torch.cuda.synchronize()
    return f, p, d, comp


@pytest.mark.parametrize("S,k,B,P_swa,P_c4", [
    (16384, 512, 4, 16, 64),    # fused lists path, 256-row slots
    (4096, 256, 3, 32, 16),     # separate path, LDS row select
    (20000, 2048, 2, 64, 128),  # separate path, multi-workgroup select (ragged last page)
])
def test_paged_equals_flat_bitwise(S, k, B, P_swa, P_c4):
    import hybrid_sparse_compressed_amd as hsa

    w = _flat_case(300 + S, B, S)
    pos = torch.tensor([4 * 199 + 3, 4 * (S - 2) + 3, 4 * 1000 + 1, -1][:B], dtype=torch.int32)
    n_cand = torch.tensor([S, S - 1, S - 77, 900][:B], dtype=torch.int32)
    swa_len = torch.tensor([128, 128, 50, 128][:B], dtype=torch.int32)
    comp_len = n_cand.clone()
    f, p, d, comp = _run_both(hsa, w, pos, n_cand, swa_len, comp_len, k, P_swa, P_c4, seed=S)
    for name, a, b in zip(("scores", "topk", "out", "lse"), f, p):
        if name == "scores":
            for s, nb in enumerate(n_cand.tolist()):
                assert torch.equal(a[s, :nb], b[s, :nb]), name
        else:
            assert torch.equal(a, b), name
    # appended entries and stored tokens
    for b in range(B):
        t = int(pos[b])
        if t < 0:
            continue
        sp = int(d["swa_map"][b, t // P_swa])
        assert torch.equal(d["state_x"][sp, t % P_swa], w["x_tok"][b])
        assert torch.equal(d["state_g"][sp, t % P_swa], w["g_tok"][b])
        if t % 4 == 3 and t // 4 < S:
            i = t // 4
            cp = int(d["c4_map"][b, i // P_c4])
            assert torch.equal(d["c4_pool"][cp, i % P_c4], comp[b, i])
            assert not torch.equal(comp[b, i], w["comp_kv"][b, i])  # the entry really changed


def test_paged_equals_flat_at_the_1m_workload():
    """c4_decode_1m (4 x 262,144 C4 entries, 2048-row list slots, the append in
    the scoring launch) on 256-row C4 pages and 64-token SWA pages."""
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w0 = workloads.c4_decode("c4_decode_1m", "cuda")
    B, S, k = w0["cfg"]["B"], w0["S"], w0["cfg"]["k"]
    g = torch.Generator().manual_seed(77)
    D = w0["cfg"]["d_qk"]
    w = dict(q=w0["q"], swa_kv=w0["swa_kv"], comp_kv=w0["comp_kv"], q_idx=w0["q_idx"], k_idx=w0["k_idx"])
    for name, shape in (("x_tok", (B, D)), ("g_tok", (B, D)), ("ring_x", (B, 4, D)), ("ring_g", (B, 4, D))):
        w[name] = torch.randn(*shape, generator=g).to(BF).cuda()
    w["bias"] = (torch.randn(4, D, generator=g) * 0.1).to(BF).cuda()
    pos = torch.tensor([4 * 1234 + 3, 4 * (S - 3) + 3, 4 * 5000 + 2, 4 * (S - 1) + 1], dtype=torch.int32)
    f, p, d, comp = _run_both(hsa, w, pos, w0["n_cand"].cpu(), w0["swa_len"].cpu(), w0["comp_len"].cpu(),
                              k, 64, 256, seed=1)
    nc = w0["n_cand"].cpu().tolist()
    for s, nb in enumerate(nc):
        assert torch.equal(f[0][s, :nb], p[0][s, :nb])
    for name, a, b in zip(("topk", "out", "lse"), f[1:], p[1:]):
        assert torch.equal(a, b), name
    for b in (0, 1):
        i = int(pos[b]) // 4
        cp = int(d["c4_map"][b, i // 256])
        assert torch.equal(d["c4_pool"][cp, i % 256], comp[b, i])


def test_freed_pages_against_the_oracle(oracle):
    """Freed indexer / C4 pages and a freed window page, S = 16,384 (fused path):
    NaN scores and no selection for freed indexer rows, top-k bit-exact against
    the oracle's select on the GPU's scores, out / lse against the oracle's
    paged attention (which leaves freed rows out)."""
    import hybrid_sparse_compressed_amd as hsa

    B, S, k, P_swa, P_c4, W = 3, 16384, 512, 16, 64, 128
    w = _flat_case(909, B, S)
    pos = torch.tensor([4 * 3000 + 3, 4 * 100 + 1, 700], dtype=torch.int32)
    n_cand = torch.tensor([S, 5000, S - 5], dtype=torch.int32)
    swa_len = torch.tensor([128, 128, 128], dtype=torch.int32)
    comp_len = torch.tensor([S, S, 9000], dtype=torch.int32)
    d = _case_from_flat(w, pos.tolist(), swa_len.tolist(), P_swa, P_c4, seed=5)
    # free: sequence 0 indexer + C4 page 7 (rows 448..511) and its window's middle page;
    # sequence 2: C4 page 3 only (its indexer rows stay candidates)
    d["kI_map"][0, 7] = -1
    d["c4_map"][0, 7] = -1
    d["c4_map"][2, 3] = -1
    mid = (int(pos[0]) - 64) // P_swa
    d["swa_map"][0, mid] = -1
    dev = w["q"].device
    note("paged step with freed pages")
    s, idx, o, l = hsa.hsa_decode_step_paged(
        None, None, None, None, None, pos.to(dev), w["q_idx"], d["kI_pool"], d["kI_map"], n_cand.to(dev),
        k, w["q"], d["swa_pool"], d["swa_map"], swa_len.to(dev), d["c4_pool"], d["c4_map"],
        comp_len.to(dev), 1.0 / 24.0, 512, W, S)
    torch.cuda.synchronize()
    sc = s.cpu().numpy()
    assert np.isnan(sc[0, 448:512]).all() and not np.isnan(sc[0, :448]).any()
    gi = idx.cpu().numpy()
    np.testing.assert_array_equal(gi, oracle.topk(sc, n_cand.numpy(), k))
    assert not ((gi[0] >= 448) & (gi[0] < 512)).any()
    cpu = lambda t: t.cpu()
    ro, rl = oracle.attn_decode_paged(
        cpu(w["q"]), cpu(d["swa_pool"]), cpu(d["swa_map"]).numpy(), P_swa, swa_len.numpy(), pos.numpy(),
        W, cpu(d["c4_pool"]), cpu(d["c4_map"]).numpy(), P_c4, comp_len.numpy(), gi, S, 1.0 / 24.0, 512)
    print(compare(o, ro, TOL_BF16, "paged out vs oracle"))
    print(compare(l, rl, TOL_BF16, "paged lse vs oracle"))
