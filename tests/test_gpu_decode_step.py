"""GPU parity: hsa_decode_step, the C4 decode layer-step with its
compression-state update (append into the C4 ring and pool, then indexer,
select and attention).

Against the oracle chain: compress_append on the rings and the pool, then
index_scores, topk and attn_decode over the updated pool.  One completing
sequence has fewer candidates than k, so every pool row it has, the new
entry included, is attended: a pool row written after the attention read it
would show in its output.  Rings must match the oracle's bit for bit, the new
entries and the attention meet the bf16 bounds, and the selected sets overlap
as in the other decode tests.  Against the two separate calls
(hsa_compress_append, then hsa_decode_sparse): everything bit-identical."""
import numpy as np
import pytest
import torch

from helpers import TOL_BF16, compare, note, round_bf16

pytestmark = pytest.mark.gpu


def _case(seed, B, S, H=64, W=128, D=576):
    g = torch.Generator().manual_seed(seed)
    bf = torch.bfloat16
    return dict(
        q=torch.randn(B, H, D, generator=g).to(bf),
        swa_kv=torch.randn(B, W, D, generator=g).to(bf),
        comp_kv=torch.randn(B, S, D, generator=g).to(bf),
        q_idx=torch.randn(B, 64, 128, generator=g).to(bf),
        k_idx=torch.randn(B, S, 128, generator=g).to(bf),
        x_tok=torch.randn(B, D, generator=g).to(bf),
        g_tok=torch.randn(B, D, generator=g).to(bf),
        bias=(torch.randn(4, D, generator=g) * 0.1).to(bf),
        ring_x=torch.randn(B, 4, D, generator=g).to(bf),
        ring_g=torch.randn(B, 4, D, generator=g).to(bf),
        scale=1.0 / 24.0,
    )


def _dev(w):
    return {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in w.items()}


def _step(hsa, d, k, pos, n_cand, swa_len, comp_len):
    return hsa.hsa_decode_step(d["x_tok"], d["g_tok"], d["bias"], d["ring_x"], d["ring_g"], pos,
                               d["q_idx"], d["k_idx"], n_cand, k, d["q"], d["swa_kv"], swa_len,
                               d["comp_kv"], comp_len, d["scale"], 512)


@pytest.mark.parametrize("S,k", [(16384, 512), (4096, 256)])  # fused lists path / separate path
def test_decode_step_against_oracle_and_separate(oracle, S, k):
    import hybrid_sparse_compressed_amd as hsa

    B = 4
    w = _case(21 + S, B, S)
    # sequence 0 completes its block at pool row 199 and has 200 candidates (fewer
    # than k: all attended); 1 completes a block near the pool's end; 2 leaves its
    # block open; 3 is idle
    pos = torch.tensor([4 * 199 + 3, 4 * (S - 2) + 3, 4 * 1000 + 1, -1], dtype=torch.int32)
    n_cand = torch.tensor([200, S - 1, S, 777], dtype=torch.int32)
    swa_len = torch.tensor([128, 128, 50, 128], dtype=torch.int32)
    comp_len = n_cand.clone()
    note("decode_step S=%d k=%d" % (S, k))
    d1, d2 = _dev(w), _dev(w)
    d1["ring_x"], d1["ring_g"], d1["comp_kv"] = (w["ring_x"].cuda(), w["ring_g"].cuda(),
                                                 w["comp_kv"].cuda())
    d2["ring_x"], d2["ring_g"], d2["comp_kv"] = (w["ring_x"].cuda(), w["ring_g"].cuda(),
                                                 w["comp_kv"].cuda())
    pd, nd, sd, cd = pos.cuda(), n_cand.cuda(), swa_len.cuda(), comp_len.cuda()
    s1, i1, o1, l1 = _step(hsa, d1, k, pd, nd, sd, cd)
    # the same work as two calls
    hsa.hsa_compress_append(d2["x_tok"], d2["g_tok"], d2["bias"], d2["ring_x"], d2["ring_g"], pd,
                            d2["comp_kv"])
    s2, i2, o2, l2 = hsa.hsa_decode_sparse(d2["q_idx"], d2["k_idx"], nd, k, d2["q"], d2["swa_kv"],
                                           sd, d2["comp_kv"], cd, d2["scale"], 512)
    torch.cuda.synchronize()
    for a, b in ((d1["ring_x"], d2["ring_x"]), (d1["ring_g"], d2["ring_g"]),
                 (d1["comp_kv"], d2["comp_kv"]), (i1, i2), (o1, o2), (l1, l2)):
        assert torch.equal(a, b), "decode_step differs from the two separate calls"
    for b, nb in enumerate(n_cand.tolist()):
        assert torch.equal(s1[b, :nb], s2[b, :nb])

    # oracle chain
    rx, rg = w["ring_x"].clone(), w["ring_g"].clone()
    pool = np.zeros((B, S, 576))
    wrote = oracle.compress_append(w["x_tok"], w["g_tok"], w["bias"], rx, rg, pos.numpy(), pool, 4)
    assert wrote == [(0, 199), (1, S - 2)]
    assert torch.equal(d1["ring_x"].cpu().view(torch.int16), rx.view(torch.int16))
    assert torch.equal(d1["ring_g"].cpu().view(torch.int16), rg.view(torch.int16))
    comp = w["comp_kv"].clone()
    for b, r in wrote:
        compare(d1["comp_kv"][b, r].cpu(), pool[b, r], TOL_BF16, "new entry %d" % b)
        comp[b, r] = round_bf16(pool[b, r])
    untouched = torch.ones(B, S, dtype=torch.bool)
    for b, r in wrote:
        untouched[b, r] = False
    assert torch.equal(d1["comp_kv"].cpu()[untouched].view(torch.int16),
                       w["comp_kv"][untouched].view(torch.int16))
    nc = n_cand.numpy()
    rs = oracle.index_scores(w["q_idx"], w["k_idx"], nc)
    ridx = oracle.topk(rs.astype(np.float32), nc, k)
    got = i1.cpu().numpy()
    assert set(got[0][got[0] >= 0].tolist()) == set(range(200))  # all of sequence 0's rows
    inter = sum(len(set(a[a >= 0].tolist()) & set(b[b >= 0].tolist())) for a, b in zip(got, ridx))
    assert inter / int((ridx >= 0).sum()) >= 0.999
    ro, rl = oracle.attn_decode(w["q"], w["swa_kv"], swa_len.numpy(), comp, comp_len.numpy(),
                                w["scale"], 512, comp_idx=got)
    print(compare(o1, ro, TOL_BF16, "decode_step out vs oracle"))
    print(compare(l1, rl, TOL_BF16, "decode_step lse vs oracle"))
    # the attention of sequence 0 saw the new entry, not the row it replaced
    ro_old, _ = oracle.attn_decode(w["q"][:1], w["swa_kv"][:1], swa_len.numpy()[:1],
                                   w["comp_kv"][:1], comp_len.numpy()[:1], w["scale"], 512,
                                   comp_idx=got[:1])
    d_new = np.abs(o1[0].float().cpu().numpy() - ro[0]).max()
    d_old = np.abs(o1[0].float().cpu().numpy() - ro_old[0]).max()
    assert d_new < d_old, (d_new, d_old)


def test_decode_step_rejects_bad_append_arguments():
    import hybrid_sparse_compressed_amd as hsa

    d = _dev(_case(5, 2, 256))
    note("decode_step argument checks")
    with pytest.raises(ValueError):
        _step(hsa, d | {"bias": d["bias"][:3]}, 64, torch.zeros(2, dtype=torch.int32, device="cuda"),
              [256, 256], [128, 128], [256, 256])
    with pytest.raises(TypeError):
        _step(hsa, d, 64, torch.zeros(2, dtype=torch.int64, device="cuda"), [256, 256],
              [128, 128], [256, 256])


@pytest.mark.parametrize("S,k", [(16384, 512), (4096, 256)])  # fused lists path / separate path
def test_decode_step_replays_from_a_hip_graph(S, k):
    """The layer-step captured once into a HIP graph (no allocation, memset or host
    synchronisation inside the call) and replayed three times, with eager work and
    synchronisations between the replays: every replay is bit-identical to an eager
    call on the same inputs.  For a fixed position the step is idempotent (the ring
    slot and the completed pool row get the same values again), and each call leaves
    the select workspace cleared for the next."""
    import hybrid_sparse_compressed_amd as hsa

    B = 4
    w = _case(31 + S, B, S)
    pos = torch.tensor([4 * 199 + 3, 4 * (S - 2) + 3, 4 * 1000 + 1, -1], dtype=torch.int32).cuda()
    n_cand = torch.tensor([200, S - 1, S, 777], dtype=torch.int32).cuda()
    swa_len = torch.tensor([128, 128, 50, 128], dtype=torch.int32).cuda()
    comp_len = n_cand.clone()
    note("decode_step graph replay S=%d k=%d" % (S, k))

    def fresh():
        d = _dev(w)
        d["ring_x"], d["ring_g"], d["comp_kv"] = (w["ring_x"].cuda(), w["ring_g"].cuda(),
                                                  w["comp_kv"].cuda())
        return d

    def outputs():
        return (torch.empty((B, S), dtype=torch.float32, device="cuda"),
                torch.empty((B, k), dtype=torch.int32, device="cuda"),
                torch.empty((B, 64, 512), dtype=torch.bfloat16, device="cuda"),
                torch.empty((B, 64), dtype=torch.float32, device="cuda"))

    from hybrid_sparse_compressed_amd import _binding

    need = _binding.lib.hsa_decode_sparse_workspace_size(B, 64, 512, 128, S, k)
    ws = torch.zeros(max(int(need), 256), dtype=torch.uint8, device="cuda")  # zeroed once

    def call(d, o):
        return hsa.hsa_decode_step(d["x_tok"], d["g_tok"], d["bias"], d["ring_x"], d["ring_g"],
                                   pos, d["q_idx"], d["k_idx"], n_cand, k, d["q"], d["swa_kv"],
                                   swa_len, d["comp_kv"], comp_len, d["scale"], 512, scores=o[0],
                                   topk_idx=o[1], out=o[2], lse=o[3], workspace=ws)

    de, oe = fresh(), outputs()
    call(de, oe)
    torch.cuda.synchronize()

    dg, og = fresh(), outputs()
    call(dg, og)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(dg, og)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in og:
            t.zero_()
        # unrelated eager work on the same buffers' device between replays
        hsa.hsa_decode_sparse(de["q_idx"], de["k_idx"], n_cand, k, de["q"], de["swa_kv"], swa_len,
                              de["comp_kv"], comp_len, de["scale"], 512)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in (("ring_x", dg["ring_x"], de["ring_x"]), ("ring_g", dg["ring_g"], de["ring_g"]),
                           ("comp_kv", dg["comp_kv"], de["comp_kv"]), ("topk", og[1], oe[1]),
                           ("out", og[2], oe[2]), ("lse", og[3], oe[3])):
            assert torch.equal(a, b), "replay %d: %s differs from the eager call" % (rep, name)
        for b, nb in enumerate(n_cand.tolist()):
            assert torch.equal(og[0][b, :nb], oe[0][b, :nb]), "replay %d: scores" % rep


def test_decode_step_at_the_1m_workload(oracle):
    """The call the bench times: hsa_decode_step at c4_decode_1m (4 sequences x
    262,144 C4 entries: 2048-row list slots, the append as extra workgroups of the
    scoring launch).  Sequence 0's token completes the block of a pool row the
    oracle selects, so the attention must read the new entry; sequence 1 completes
    a block near the pool's end, 2 leaves its block open, 3 is idle.  Checks: the
    two separate calls bit for bit, rings bit for bit and new entries against the
    oracle's append, top-k bit-exact against the oracle's select on the GPU's own
    fp32 scores, overlap with the oracle's fp64 chain, and out / lse against the
    oracle's attention over the updated pool."""
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    w = workloads.c4_decode("c4_decode_1m", "cuda")
    B, S, k = w["cfg"]["B"], w["S"], w["cfg"]["k"]
    D = w["cfg"]["d_qk"]
    nc = w["n_cand"].cpu().numpy()
    note("decode_step 1m: oracle scores")
    rs = oracle.index_scores(w["q_idx"].cpu(), w["k_idx"].cpu(), nc)
    ridx = oracle.topk(rs.astype(np.float32), nc, k)
    r_sel = int(ridx[0][k // 2])  # a row the oracle selects for sequence 0
    g = torch.Generator().manual_seed(404)
    bf = torch.bfloat16
    app = dict(x_tok=torch.randn(B, D, generator=g).to(bf), g_tok=torch.randn(B, D, generator=g).to(bf),
               bias=(torch.randn(4, D, generator=g) * 0.1).to(bf),
               ring_x=torch.randn(B, 4, D, generator=g).to(bf),
               ring_g=torch.randn(B, 4, D, generator=g).to(bf))
    pos = torch.tensor([4 * r_sel + 3, 4 * (S - 3) + 3, 4 * 5000 + 2, -1], dtype=torch.int32)
    comp0 = w["comp_kv"].clone()
    d1 = {kk: v.cuda() for kk, v in app.items()}
    d2 = {kk: v.cuda() for kk, v in app.items()}
    pd = pos.cuda()
    note("decode_step 1m: fused step")
    s1, i1, o1, l1 = hsa.hsa_decode_step(d1["x_tok"], d1["g_tok"], d1["bias"], d1["ring_x"],
                                         d1["ring_g"], pd, w["q_idx"], w["k_idx"], w["n_cand"], k,
                                         w["q"], w["swa_kv"], w["swa_len"], w["comp_kv"],
                                         w["comp_len"], w["scale"], 512)
    torch.cuda.synchronize()
    pool1 = w["comp_kv"].clone()
    w["comp_kv"].copy_(comp0)
    note("decode_step 1m: separate calls")
    hsa.hsa_compress_append(d2["x_tok"], d2["g_tok"], d2["bias"], d2["ring_x"], d2["ring_g"], pd,
                            w["comp_kv"])
    s2, i2, o2, l2 = hsa.hsa_decode_sparse(w["q_idx"], w["k_idx"], w["n_cand"], k, w["q"],
                                           w["swa_kv"], w["swa_len"], w["comp_kv"], w["comp_len"],
                                           w["scale"], 512)
    torch.cuda.synchronize()
    for name, a, b in (("ring_x", d1["ring_x"], d2["ring_x"]), ("ring_g", d1["ring_g"], d2["ring_g"]),
                       ("pool", pool1, w["comp_kv"]), ("scores", s1, s2), ("topk", i1, i2),
                       ("out", o1, o2), ("lse", l1, l2)):
        assert torch.equal(a, b), "decode_step differs from the two separate calls: " + name

    # top-k: bit-exact against the oracle's select on the GPU's own scores
    got = i1.cpu().numpy()
    np.testing.assert_array_equal(got, oracle.topk(s1.cpu().numpy(), nc, k))
    assert r_sel in set(got[0].tolist())
    inter = sum(len(set(a[a >= 0].tolist()) & set(b[b >= 0].tolist())) for a, b in zip(got, ridx))
    ov = inter / int((ridx >= 0).sum())
    print("selected-set overlap %.6f" % ov)
    assert ov >= 0.999

    # the append: rings, new entries, untouched rows
    rx, rg = app["ring_x"].clone(), app["ring_g"].clone()
    new = np.zeros((B, S, D))
    wrote = oracle.compress_append(app["x_tok"], app["g_tok"], app["bias"], rx, rg, pos.numpy(),
                                   new, 4)
    assert wrote == [(0, r_sel), (1, S - 3)]
    assert torch.equal(d1["ring_x"].cpu().view(torch.int16), rx.view(torch.int16))
    assert torch.equal(d1["ring_g"].cpu().view(torch.int16), rg.view(torch.int16))
    comp = comp0.cpu()
    for b, r in wrote:
        compare(pool1[b, r].cpu(), new[b, r], TOL_BF16, "new entry %d" % b)
        comp[b, r] = round_bf16(new[b, r])
    changed = (pool1 != comp0).any(dim=2).nonzero().cpu().tolist()
    assert all(tuple(x) in set(wrote) for x in changed)

    ro, rl = oracle.attn_decode(w["q"].cpu(), w["swa_kv"].cpu(), w["swa_len"].cpu().numpy(), comp,
                                w["comp_len"].cpu().numpy(), w["scale"], 512, comp_idx=got)
    print(compare(o1, ro, TOL_BF16, "decode_step 1m out vs oracle"))
    print(compare(l1, rl, TOL_BF16, "decode_step 1m lse vs oracle"))
    # sequence 0 attended the new entry, not the row it replaced
    ro_old, _ = oracle.attn_decode(w["q"][:1].cpu(), w["swa_kv"][:1].cpu(),
                                   w["swa_len"][:1].cpu().numpy(), comp0[:1].cpu(),
                                   w["comp_len"][:1].cpu().numpy(), w["scale"], 512, comp_idx=got[:1])
    d_new = np.abs(o1[0].float().cpu().numpy() - ro[0]).max()
    d_old = np.abs(o1[0].float().cpu().numpy() - ro_old[0]).max()
    assert d_new < d_old, (d_new, d_old)
