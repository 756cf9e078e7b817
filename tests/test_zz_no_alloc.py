"""GPU parity: hsa_decode_step_noalloc, the decode layer-step on the library's
own fixed scratch (no workspace argument), against hsa_decode_step with a
workspace of its own, called through the C ABI.

Three calls in a row on the same scratch, each smaller than or differently laid
out from the one before: the 1M-context workload (4 x 262,144 C4 entries, the
fused list path), then 2 x 40,000 entries (the fused path with another
workspace layout), then 8 x 13,000 entries with k = 2048 (the separate
multi-workgroup select, which needs its whole workspace zero).  Each result
must equal the workspace call's bit for bit: the same kernels run on the same
inputs."""
import pytest
import torch

from helpers import note

pytestmark = pytest.mark.gpu


def _append_inputs(B, D, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    bf = torch.bfloat16
    return dict(x_tok=torch.randn(B, D, generator=g, device="cuda").to(bf),
                g_tok=torch.randn(B, D, generator=g, device="cuda").to(bf),
                bias=(torch.randn(4, D, generator=g, device="cuda") * 0.1).to(bf),
                ring_x=torch.randn(B, 4, D, generator=g, device="cuda").to(bf),
                ring_g=torch.randn(B, 4, D, generator=g, device="cuda").to(bf))


def _decode_inputs(B, S, seed, H=64, W=128, D=576):
    g = torch.Generator(device="cuda").manual_seed(seed)
    bf = torch.bfloat16
    return dict(q=torch.randn(B, H, D, generator=g, device="cuda").to(bf),
                swa_kv=torch.randn(B, W, D, generator=g, device="cuda").to(bf),
                comp_kv=torch.randn(B, S, D, generator=g, device="cuda").to(bf),
                q_idx=torch.randn(B, 64, 128, generator=g, device="cuda").to(bf),
                k_idx=torch.randn(B, S, 128, generator=g, device="cuda").to(bf),
                swa_len=torch.full((B,), W, dtype=torch.int32, device="cuda"),
                comp_len=torch.full((B,), S, dtype=torch.int32, device="cuda"),
                n_cand=torch.full((B,), S, dtype=torch.int32, device="cuda"),
                scale=1.0 / 24.0)


def _run_pair(hsa, w, a, pos, k, label):
    """The same step through hsa_decode_step (own zeroed workspace) and
    hsa_decode_step_noalloc, on separate copies of the state they update."""
    B, S = w["k_idx"].shape[0], w["k_idx"].shape[1]
    H = w["q"].shape[1]
    states = []
    for _ in range(2):
        states.append(dict(ring_x=a["ring_x"].clone(), ring_g=a["ring_g"].clone(),
                           comp_kv=w["comp_kv"].clone()))
    outs = []
    for use_static, st in zip((False, True), states):
        o = (torch.empty((B, S), dtype=torch.float32, device="cuda"),
             torch.empty((B, k), dtype=torch.int32, device="cuda"),
             torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda"),
             torch.empty((B, H), dtype=torch.float32, device="cuda"))
        note("%s: %s" % (label, "noalloc" if use_static else "workspace"))
        if use_static:
            hsa.hsa_decode_step_noalloc(a["x_tok"], a["g_tok"], a["bias"], st["ring_x"], st["ring_g"],
                                        pos, w["q_idx"], w["k_idx"], w["n_cand"], k, w["q"],
                                        w["swa_kv"], w["swa_len"], st["comp_kv"], w["comp_len"],
                                        w["scale"], 512, *o)
        else:
            hsa.hsa_decode_step(a["x_tok"], a["g_tok"], a["bias"], st["ring_x"], st["ring_g"], pos,
                                w["q_idx"], w["k_idx"], w["n_cand"], k, w["q"], w["swa_kv"],
                                w["swa_len"], st["comp_kv"], w["comp_len"], w["scale"], 512,
                                scores=o[0], topk_idx=o[1], out=o[2], lse=o[3],
                                workspace=torch.zeros(
                                    hsa.lib.hsa_decode_sparse_workspace_size(B, H, 512, 128, S, k),
                                    dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        outs.append(o)
    (s1, i1, o1, l1), (s2, i2, o2, l2) = outs
    n = w["n_cand"].cpu().tolist()
    for b in range(B):
        assert torch.equal(s1[b, :n[b]], s2[b, :n[b]]), label + ": scores"
    assert torch.equal(i1, i2), label + ": top-k indices"
    assert torch.equal(o1, o2), label + ": out"
    assert torch.equal(l1, l2), label + ": lse"
    for key in ("ring_x", "ring_g", "comp_kv"):
        assert torch.equal(states[0][key], states[1][key]), label + ": " + key
    assert (i2 >= 0).all() or (w["n_cand"] < k).any()


def test_noalloc_step_matches_the_workspace_call_across_sizes():
    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    # 1. the 1M-context workload, a completing position
    w = workloads.c4_decode("c4_decode_1m", "cuda")
    S = w["S"]
    a = _append_inputs(4, 576, 11)
    pos = torch.full((4,), 4 * (S - 1) + 3, dtype=torch.int32, device="cuda")
    _run_pair(hsa, w, a, pos, 512, "1m")
    del w
    torch.cuda.empty_cache()
    # 2. smaller: 2 x 40,000, another layout of the same fused path, ragged counts
    w = _decode_inputs(2, 40000, 12)
    w["n_cand"] = torch.tensor([40000, 31111], dtype=torch.int32, device="cuda")
    a = _append_inputs(2, 576, 13)
    pos = torch.tensor([4 * 100 + 3, 4 * 7 + 1], dtype=torch.int32, device="cuda")
    _run_pair(hsa, w, a, pos, 512, "40k")
    # 3. the separate multi-workgroup select (k = 2048, 8 sequences)
    w = _decode_inputs(8, 13000, 14)
    a = _append_inputs(8, 576, 15)
    pos = torch.full((8,), 4 * 12999 + 3, dtype=torch.int32, device="cuda")
    _run_pair(hsa, w, a, pos, 2048, "13k-k2048")
