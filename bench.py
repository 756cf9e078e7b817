"""Decode layer-step benchmark of the hybrid sparse-attention hot path on one MI355X.

Workload (c4_decode_1m): 4 sequences x 1,048,576 tokens, 262,144 C4 entries
each, 64 heads over a 576-wide latent (value 512), window 128, indexer
64 heads x 128, top-512; synthetic seeded inputs resident in HBM.

One step = one decode layer-step: indexer scores over every C4 key, exact
radix top-512 select, and the SWA + selected-C4 attention with split-KV merge,
together with the decode-time compression state update, all in one
hsa_decode_step call (scoring, which also leaves per-2048-candidate lists
and carries the compression-state append as extra workgroups; attention that
finishes the select from the lists; merge): each
sequence's new token enters its 4-token ring and on every 4th step completes
the block, whose C4 entry is written to the pool before the attention runs.
Two copies of the
indexer inputs alternate between steps so the 268 MB key stream is larger
than the on-die cache across a pair of steps.

After the metric, "rows" measures every other row of the path at its own
full-size workload (compressor, prefill indexer + top-k and prefill attention
at prefill_32k, dense C128 decode, fused sparse decode at c4_decode_64k, the
compression-state append at the C4 and C128 decode batches), each against its
own roofline; --no-rows skips them.

Prints ONE JSON line (rank 0).  --gpus N > 1 is not supported: the path is
measured on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "hybrid-attn decode layer-steps/s + achieved HBM GB/s (C4 top-512, 1M ctx)"
HBM_PEAK_GBPS = 8000.0
PMC_FILE = os.path.join(ROOT, "profiles", "score_kernel_c4_decode_1m_pmc.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=12)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time over which the oracle layer-step is repeated")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the per-row measurements at the other workloads")
    ap.add_argument("--rows-only", action="store_true",
                    help="only the per-row measurements (a JSON object of rows), for profiling them")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before warm-up, run three plain device copies of this many MiB, so that "
                         "a hardware byte counter can be scaled by a transfer of known size")
    return ap.parse_args()


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def score_kernel_sources():
    c = os.path.join(ROOT, "hybrid_sparse_compressed_amd", "csrc")
    return [os.path.join(c, f) for f in ("index_topk.hip", "hsa_common.hpp", "hsa_internal.hpp",
                                         "select.hpp", "compress_append.hpp")]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the hot path on one GPU only; --gpus %d is not supported "
              "(the multi-GPU sharding is a design note, not a built path)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    import hybrid_sparse_compressed_amd as hsa
    from hybrid_sparse_compressed_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.rows_only:
        if args.copy_calibration_mib > 0:
            copy_calibration(torch, dev, args.copy_calibration_mib)
        print(json.dumps({"rows": other_rows(hsa, workloads)}), flush=True)
        return
    name = "c4_decode_1m"
    w = workloads.c4_decode(name, dev)
    c = w["cfg"]
    B, S, k, H, d_qk, d_v, W = c["B"], w["S"], c["k"], c["H"], c["d_qk"], c["d_v"], c["W"]
    H_I, d_I = c["H_I"], c["d_I"]
    # second copy of the indexer inputs (different seed), alternated per step
    g2 = torch.Generator(device=dev).manual_seed(c["seed"] + 100)
    k_idx2 = torch.randn(w["k_idx"].shape, generator=g2, device=dev).to(torch.bfloat16)
    q_idx2 = torch.randn(w["q_idx"].shape, generator=g2, device=dev).to(torch.bfloat16)
    workloads.plant_duplicate_rows(k_idx2, c["dup_frac"], workloads._Draw(c["seed"] + 100, dev))
    sets = [(w["q_idx"], w["k_idx"]), (q_idx2, k_idx2)]
    # decode-time compression state: every step appends each sequence's token to its
    # 4-token ring; one step in four completes the block and writes its C4 entry
    xt = torch.randn((B, d_qk), generator=g2, device=dev).to(torch.bfloat16)
    gt = torch.randn((B, d_qk), generator=g2, device=dev).to(torch.bfloat16)
    bb = (torch.randn((4, d_qk), generator=g2, device=dev) * 0.1).to(torch.bfloat16)
    ring_x = torch.randn((B, 4, d_qk), generator=g2, device=dev).to(torch.bfloat16)
    ring_g = torch.randn((B, 4, d_qk), generator=g2, device=dev).to(torch.bfloat16)
    # positions at the end of the context: the completed block's entry lands in the
    # C4 pool's last row
    pos4 = [torch.full((B,), 4 * (S - 1) + j, dtype=torch.int32, device=dev) for j in range(4)]

    stream = torch.cuda.current_stream()
    scores = torch.empty((B, S), dtype=torch.float32, device=dev)
    idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    out = torch.empty((B, H, d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(256, hsa.lib.hsa_decode_sparse_workspace_size(B, H, d_v, W, S, k)),
                     dtype=torch.uint8, device=dev)

    def step(i):
        qi, ki = sets[i & 1]
        hsa.hsa_decode_step(xt, gt, bb, ring_x, ring_g, pos4[i & 3], qi, ki, w["n_cand"], k,
                            w["q"], w["swa_kv"], w["swa_len"], w["comp_kv"], w["comp_len"],
                            w["scale"], d_v, scores=scores, topk_idx=idx, out=out, lse=lse,
                            workspace=ws)

    if args.copy_calibration_mib > 0:
        copy_calibration(torch, dev, args.copy_calibration_mib)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    fams = {"compress": hsa.HSA_PROF_COMPRESS, "score": hsa.HSA_PROF_SCORE,
            "select": hsa.HSA_PROF_SELECT, "attn": hsa.HSA_PROF_ATTN, "merge": hsa.HSA_PROF_MERGE}

    # timed region (value): nothing but the steps between the two synchronisations
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_per_step = ms_total / args.steps

    def instrumented(mask):
        """The same steps again with the library's event pair around each launch of the
        kernel families in mask (on the stream the kernels run on)."""
        for f in fams.values():
            hsa.hsa_profile_read(f, reset=True)
        hsa.hsa_profile_enable(mask)
        torch.cuda.synchronize()
        ti = time.perf_counter()
        for i in range(args.steps):
            step(args.warmup + i)
        torch.cuda.synchronize()
        hsa.hsa_profile_enable(0)
        ms = (time.perf_counter() - ti) * 1000.0 / args.steps
        got = {}
        for nm, f in fams.items():
            if mask & f:
                tot, n = hsa.hsa_profile_read(f)
                got[nm] = {"avg_us": round(1000.0 * tot / n, 3) if n else None, "launches": n}
        return ms, got

    # one pass with every kernel family's event pair: the per-kernel breakdown and
    # the dominant kernel's duration come from the same launches
    ms_instr, breakdown = instrumented(sum(fams.values()))

    # what the memory system delivers to the scoring kernel's launch shape: a plain
    # read of the same key bytes (512 workgroups, one contiguous 512 KB part each;
    # the two copies alternating as in the steps), timed by the same event pairs
    stream_us = None
    kb = [sets[0][1], sets[1][1]]
    if (kb[0].numel() * kb[0].element_size()) % (16 << 20) == 0:
        sink = torch.empty(4096, dtype=torch.uint8, device=dev)
        for i in range(8):
            hsa.hsa_stream_read(kb[i & 1], sink)
        torch.cuda.synchronize()
        hsa.hsa_profile_read(hsa.HSA_PROF_STREAM, reset=True)
        hsa.hsa_profile_enable(hsa.HSA_PROF_STREAM)
        for i in range(args.steps):
            hsa.hsa_stream_read(kb[i & 1], sink)
        torch.cuda.synchronize()
        hsa.hsa_profile_enable(0)
        tot, n = hsa.hsa_profile_read(hsa.HSA_PROF_STREAM, reset=True)
        stream_us = round(1000.0 * tot / n, 3) if n else None

    # roofline of the dominant kernel (indexer scoring): algorithmic bytes per launch
    alg_bytes = B * S * d_I * 2 + B * H_I * d_I * 2
    score_us = breakdown["score"]["avg_us"]
    achieved = alg_bytes / (score_us * 1e-6) / 1e9
    traffic = None
    if os.path.exists(PMC_FILE):
        pmc = json.load(open(PMC_FILE))
        if pmc.get("source_hash") == source_hash(score_kernel_sources()):
            traffic = pmc.get("hbm_bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "scope": "dominant kernel",
                "kernel": "score_kernel (indexer scores, first-digit histogram, candidate lists)",
                "avg_us": score_us, "alg_bytes_per_launch": alg_bytes}
    if stream_us:
        kbytes = kb[0].numel() * kb[0].element_size()
        roofline["plain_read"] = {
            "what": "hsa_stream_read of the same %d key bytes in the same launch shape" % kbytes,
            "avg_us": stream_us, "GBps": round(kbytes / (stream_us * 1e-6) / 1e9, 1),
            "score_kernel_vs_plain_read": round(stream_us / score_us, 4)}

    # the whole layer-step against the same peak: its algorithmic bytes over the
    # timed step time (the metric's own roofline)
    step_bytes = (B * S * d_I * 2 + B * (W + k) * d_qk * 2 + B * H * d_qk * 2 + B * H * d_v * 2
                  + B * H_I * d_I * 2 + B * k * 4)
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    step_roofline = {"bound": "hbm", "achieved": round(step_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(step_gbps / HBM_PEAK_GBPS, 4),
                     "scope": "whole decode layer-step (value)", "alg_bytes_per_step": step_bytes,
                     "us_per_step": round(ms_per_step * 1000.0, 2)}
    value = 1000.0 / ms_per_step
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_instrumented": round(ms_instr, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1); 1% duplicated indexer key rows)",
        "config": {"workload": name, "batch": B, "context": c["L"], "c4_entries": S, "heads": H,
                   "latent": d_qk, "value_dim": d_v, "window": W, "topk": k,
                   "indexer": "%dx%d" % (H_I, d_I)},
        "achieved_GBps": round(step_gbps, 1),
        "alg_bytes_per_step": step_bytes,
        "breakdown_us": breakdown,
        "roofline": roofline,
        "step_roofline": step_roofline,
        "cpu_baseline": None,
    }

    if not args.no_rows:
        res["rows"] = other_rows(hsa, workloads)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def copy_calibration(torch, dev, mib):
    """Three plain device copies of mib MiB: a transfer of known size for scaling the
    hardware byte counters."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


ROW_WARM_MS = 40.0


def _warm(torch, fn, warm_ms=ROW_WARM_MS):
    """Back-to-back calls of fn() for at least warm_ms of wall time.  The GPU's
    core clock ramps up over a few tens of milliseconds of sustained work (an
    MI355X prefill attention call measured 2.93 ms right after an idle pause and
    2.32 ms ten calls later), so every row is timed at its steady-state clock."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= warm_ms:
                break
    torch.cuda.synchronize()


def _median_us(torch, fn, reps, inner=1):
    """Median time per call of fn() on the current stream, in microseconds: reps
    measurements of `inner` back-to-back calls each (after a steady-state warm-up,
    _warm), so that short calls are timed as a stream of calls, not with the host's
    launch latency."""
    _warm(torch, fn)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        e0.record()
        for _ in range(inner):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1000.0 / inner)
    ts.sort()
    return ts[len(ts) // 2]


def _graph_us(torch, fn, reps, inner):
    """Median time per call of fn() for calls of a few microseconds: `inner` calls are
    captured once into a HIP graph (after one eager warm-up call), and each of the reps
    measurements replays it, so the host's per-call cost does not set the pace."""
    fn()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(inner):
            fn()
    _warm(torch, g.replay)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1000.0 / inner)
    ts.sort()
    return ts[len(ts) // 2]


def _row(workload, us, bound, alg, unit, peak, **extra):
    if unit == "GB/s":
        achieved = alg / (us * 1e-6) / 1e9
    else:  # TFLOP/s
        achieved = alg / (us * 1e-6) / 1e12
    r = {"workload": workload, "us": round(us, 2), "bound": bound, "alg": alg,
         "achieved": round(achieved, 1), "unit": unit, "peak": peak,
         "frac": round(achieved / peak, 4)}
    r.update(extra)
    return r


def other_rows(hsa, workloads):
    """Each row of the path at its own full-size workload (whole calls, median of a few):
    the compressor and the prefill chain at prefill_32k (compress -> indexer + top-k over
    16,384 queries -> prefill attention over their own top-512), the dense C128 decode at
    c128_dense_decode, and the fused sparse decode at c4_decode_64k."""
    import torch

    rows = {}
    w = workloads.prefill("cuda")
    n_seq, T, D = 8, 32768, 576
    c4 = torch.empty((n_seq, T // 4, D), dtype=torch.bfloat16, device="cuda")
    c128 = torch.empty((n_seq, T // 128, D), dtype=torch.bfloat16, device="cuda")
    # each call reads x and its gate once and writes the entries once
    for m, g, b, out, key in ((4, w["gate4"], w["bias4"], c4, "a1_compress_c4"),
                              (128, w["gate128"], w["bias128"], c128, "a1_compress_c128")):
        us = _median_us(torch, lambda: hsa.hsa_compress(w["x"], g, b, m, out=out), 5, 5)
        alg = 2 * n_seq * T * D * 2 + m * D * 2 + n_seq * (T // m) * D * 2
        rows[key] = _row("prefill_32k", us, "hbm", alg, "GB/s", HBM_PEAK_GBPS)
    Nq, S, k = 16384, T // 4, 512
    scores = torch.empty((Nq, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((Nq, k), dtype=torch.int32, device="cuda")
    us = _median_us(torch, lambda: hsa.hsa_index_topk(w["q_idx"], w["k_idx"], w["n_cand"], k,
                                                      q_seq=w["q_seq"], scores=scores,
                                                      topk_idx=idx), 5)
    # q_I read once, K_I once, the indices written once (the fp32 score round trip,
    # 2 x 536.9 MB, is the implementation's and not counted)
    alg = Nq * 64 * 128 * 2 + n_seq * S * 128 * 2 + Nq * k * 4
    n_cand = w["n_cand"].double().sum().item()
    rows["a2_a3_index_topk"] = _row("prefill_32k", us, "hbm", alg, "GB/s", HBM_PEAK_GBPS,
                                    queries=Nq, per_head_tflop=round(n_cand * 64 * 128 * 2 / 1e12, 3))
    out = torch.empty((n_seq, 2048, 64, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((n_seq, 2048, 64), dtype=torch.float32, device="cuda")
    us = _median_us(torch, lambda: hsa.hsa_attn_prefill(w["q"], w["x"], c4, w["q_start"], 128, 4,
                                                        w["scale"], 512, comp_idx=idx, out=out,
                                                        lse=lse), 5)
    flop = Nq * 64 * (128 + k) * (576 + 512) * 2
    rows["a5_prefill_attention"] = _row("prefill_32k", us, "mfma", flop, "TFLOP/s", 2500.0)
    del w, c4, c128, scores, idx, out, lse
    torch.cuda.empty_cache()

    d = workloads.c128_dense_decode("cuda")
    lens = d["lengths"]
    alg = sum((128 + L // 128) * 1152 + 139264 for L in lens)
    outd = torch.empty((len(lens), 64, 512), dtype=torch.bfloat16, device="cuda")
    lsed = torch.empty((len(lens), 64), dtype=torch.float32, device="cuda")
    us = _median_us(torch, lambda: hsa.hsa_attn_decode(d["q"], d["swa_kv"], d["swa_len"],
                                                       d["comp_kv"], d["comp_len"], d["scale"],
                                                       512, out=outd, lse=lsed), 7, 20)
    rows["a4_dense_decode_c128"] = _row("c128_dense_decode", us, "hbm", alg, "GB/s",
                                        HBM_PEAK_GBPS)
    del d
    e = workloads.c4_decode("c4_decode_64k", "cuda")
    sc = torch.empty((1, e["comp_kv"].shape[1]), dtype=torch.float32, device="cuda")
    ix = torch.empty((1, 512), dtype=torch.int32, device="cuda")
    oe = torch.empty((1, 64, 512), dtype=torch.bfloat16, device="cuda")
    le = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    us = _median_us(torch, lambda: hsa.hsa_decode_sparse(e["q_idx"], e["k_idx"], e["n_cand"], 512,
                                                         e["q"], e["swa_kv"], e["swa_len"],
                                                         e["comp_kv"], e["comp_len"], e["scale"],
                                                         512, scores=sc, topk_idx=ix, out=oe,
                                                         lse=le), 7, 20)
    rows["a2_a3_a4_decode_c4_64k"] = _row("c4_decode_64k", us, "hbm", 5089280, "GB/s",
                                          HBM_PEAK_GBPS)
    del e
    rows.update(append_rows(hsa, torch))
    torch.cuda.empty_cache()
    rows.update(paged_step_rows(hsa, workloads, torch))
    torch.cuda.empty_cache()
    return rows


def paged_step_rows(hsa, workloads, torch):
    """The metric's layer-step on paged pools: c4_decode_1m with the indexer keys and
    the C4 pool on shuffled 256-row pages and the window and compression state on
    64-token SWA pages (only the pages the window and the open block use resident),
    timed next to the same step on the flat pools (same inputs, same bytes)."""
    w = workloads.c4_decode("c4_decode_1m", "cuda")
    c = w["cfg"]
    B, S, k, H, D, W = c["B"], w["S"], c["k"], c["H"], c["d_qk"], c["W"]
    g = torch.Generator().manual_seed(11)
    bf = torch.bfloat16

    def paged(flat, P):
        n = flat.shape[1] // P
        perm = torch.randperm(B * n, generator=g).cuda()
        pool = torch.empty((B * n, P, flat.shape[2]), dtype=bf, device="cuda")
        pool[perm] = flat.reshape(B * n, P, flat.shape[2])
        return pool, perm.reshape(B, n).to(torch.int32)

    kI, kmap = paged(w["k_idx"], 256)
    c4, cmap = paged(w["comp_kv"], 256)
    P = 64
    pos = torch.full((B,), 4 * (S - 1) + 3, dtype=torch.int32, device="cuda")
    last = (4 * (S - 1) + 3) // P
    smap = torch.full((B, last + 1), -1, dtype=torch.int32)
    for b in range(B):  # the window (128 tokens) and the open block: the last three pages
        for j in range(3):
            smap[b, last - j] = 3 * b + j
    smap = smap.cuda()
    swa = torch.randn((3 * B, P, D), device="cuda").to(bf)
    sx, sg = torch.randn_like(swa, dtype=torch.float32).to(bf), torch.randn_like(swa, dtype=torch.float32).to(bf)
    xt = torch.randn((B, D), device="cuda").to(bf)
    gt = torch.randn((B, D), device="cuda").to(bf)
    bias = (torch.randn((4, D), device="cuda") * 0.1).to(bf)
    rx, rg = torch.randn((B, 4, D), device="cuda").to(bf), torch.randn((B, 4, D), device="cuda").to(bf)
    sc = torch.empty((B, S), dtype=torch.float32, device="cuda")
    ix = torch.empty((B, k), dtype=torch.int32, device="cuda")
    o = torch.empty((B, H, 512), dtype=bf, device="cuda")
    l = torch.empty((B, H), dtype=torch.float32, device="cuda")
    us = _median_us(torch, lambda: hsa.hsa_decode_step_paged(
        xt, gt, bias, sx, sg, pos, w["q_idx"], kI, kmap, w["n_cand"], k, w["q"], swa, smap,
        w["swa_len"], c4, cmap, w["comp_len"], w["scale"], 512, W, S, scores=sc, topk_idx=ix,
        out=o, lse=l), 7, 20)
    flat_us = _median_us(torch, lambda: hsa.hsa_decode_step(
        xt, gt, bias, rx, rg, pos, w["q_idx"], w["k_idx"], w["n_cand"], k, w["q"], w["swa_kv"],
        w["swa_len"], w["comp_kv"], w["comp_len"], w["scale"], 512, scores=sc, topk_idx=ix,
        out=o, lse=l), 7, 20)
    alg = (B * S * 128 * 2 + B * (W + k) * D * 2 + B * H * D * 2 + B * H * 512 * 2
           + B * 64 * 128 * 2 + B * k * 4)
    rows = {"f2_decode_step_paged_c4_1m": _row("c4_decode_1m", us, "hbm", alg, "GB/s", HBM_PEAK_GBPS,
                                               flat_us=round(flat_us, 2), page_rows={"swa": P, "c4": 256})}
    # the weighted, activated indexer heads (MFMA per head) on the same workload,
    # without the append, next to the unit-weight call
    hw = (torch.rand((B, 64), generator=g) * 2.0 - 0.3).float().cuda()
    wus = _median_us(torch, lambda: hsa.hsa_decode_sparse_weighted(
        w["q_idx"], hw, w["k_idx"], w["n_cand"], k, w["q"], w["swa_kv"], w["swa_len"], w["comp_kv"],
        w["comp_len"], w["scale"], 512, scores=sc, topk_idx=ix, out=o, lse=l), 7, 20)
    uus = _median_us(torch, lambda: hsa.hsa_decode_sparse(
        w["q_idx"], w["k_idx"], w["n_cand"], k, w["q"], w["swa_kv"], w["swa_len"], w["comp_kv"],
        w["comp_len"], w["scale"], 512, scores=sc, topk_idx=ix, out=o, lse=l), 7, 20)
    rows["f3_decode_sparse_weighted_heads_c4_1m"] = _row(
        "c4_decode_1m", wus, "hbm", alg, "GB/s", HBM_PEAK_GBPS, unit_weight_us=round(uus, 2),
        mfma_tflop=round(B * S * 64 * 128 * 2 / 1e12, 4))
    return rows


def append_rows(hsa, torch):
    """Decode-time compression state: one token per sequence appended to its ring,
    at the C4 decode batch (4 sequences, m=4) and the C128 one (32 sequences, m=128),
    latent 576 bf16, both for a call that completes every sequence's block and for
    one that does not.  Positions sit at the end of the long contexts."""
    rows = {}
    D = 576
    g = torch.Generator(device="cuda").manual_seed(5)
    for B, m, n_blocks, key in ((4, 4, 262144, "c4"), (32, 128, 1024, "c128")):
        rx = torch.randn(B, m, D, device="cuda", generator=g).to(torch.bfloat16)
        rg = torch.randn(B, m, D, device="cuda", generator=g).to(torch.bfloat16)
        xt = torch.randn(B, D, device="cuda", generator=g).to(torch.bfloat16)
        gt = torch.randn(B, D, device="cuda", generator=g).to(torch.bfloat16)
        bias = (torch.randn(m, D, device="cuda", generator=g) * 0.1).to(torch.bfloat16)
        pool = torch.empty(B, n_blocks, D, dtype=torch.bfloat16, device="cuda")
        last = (n_blocks - 1) * m
        for tag, p in (("complete", last + m - 1), ("open", last)):
            pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
            us = _graph_us(torch, lambda: hsa.hsa_compress_append(xt, gt, bias, rx, rg, pos, pool),
                           7, 50)
            # token in (x, g), ring slot out (x, g); on completion the other m-1 ring
            # rows in, the entry out, and the bias once
            per_seq = 4 * D * 2 + ((2 * (m - 1) + 1) * D * 2 if tag == "complete" else 0)
            alg = B * per_seq + (m * D * 2 if tag == "complete" else 0)
            rows["f1_compress_append_%s_%s" % (key, tag)] = _row(
                "c4_decode_1m" if key == "c4" else "c128_dense_decode", us, "hbm", alg, "GB/s",
                HBM_PEAK_GBPS)
        del rx, rg, pool
    return rows


def cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(w, min_seconds):
    """The oracle's whole decode layer-step (all sequences), repeated for ~min_seconds."""
    import numpy as np
    import torch

    import oracle

    oracle.build(force=False)
    c = w["cfg"]
    k = c["k"]
    q_idx, k_idx = w["q_idx"].cpu(), w["k_idx"].cpu()
    q, swa, comp = w["q"].cpu(), w["swa_kv"].cpu(), w["comp_kv"].cpu()
    n_cand = w["n_cand"].cpu().numpy()
    swa_len, comp_len = w["swa_len"].cpu().numpy(), w["comp_len"].cpu().numpy()
    B, S, D = comp.shape
    g = torch.Generator().manual_seed(5)
    xt, gt = (torch.randn(B, D, generator=g).to(torch.bfloat16) for _ in range(2))
    bias = (torch.randn(4, D, generator=g) * 0.1).to(torch.bfloat16)
    ring_x, ring_g = (torch.randn(B, 4, D, generator=g).to(torch.bfloat16) for _ in range(2))
    pool = np.zeros((B, S, D))  # zero pages: only the rows written get memory
    reps, t = 0, time.perf_counter()
    while True:
        pos = np.full(B, 4 * (S - 1) + (reps & 3), np.int32)
        oracle.compress_append(xt, gt, bias, ring_x, ring_g, pos, pool, 4)
        sc = oracle.index_scores(q_idx, k_idx, n_cand)
        idx = oracle.topk(sc.astype(np.float32), n_cand, k)
        oracle.attn_decode(q, swa, swa_len, comp, comp_len, w["scale"], c["d_v"], comp_idx=idx)
        reps += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds:
            break
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        cores = min(cores, int(omp))
    return {"value": round(reps / dt, 5), "unit": "layer-steps/s", "cores": cores,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "%d repetition(s) of the whole c4_decode_1m layer-step (compression-state "
                      "append, fp64 scores over all 4 x 262,144 C4 keys, select, attention) in "
                      "%.1f s" % (reps, dt)}


if __name__ == "__main__":
    main()
