"""Seeded synthetic inputs for the hybrid sparse-attention hot path.

This module holds no arithmetic of the method: it only draws seeded random
tensors with the shapes, dtypes and structure of the workloads below and
hands them to both the HIP library and the CPU oracle.  Values are drawn in
fp32 (torch's seeded generator on the chosen device) and rounded to the
storage dtype by torch's round-to-nearest-even cast.

Workloads (shapes of the decode/prefill layer, one GPU):
  tiny_fp32_decode : fp32, 1 sequence, 1024 tokens, 8 heads x d 128 over one
                     latent KV head (d_v = d_qk = 128), window 128, C4 over the
                     1024 tokens (256 entries), indexer 1 head x d 64, top-64.
  c4_decode_64k    : bf16, 1 sequence, 65,536 tokens (16,384 C4 entries),
                     64 heads, latent 576 (value 512), window 128, indexer
                     64 heads x d 128, top-512.
  c128_dense_decode: bf16, 32 sequences with lengths uniform in
                     [16,384, 131,072] (up to 1024 C128 entries), 64 heads,
                     latent 576/512, window 128, all compressed entries.
  c4_decode_1m     : bf16, 4 sequences of 1,048,576 tokens (262,144 C4
                     entries each), 64 heads, latent 576/512, window 128,
                     indexer 64 x 128, top-512; 1 % of the indexer key rows of
                     each sequence are exact copies of other rows (planted
                     score ties).
  prefill_32k      : bf16, 8 sequences x 32,768 tokens, latent 576; C4 and
                     C128 compression of every complete block, then the last
                     2048 query positions of each sequence attend to their
                     causal window of 128 plus their own top-512 C4 entries.
Gates ~ N(0, 1), biases ~ N(0, 0.1^2) (standard deviation 0.1), everything
else ~ N(0, 1).
"""
from __future__ import annotations

import math

import torch

WORKLOADS = {
    "tiny_fp32_decode": dict(B=1, L=1024, H=8, d_qk=128, d_v=128, W=128, m=4, H_I=1, d_I=64,
                             k=64, dtype="fp32", seed=1001),
    "c4_decode_64k": dict(B=1, L=65536, H=64, d_qk=576, d_v=512, W=128, m=4, H_I=64, d_I=128,
                          k=512, dtype="bf16", seed=1002),
    "c128_dense_decode": dict(B=32, L_min=16384, L_max=131072, H=64, d_qk=576, d_v=512, W=128,
                              m=128, dtype="bf16", seed=1003),
    "c4_decode_1m": dict(B=4, L=1048576, H=64, d_qk=576, d_v=512, W=128, m=4, H_I=64, d_I=128,
                         k=512, dtype="bf16", dup_frac=0.01, seed=1004),
    "prefill_32k": dict(n_seq=8, T=32768, n_q=2048, H=64, d_qk=576, d_v=512, W=128, H_I=64,
                        d_I=128, k=512, dtype="bf16", seed=1005),
}

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


class _Draw:
    """Seeded N(0, std^2) draws in a fixed order, cast to the storage dtype."""

    def __init__(self, seed: int, device):
        self.device = torch.device(device)
        self.g = torch.Generator(device=self.device)
        self.g.manual_seed(seed)
        self.cpu = torch.Generator()
        self.cpu.manual_seed(seed + 7919)

    def normal(self, shape, dtype, std=1.0, chunk_dim0=False):
        if not chunk_dim0:
            t = torch.randn(shape, generator=self.g, device=self.device, dtype=torch.float32)
            if std != 1.0:
                t.mul_(std)
            return t.to(dtype)
        out = torch.empty(shape, dtype=dtype, device=self.device)
        for i in range(shape[0]):  # bounded fp32 temporaries for large tensors
            t = torch.randn(shape[1:], generator=self.g, device=self.device, dtype=torch.float32)
            if std != 1.0:
                t.mul_(std)
            out[i].copy_(t.to(dtype))
        return out

    def ints(self, lo, hi, n):
        """n integers uniform in [lo, hi] (inclusive), drawn on the CPU."""
        return torch.randint(lo, hi + 1, (n,), generator=self.cpu, dtype=torch.int64)

    def perm(self, n):
        return torch.randperm(n, generator=self.cpu)


def _i32(vals, device):
    return torch.as_tensor(vals, dtype=torch.int32, device=device)


def plant_duplicate_rows(k_idx: torch.Tensor, frac: float, draw: _Draw):
    """Overwrite `frac` of the rows of each sequence with copies of other rows."""
    B, S, _ = k_idx.shape
    n = int(S * frac)
    for b in range(B):
        dst = draw.perm(S)[:n].to(k_idx.device)
        src = draw.ints(0, S - 1, n).to(k_idx.device)
        k_idx[b, dst] = k_idx[b, src]
    return k_idx


def tiny_fp32_decode(device="cpu"):
    c = WORKLOADS["tiny_fp32_decode"]
    d = _Draw(c["seed"], device)
    dt = _DT[c["dtype"]]
    B, L, D = c["B"], c["L"], c["d_qk"]
    S = L // c["m"]
    x = d.normal((B, L, D), dt)
    gate = d.normal((B, L, D), dt)
    bias = d.normal((c["m"], D), dt, std=0.1)
    q = d.normal((B, c["H"], D), dt)
    q_idx = d.normal((B, c["H_I"], c["d_I"]), dt)
    k_idx = d.normal((B, S, c["d_I"]), dt)
    # token t sits in ring slot t mod W; the last W tokens fill slots 0..W-1 in order
    swa = x[:, L - c["W"]:, :].clone()
    return dict(cfg=c, x=x, gate=gate, bias=bias, q=q, q_idx=q_idx, k_idx=k_idx, swa_kv=swa,
                swa_len=_i32([c["W"]] * B, device), n_cand=_i32([S] * B, device),
                comp_len=_i32([S] * B, device), S=S, scale=1.0 / math.sqrt(D))


def c4_decode(name="c4_decode_1m", device="cpu", B=None, L=None):
    """Decode-layer inputs of the C4 workloads (B and L may be overridden for small tests)."""
    c = dict(WORKLOADS[name])
    if B is not None:
        c["B"] = B
    if L is not None:
        c["L"] = L
    d = _Draw(c["seed"], device)
    dt = _DT[c["dtype"]]
    B, L = c["B"], c["L"]
    S = L // c["m"]
    q = d.normal((B, c["H"], c["d_qk"]), dt)
    swa = d.normal((B, c["W"], c["d_qk"]), dt)
    comp = d.normal((B, S, c["d_qk"]), dt, chunk_dim0=True)
    q_idx = d.normal((B, c["H_I"], c["d_I"]), dt)
    k_idx = d.normal((B, S, c["d_I"]), dt, chunk_dim0=True)
    if c.get("dup_frac"):
        plant_duplicate_rows(k_idx, c["dup_frac"], d)
    return dict(cfg=c, q=q, swa_kv=swa, comp_kv=comp, q_idx=q_idx, k_idx=k_idx,
                swa_len=_i32([min(L, c["W"])] * B, device), comp_len=_i32([S] * B, device),
                n_cand=_i32([S] * B, device), S=S, scale=1.0 / math.sqrt(c["d_qk"]))


def c128_dense_decode(device="cpu", B=None):
    c = dict(WORKLOADS["c128_dense_decode"])
    if B is not None:
        c["B"] = B
    d = _Draw(c["seed"], device)
    dt = _DT[c["dtype"]]
    B = c["B"]
    lens = d.ints(c["L_min"], c["L_max"], B)
    S_max = c["L_max"] // c["m"]
    q = d.normal((B, c["H"], c["d_qk"]), dt)
    swa = d.normal((B, c["W"], c["d_qk"]), dt)
    comp = d.normal((B, S_max, c["d_qk"]), dt, chunk_dim0=True)
    return dict(cfg=c, q=q, swa_kv=swa, comp_kv=comp, lengths=lens.tolist(),
                swa_len=_i32([c["W"]] * B, device),
                comp_len=_i32((lens // c["m"]).tolist(), device), S_max=S_max,
                scale=1.0 / math.sqrt(c["d_qk"]))


def prefill(device="cpu", n_seq=None, T=None, n_q=None):
    """Prefill-chunk inputs (sizes may be overridden for small tests)."""
    c = dict(WORKLOADS["prefill_32k"])
    for key, v in (("n_seq", n_seq), ("T", T), ("n_q", n_q)):
        if v is not None:
            c[key] = v
    d = _Draw(c["seed"], device)
    dt = _DT[c["dtype"]]
    n_seq, T, n_q, D = c["n_seq"], c["T"], c["n_q"], c["d_qk"]
    x = d.normal((n_seq, T, D), dt, chunk_dim0=True)
    gate4 = d.normal((n_seq, T, D), dt, chunk_dim0=True)
    gate128 = d.normal((n_seq, T, D), dt, chunk_dim0=True)
    bias4 = d.normal((4, D), dt, std=0.1)
    bias128 = d.normal((128, D), dt, std=0.1)
    q = d.normal((n_seq, n_q, c["H"], D), dt, chunk_dim0=True)
    q_idx = d.normal((n_seq * n_q, c["H_I"], c["d_I"]), dt)
    k_idx = d.normal((n_seq, T // 4, c["d_I"]), dt, chunk_dim0=True)
    q_start = T - n_q
    pos = torch.arange(q_start, T, dtype=torch.int64)
    n_cand = ((pos + 1) // 4).repeat(n_seq).to(torch.int32).to(device)
    q_seq = torch.arange(n_seq, dtype=torch.int32).repeat_interleave(n_q).to(device)
    return dict(cfg=c, x=x, gate4=gate4, gate128=gate128, bias4=bias4, bias128=bias128, q=q,
                q_idx=q_idx, k_idx=k_idx, q_start=q_start, n_cand=n_cand, q_seq=q_seq,
                scale=1.0 / math.sqrt(D))


def topk_scores(Nq, S, device="cpu", seed=2001, dup_frac=0.01):
    """fp32 N(0,1) scores with `dup_frac` of each row overwritten by copies of other entries."""
    d = _Draw(seed, device)
    s = torch.randn((Nq, S), generator=d.g, device=d.device, dtype=torch.float32)
    n = int(S * dup_frac)
    for i in range(Nq):
        dst = d.perm(S)[:n].to(s.device)
        src = d.ints(0, S - 1, n).to(s.device)
        s[i, dst] = s[i, src]
    return s
