"""CPU oracle for the hybrid sparse-attention hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``hybrid_sparse_compressed_amd``) never imports, links or calls it.

The arithmetic lives in ``oracle.c`` (plain C loops, fp64 accumulation); this
module only builds it with gcc and marshals numpy / CPU-torch arrays into it.
Each wrapper's docstring names the definition it follows; the C file carries
the citations of the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# the same source built with AddressSanitizer and UndefinedBehaviorSanitizer; a
# process that sets ORACLE_SANITIZED=1 (and preloads the two runtimes) loads it
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
if os.environ.get("ORACLE_SANITIZED") == "1":
    _LIB = _LIB_SAN

OR_F64, OR_F32, OR_BF16 = 0, 1, 2


def build(force: bool = True, sanitized: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, -O2, OpenMP), or with
    sanitized=True into liboracle_san.so with -fsanitize=address,undefined (every
    report fatal)."""
    lib = _LIB_SAN if sanitized else _LIB
    if force or not os.path.exists(lib):
        tmp = lib + ".tmp%d" % os.getpid()
        flags = ["-O2"]
        if sanitized:
            flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                     "-fno-sanitize-recover=all"]
        cmd = ["gcc", *flags, "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.oracle_compress.argtypes = [I, P, P, P, P, I, I, I, I]
        lib.oracle_index_scores.argtypes = [I, P, P, P, P, P, I, I, I, I, I]
        lib.oracle_topk.argtypes = [P, P, P, I, I, I]
        lib.oracle_attn_decode.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, D]
        lib.oracle_attn_prefill.argtypes = [I, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I,
                                            I, D, P, I]
        for f in (lib.oracle_compress, lib.oracle_index_scores, lib.oracle_topk,
                  lib.oracle_attn_decode, lib.oracle_attn_prefill):
            f.restype = I
        _lib = lib
    return _lib


def _elem(arr):
    """Return (element-type code, contiguous numpy array) for a float input.

    Accepts numpy float64/float32 arrays and CPU torch tensors of float64,
    float32 or bfloat16 (passed as their raw 16-bit patterns)."""
    try:
        import torch
    except ImportError:  # pragma: no cover - torch is always present here
        torch = None
    if torch is not None and isinstance(arr, torch.Tensor):
        t = arr.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return OR_BF16, t.view(torch.int16).numpy().view(np.uint16)
        arr = t.numpy()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.float64:
        return OR_F64, a
    if a.dtype == np.float32:
        return OR_F32, a
    raise TypeError("oracle inputs must be float64, float32 or bfloat16, got %s" % a.dtype)


def _same_et(*arrs):
    out = [_elem(a) for a in arrs if a is not None]
    ets = {e for e, _ in out}
    if len(ets) != 1:
        raise TypeError("oracle inputs must share one element type")
    return out[0][0], [a for _, a in out]


def _i32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError("%s rejected its arguments (code %d)" % (name, rc))


def compress(x, gate, bias, m):
    """Block compressor: out[b,i,d] = sum_j softmax_j(gate+bias)[j] * x[b,m*i+j,d].

    x, gate: [B, T, D]; bias: [m, D] -> float64 [B, T//m, D]."""
    et, (xa, ga, ba) = _same_et(x, gate, bias)
    B, T, D = xa.shape
    if ga.shape != (B, T, D) or ba.shape != (m, D):
        raise ValueError("compress: shape mismatch")
    out = np.empty((B, T // m, D), dtype=np.float64)
    _check(_load().oracle_compress(et, _p(xa), _p(ga), _p(ba), _p(out), B, T, D, m), "compress")
    return out


def compress_append(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, m):
    """Decode-time compression state: append one token per sequence.

    [NK "DeepSeek V4 的新架构", five state classes] and [KD "Arquitectura del
    Sistema", compression-state ring buffers]: an entry of the compressed pool
    exists once the whole block of m tokens behind it has arrived; until then
    the block's tokens wait in a per-sequence ring.  State of sequence b:
    ring_x[b], ring_g[b] ([m, D]) hold the latents and gate logits of the open
    block, slot = position mod m.  The token of sequence b has position
    p = pos[b] (tokens before it; the caller advances its positions).  It is
    stored in slot p mod m; if that slot is the block's last one the ring holds
    tokens p-m+1 .. p in order and compress() of it becomes pool[b, p div m]
    (unless p div m is past the pool's last row).  A sequence with pos[b] < 0
    takes no token.

    x_tok, g_tok: [B, D]; bias: [m, D]; ring_x, ring_g: [B, m, D], same element
    type as the tokens (CPU torch tensors or numpy arrays, updated in place);
    pos: int32 [B]; pool: float64 numpy [B, S_max, D] (completed rows written).
    Returns the (b, row) pairs written to pool."""
    B = x_tok.shape[0]
    if tuple(ring_x.shape) != (B, m, x_tok.shape[1]) or tuple(ring_g.shape) != tuple(ring_x.shape):
        raise ValueError("compress_append: ring shape mismatch")
    written = []
    for b in range(B):
        p = int(pos[b])
        if p < 0:
            continue
        ring_x[b, p % m] = x_tok[b]
        ring_g[b, p % m] = g_tok[b]
        if p % m == m - 1 and p // m < pool.shape[1]:
            pool[b, p // m] = compress(ring_x[b:b + 1], ring_g[b:b + 1], bias, m)[0, 0]
            written.append((b, p // m))
    return written


def index_scores(q_idx, k_idx, n_cand, q_seq=None):
    """Indexer scores: sum over heads and channels of q_idx[q,h,e]*k_idx[seq(q),s,e].

    q_idx: [Nq, H_I, d_I]; k_idx: [B, S_max, d_I]; n_cand: [Nq] -> float64
    [Nq, S_max], NaN where s >= n_cand[q]."""
    et, (qa, ka) = _same_et(q_idx, k_idx)
    Nq, H_I, d_I = qa.shape
    B, S_max, d2 = ka.shape
    if d2 != d_I:
        raise ValueError("index_scores: d_I mismatch")
    nc, qs = _i32(n_cand), _i32(q_seq)
    out = np.empty((Nq, S_max), dtype=np.float64)
    _check(_load().oracle_index_scores(et, _p(qa), _p(ka), _p(qs), _p(nc), _p(out), Nq, B, H_I,
                                       d_I, S_max), "index_scores")
    return out


def topk(scores_f32, n_cand, k):
    """First min(k, n) candidates under (score desc, index asc), indices ascending, -1 padded.

    scores_f32: [Nq, S_max] float32 (values compared exactly as fp32)."""
    s = np.ascontiguousarray(np.asarray(scores_f32, dtype=np.float32))
    if s.ndim == 1:
        s = s[None, :]
    Nq, S_max = s.shape
    nc = _i32(n_cand).reshape(-1)
    if nc.shape[0] != Nq:
        raise ValueError("topk: n_cand length mismatch")
    out = np.empty((Nq, k), dtype=np.int32)
    _check(_load().oracle_topk(_p(s), _p(nc), _p(out), Nq, S_max, k), "topk")
    return out


def attn_decode(q, swa_kv, swa_len, comp_kv, comp_len, scale, d_v, comp_idx=None):
    """Decode attention: one softmax over SWA slots plus sparse (comp_idx) or dense rows.

    q: [B, H, d_qk]; swa_kv: [B, W, d_qk]; comp_kv: [B, S_max, d_qk];
    comp_idx: [B, k] or None -> (out float64 [B, H, d_v], lse float64 [B, H])."""
    et, (qa, sa, ca) = _same_et(q, swa_kv, comp_kv)
    B, H, d_qk = qa.shape
    W = sa.shape[1]
    S_max = ca.shape[1]
    ci = _i32(comp_idx)
    k = 0 if ci is None else ci.shape[1]
    sl, cl = _i32(swa_len), _i32(comp_len)
    out = np.empty((B, H, d_v), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    _check(_load().oracle_attn_decode(et, _p(qa), _p(sa), _p(sl), _p(ca), _p(ci), _p(cl),
                                      _p(out), _p(lse), B, H, d_qk, d_v, W, S_max, k,
                                      float(scale)), "attn_decode")
    return out, lse


def attn_prefill(q, kv, comp_kv, q_start, W, m, scale, d_v, comp_idx=None, sel=None):
    """Prefill attention for queries at positions q_start.. of each sequence.

    q: [n_seq, n_q, H, d_qk]; kv: [n_seq, T, d_qk]; comp_kv: [n_seq, S_max, d_qk];
    comp_idx: [n_seq*n_q, k] or None; sel: flat query ids (default: all)
    -> (out float64 [n_sel, H, d_v], lse float64 [n_sel, H])."""
    et, (qa, ka, ca) = _same_et(q, kv, comp_kv)
    n_seq, n_q, H, d_qk = qa.shape
    T = ka.shape[1]
    S_max = ca.shape[1]
    ci = _i32(comp_idx)
    k = 0 if ci is None else ci.shape[1]
    sl = _i32(np.arange(n_seq * n_q) if sel is None else sel).reshape(-1)
    out = np.empty((sl.shape[0], H, d_v), dtype=np.float64)
    lse = np.empty((sl.shape[0], H), dtype=np.float64)
    _check(_load().oracle_attn_prefill(et, _p(qa), _p(ka), _p(ca), _p(ci), _p(out), _p(lse),
                                       n_seq, n_q, q_start, T, H, d_qk, d_v, W, S_max, k, m,
                                       float(scale), _p(sl), sl.shape[0]), "attn_prefill")
    return out, lse
