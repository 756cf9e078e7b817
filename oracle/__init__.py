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
        lib.oracle_compress_overlap.argtypes = [I, P, P, P, P, I, I, I, I]
        lib.oracle_index_scores.argtypes = [I, P, P, P, P, P, I, I, I, I, I]
        lib.oracle_index_scores_weighted.argtypes = [I, P, P, P, P, P, P, I, I, I, I, I]
        lib.oracle_topk.argtypes = [P, P, P, I, I, I]
        lib.oracle_attn_decode.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, D]
        lib.oracle_attn_prefill.argtypes = [I, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I,
                                            I, D, P, I]
        for f in (lib.oracle_compress, lib.oracle_compress_overlap, lib.oracle_index_scores,
                  lib.oracle_index_scores_weighted,
                  lib.oracle_topk,
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


def compress_overlap(x, gate, bias, m):
    """Overlapping-block compressor (method variant): entry i over tokens
    m(i-1) .. m(i+1)-1 that exist, bias [2m, D] (row j for token m(i-1)+j).

    x, gate: [B, T, D]; bias: [2m, D] -> float64 [B, T//m, D]."""
    et, (xa, ga, ba) = _same_et(x, gate, bias)
    B, T, D = xa.shape
    if ga.shape != (B, T, D) or ba.shape != (2 * m, D):
        raise ValueError("compress_overlap: shape mismatch")
    out = np.empty((B, T // m, D), dtype=np.float64)
    _check(_load().oracle_compress_overlap(et, _p(xa), _p(ga), _p(ba), _p(out), B, T, D, m),
           "compress_overlap")
    return out


def compress_append_overlap(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, m):
    """Decode-time state of the overlapping compressor: the ring keeps the last
    2m tokens (slot = position mod 2m).  The token of sequence b at p = pos[b]
    >= 0 is stored in slot p mod 2m; if it completes block i = p div m (and
    i < S_max) the entry is compress_overlap of tokens m(i-1) .. p, read from
    the ring (tokens before 0 do not exist).
    ring_x, ring_g: [B, 2m, D] (updated in place); pool: float64 [B, S_max, D].
    Returns the (b, row) pairs written."""
    B = x_tok.shape[0]
    if tuple(ring_x.shape) != (B, 2 * m, x_tok.shape[1]) or tuple(ring_g.shape) != tuple(ring_x.shape):
        raise ValueError("compress_append_overlap: ring shape mismatch")
    written = []
    for b in range(B):
        p = int(pos[b])
        if p < 0:
            continue
        ring_x[b, p % (2 * m)] = x_tok[b]
        ring_g[b, p % (2 * m)] = g_tok[b]
        i = p // m
        if p % m != m - 1 or i >= pool.shape[1]:
            continue
        t0 = max(0, m * (i - 1))
        toks = list(range(t0, p + 1))
        slots = [t % (2 * m) for t in toks]
        seq_x = ring_x[b][slots][None]
        seq_g = ring_g[b][slots][None]
        if i == 0:  # one block: the whole window is entry 0 of a length-m sequence
            pool[b, i] = compress_overlap(seq_x, seq_g, bias, m)[0, 0]
        else:       # two blocks: entry 1 of a length-2m sequence is the window
            pool[b, i] = compress_overlap(seq_x, seq_g, bias, m)[0, 1]
        written.append((b, i))
    return written


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


def index_scores_weighted(q_idx, w, k_idx, n_cand, q_seq=None):
    """Weighted, activated indexer heads (method variant):
    sum_h w[q,h] * max(0, q_idx[q,h,:] . k_idx[seq(q),s,:]).

    q_idx: [Nq, H_I, d_I]; w: [Nq, H_I] (taken as fp32); k_idx: [B, S_max, d_I];
    n_cand: [Nq] -> float64 [Nq, S_max], NaN where s >= n_cand[q]."""
    et, (qa, ka) = _same_et(q_idx, k_idx)
    Nq, H_I, d_I = qa.shape
    B, S_max, d2 = ka.shape
    wa = np.ascontiguousarray(np.asarray(w.float() if hasattr(w, "float") else w, dtype=np.float32))
    if d2 != d_I or wa.shape != (Nq, H_I):
        raise ValueError("index_scores_weighted: shape mismatch")
    nc, qs = _i32(n_cand), _i32(q_seq)
    out = np.empty((Nq, S_max), dtype=np.float64)
    _check(_load().oracle_index_scores_weighted(et, _p(qa), _p(wa), _p(ka), _p(qs), _p(nc),
                                                _p(out), Nq, B, H_I, d_I, S_max),
           "index_scores_weighted")
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


# ---- paged pools --------------------------------------------------------------
# [KD "Arquitectura del Sistema", ShadowRadix paragraph] and [NK "推理侧优化",
# shadow radix cache bullet]: every pool is addressed through its own index
# map ("shadow") from a sequence's virtual rows to physical storage, so pools
# live and die independently (SWA pages go once the window has passed them).
# Reading (the pages give no layout): a pool is [pool_pages, P, D]; row r of
# sequence b is pool[page_map[b, r // P], r % P]; a page past the map or a map
# entry outside [0, pool_pages) is not resident.  SWA rows are indexed by
# token position, C4 KV and indexer-key rows by entry; the compression state
# of token t sits at t's SWA row in two state pools shaped like the SWA pool.
# These functions only resolve the maps and then call the definitions above.

def paged_rows(pool, page_map_b, n_rows, page_rows, fill=np.nan):
    """Rows 0 .. n_rows-1 of one sequence of a paged pool.

    pool: [pool_pages, P, D] (torch CPU or numpy); page_map_b: the sequence's
    map entries.  Returns (rows float64 [n_rows, D], resident bool [n_rows]);
    rows that are not resident hold `fill`."""
    pa = np.asarray(pool.float() if hasattr(pool, "float") else pool, dtype=np.float64)
    pm = np.asarray(page_map_b, dtype=np.int64).reshape(-1)
    r = np.arange(n_rows)
    j = r // page_rows
    page = np.where(j < pm.shape[0], pm[np.minimum(j, max(pm.shape[0] - 1, 0))], -1)
    resident = (page >= 0) & (page < pa.shape[0])
    rows = np.full((n_rows, pa.shape[2]), fill, dtype=np.float64)
    rows[resident] = pa[page[resident], (r % page_rows)[resident]]
    return rows, resident


def physical_row(page_map_b, r, page_rows, pool_pages):
    """(page, offset) of row r of one sequence, or None when it is not resident."""
    pm = np.asarray(page_map_b).reshape(-1)
    j = r // page_rows
    if r < 0 or j >= pm.shape[0] or not (0 <= int(pm[j]) < pool_pages):
        return None
    return int(pm[j]), r % page_rows


def compress_append_paged(x_tok, g_tok, bias, state_x, state_g, pos, swa_map, c4_map,
                          swa_page_rows, c4_page_rows, c4_pool_pages, S_max, m=4):
    """Decode-time compression state on paged pools (m = 4).

    The token of sequence b at p = pos[b] >= 0 is stored at its SWA row of the
    state pools (state_x, state_g: [swa_pool_pages, P, D], updated in place);
    when p mod m == m-1 and i = p div m < S_max, the entry of tokens p-m+1 .. p
    (compress() of their state rows) is due at C4 row i.  A token whose SWA
    row is not resident is not stored; an entry whose C4 row (or a state row of
    its block) is not resident is not formed.
    Returns [(b, i, (page, offset), entry float64 [D])] for the entries formed."""
    written = []
    n_pages = state_x.shape[0]
    for b in range(x_tok.shape[0]):
        p = int(pos[b])
        if p < 0:
            continue
        at = physical_row(swa_map[b], p, swa_page_rows, n_pages)
        if at is None:
            continue
        state_x[at[0], at[1]] = x_tok[b]
        state_g[at[0], at[1]] = g_tok[b]
        i = p // m
        if p % m != m - 1 or i >= S_max:
            continue
        dest = physical_row(c4_map[b], i, c4_page_rows, c4_pool_pages)
        rows = [physical_row(swa_map[b], t, swa_page_rows, n_pages) for t in range(p - m + 1, p + 1)]
        if dest is None or any(a is None for a in rows):
            continue
        rx = state_x[[a[0] for a in rows], [a[1] for a in rows]][None, None]
        rg = state_g[[a[0] for a in rows], [a[1] for a in rows]][None, None]
        # one block of m tokens: [1, m, D]
        entry = compress(rx.reshape(1, m, -1), rg.reshape(1, m, -1), bias, m)[0, 0]
        written.append((b, i, dest, entry))
    return written


def index_scores_paged(q_idx, kI_pool, kI_map, c4_page_rows, n_cand, S_max):
    """index_scores over indexer-key rows reached through the kI shadow; a row
    that is not resident is all-NaN, so its score is NaN."""
    B = q_idx.shape[0]
    keys = np.stack([paged_rows(kI_pool, kI_map[b], S_max, c4_page_rows)[0] for b in range(B)])
    return index_scores(q_idx.double() if hasattr(q_idx, "double") else np.asarray(q_idx, np.float64),
                        keys, n_cand)


def attn_decode_paged(q, swa_pool, swa_map, swa_page_rows, swa_len, pos, W, c4_pool, c4_map,
                      c4_page_rows, comp_len, comp_idx, S_max, scale, d_v):
    """attn_decode (sparse) with the window = the n = clamp(swa_len[b], 0, W)
    tokens pos[b]-n+1 .. pos[b] (none when pos[b] < 0) and the listed C4 rows
    (i < comp_len[b]), each read through its shadow; rows that are not resident
    are left out."""
    qa = np.asarray(q.double() if hasattr(q, "double") else q, dtype=np.float64)
    B, H, d_qk = qa.shape
    sp = np.asarray(swa_pool.float() if hasattr(swa_pool, "float") else swa_pool, dtype=np.float64)
    win = np.zeros((B, W, d_qk))
    n_win = np.zeros(B, dtype=np.int32)
    comp = np.zeros((B, S_max, d_qk))
    ci = np.array(comp_idx, dtype=np.int32, copy=True)
    for b in range(B):
        p = int(pos[b])
        n = min(max(int(swa_len[b]), 0), W) if p >= 0 else 0
        kept = []
        for t in range(p - n + 1, p + 1):
            at = physical_row(swa_map[b], t, swa_page_rows, sp.shape[0])
            if at is not None:
                kept.append(sp[at[0], at[1]])
        for j, row in enumerate(kept):
            win[b, j] = row
        n_win[b] = len(kept)
        crow, cres = paged_rows(c4_pool, c4_map[b], S_max, c4_page_rows, fill=0.0)
        comp[b] = crow
        for j in range(ci.shape[1]):
            if 0 <= ci[b, j] < S_max and not cres[ci[b, j]]:
                ci[b, j] = -1
    return attn_decode(qa, win, n_win, comp, np.asarray(comp_len, dtype=np.int32), scale, d_v,
                       comp_idx=ci)
