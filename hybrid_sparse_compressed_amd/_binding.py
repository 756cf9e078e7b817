"""ctypes binding of libhsa_attn.so.

Argument marshalling only: these functions check tensor placement, dtype and
contiguity, allocate outputs / workspaces with torch when the caller passes
none, and call the C entry point of the same name on the current HIP stream.
Every step of the computation runs in the library's kernels.  If the shared
library is missing the import fails loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhsa_attn.so")

HSA_OK, HSA_ERR_INVALID_ARG, HSA_ERR_UNSUPPORTED, HSA_ERR_WORKSPACE, HSA_ERR_HIP = range(5)
HSA_F32, HSA_BF16 = 0, 1

EXPORTED = (
    "hsa_strerror", "hsa_version", "hsa_compress", "hsa_compress_append",
    "hsa_index_topk_workspace_size",
    "hsa_index_topk", "hsa_attn_decode_workspace_size", "hsa_attn_decode",
    "hsa_attn_prefill_workspace_size", "hsa_attn_prefill", "hsa_decode_sparse_workspace_size",
    "hsa_decode_sparse", "hsa_decode_step", "hsa_decode_step_noalloc", "hsa_decode_step_paged",
    "hsa_index_topk_weighted", "hsa_decode_sparse_weighted", "hsa_compress_overlap",
    "hsa_compress_append_overlap", "hsa_profile_enable", "hsa_profile_read", "hsa_stream_read",
)
HSA_PROF_COMPRESS, HSA_PROF_SCORE, HSA_PROF_SELECT, HSA_PROF_ATTN, HSA_PROF_MERGE = 1, 2, 4, 8, 16
HSA_PROF_STREAM = 32


class PageMaps(ctypes.Structure):
    """hsa_page_maps: the shadows of one paged decode call (device map pointers)."""
    _fields_ = [("swa_map", ctypes.c_void_p), ("swa_map_pages", ctypes.c_int32),
                ("swa_page_rows", ctypes.c_int32), ("swa_pool_pages", ctypes.c_int32),
                ("c4_map", ctypes.c_void_p), ("kI_map", ctypes.c_void_p),
                ("c4_map_pages", ctypes.c_int32), ("c4_page_rows", ctypes.c_int32),
                ("c4_pool_pages", ctypes.c_int32), ("kI_pool_pages", ctypes.c_int32)]


class HsaError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__("%s failed: %s (%d)" % (fn, strerror(code), code))
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libhsa_attn.so is not built (expected at %s); run "
            "`python -m hybrid_sparse_compressed_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, U32, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t,
                          ctypes.c_float)
    I = ctypes.c_int
    lib.hsa_strerror.argtypes = [I]
    lib.hsa_strerror.restype = ctypes.c_char_p
    lib.hsa_version.argtypes = []
    lib.hsa_version.restype = I
    lib.hsa_compress.argtypes = [I, P, P, P, P, I32, I32, I32, I32, P]
    lib.hsa_compress.restype = I
    lib.hsa_compress_append.argtypes = [I, P, P, P, P, P, P, P, I32, I32, I32, I32, P]
    lib.hsa_compress_append.restype = I
    lib.hsa_index_topk_workspace_size.argtypes = [I32, I32, I32]
    lib.hsa_index_topk_workspace_size.restype = SZ
    lib.hsa_index_topk.argtypes = [I, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, U32, P, SZ, P]
    lib.hsa_index_topk.restype = I
    lib.hsa_attn_decode_workspace_size.argtypes = [I32, I32, I32, I32]
    lib.hsa_attn_decode_workspace_size.restype = SZ
    lib.hsa_attn_decode.argtypes = [I, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                    F, P, SZ, P]
    lib.hsa_attn_decode.restype = I
    lib.hsa_decode_sparse_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.hsa_decode_sparse_workspace_size.restype = SZ
    lib.hsa_decode_sparse.argtypes = [I, P, P, P, P, P, P, P, P, P, P, P, P] + [I32] * 9 + [F, P, SZ, P]
    lib.hsa_decode_sparse.restype = I
    lib.hsa_decode_step.argtypes = [I] + [P] * 18 + [I32] * 9 + [F, P, SZ, P]
    lib.hsa_decode_step.restype = I
    lib.hsa_decode_step_noalloc.argtypes = [I] + [P] * 18 + [I32] * 9 + [F, P]
    lib.hsa_decode_step_noalloc.restype = I
    lib.hsa_decode_step_paged.argtypes = [I] + [P] * 16 + [ctypes.POINTER(PageMaps), P, P] + \
        [I32] * 9 + [F, P, SZ, P]
    lib.hsa_decode_step_paged.restype = I
    lib.hsa_compress_overlap.argtypes = [I, P, P, P, P, I32, I32, I32, I32, P]
    lib.hsa_compress_overlap.restype = I
    lib.hsa_compress_append_overlap.argtypes = [I, P, P, P, P, P, P, P, I32, I32, I32, I32, P]
    lib.hsa_compress_append_overlap.restype = I
    lib.hsa_index_topk_weighted.argtypes = [I, P, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, P,
                                            SZ, P]
    lib.hsa_index_topk_weighted.restype = I
    lib.hsa_decode_sparse_weighted.argtypes = [I] + [P] * 13 + [I32] * 9 + [F, P, SZ, P]
    lib.hsa_decode_sparse_weighted.restype = I
    lib.hsa_attn_prefill_workspace_size.argtypes = [I32, I32, I32, I32]
    lib.hsa_attn_prefill_workspace_size.restype = SZ
    lib.hsa_attn_prefill.argtypes = [I, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32,
                                     I32, I32, I32, F, P, SZ, P]
    lib.hsa_attn_prefill.restype = I
    lib.hsa_profile_enable.argtypes = [ctypes.c_uint]
    lib.hsa_profile_enable.restype = I
    lib.hsa_profile_read.argtypes = [ctypes.c_uint, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_longlong), I]
    lib.hsa_profile_read.restype = I
    lib.hsa_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
    lib.hsa_stream_read.restype = I
    return lib


lib = _load()


def strerror(code: int) -> str:
    return lib.hsa_strerror(int(code)).decode()


def _check(fn, code):
    if code != HSA_OK:
        raise HsaError(fn, code)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return HSA_F32
    if t.dtype == torch.bfloat16:
        return HSA_BF16
    raise TypeError("expected float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libhsa_attn must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libhsa_attn must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _i32(t, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        t = torch.as_tensor(t, dtype=torch.int32)
    if t.dtype != torch.int32:
        raise TypeError("index/length tensors must be int32")
    return t.to(device).contiguous()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Workspace:
    """Device buffers reused across calls, one per (purpose, device, stream).

    The top-k workspace must be zero-filled before its first use and every
    completed call leaves it zero-filled again, so it is never shared with a
    purpose that leaves data behind (the decode split partials)."""

    _cache: dict = {}

    @classmethod
    def get(cls, purpose: str, nbytes: int, device, stream) -> torch.Tensor | None:
        if nbytes == 0:
            return None
        key = (purpose, str(device), stream.cuda_stream if stream is not None else 0)
        buf = cls._cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
            cls._cache[key] = buf
        return buf

    @classmethod
    def discard(cls, buf) -> None:
        """Forget a cached buffer (after a failed call its contents are unknown, and
        a zero-filled one is made on the next request)."""
        for key, v in list(cls._cache.items()):
            if v is buf:
                del cls._cache[key]


def _call_with_workspace(name, rc_fn, workspace, cached):
    """Run one C call; if it fails and the workspace came from the cache, drop it."""
    code = rc_fn()
    if code != HSA_OK and cached:
        Workspace.discard(workspace)
    _check(name, code)


def hsa_compress(x, gate, bias, m, out=None, stream=None):
    """out[b,i,:] = sum_j softmax_j(gate[b,m*i+j,:] + bias[j,:]) * x[b,m*i+j,:]."""
    B, T, D = x.shape
    if out is None:
        out = torch.empty((B, T // m, D), dtype=x.dtype, device=x.device)
    for t in (gate, bias, out):
        if t.dtype != x.dtype:
            raise TypeError("hsa_compress: all tensors must share one dtype")
    if gate.shape != x.shape or tuple(bias.shape) != (m, D) or tuple(out.shape) != (B, T // m, D):
        raise ValueError("hsa_compress: shape mismatch")
    _check("hsa_compress", lib.hsa_compress(_dt(x), _ptr(x), _ptr(gate), _ptr(bias), _ptr(out),
                                            B, T, D, m, _stream(stream)))
    return out


def hsa_compress_append(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, stream=None):
    """Store each sequence's token into ring slot pos mod m; a token that
    completes its block writes that block's entry to pool[b, pos // m].

    x_tok, g_tok: [B, D]; bias: [m, D]; ring_x, ring_g: [B, m, D] (updated in
    place); pos: [B] int32 (read only, < 0 = idle); pool: [B, S_max, D]."""
    B, D = x_tok.shape
    m = bias.shape[0]
    S_max = pool.shape[1]
    for t in (g_tok, bias, ring_x, ring_g, pool):
        if t.dtype != x_tok.dtype:
            raise TypeError("hsa_compress_append: all float tensors must share one dtype")
    if (tuple(g_tok.shape) != (B, D) or tuple(bias.shape) != (m, D)
            or tuple(ring_x.shape) != (B, m, D) or tuple(ring_g.shape) != (B, m, D)
            or tuple(pool.shape) != (B, S_max, D) or tuple(pos.shape) != (B,)):
        raise ValueError("hsa_compress_append: shape mismatch")
    if pos.dtype != torch.int32:
        raise TypeError("hsa_compress_append: pos must be int32")
    _check("hsa_compress_append",
           lib.hsa_compress_append(_dt(x_tok), _ptr(x_tok), _ptr(g_tok), _ptr(bias), _ptr(ring_x),
                                   _ptr(ring_g), _ptr(pos), _ptr(pool), B, D, m, S_max,
                                   _stream(stream)))
    return pool


def hsa_compress_overlap(x, gate, bias, m, out=None, stream=None):
    """Overlapping blocks: out[b,i,:] = sum_j softmax_j(gate[b,t_j,:] + bias[j,:]) * x[b,t_j,:]
    over the tokens t_j = m*(i-1)+j >= 0, j < 2m; bias: [2m, D]."""
    B, T, D = x.shape
    if out is None:
        out = torch.empty((B, T // m, D), dtype=x.dtype, device=x.device)
    for t in (gate, bias, out):
        if t.dtype != x.dtype:
            raise TypeError("hsa_compress_overlap: all tensors must share one dtype")
    if gate.shape != x.shape or tuple(bias.shape) != (2 * m, D) or tuple(out.shape) != (B, T // m, D):
        raise ValueError("hsa_compress_overlap: shape mismatch")
    _check("hsa_compress_overlap", lib.hsa_compress_overlap(
        _dt(x), _ptr(x), _ptr(gate), _ptr(bias), _ptr(out), B, T, D, m, _stream(stream)))
    return out


def hsa_compress_append_overlap(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, stream=None):
    """Decode-time state of the overlapping compressor: ring of the last 2m tokens
    (slot pos mod 2m); the token completing block i writes entry i (blocks i-1, i).

    x_tok, g_tok: [B, D]; bias: [2m, D]; ring_x, ring_g: [B, 2m, D]; pos: [B] int32;
    pool: [B, S_max, D]."""
    B, D = x_tok.shape
    m = bias.shape[0] // 2
    S_max = pool.shape[1]
    for t in (g_tok, bias, ring_x, ring_g, pool):
        if t.dtype != x_tok.dtype:
            raise TypeError("hsa_compress_append_overlap: all float tensors must share one dtype")
    if (bias.shape[0] != 2 * m or tuple(g_tok.shape) != (B, D) or tuple(bias.shape) != (2 * m, D)
            or tuple(ring_x.shape) != (B, 2 * m, D) or tuple(ring_g.shape) != (B, 2 * m, D)
            or tuple(pool.shape) != (B, S_max, D) or tuple(pos.shape) != (B,)):
        raise ValueError("hsa_compress_append_overlap: shape mismatch")
    if pos.dtype != torch.int32:
        raise TypeError("hsa_compress_append_overlap: pos must be int32")
    _check("hsa_compress_append_overlap", lib.hsa_compress_append_overlap(
        _dt(x_tok), _ptr(x_tok), _ptr(g_tok), _ptr(bias), _ptr(ring_x), _ptr(ring_g), _ptr(pos),
        _ptr(pool), B, D, m, S_max, _stream(stream)))
    return pool


def hsa_index_topk(q_idx, k_idx, n_cand, k, q_seq=None, scores=None, topk_idx=None,
                   workspace=None, stream=None, S_max=None):
    """Indexer scores + top-k.  q_idx=None selects from the given `scores`.

    q_idx: [Nq, H_I, d_I]; k_idx: [B, S_max, d_I]; n_cand: [Nq] int32.
    Returns (scores [Nq, S_max] fp32, topk_idx [Nq, k] int32)."""
    return _index_topk(q_idx, None, k_idx, n_cand, k, q_seq, scores, topk_idx, workspace, stream)


def hsa_index_topk_weighted(q_idx, head_w, k_idx, n_cand, k, q_seq=None, scores=None,
                            topk_idx=None, workspace=None, stream=None):
    """hsa_index_topk with weighted, activated heads: head_w [Nq, H_I] fp32 (device),
    score = sum_h head_w[q, h] * max(0, q_idx[q, h] . k).  bf16, d_I = 128."""
    if head_w is None or head_w.dtype != torch.float32 or tuple(head_w.shape) != tuple(q_idx.shape[:2]):
        raise ValueError("hsa_index_topk_weighted: head_w must be fp32 [Nq, H_I]")
    return _index_topk(q_idx, head_w, k_idx, n_cand, k, q_seq, scores, topk_idx, workspace, stream)


def _index_topk(q_idx, head_w, k_idx, n_cand, k, q_seq, scores, topk_idx, workspace, stream):
    if q_idx is not None:
        Nq, H_I, d_I = q_idx.shape
        B, S_max, d2 = k_idx.shape
        if d2 != d_I or k_idx.dtype != q_idx.dtype:
            raise ValueError("hsa_index_topk: q_idx / k_idx mismatch")
        dev = q_idx.device
        dt = _dt(q_idx)
    else:
        if scores is None:
            raise ValueError("hsa_index_topk: select-only mode needs scores")
        Nq, S_max = scores.shape
        B, H_I, d_I, dev, dt = 1, 1, 1, scores.device, HSA_F32
    n_cand = _i32(n_cand, dev)
    q_seq = _i32(q_seq, dev)
    if scores is None:
        scores = torch.empty((Nq, S_max), dtype=torch.float32, device=dev)
    if scores.dtype != torch.float32 or tuple(scores.shape) != (Nq, S_max):
        raise ValueError("hsa_index_topk: scores must be fp32 [Nq, S_max]")
    if topk_idx is None:
        topk_idx = torch.empty((Nq, k), dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream() if stream is None else stream
    need = lib.hsa_index_topk_workspace_size(Nq, S_max, k)
    cached = workspace is None
    if cached:
        workspace = Workspace.get("topk", need, dev, st)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if head_w is None:
        _call_with_workspace("hsa_index_topk", lambda: lib.hsa_index_topk(
            dt, _ptr(q_idx), _ptr(k_idx), B, _ptr(q_seq), _ptr(n_cand), _ptr(scores),
            _ptr(topk_idx), Nq, H_I, d_I, S_max, k, 0, _ptr(workspace), wsz, _stream(st)),
            workspace, cached)
    else:
        _call_with_workspace("hsa_index_topk_weighted", lambda: lib.hsa_index_topk_weighted(
            dt, _ptr(q_idx), _ptr(head_w), _ptr(k_idx), B, _ptr(q_seq), _ptr(n_cand),
            _ptr(scores), _ptr(topk_idx), Nq, H_I, d_I, S_max, k, _ptr(workspace), wsz,
            _stream(st)), workspace, cached)
    return scores, topk_idx


def hsa_attn_decode(q, swa_kv, swa_len, comp_kv, comp_len, scale, d_v, comp_idx=None, out=None,
                    lse=None, workspace=None, stream=None):
    """One softmax over the SWA ring plus sparse (comp_idx) or dense compressed rows.

    q: [B, H, d_qk]; swa_kv: [B, W, d_qk]; comp_kv: [B, S_max, d_qk]; comp_idx: [B, k]
    int32 or None.  Returns (out [B, H, d_v], lse [B, H] fp32)."""
    B, H, d_qk = q.shape
    W = swa_kv.shape[1]
    S_max = comp_kv.shape[1]
    dev = q.device
    swa_len, comp_len, comp_idx = _i32(swa_len, dev), _i32(comp_len, dev), _i32(comp_idx, dev)
    k = 0 if comp_idx is None else comp_idx.shape[1]
    if out is None:
        out = torch.empty((B, H, d_v), dtype=q.dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream() if stream is None else stream
    need = lib.hsa_attn_decode_workspace_size(B, H, d_v, W + (k if comp_idx is not None else S_max))
    if workspace is None:
        workspace = Workspace.get("attn_decode", need, dev, st)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("hsa_attn_decode", lib.hsa_attn_decode(
        _dt(q), _ptr(q), _ptr(swa_kv), _ptr(swa_len), _ptr(comp_kv), _ptr(comp_idx),
        _ptr(comp_len), _ptr(out), _ptr(lse), B, H, d_qk, d_v, W, S_max, k, float(scale),
        _ptr(workspace), wsz, _stream(st)))
    return out, lse


def hsa_decode_sparse(q_idx, k_idx, n_cand, k, q, swa_kv, swa_len, comp_kv, comp_len, scale, d_v,
                      scores=None, topk_idx=None, out=None, lse=None, workspace=None, stream=None):
    """The C4 decode layer-step in one call (query b reads sequence b): indexer
    scores, exact top-k, and the SWA + selected-row attention.

    q_idx: [B, H_I, d_I]; k_idx: [B, S_max, d_I]; q: [B, H, d_qk]; swa_kv: [B, W, d_qk];
    comp_kv: [B, S_max, d_qk].  Returns (scores, topk_idx, out, lse)."""
    return _decode_sparse(q_idx, None, k_idx, n_cand, k, q, swa_kv, swa_len, comp_kv, comp_len,
                          scale, d_v, scores, topk_idx, out, lse, workspace, stream)


def hsa_decode_sparse_weighted(q_idx, head_w, k_idx, n_cand, k, q, swa_kv, swa_len, comp_kv,
                               comp_len, scale, d_v, scores=None, topk_idx=None, out=None,
                               lse=None, workspace=None, stream=None):
    """hsa_decode_sparse with the weighted, activated indexer heads of
    hsa_index_topk_weighted (head_w [B, H_I] fp32)."""
    if head_w is None or head_w.dtype != torch.float32 or tuple(head_w.shape) != tuple(q_idx.shape[:2]):
        raise ValueError("hsa_decode_sparse_weighted: head_w must be fp32 [B, H_I]")
    return _decode_sparse(q_idx, head_w, k_idx, n_cand, k, q, swa_kv, swa_len, comp_kv, comp_len,
                          scale, d_v, scores, topk_idx, out, lse, workspace, stream)


def _decode_sparse(q_idx, head_w, k_idx, n_cand, k, q, swa_kv, swa_len, comp_kv, comp_len, scale,
                   d_v, scores, topk_idx, out, lse, workspace, stream):
    B, H_I, d_I = q_idx.shape
    _, S_max, _ = k_idx.shape
    _, H, d_qk = q.shape
    W = swa_kv.shape[1]
    if comp_kv.shape[1] != S_max or k_idx.dtype != q_idx.dtype or q.dtype != q_idx.dtype:
        raise ValueError("hsa_decode_sparse: shape or dtype mismatch")
    dev = q.device
    n_cand, swa_len, comp_len = _i32(n_cand, dev), _i32(swa_len, dev), _i32(comp_len, dev)
    if scores is None:
        scores = torch.empty((B, S_max), dtype=torch.float32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, H, d_v), dtype=q.dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream() if stream is None else stream
    need = lib.hsa_decode_sparse_workspace_size(B, H, d_v, W, S_max, k)
    cached = workspace is None
    if cached:
        # the select part sits at the front and must be zero-filled, so a
        # cached buffer serves one layout only
        workspace = Workspace.get("decode_sparse:%d:%d:%d:%d:%d" % (B, H, d_v, W, S_max * 4096 + k),
                                  need, dev, st)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if head_w is None:
        _call_with_workspace("hsa_decode_sparse", lambda: lib.hsa_decode_sparse(
            _dt(q), _ptr(q_idx), _ptr(k_idx), _ptr(n_cand), _ptr(scores), _ptr(topk_idx), _ptr(q),
            _ptr(swa_kv), _ptr(swa_len), _ptr(comp_kv), _ptr(comp_len), _ptr(out), _ptr(lse), B,
            H_I, d_I, H, d_qk, d_v, W, S_max, k, float(scale), _ptr(workspace), wsz, _stream(st)),
            workspace, cached)
    else:
        _call_with_workspace("hsa_decode_sparse_weighted", lambda: lib.hsa_decode_sparse_weighted(
            _dt(q), _ptr(q_idx), _ptr(head_w), _ptr(k_idx), _ptr(n_cand), _ptr(scores),
            _ptr(topk_idx), _ptr(q), _ptr(swa_kv), _ptr(swa_len), _ptr(comp_kv), _ptr(comp_len),
            _ptr(out), _ptr(lse), B, H_I, d_I, H, d_qk, d_v, W, S_max, k, float(scale),
            _ptr(workspace), wsz, _stream(st)), workspace, cached)
    return scores, topk_idx, out, lse


def hsa_decode_step(x_tok, g_tok, bias, ring_x, ring_g, pos, q_idx, k_idx, n_cand, k, q, swa_kv,
                    swa_len, comp_kv, comp_len, scale, d_v, scores=None, topk_idx=None, out=None,
                    lse=None, workspace=None, stream=None):
    """hsa_compress_append (C4: m = 4, into comp_kv) followed by hsa_decode_sparse, in
    one call.  x_tok, g_tok: [B, d_qk]; bias: [4, d_qk]; ring_x, ring_g: [B, 4, d_qk]
    (updated); pos: [B] int32 (read only); comp_kv: [B, S_max, d_qk] (completed rows
    written); other arguments as hsa_decode_sparse.  Returns (scores, topk_idx, out, lse)."""
    B, H_I, d_I = q_idx.shape
    _, S_max, _ = k_idx.shape
    _, H, d_qk = q.shape
    W = swa_kv.shape[1]
    if comp_kv.shape[1] != S_max or k_idx.dtype != q_idx.dtype or q.dtype != q_idx.dtype:
        raise ValueError("hsa_decode_step: shape or dtype mismatch")
    for t in (x_tok, g_tok, bias, ring_x, ring_g, comp_kv):
        if t.dtype != q.dtype:
            raise TypeError("hsa_decode_step: append tensors must have the query dtype")
    if (tuple(x_tok.shape) != (B, d_qk) or tuple(g_tok.shape) != (B, d_qk)
            or tuple(bias.shape) != (4, d_qk) or tuple(ring_x.shape) != (B, 4, d_qk)
            or tuple(ring_g.shape) != (B, 4, d_qk) or tuple(pos.shape) != (B,)):
        raise ValueError("hsa_decode_step: append shape mismatch")
    if pos.dtype != torch.int32:
        raise TypeError("hsa_decode_step: pos must be int32")
    dev = q.device
    n_cand, swa_len, comp_len = _i32(n_cand, dev), _i32(swa_len, dev), _i32(comp_len, dev)
    if scores is None:
        scores = torch.empty((B, S_max), dtype=torch.float32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, H, d_v), dtype=q.dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream() if stream is None else stream
    need = lib.hsa_decode_sparse_workspace_size(B, H, d_v, W, S_max, k)
    cached = workspace is None
    if cached:
        workspace = Workspace.get("decode_sparse:%d:%d:%d:%d:%d" % (B, H, d_v, W, S_max * 4096 + k),
                                  need, dev, st)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call_with_workspace("hsa_decode_step", lambda: lib.hsa_decode_step(
        _dt(q), _ptr(x_tok), _ptr(g_tok), _ptr(bias), _ptr(ring_x), _ptr(ring_g), _ptr(pos),
        _ptr(q_idx), _ptr(k_idx), _ptr(n_cand), _ptr(scores), _ptr(topk_idx), _ptr(q),
        _ptr(swa_kv), _ptr(swa_len), _ptr(comp_kv), _ptr(comp_len), _ptr(out), _ptr(lse), B, H_I,
        d_I, H, d_qk, d_v, W, S_max, k, float(scale), _ptr(workspace), wsz, _stream(st)),
        workspace, cached)
    return scores, topk_idx, out, lse


def hsa_decode_step_paged(x_tok, g_tok, bias, state_x, state_g, pos, q_idx, kI_pool, kI_map,
                          n_cand, k, q, swa_pool, swa_map, swa_len, c4_pool, c4_map, comp_len,
                          scale, d_v, W, S_max, scores=None, topk_idx=None, out=None, lse=None,
                          workspace=None, stream=None):
    """hsa_decode_step on paged pools (x_tok None: no append, as hsa_decode_sparse).

    Pools: swa_pool, state_x, state_g [swa_pool_pages, P_swa, d_qk]; c4_pool
    [c4_pool_pages, P_c4, d_qk]; kI_pool [kI_pool_pages, P_c4, d_I].  Shadows
    (int32 device tensors): swa_map [B, swa_map_pages], c4_map and kI_map
    [B, c4_map_pages].  pos: [B] int32, the query token positions.  Window: the
    swa_len[b] (<= W) tokens ending at pos[b].  Returns (scores, topk_idx, out, lse)."""
    B, H_I, d_I = q_idx.shape
    _, H, d_qk = q.shape
    if kI_pool.dtype != q_idx.dtype or q.dtype != q_idx.dtype or swa_pool.dtype != q.dtype \
            or c4_pool.dtype != q.dtype:
        raise TypeError("hsa_decode_step_paged: pools must have the query dtype")
    if swa_pool.dim() != 3 or c4_pool.dim() != 3 or kI_pool.dim() != 3:
        raise ValueError("hsa_decode_step_paged: pools are [pages, rows, D]")
    if kI_pool.shape[1] != c4_pool.shape[1] or kI_map.shape != c4_map.shape:
        raise ValueError("hsa_decode_step_paged: kI and C4 shadows must share the page size")
    for t in (pos, swa_map, c4_map, kI_map):
        if t.dtype != torch.int32:
            raise TypeError("hsa_decode_step_paged: pos and maps must be int32")
    if x_tok is not None:
        for t in (x_tok, g_tok, bias, state_x, state_g):
            if t.dtype != q.dtype:
                raise TypeError("hsa_decode_step_paged: append tensors must have the query dtype")
        if (tuple(x_tok.shape) != (B, d_qk) or tuple(g_tok.shape) != (B, d_qk)
                or tuple(bias.shape) != (4, d_qk) or tuple(state_x.shape) != tuple(swa_pool.shape)
                or tuple(state_g.shape) != tuple(swa_pool.shape)):
            raise ValueError("hsa_decode_step_paged: append shape mismatch")
    maps = PageMaps(_ptr(swa_map).value, swa_map.shape[1], swa_pool.shape[1], swa_pool.shape[0],
                    _ptr(c4_map).value, _ptr(kI_map).value, c4_map.shape[1], c4_pool.shape[1],
                    c4_pool.shape[0], kI_pool.shape[0])
    dev = q.device
    n_cand, swa_len, comp_len = _i32(n_cand, dev), _i32(swa_len, dev), _i32(comp_len, dev)
    if scores is None:
        scores = torch.empty((B, S_max), dtype=torch.float32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, H, d_v), dtype=q.dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream() if stream is None else stream
    need = lib.hsa_decode_sparse_workspace_size(B, H, d_v, W, S_max, k)
    cached = workspace is None
    if cached:
        workspace = Workspace.get("decode_sparse:%d:%d:%d:%d:%d" % (B, H, d_v, W, S_max * 4096 + k),
                                  need, dev, st)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call_with_workspace("hsa_decode_step_paged", lambda: lib.hsa_decode_step_paged(
        _dt(q), _ptr(x_tok), _ptr(g_tok), _ptr(bias), _ptr(state_x), _ptr(state_g), _ptr(pos),
        _ptr(q_idx), _ptr(kI_pool), _ptr(n_cand), _ptr(scores), _ptr(topk_idx), _ptr(q),
        _ptr(swa_pool), _ptr(swa_len), _ptr(c4_pool), _ptr(comp_len), ctypes.byref(maps),
        _ptr(out), _ptr(lse), B, H_I, d_I, H, d_qk, d_v, W, S_max, k, float(scale),
        _ptr(workspace), wsz, _stream(st)), workspace, cached)
    return scores, topk_idx, out, lse


def hsa_decode_step_noalloc(x_tok, g_tok, bias, ring_x, ring_g, pos, q_idx, k_idx, n_cand, k, q,
                            swa_kv, swa_len, comp_kv, comp_len, scale, d_v, scores, topk_idx,
                            out, lse, stream=None):
    """hsa_decode_step without a workspace (the library's own fixed scratch): for
    callers that cannot allocate, so every output is passed in.  Arguments and
    results as hsa_decode_step; n_cand, swa_len and comp_len must be int32 device
    tensors already."""
    B, H_I, d_I = q_idx.shape
    _, S_max, _ = k_idx.shape
    _, H, d_qk = q.shape
    W = swa_kv.shape[1]
    for name, t, shape, dt in (("scores", scores, (B, S_max), torch.float32),
                               ("topk_idx", topk_idx, (B, k), torch.int32),
                               ("out", out, (B, H, d_v), q.dtype), ("lse", lse, (B, H), torch.float32)):
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous():
            raise ValueError("hsa_decode_step_noalloc: %s must be a contiguous %s %s" % (name, dt, shape))
    for name, t in (("pos", pos), ("n_cand", n_cand), ("swa_len", swa_len), ("comp_len", comp_len)):
        if t.dtype != torch.int32 or tuple(t.shape) != (B,) or t.device != q.device:
            raise TypeError("hsa_decode_step_noalloc: %s must be int32 [B] on the query's device" % name)
    if comp_kv.shape[1] != S_max or k_idx.dtype != q_idx.dtype or q.dtype != q_idx.dtype:
        raise ValueError("hsa_decode_step_noalloc: shape or dtype mismatch")
    for t in (x_tok, g_tok, bias, ring_x, ring_g, comp_kv):
        if t.dtype != q.dtype:
            raise TypeError("hsa_decode_step_noalloc: append tensors must have the query dtype")
    if (tuple(x_tok.shape) != (B, d_qk) or tuple(g_tok.shape) != (B, d_qk)
            or tuple(bias.shape) != (4, d_qk) or tuple(ring_x.shape) != (B, 4, d_qk)
            or tuple(ring_g.shape) != (B, 4, d_qk)):
        raise ValueError("hsa_decode_step_noalloc: append shape mismatch")
    st = torch.cuda.current_stream() if stream is None else stream
    _check("hsa_decode_step_noalloc", lib.hsa_decode_step_noalloc(
        _dt(q), _ptr(x_tok), _ptr(g_tok), _ptr(bias), _ptr(ring_x), _ptr(ring_g), _ptr(pos),
        _ptr(q_idx), _ptr(k_idx), _ptr(n_cand), _ptr(scores), _ptr(topk_idx), _ptr(q),
        _ptr(swa_kv), _ptr(swa_len), _ptr(comp_kv), _ptr(comp_len), _ptr(out), _ptr(lse), B, H_I,
        d_I, H, d_qk, d_v, W, S_max, k, float(scale), _stream(st)))
    return scores, topk_idx, out, lse


def hsa_attn_prefill(q, kv, comp_kv, q_start, W, m, scale, d_v, comp_idx=None, out=None,
                     lse=None, stream=None):
    """Chunked prefill: causal SWA window plus sparse (comp_idx) or dense visible rows.

    q: [n_seq, n_q, H, d_qk]; kv: [n_seq, T, d_qk]; comp_kv: [n_seq, S_max, d_qk];
    comp_idx: [n_seq*n_q, k] int32 or None.  Returns (out [n_seq, n_q, H, d_v], lse)."""
    n_seq, n_q, H, d_qk = q.shape
    T = kv.shape[1]
    S_max = comp_kv.shape[1]
    dev = q.device
    comp_idx = _i32(comp_idx, dev)
    k = 0 if comp_idx is None else comp_idx.shape[1]
    if out is None:
        out = torch.empty((n_seq, n_q, H, d_v), dtype=q.dtype, device=dev)
    if lse is None:
        lse = torch.empty((n_seq * n_q, H), dtype=torch.float32, device=dev)
    _check("hsa_attn_prefill", lib.hsa_attn_prefill(
        _dt(q), _ptr(q), _ptr(kv), _ptr(comp_kv), _ptr(comp_idx), _ptr(out), _ptr(lse), n_seq,
        n_q, q_start, T, H, d_qk, d_v, W, S_max, k, m, float(scale), None, 0, _stream(stream)))
    return out, lse


def hsa_profile_enable(family_mask: int) -> None:
    """Arm event timing for the kernel families in family_mask (0 disarms)."""
    _check("hsa_profile_enable", lib.hsa_profile_enable(int(family_mask)))


def hsa_profile_read(family: int, reset: bool = False):
    """(total milliseconds, launch count) recorded so far for one kernel family."""
    ms, n = ctypes.c_double(), ctypes.c_longlong()
    _check("hsa_profile_read", lib.hsa_profile_read(int(family), ctypes.byref(ms), ctypes.byref(n),
                                                    1 if reset else 0))
    return ms.value, n.value


def hsa_stream_read(src, sink=None, stream=None):
    """Plain read of the whole of src (a device tensor whose size is a multiple of
    16 MiB) in the decode scoring kernel's launch shape: a read-bandwidth reference
    for that kernel.  sink: 4096-byte device scratch (allocated when None)."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("hsa_stream_read: src must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(4096, dtype=torch.uint8, device=src.device)
    _check("hsa_stream_read", lib.hsa_stream_read(_ptr(src), src.numel() * src.element_size(),
                                                  _ptr(sink), _stream(stream)))
    return sink
