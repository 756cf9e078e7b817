"""The C-ABI library loads, exports every entry point its header declares, and
rejects bad arguments on the host with the documented status codes (nothing
here launches a kernel, so it runs without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsa_attn.h")


@pytest.fixture(scope="module")
def hsa():
    import hybrid_sparse_compressed_amd as h

    return h


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = _declared()
    for n in ("hsa_compress", "hsa_index_topk", "hsa_attn_decode", "hsa_attn_prefill"):
        assert n in names


def test_every_declared_symbol_is_exported(hsa):
    from hybrid_sparse_compressed_amd import _binding

    raw = ctypes.CDLL(_binding.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name
    assert sorted(hsa.EXPORTED) == _declared()


def test_status_strings_and_version(hsa):
    assert hsa.strerror(0) == "HSA_OK"
    assert hsa.strerror(3) == "HSA_ERR_WORKSPACE"
    assert hsa.strerror(99) == "HSA_ERR_UNKNOWN"
    assert hsa.lib.hsa_version() >= 100


def test_workspace_sizes(hsa):
    lib = hsa.lib
    assert lib.hsa_index_topk_workspace_size(4, 8192, 512) == 0  # LDS-resident select
    big = lib.hsa_index_topk_workspace_size(4, 262144, 512)
    assert big >= 4 * (262144 * 8 + 2048 * 4 + 512 * 4)
    assert lib.hsa_index_topk_workspace_size(0, 10, 10) == 0
    assert lib.hsa_attn_decode_workspace_size(4, 64, 512, 640) > 0
    assert lib.hsa_attn_prefill_workspace_size(8, 2048, 64, 512) == 0


P = ctypes.c_void_p
A = P(4096)  # aligned, never dereferenced: every call below is rejected first
MIS = P(4097)


@pytest.mark.parametrize(
    "args,code",
    [
        ((1, None, A, A, A, 1, 8, 8, 4, None), 1),    # null x
        ((7, A, A, A, A, 1, 8, 8, 4, None), 1),       # bad dtype
        ((1, A, A, A, A, 1, 8, 8, 0, None), 1),       # m = 0
        ((1, A, A, A, A, 1, 3, 8, 4, None), 1),       # T < m
        ((1, MIS, A, A, A, 1, 8, 8, 4, None), 1),     # misaligned
        ((1, A, A, A, A, 1, 8, 7, 4, None), 2),       # 7 bf16 channels: not 16-byte rows
    ],
)
def test_compress_rejects(hsa, args, code):
    assert hsa.lib.hsa_compress(*args) == code


def _topk(hsa, **kw):
    a = dict(dtype=1, q=A, k=A, B=4, q_seq=None, n_cand=A, scores=A, idx=A, Nq=4, H_I=64, d_I=128,
             S_max=1000, kk=64, flags=0, ws=None, wsz=0)
    a.update(kw)
    return hsa.lib.hsa_index_topk(a["dtype"], a["q"], a["k"], a["B"], a["q_seq"], a["n_cand"],
                                  a["scores"], a["idx"], a["Nq"], a["H_I"], a["d_I"],
                                  a["S_max"], a["kk"], a["flags"], a["ws"], a["wsz"], None)


def test_index_topk_rejects(hsa):
    assert _topk(hsa, flags=1) == 1
    assert _topk(hsa, kk=0) == 1
    assert _topk(hsa, kk=4096) == 1
    assert _topk(hsa, n_cand=None) == 1
    assert _topk(hsa, Nq=5) == 1               # no q_seq and more queries than sequences
    assert _topk(hsa, d_I=100) == 2            # 200-byte key rows
    assert _topk(hsa, S_max=300000) == 3       # multi-workgroup path needs a workspace
    assert _topk(hsa, S_max=300000, ws=A, wsz=16) == 3
    assert _topk(hsa, q=MIS) == 1


def _dec(hsa, **kw):
    a = dict(dtype=1, q=A, swa=A, swa_len=A, comp=A, idx=A, comp_len=A, out=A, lse=A, B=4, H=64,
             d_qk=576, d_v=512, W=128, S_max=1000, k=512, scale=0.04, ws=None, wsz=0)
    a.update(kw)
    return hsa.lib.hsa_attn_decode(a["dtype"], a["q"], a["swa"], a["swa_len"], a["comp"],
                                   a["idx"], a["comp_len"], a["out"], a["lse"], a["B"], a["H"],
                                   a["d_qk"], a["d_v"], a["W"], a["S_max"], a["k"], a["scale"],
                                   a["ws"], a["wsz"], None)


def test_attn_decode_rejects(hsa):
    assert _dec(hsa, d_v=600) == 1
    assert _dec(hsa, q=None) == 1
    assert _dec(hsa, scale=float("nan")) == 1
    assert _dec(hsa, W=0) == 1
    assert _dec(hsa, dtype=0) == 2                 # fp32 at 576/512 is not built
    assert _dec(hsa, d_qk=256, d_v=256) == 2
    assert _dec(hsa) == 3                          # split partials need a workspace


def test_attn_prefill_rejects(hsa):
    lib = hsa.lib

    def call(**kw):
        a = dict(dtype=1, q=A, kv=A, comp=A, idx=A, out=A, lse=A, n_seq=8, n_q=2048,
                 q_start=30720, T=32768, H=64, d_qk=576, d_v=512, W=128, S_max=8192, k=512, m=4,
                 scale=0.04)
        a.update(kw)
        return lib.hsa_attn_prefill(a["dtype"], a["q"], a["kv"], a["comp"], a["idx"], a["out"],
                                    a["lse"], a["n_seq"], a["n_q"], a["q_start"], a["T"], a["H"],
                                    a["d_qk"], a["d_v"], a["W"], a["S_max"], a["k"], a["m"],
                                    a["scale"], None, 0, None)

    assert call(q_start=30721) == 1   # last query beyond T
    assert call(m=0) == 1
    assert call(kv=None) == 1
    assert call(d_qk=64, d_v=64) == 2


def test_decode_step_noalloc_rejects(hsa):
    """The no-allocation decode step rejects sizes whose workspace need exceeds its
    fixed scratch (HSA_ERR_WORKSPACE) and bad arguments, launching nothing."""
    lib = hsa.lib

    def call(**kw):
        a = dict(dtype=1, B=4, H_I=64, d_I=128, H=64, d_qk=576, d_v=512, W=128, S_max=262144,
                 k=512, x_tok=A, comp=A)
        a.update(kw)
        ptrs = [a["x_tok"], A, A, A, A, A, A, A, A, A, A, A, A, A, a["comp"], A, A, A]
        return lib.hsa_decode_step_noalloc(a["dtype"], *ptrs, a["B"], a["H_I"], a["d_I"], a["H"],
                                           a["d_qk"], a["d_v"], a["W"], a["S_max"], a["k"], 0.04,
                                           None)

    need = lib.hsa_decode_sparse_workspace_size(4, 64, 512, 128, 262144, 512)
    assert 0 < need <= 32 << 20                      # the 1M-context step fits the scratch
    assert call(B=8) == 3                             # twice that does not
    assert call(S_max=4000000, B=1) == 3
    assert call(x_tok=None) == 1
    assert call(comp=MIS) == 1
    assert call(k=0) == 1


def test_decode_step_paged_rejects_bad_shadows(hsa):
    """The paged step checks its map description on the host: page sizes that
    are not powers of two in [16, 4096], empty maps or pools, a C4 shadow too
    short for S_max, missing maps or positions (HSA_ERR_INVALID_ARG, nothing
    launched)."""
    lib = hsa.lib
    from hybrid_sparse_compressed_amd._binding import PageMaps

    def call(maps=True, pos=A, **kw):
        m = dict(swa_map=A.value, swa_map_pages=8, swa_page_rows=16, swa_pool_pages=4, c4_map=A.value,
                 kI_map=A.value, c4_map_pages=64, c4_page_rows=256, c4_pool_pages=300,
                 kI_pool_pages=300)
        m.update(kw)
        pm = PageMaps(**m)
        ptrs = [A, A, A, A, A, pos, A, A, A, A, A, A, A, A, A, A]
        return lib.hsa_decode_step_paged(1, *ptrs, ctypes.byref(pm) if maps else None, A, A, 4, 64,
                                         128, 64, 576, 512, 128, 16384, 512, 0.04, None, 0, None)

    assert call(swa_page_rows=24) == 1
    assert call(swa_page_rows=8) == 1
    assert call(c4_page_rows=8192) == 1
    assert call(c4_map_pages=63) == 1      # 63 * 256 rows < S_max = 16384
    assert call(swa_map_pages=0) == 1
    assert call(kI_pool_pages=0) == 1
    assert call(c4_map=None) == 1
    assert call(maps=False) == 1
    assert call(pos=None) == 1
    assert call() == 3                     # well-formed: only the workspace is missing


def test_stream_read_rejects_bad_arguments(hsa):
    lib = hsa.lib
    mib16 = 16 << 20
    assert lib.hsa_stream_read(None, mib16, A, None) == 1
    assert lib.hsa_stream_read(A, mib16, None, None) == 1
    assert lib.hsa_stream_read(P(4097), mib16, A, None) == 1  # misaligned source
    assert lib.hsa_stream_read(A, mib16, P(4100), None) == 1  # misaligned sink
    assert lib.hsa_stream_read(A, 0, A, None) == 1
    assert lib.hsa_stream_read(A, mib16 + 4096, A, None) == 1  # not a multiple of 16 MiB
