"""hybrid_sparse_compressed_amd -- MI355X (gfx950) hybrid sparse-attention hot path.

The compute lives in libhsa_attn.so (hand-written HIP kernels behind a C ABI,
declared in include/hsa_attn.h).  This package holds that library's sources
(csrc/), its build script (build.py), a ctypes binding with the C entry
points' names (_binding.py) and the seeded synthetic workload generators
(workloads.py, which holds no arithmetic of the method).

Touching any binding name (``hsa_compress`` ...) loads the library and raises
ImportError if it has not been built; there is no fallback path.
"""

_BINDING_NAMES = (
    "EXPORTED", "HSA_BF16", "HSA_F32", "HsaError", "Workspace", "hsa_attn_decode",
    "hsa_attn_prefill", "hsa_compress", "hsa_compress_append", "hsa_index_topk",
    "hsa_decode_sparse", "hsa_decode_step", "hsa_decode_step_noalloc", "hsa_decode_step_paged",
    "PageMaps", "hsa_index_topk_weighted", "hsa_decode_sparse_weighted", "hsa_compress_overlap",
    "hsa_compress_append_overlap", "lib", "strerror",
    "hsa_profile_enable", "hsa_profile_read", "HSA_PROF_COMPRESS", "HSA_PROF_SCORE",
    "HSA_PROF_SELECT", "HSA_PROF_ATTN", "HSA_PROF_MERGE", "HSA_PROF_STREAM", "hsa_stream_read",
)

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _binding

        return getattr(_binding, name)
    raise AttributeError(name)
