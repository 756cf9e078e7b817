// api.hip -- the extern "C" boundary of libhsa_attn.so.  Every entry point
// validates its arguments on the host, returns a status code without
// launching anything when they are rejected, and otherwise enqueues the
// kernels on the caller's stream.  No exception crosses this boundary.
#include "../../include/hsa_attn.h"
#include "hsa_internal.hpp"

#include <stdint.h>

#include <mutex>

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int dt) { return dt == HSA_F32 || dt == HSA_BF16; }
int esize(int dt) { return dt == HSA_F32 ? 4 : 2; }
hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int finish(hipError_t e) { return e == hipSuccess ? HSA_OK : HSA_ERR_HIP; }

}  // namespace

extern "C" {

const char* hsa_strerror(int status) {
    switch (status) {
        case HSA_OK: return "HSA_OK";
        case HSA_ERR_INVALID_ARG: return "HSA_ERR_INVALID_ARG";
        case HSA_ERR_UNSUPPORTED: return "HSA_ERR_UNSUPPORTED";
        case HSA_ERR_WORKSPACE: return "HSA_ERR_WORKSPACE";
        case HSA_ERR_HIP: return "HSA_ERR_HIP";
        default: return "HSA_ERR_UNKNOWN";
    }
}

int hsa_version(void) { return 100; }

int hsa_compress(int dtype, const void* x, const void* gate, const void* bias, void* out,
                 int32_t B, int32_t T, int32_t D, int32_t m, void* stream) {
    try {
        if (!dtype_ok(dtype)) return HSA_ERR_INVALID_ARG;
        if (!x || !gate || !bias || !out) return HSA_ERR_INVALID_ARG;
        if (!aligned16(x) || !aligned16(gate) || !aligned16(bias) || !aligned16(out))
            return HSA_ERR_INVALID_ARG;
        if (B < 1 || D < 1 || m < 1 || m > 1024 || T < m) return HSA_ERR_INVALID_ARG;
        if ((D * esize(dtype)) % 16 != 0) return HSA_ERR_UNSUPPORTED;
        return finish(hsa::launch_compress(dtype, x, gate, bias, out, B, T, D, m, as_stream(stream)));
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

int hsa_compress_append(int dtype, const void* x_tok, const void* g_tok, const void* bias,
                        void* ring_x, void* ring_g, const int32_t* pos, void* pool, int32_t B,
                        int32_t D, int32_t m, int32_t S_max, void* stream) {
    try {
        if (!dtype_ok(dtype)) return HSA_ERR_INVALID_ARG;
        if (!x_tok || !g_tok || !bias || !ring_x || !ring_g || !pos || !pool)
            return HSA_ERR_INVALID_ARG;
        if (!aligned16(x_tok) || !aligned16(g_tok) || !aligned16(bias) || !aligned16(ring_x) ||
            !aligned16(ring_g) || !aligned16(pool))
            return HSA_ERR_INVALID_ARG;
        if (B < 1 || D < 1 || m < 1 || m > 1024 || S_max < 1) return HSA_ERR_INVALID_ARG;
        if ((D * esize(dtype)) % 16 != 0) return HSA_ERR_UNSUPPORTED;
        if ((long long)D * esize(dtype) / 16 > 65535LL * 256) return HSA_ERR_UNSUPPORTED;
        return finish(hsa::launch_compress_append(dtype, x_tok, g_tok, bias, ring_x, ring_g, pos,
                                                  pool, B, D, m, S_max, as_stream(stream)));
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

int hsa_compress_overlap(int dtype, const void* x, const void* gate, const void* bias, void* out,
                         int32_t B, int32_t T, int32_t D, int32_t m, void* stream) {
    try {
        if (!dtype_ok(dtype)) return HSA_ERR_INVALID_ARG;
        if (!x || !gate || !bias || !out) return HSA_ERR_INVALID_ARG;
        if (!aligned16(x) || !aligned16(gate) || !aligned16(bias) || !aligned16(out))
            return HSA_ERR_INVALID_ARG;
        if (B < 1 || D < 1 || m < 1 || T < m) return HSA_ERR_INVALID_ARG;
        if (m > 4 || (D * esize(dtype)) % 16 != 0) return HSA_ERR_UNSUPPORTED;
        return finish(hsa::launch_compress_overlap(dtype, x, gate, bias, out, B, T, D, m,
                                                   as_stream(stream)));
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

int hsa_compress_append_overlap(int dtype, const void* x_tok, const void* g_tok, const void* bias,
                                void* ring_x, void* ring_g, const int32_t* pos, void* pool,
                                int32_t B, int32_t D, int32_t m, int32_t S_max, void* stream) {
    try {
        if (!dtype_ok(dtype)) return HSA_ERR_INVALID_ARG;
        if (!x_tok || !g_tok || !bias || !ring_x || !ring_g || !pos || !pool)
            return HSA_ERR_INVALID_ARG;
        if (!aligned16(x_tok) || !aligned16(g_tok) || !aligned16(bias) || !aligned16(ring_x) ||
            !aligned16(ring_g) || !aligned16(pool))
            return HSA_ERR_INVALID_ARG;
        if (B < 1 || D < 1 || m < 1 || S_max < 1) return HSA_ERR_INVALID_ARG;
        if (m > 4 || (D * esize(dtype)) % 16 != 0) return HSA_ERR_UNSUPPORTED;
        if ((long long)D * esize(dtype) / 16 > 65535LL * 256) return HSA_ERR_UNSUPPORTED;
        return finish(hsa::launch_compress_append_overlap(dtype, x_tok, g_tok, bias, ring_x, ring_g,
                                                          pos, pool, B, D, m, S_max,
                                                          as_stream(stream)));
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

size_t hsa_index_topk_workspace_size(int32_t Nq, int32_t S_max, int32_t k) {
    if (Nq < 1 || S_max < 1 || k < 1) return 0;
    return hsa::topk_workspace_bytes(Nq, S_max, k);
}

int hsa_index_topk(int dtype, const void* q_idx, const void* k_idx, int32_t B,
                   const int32_t* q_seq, const int32_t* n_cand, float* scores,
                   int32_t* topk_idx, int32_t Nq, int32_t H_I, int32_t d_I, int32_t S_max,
                   int32_t k, uint32_t flags, void* workspace, size_t workspace_bytes,
                   void* stream) {
    try {
        if (flags != 0) return HSA_ERR_INVALID_ARG;
        if (!n_cand || !scores || !topk_idx) return HSA_ERR_INVALID_ARG;
        if (Nq < 1 || S_max < 1 || k < 1 || k > hsa::kTopkMaxK) return HSA_ERR_INVALID_ARG;
        if (S_max > hsa::kTopkMaxSegments * 4096) return HSA_ERR_UNSUPPORTED;
        if (q_idx) {
            if (!dtype_ok(dtype) || !k_idx || B < 1 || H_I < 1 || d_I < 1) return HSA_ERR_INVALID_ARG;
            if (!aligned16(q_idx) || !aligned16(k_idx)) return HSA_ERR_INVALID_ARG;
            if (!q_seq && Nq > B) return HSA_ERR_INVALID_ARG;
            const int row_bytes = d_I * esize(dtype);
            if (row_bytes != 128 && row_bytes != 256 && row_bytes != 512) return HSA_ERR_UNSUPPORTED;
        }
        const size_t need = hsa::topk_workspace_bytes(Nq, S_max, k);
        if (need > 0 && (!workspace || workspace_bytes < need)) return HSA_ERR_WORKSPACE;
        return finish(hsa::launch_index_topk(dtype, q_idx, k_idx, B, q_seq, n_cand, scores,
                                             topk_idx, Nq, H_I, d_I, S_max, k, workspace,
                                             as_stream(stream)));
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

}  // extern "C"

namespace {
// Shape of the weighted, activated indexer heads: bf16, 128-wide keys, H_I a
// multiple of 16 up to 64, fp32 weights 4-byte aligned.
int weighted_heads_ok(int dtype, int32_t H_I, int32_t d_I, const float* head_w) {
    if (!head_w || (reinterpret_cast<uintptr_t>(head_w) & 3u) != 0) return HSA_ERR_INVALID_ARG;
    if (dtype != HSA_BF16 || d_I != 128 || H_I < 16 || H_I % 16 != 0 || H_I > 64)
        return HSA_ERR_UNSUPPORTED;
    return HSA_OK;
}
}  // namespace

extern "C" {

int hsa_index_topk_weighted(int dtype, const void* q_idx, const float* head_w, const void* k_idx,
                            int32_t B, const int32_t* q_seq, const int32_t* n_cand, float* scores,
                            int32_t* topk_idx, int32_t Nq, int32_t H_I, int32_t d_I,
                            int32_t S_max, int32_t k, void* workspace, size_t workspace_bytes,
                            void* stream) {
    try {
        if (!q_idx || !dtype_ok(dtype)) return HSA_ERR_INVALID_ARG;
        if (!n_cand || !scores || !topk_idx || !k_idx) return HSA_ERR_INVALID_ARG;
        if (Nq < 1 || B < 1 || H_I < 1 || d_I < 1 || S_max < 1 || k < 1 || k > hsa::kTopkMaxK)
            return HSA_ERR_INVALID_ARG;
        if (!aligned16(q_idx) || !aligned16(k_idx)) return HSA_ERR_INVALID_ARG;
        if (!q_seq && Nq > B) return HSA_ERR_INVALID_ARG;
        const int wok = weighted_heads_ok(dtype, H_I, d_I, head_w);
        if (wok != HSA_OK) return wok;
        if (S_max > hsa::kTopkMaxSegments * 4096) return HSA_ERR_UNSUPPORTED;
        const size_t need = hsa::topk_workspace_bytes(Nq, S_max, k);
        if (need > 0 && (!workspace || workspace_bytes < need)) return HSA_ERR_WORKSPACE;
        return finish(hsa::launch_index_topk(dtype, q_idx, k_idx, B, q_seq, n_cand, scores,
                                             topk_idx, Nq, H_I, d_I, S_max, k, workspace,
                                             as_stream(stream), nullptr, head_w));
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

size_t hsa_attn_decode_workspace_size(int32_t B, int32_t H, int32_t d_v, int32_t max_rows) {
    if (B < 1 || H < 1 || d_v < 1 || max_rows < 1) return 0;
    return hsa::decode_workspace_bytes(B, H, d_v, max_rows, true);
}

int hsa_attn_decode(int dtype, const void* q, const void* swa_kv, const int32_t* swa_len,
                    const void* comp_kv, const int32_t* comp_idx, const int32_t* comp_len,
                    void* out, float* lse, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                    int32_t W, int32_t S_max, int32_t k, float scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
    try {
        if (!dtype_ok(dtype)) return HSA_ERR_INVALID_ARG;
        if (!q || !swa_kv || !swa_len || !comp_len || !out) return HSA_ERR_INVALID_ARG;
        if (S_max > 0 && !comp_kv) return HSA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(swa_kv) || !aligned16(out) || (comp_kv && !aligned16(comp_kv)))
            return HSA_ERR_INVALID_ARG;
        if (B < 1 || H < 1 || H > 1024 || d_qk < 1 || d_v < 1 || d_v > d_qk || W < 1 || S_max < 0)
            return HSA_ERR_INVALID_ARG;
        if (comp_idx && (k < 1 || k > (1 << 20))) return HSA_ERR_INVALID_ARG;
        if (!(scale == scale)) return HSA_ERR_INVALID_ARG;
        if (!hsa::attn_shape_supported(dtype, d_qk, d_v)) return HSA_ERR_UNSUPPORTED;
        const int max_rows = W + (comp_idx ? k : S_max);
        const size_t need = hsa::decode_workspace_bytes(B, H, d_v, max_rows, comp_idx == nullptr);
        if (need > 0 && (!workspace || workspace_bytes < need)) return HSA_ERR_WORKSPACE;
        return finish(hsa::launch_attn_decode(dtype, q, swa_kv, swa_len, comp_kv, comp_idx,
                                              comp_len, out, lse, B, H, d_qk, d_v, W, S_max,
                                              comp_idx ? k : 0, scale, workspace,
                                              as_stream(stream)));
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t hsa_decode_sparse_workspace_size(int32_t B, int32_t H, int32_t d_v, int32_t W,
                                        int32_t S_max, int32_t k) {
    if (B < 1 || H < 1 || d_v < 1 || W < 1 || S_max < 1 || k < 1) return 0;
    return round256(hsa::topk_workspace_bytes(B, S_max, k)) + hsa::decode_workspace_bytes(B, H, d_v, W + k, false);
}

namespace {

// hsa_decode_sparse, preceded by the decode-time C4 append of `job` when it is
// not null (its arguments already checked).  clear_ws: the workspace holds
// unknown contents, so the words the chosen path needs at zero are cleared
// first (by fill kernels on the stream, after every argument check).
int decode_sparse_impl(int dtype, const void* q_idx, const void* k_idx, const int32_t* n_cand,
                       float* scores, int32_t* topk_idx, const void* q, const void* swa_kv,
                       const int32_t* swa_len, const void* comp_kv, const int32_t* comp_len,
                       void* out, float* lse, int32_t B, int32_t H_I, int32_t d_I, int32_t H,
                       int32_t d_qk, int32_t d_v, int32_t W, int32_t S_max, int32_t k,
                       float scale, void* workspace, size_t workspace_bytes, void* stream,
                       const hsa::AppendJob* job, bool clear_ws = false,
                       const hsa::Paging* pg = nullptr, const float* head_w = nullptr) {
    // indexer + select arguments (as hsa_index_topk with Nq = B, no q_seq)
    if (!dtype_ok(dtype) || !q_idx || !k_idx || !n_cand || !scores || !topk_idx)
        return HSA_ERR_INVALID_ARG;
    if (B < 1 || H_I < 1 || d_I < 1 || S_max < 1 || k < 1 || k > hsa::kTopkMaxK)
        return HSA_ERR_INVALID_ARG;
    if (S_max > hsa::kTopkMaxSegments * 4096) return HSA_ERR_UNSUPPORTED;
    if (!aligned16(q_idx) || !aligned16(k_idx)) return HSA_ERR_INVALID_ARG;
    const int row_bytes = d_I * esize(dtype);
    if (row_bytes != 128 && row_bytes != 256 && row_bytes != 512) return HSA_ERR_UNSUPPORTED;
    if (head_w) {
        const int wok = weighted_heads_ok(dtype, H_I, d_I, head_w);
        if (wok != HSA_OK) return wok;
    }
    // attention arguments (as hsa_attn_decode, sparse mode)
    if (!q || !swa_kv || !swa_len || !comp_kv || !comp_len || !out) return HSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(swa_kv) || !aligned16(out) || !aligned16(comp_kv))
        return HSA_ERR_INVALID_ARG;
    if (H < 1 || H > 1024 || d_qk < 1 || d_v < 1 || d_v > d_qk || W < 1) return HSA_ERR_INVALID_ARG;
    if (!(scale == scale)) return HSA_ERR_INVALID_ARG;
    if (!hsa::attn_shape_supported(dtype, d_qk, d_v)) return HSA_ERR_UNSUPPORTED;
    const size_t need = hsa_decode_sparse_workspace_size(B, H, d_v, W, S_max, k);
    if (!workspace || workspace_bytes < need) return HSA_ERR_WORKSPACE;
    hipStream_t st = as_stream(stream);
    uint8_t* ws_sel = static_cast<uint8_t*>(workspace);
    uint8_t* ws_attn = ws_sel + round256(hsa::topk_workspace_bytes(B, S_max, k));
    const bool fused = S_max > hsa::kRowSelectCap && hsa::index_lists_apply(S_max, k, B) &&
                       hsa::fused_decode_supported(B, H, W, k);
    if (clear_ws) {
        // fused: only the first-digit histograms must start at zero (every other
        // word is written before it is read); the separate multi-workgroup
        // select needs its whole workspace zero; the LDS row select needs none
        hipError_t e = hipSuccess;
        if (fused)
            e = hsa::launch_clear_select_hist(ws_sel, B, S_max, k, st);
        else
            e = hsa::launch_zero_words(ws_sel, hsa::topk_workspace_bytes(B, S_max, k) / 4, st);
        if (e != hipSuccess) return finish(e);
    }
    if (fused) {
        // the append rides in the scoring launch, which ends before the attention
        // reads the pool; scoring never reads it
        hipError_t e = hsa::launch_index_lists(dtype, q_idx, k_idx, B, n_cand, scores, B, H_I,
                                               d_I, S_max, k, ws_sel, job, st,
                                               pg ? &pg->kI : nullptr, head_w);
        if (e != hipSuccess) return finish(e);
        e = hsa::launch_attn_decode_fused(dtype, q, swa_kv, swa_len, comp_kv, comp_len, n_cand,
                                          ws_sel, scores, topk_idx, out, lse, B, H, d_qk, d_v, W,
                                          S_max, k, scale, ws_attn, st, pg);
        // the scoring launch counted into the histograms that the merge would have
        // cleared: leave the workspace ready for the next call all the same
        if (e != hipSuccess) (void)hsa::launch_clear_select_hist(ws_sel, B, S_max, k, st);
        return finish(e);
    }
    if (job) {
        hipError_t e = job->swa.map
                           ? hsa::launch_compress_append_paged(dtype, *job, st)
                           : hsa::launch_compress_append(dtype, job->x_tok, job->g_tok, job->bias,
                                                         job->ring_x, job->ring_g, job->pos,
                                                         job->pool, job->B, job->D, 4, job->S_max, st);
        if (e != hipSuccess) return finish(e);
    }
    hipError_t e = hsa::launch_index_topk(dtype, q_idx, k_idx, B, nullptr, n_cand, scores,
                                          topk_idx, B, H_I, d_I, S_max, k, ws_sel, st,
                                          pg ? &pg->kI : nullptr, head_w);
    if (e != hipSuccess) return finish(e);
    return finish(hsa::launch_attn_decode(dtype, q, swa_kv, swa_len, comp_kv, topk_idx,
                                          comp_len, out, lse, B, H, d_qk, d_v, W, S_max, k,
                                          scale, ws_attn, st, pg));
}

}  // namespace

int hsa_decode_sparse(int dtype, const void* q_idx, const void* k_idx, const int32_t* n_cand,
                      float* scores, int32_t* topk_idx, const void* q, const void* swa_kv,
                      const int32_t* swa_len, const void* comp_kv, const int32_t* comp_len,
                      void* out, float* lse, int32_t B, int32_t H_I, int32_t d_I, int32_t H,
                      int32_t d_qk, int32_t d_v, int32_t W, int32_t S_max, int32_t k,
                      float scale, void* workspace, size_t workspace_bytes, void* stream) {
    try {
        return decode_sparse_impl(dtype, q_idx, k_idx, n_cand, scores, topk_idx, q, swa_kv,
                                  swa_len, comp_kv, comp_len, out, lse, B, H_I, d_I, H, d_qk, d_v,
                                  W, S_max, k, scale, workspace, workspace_bytes, stream, nullptr);
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

int hsa_decode_sparse_weighted(int dtype, const void* q_idx, const float* head_w,
                               const void* k_idx, const int32_t* n_cand, float* scores,
                               int32_t* topk_idx, const void* q, const void* swa_kv,
                               const int32_t* swa_len, const void* comp_kv,
                               const int32_t* comp_len, void* out, float* lse, int32_t B,
                               int32_t H_I, int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v,
                               int32_t W, int32_t S_max, int32_t k, float scale, void* workspace,
                               size_t workspace_bytes, void* stream) {
    try {
        if (!head_w) return HSA_ERR_INVALID_ARG;
        return decode_sparse_impl(dtype, q_idx, k_idx, n_cand, scores, topk_idx, q, swa_kv,
                                  swa_len, comp_kv, comp_len, out, lse, B, H_I, d_I, H, d_qk, d_v,
                                  W, S_max, k, scale, workspace, workspace_bytes, stream, nullptr,
                                  false, nullptr, head_w);
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

int hsa_decode_step(int dtype, const void* x_tok, const void* g_tok, const void* bias,
                    void* ring_x, void* ring_g, const int32_t* pos, const void* q_idx,
                    const void* k_idx, const int32_t* n_cand, float* scores, int32_t* topk_idx,
                    const void* q, const void* swa_kv, const int32_t* swa_len, void* comp_kv,
                    const int32_t* comp_len, void* out, float* lse, int32_t B, int32_t H_I,
                    int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v, int32_t W, int32_t S_max,
                    int32_t k, float scale, void* workspace, size_t workspace_bytes,
                    void* stream) {
    try {
        // append arguments (as hsa_compress_append with m = 4, pool = comp_kv, D = d_qk)
        if (!dtype_ok(dtype)) return HSA_ERR_INVALID_ARG;
        if (!x_tok || !g_tok || !bias || !ring_x || !ring_g || !pos || !comp_kv)
            return HSA_ERR_INVALID_ARG;
        if (!aligned16(x_tok) || !aligned16(g_tok) || !aligned16(bias) || !aligned16(ring_x) ||
            !aligned16(ring_g) || !aligned16(comp_kv))
            return HSA_ERR_INVALID_ARG;
        if (B < 1 || d_qk < 1 || S_max < 1) return HSA_ERR_INVALID_ARG;
        if ((d_qk * esize(dtype)) % 16 != 0) return HSA_ERR_UNSUPPORTED;
        const hsa::AppendJob job{x_tok, g_tok, bias, ring_x, ring_g, pos, comp_kv, B, d_qk, S_max};
        return decode_sparse_impl(dtype, q_idx, k_idx, n_cand, scores, topk_idx, q, swa_kv,
                                  swa_len, comp_kv, comp_len, out, lse, B, H_I, d_I, H, d_qk, d_v,
                                  W, S_max, k, scale, workspace, workspace_bytes, stream, &job);
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

int hsa_decode_step_paged(int dtype, const void* x_tok, const void* g_tok, const void* bias,
                          void* state_x, void* state_g, const int32_t* pos, const void* q_idx,
                          const void* kI_pool, const int32_t* n_cand, float* scores,
                          int32_t* topk_idx, const void* q, const void* swa_pool,
                          const int32_t* swa_len, void* c4_pool, const int32_t* comp_len,
                          const hsa_page_maps* maps, void* out, float* lse, int32_t B,
                          int32_t H_I, int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v,
                          int32_t W, int32_t S_max, int32_t k, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
    try {
        if (!dtype_ok(dtype) || !maps || !pos) return HSA_ERR_INVALID_ARG;
        const hsa_page_maps& m = *maps;
        auto page_rows_ok = [](int32_t v) { return v >= 16 && v <= 4096 && (v & (v - 1)) == 0; };
        if (!m.swa_map || !m.c4_map || !m.kI_map) return HSA_ERR_INVALID_ARG;
        if (!page_rows_ok(m.swa_page_rows) || !page_rows_ok(m.c4_page_rows)) return HSA_ERR_INVALID_ARG;
        if (m.swa_map_pages < 1 || m.c4_map_pages < 1 || m.swa_pool_pages < 1 ||
            m.c4_pool_pages < 1 || m.kI_pool_pages < 1)
            return HSA_ERR_INVALID_ARG;
        if (B < 1 || S_max < 1 || d_qk < 1) return HSA_ERR_INVALID_ARG;
        if ((long long)m.c4_map_pages * m.c4_page_rows < S_max) return HSA_ERR_INVALID_ARG;
        hsa::Paging pg;
        pg.swa = {m.swa_map, m.swa_map_pages, __builtin_ctz((unsigned)m.swa_page_rows), m.swa_pool_pages};
        pg.c4 = {m.c4_map, m.c4_map_pages, __builtin_ctz((unsigned)m.c4_page_rows), m.c4_pool_pages};
        pg.kI = {m.kI_map, m.c4_map_pages, __builtin_ctz((unsigned)m.c4_page_rows), m.kI_pool_pages};
        pg.pos = pos;
        hsa::AppendJob job{};
        if (x_tok) {
            // append arguments (as hsa_decode_step, the rings replaced by the state pools)
            if (!g_tok || !bias || !state_x || !state_g || !c4_pool) return HSA_ERR_INVALID_ARG;
            if (!aligned16(x_tok) || !aligned16(g_tok) || !aligned16(bias) || !aligned16(state_x) ||
                !aligned16(state_g) || !aligned16(c4_pool))
                return HSA_ERR_INVALID_ARG;
            if ((d_qk * esize(dtype)) % 16 != 0) return HSA_ERR_UNSUPPORTED;
            job = hsa::AppendJob{x_tok, g_tok, bias, state_x, state_g, pos, c4_pool, B, d_qk, S_max,
                                 pg.swa, pg.c4};
        }
        return decode_sparse_impl(dtype, q_idx, kI_pool, n_cand, scores, topk_idx, q, swa_pool,
                                  swa_len, c4_pool, comp_len, out, lse, B, H_I, d_I, H, d_qk, d_v,
                                  W, S_max, k, scale, workspace, workspace_bytes, stream,
                                  x_tok ? &job : nullptr, false, &pg);
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

}  // extern "C"

namespace {

// Scratch of hsa_decode_step_noalloc: device memory of the library itself, one
// copy per GPU, held until the process ends.  In host code this name is only a
// stand-in: the kernels get the per-device address that hipGetSymbolAddress
// returns (scratch_addr below), never the name itself.
static __device__ __align__(256) uint8_t scratch[HSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxScratchDevices];

// The device address of `scratch` on device `dev`, looked up on the first call
// for that device with that device current, then kept.
hipError_t scratch_addr(int dev, void** out) {
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int hsa_decode_step_noalloc(int dtype, const void* x_tok, const void* g_tok, const void* bias,
                            void* ring_x, void* ring_g, const int32_t* pos, const void* q_idx,
                            const void* k_idx, const int32_t* n_cand, float* scores,
                            int32_t* topk_idx, const void* q, const void* swa_kv,
                            const int32_t* swa_len, void* comp_kv, const int32_t* comp_len,
                            void* out, float* lse, int32_t B, int32_t H_I, int32_t d_I, int32_t H,
                            int32_t d_qk, int32_t d_v, int32_t W, int32_t S_max, int32_t k,
                            float scale, void* stream) {
    try {
        // append arguments (as hsa_decode_step); the rest is checked by the step itself
        if (!dtype_ok(dtype)) return HSA_ERR_INVALID_ARG;
        if (!x_tok || !g_tok || !bias || !ring_x || !ring_g || !pos || !comp_kv)
            return HSA_ERR_INVALID_ARG;
        if (!aligned16(x_tok) || !aligned16(g_tok) || !aligned16(bias) || !aligned16(ring_x) ||
            !aligned16(ring_g) || !aligned16(comp_kv))
            return HSA_ERR_INVALID_ARG;
        if (B < 1 || d_qk < 1 || S_max < 1) return HSA_ERR_INVALID_ARG;
        if ((d_qk * esize(dtype)) % 16 != 0) return HSA_ERR_UNSUPPORTED;
        const size_t need = hsa_decode_sparse_workspace_size(B, H, d_v, W, S_max, k);
        if (need == 0) return HSA_ERR_INVALID_ARG;
        if (need > (size_t)HSA_NOALLOC_SCRATCH_BYTES) return HSA_ERR_WORKSPACE;
        hipStream_t st = as_stream(stream);
        int dev = 0;
        hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
        if (e != hipSuccess) return HSA_ERR_HIP;
        void* ws = nullptr;
        if (scratch_addr(dev, &ws) != hipSuccess) return HSA_ERR_HIP;
        const hsa::AppendJob job{x_tok, g_tok, bias, ring_x, ring_g, pos, comp_kv, B, d_qk, S_max};
        return decode_sparse_impl(dtype, q_idx, k_idx, n_cand, scores, topk_idx, q, swa_kv,
                                  swa_len, comp_kv, comp_len, out, lse, B, H_I, d_I, H, d_qk, d_v,
                                  W, S_max, k, scale, ws, (size_t)HSA_NOALLOC_SCRATCH_BYTES,
                                  stream, &job, true);
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

size_t hsa_attn_prefill_workspace_size(int32_t n_seq, int32_t n_q, int32_t H, int32_t d_v) {
    (void)n_seq; (void)n_q; (void)H; (void)d_v;
    return 0;
}

int hsa_attn_prefill(int dtype, const void* q, const void* kv, const void* comp_kv,
                     const int32_t* comp_idx, void* out, float* lse, int32_t n_seq,
                     int32_t n_q, int32_t q_start, int32_t T, int32_t H, int32_t d_qk,
                     int32_t d_v, int32_t W, int32_t S_max, int32_t k, int32_t m, float scale,
                     void* workspace, size_t workspace_bytes, void* stream) {
    (void)workspace; (void)workspace_bytes;
    try {
        if (!dtype_ok(dtype)) return HSA_ERR_INVALID_ARG;
        if (!q || !kv || !out) return HSA_ERR_INVALID_ARG;
        if (S_max > 0 && !comp_kv) return HSA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || (comp_kv && !aligned16(comp_kv)))
            return HSA_ERR_INVALID_ARG;
        if (n_seq < 1 || n_q < 1 || q_start < 0 || T < 1 || (int64_t)q_start + n_q > T || H < 1 ||
            H > 1024 || d_qk < 1 || d_v < 1 || d_v > d_qk || W < 1 || S_max < 0 || m < 1)
            return HSA_ERR_INVALID_ARG;
        if (comp_idx && (k < 1 || k > (1 << 20))) return HSA_ERR_INVALID_ARG;
        if (!(scale == scale)) return HSA_ERR_INVALID_ARG;
        if (!hsa::attn_shape_supported(dtype, d_qk, d_v)) return HSA_ERR_UNSUPPORTED;
        if ((int64_t)n_q > 0x7fffffff || (int64_t)n_seq > 65535) return HSA_ERR_UNSUPPORTED;
        return finish(hsa::launch_attn_prefill(dtype, q, kv, comp_kv, comp_idx, out, lse, n_seq,
                                               n_q, q_start, T, H, d_qk, d_v, W, S_max,
                                               comp_idx ? k : 0, m, scale, as_stream(stream)));
    } catch (...) {
        return HSA_ERR_HIP;
    }
}

}  // extern "C"
