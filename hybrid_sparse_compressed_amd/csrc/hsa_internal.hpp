// hsa_internal.hpp -- launchers shared between the kernel translation units
// and the C-ABI layer (api.hip).  Arguments are already validated by the
// caller; every launcher enqueues on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hsa {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// ---- optional kernel timing (profile.hip) ----
// Kernel families, same values as HSA_PROF_* in hsa_attn.h.
constexpr unsigned kProfCompress = 1u, kProfScore = 2u, kProfSelect = 4u, kProfAttn = 8u,
                   kProfMerge = 16u;
// Records a HIP event on `st` when constructed and another when destroyed, if
// the family is armed; wrap exactly one kernel launch in its scope.
class ProfScope {
  public:
    ProfScope(unsigned family, hipStream_t st);
    ~ProfScope();
    ProfScope(const ProfScope&) = delete;
    ProfScope& operator=(const ProfScope&) = delete;

  private:
    unsigned family_;
    hipStream_t st_;
    int slot_;
};

// ---- paged pools ----
// A pool kept in physical pages of 2^lg rows: row r of sequence b lives at
// physical row map[b * pages + (r >> lg)] * 2^lg + (r mod 2^lg).  A logical
// page past `pages`, or a map entry outside [0, pool_pages), is not resident:
// its rows do not exist.  map == nullptr: the flat layout [B, rows, D].
struct PoolMap {
    const int32_t* map;
    int pages;       // map entries per sequence
    int lg;          // log2 of the rows per page
    int pool_pages;  // physical pages of the pool
};
// Physical row of row r of sequence b, or -1 when it is not resident.
__device__ __forceinline__ long long paged_row(const PoolMap& m, int b, long long r) {
    const long long j = r >> m.lg;
    if (r < 0 || j >= m.pages) return -1;
    const int pg = m.map[(size_t)b * m.pages + (size_t)j];
    if (pg < 0 || pg >= m.pool_pages) return -1;
    return ((long long)pg << m.lg) | (r & ((1LL << m.lg) - 1));
}
// The shadows of one decode call: SWA rows are token-indexed (token t of the
// sequence is row t; the compression-state rows of a token sit at the same
// physical row of their own pools), C4 KV and indexer-key rows are indexed by
// entry.  pos[b] is the position of sequence b's query token (< 0: none).
struct Paging {
    PoolMap swa, c4, kI;
    const int32_t* pos;
};

// ---- compressor ----
hipError_t launch_compress(int dtype, const void* x, const void* g, const void* bias, void* out,
                           int B, int T_len, int D, int m, hipStream_t st);
// Decode-time compression state: one token per sequence into its ring, the
// block's entry written to the pool when the token completes it.
hipError_t launch_compress_append(int dtype, const void* x_tok, const void* g_tok,
                                  const void* bias, void* ring_x, void* ring_g,
                                  const int32_t* pos, void* pool, int B, int D, int m, int S_max,
                                  hipStream_t st);

// Overlapping blocks (method variant), m <= 4: entry i over blocks i-1 and i
// with a bias of 2m rows; the decode-time ring keeps the last 2m tokens.
hipError_t launch_compress_overlap(int dtype, const void* x, const void* g, const void* bias,
                                   void* out, int B, int T_len, int D, int m, hipStream_t st);
hipError_t launch_compress_append_overlap(int dtype, const void* x_tok, const void* g_tok,
                                          const void* bias, void* ring_x, void* ring_g,
                                          const int32_t* pos, void* pool, int B, int D, int m,
                                          int S_max, hipStream_t st);

// ---- indexer + top-k ----
// Candidate lists up to this length are selected by one workgroup per query
// with every key resident in LDS; longer ones use the multi-workgroup path
// (histogram pass fused into scoring, then a filter + final select).
constexpr int kRowSelectCap = 12288;
constexpr int kTopkMaxK = 2048;
constexpr int kTopkMaxSegments = 1024;  // multi-workgroup select: S_max <= 1024 * 4096
size_t topk_workspace_bytes(int Nq, int S_max, int k);
// kI != nullptr with kI->map set: k_idx is the paged indexer-key pool (a row
// that is not resident scores NaN).  head_w != nullptr: weighted, activated
// heads, sum_h head_w[q, h] * max(0, q_h . k) (bf16, d_I = 128, H_I a multiple
// of 16 up to 64; the caller checks the shape).
hipError_t launch_index_topk(int dtype, const void* q_idx, const void* k_idx, int B,
                             const int32_t* q_seq, const int32_t* n_cand, float* scores,
                             int32_t* topk_idx, int Nq, int H_I, int d_I, int S_max, int k,
                             void* ws, hipStream_t st, const PoolMap* kI = nullptr,
                             const float* head_w = nullptr);
// A decode-time C4 append (block length 4) handed to a decode layer-step:
// the arguments of launch_compress_append with m = 4.
// Paged (swa.map != nullptr): ring_x / ring_g are the compression-state pools,
// whose row of token t is the SWA row of t, and pool is the paged C4 pool.
struct AppendJob {
    const void* x_tok;
    const void* g_tok;
    const void* bias;
    void* ring_x;
    void* ring_g;
    const int32_t* pos;
    void* pool;
    int B, D, S_max;
    PoolMap swa, c4;
};
// launch_compress_append for a paged job (m = 4).
hipError_t launch_compress_append_paged(int dtype, const AppendJob& job, hipStream_t st);
// Scoring with the first-digit histogram and each scoring workgroup's
// candidate list, for S_max > kRowSelectCap where sel::lists_apply holds: the
// select is finished by the fused decode attention.  job != nullptr: the
// append runs as extra workgroups of the same launch.
bool index_lists_apply(int S_max, int k, int Nq);
// Zero the first-digit histograms of Nq queries in a top-k workspace (after a
// scoring launch whose select did not run).
hipError_t launch_clear_select_hist(void* ws, int Nq, int S_max, int k, hipStream_t st);
// Zero `words` 32-bit words at p (16-byte aligned) with a fill kernel.
hipError_t launch_zero_words(void* p, size_t words, hipStream_t st);
hipError_t launch_index_lists(int dtype, const void* q_idx, const void* k_idx, int B,
                              const int32_t* n_cand, float* scores, int Nq, int H_I, int d_I,
                              int S_max, int k, void* ws, const AppendJob* job, hipStream_t st,
                              const PoolMap* kI = nullptr, const float* head_w = nullptr);

// ---- attention ----
struct DecodePlan {
    int max_rows;  // W + (sparse ? k : S_max)
    int rows_per_split;
    int n_split;
};
DecodePlan plan_decode(int B, int H, int max_rows);
// dense: the call may take the dense 64-head path (its device-planned splits)
size_t decode_workspace_bytes(int B, int H, int d_v, int max_rows, bool dense);
bool attn_shape_supported(int dtype, int d_qk, int d_v);
// pg != nullptr (sparse mode only): swa_kv and comp_kv are the paged SWA and
// C4 pools; the window of sequence b is the swa_len[b] tokens ending at
// pg->pos[b] (clamped to W), rows that are not resident skipped.
hipError_t launch_attn_decode(int dtype, const void* q, const void* swa_kv,
                              const int32_t* swa_len, const void* comp_kv,
                              const int32_t* comp_idx, const int32_t* comp_len, void* out,
                              float* lse, int B, int H, int d_qk, int d_v, int W, int S_max,
                              int k, float scale, void* ws, hipStream_t st,
                              const Paging* pg = nullptr);
// Fused sparse decode after launch_index_lists (one query per sequence):
// finishes the select inside the attention kernel (from the lists, or from
// the score rows when a list is short), writes topk_out ascending, and clears
// the first-digit histogram in the merge kernel.
bool fused_decode_supported(int B, int H, int W, int k);
hipError_t launch_attn_decode_fused(int dtype, const void* q, const void* swa_kv,
                                    const int32_t* swa_len, const void* comp_kv,
                                    const int32_t* comp_len, const int32_t* n_cand, void* sel_ws,
                                    const float* scores, int32_t* topk_out, void* out, float* lse, int B, int H,
                                    int d_qk, int d_v, int W, int S_max, int k, float scale,
                                    void* ws, hipStream_t st, const Paging* pg = nullptr);
hipError_t launch_attn_prefill(int dtype, const void* q, const void* kv, const void* comp_kv,
                               const int32_t* comp_idx, void* out, float* lse, int n_seq,
                               int n_q, int q_start, int T_len, int H, int d_qk, int d_v, int W,
                               int S_max, int k, int m, float scale, hipStream_t st);

}  // namespace hsa
