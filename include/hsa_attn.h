/*
 * hsa_attn.h -- C ABI of the MI355X (gfx950) hybrid sparse-attention library
 * (libhsa_attn.so): block KV compressor, indexer scores + top-k select, and the
 * fused attention over the sliding window plus selected (C4) or all (C128)
 * compressed rows.
 *
 * Pages cited (titles as published; sections named as on the page):
 *   [KD] "DeepSeek-V4: optimizacion de inferencia y RL para modelos con
 *        atencion hibrida y FP4" (kerneldigest.dev)
 *   [LH] "DeepSeek-V4: SGLang va Miles mang den ho tro Day-0 cho suy luan
 *        nhanh va Hoc tang cuong" (lehuy.net)
 *   [NK] "与 SGLang 团队聊 DeepSeek V4:混合注意力的推理与 RL 训练适配"
 *        (nolimitkun.github.io AI-KOL wiki)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *    tensors), row-major and contiguous, 16-byte aligned.  Index, length and
 *    count arrays are int32 in device memory.
 *  - dtype (HSA_F32 or HSA_BF16) is the storage type of every floating-point
 *    tensor argument except `scores` and `lse`, which are always fp32.  All
 *    arithmetic is fp32 (bf16 inputs are widened exactly; bf16 outputs are
 *    rounded to nearest even).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call checks
 *    its arguments on the host, enqueues its kernels on `stream` and returns
 *    without synchronising.  Faults inside a kernel surface at the caller's
 *    next synchronisation.
 *  - Ownership: the caller owns every buffer, including the workspace.  The
 *    library allocates no device memory and keeps no pointer after returning.
 *  - Errors: a rejected call returns a nonzero hsa_status_code and launches
 *    nothing.  HSA_ERR_HIP means a launch failed (hipGetLastError).  No C++
 *    exception crosses this boundary.
 *  - Outputs must not alias inputs, except `scores` in select-only mode.
 *  - Identical inputs give bitwise-identical outputs (no floating-point
 *    atomics; every reduction has a fixed order).
 *  - Re-entrant; calls that share one workspace must not overlap in time.
 *
 * Interface notes: every entry point returns an int holding an
 * hsa_status_code (the ABI does not depend on the size of an enum type);
 * the status-string call is hsa_strerror because the ROCm runtime already
 * exports a symbol named hsa_status_string; hsa_index_topk takes B, the
 * number of key sequences, so that q_seq can be checked against it;
 * hsa_attn_prefill takes the block length m, which sets when a compressed
 * row becomes visible; prefill attention needs no scratch memory, so its
 * workspace size is 0.
 */
#ifndef HSA_ATTN_H
#define HSA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HSA_OK = 0,
    HSA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, bad flag   */
    HSA_ERR_UNSUPPORTED = 2, /* valid but not built (shape/dtype combination) */
    HSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required    */
    HSA_ERR_HIP = 4          /* a HIP launch reported an error                */
} hsa_status_code;

typedef enum { HSA_F32 = 0, HSA_BF16 = 1 } hsa_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char *hsa_strerror(int status);

/* Library version as 10000*major + 100*minor + patch. */
int hsa_version(void);

/*
 * hsa_compress -- block KV compressor.
 *
 * [NK "推理侧优化", Kernel fusion bullet]: the compression chain is
 * read -> add -> softmax -> multiply -> write back, fused into one on-chip
 * pass ([KD "Arquitectura del Sistema"], Flash Compressor).
 * [NK "DeepSeek V4 的新架构"]: an entry is produced once every m = 4 (C4) or
 * m = 128 (C128) tokens.
 *
 *   out[b, i, d] = sum_{j<m} softmax_j(gate[b, m*i+j, d] + bias[j, d]) * x[b, m*i+j, d]
 *
 * for every complete block i < T/m (a trailing partial block is ignored),
 * softmax taken over j separately for each channel d.
 *
 *   x, gate : [B, T, D]   dtype     (x: token latents, gate: per-token gate logits)
 *   bias    : [m, D]      dtype     (per-position-in-block bias, shared by all blocks)
 *   out     : [B, T/m, D] dtype
 *   Sizes   : B >= 1, T >= m, D >= 1 with D*sizeof(dtype) a multiple of 16, 1 <= m <= 1024.
 */
int hsa_compress(int dtype, const void *x, const void *gate, const void *bias, void *out,
                 int32_t B, int32_t T, int32_t D, int32_t m, void *stream);

/*
 * hsa_compress_append -- decode-time compression state, one token per sequence.
 *
 * [NK "DeepSeek V4 的新架构"]: besides the SWA, C4 and C128 pools a decoder
 * keeps, for C4 and for C128, the in-flight tokens of the block not yet
 * compressed; an entry is formed each time 4 (128) tokens have arrived.
 * [KD "Arquitectura del Sistema"]: these compression states live in ring
 * buffers of their own.
 *
 * For each sequence b with p = pos[b] >= 0 (the token's position: the number
 * of tokens of b before it):
 *   1. ring_x[b, p mod m, :] = x_tok[b, :];  ring_g[b, p mod m, :] = g_tok[b, :]
 *   2. if p mod m == m - 1 (the token completes block i = p div m) and i < S_max:
 *        pool[b, i, d] = sum_{j<m} softmax_j(ring_g[b, j, d] + bias[j, d]) * ring_x[b, j, d]
 *      with the ring as left by step 1 -- the hsa_compress entry of that block.
 * A sequence with pos[b] < 0 is left alone (its token is not read).  pos is
 * read only: the caller advances its positions between calls.  Pool rows of
 * blocks not completed by this call are not touched.
 *
 *   x_tok, g_tok   : [B, D]          dtype  (latent and gate logits of the new token)
 *   bias           : [m, D]          dtype
 *   ring_x, ring_g : [B, m, D]       dtype  in/out, owned by the caller, kept between
 *                                           calls; slot j of an open block holds its
 *                                           token at position (block start + j)
 *   pos            : [B]             int32  device memory
 *   pool           : [B, S_max, D]   dtype  out (completed rows only)
 *   Sizes          : B >= 1, D >= 1 with D*sizeof(dtype) a multiple of 16, 1 <= m <= 1024,
 *                    S_max >= 1.  Buffers must not overlap.  All float pointers 16-byte
 *                    aligned (HSA_ERR_INVALID_ARG otherwise).
 */
int hsa_compress_append(int dtype, const void *x_tok, const void *g_tok, const void *bias,
                        void *ring_x, void *ring_g, const int32_t *pos, void *pool, int32_t B,
                        int32_t D, int32_t m, int32_t S_max, void *stream);

/*
 * hsa_compress_overlap, hsa_compress_append_overlap -- the block compressor
 * with overlapping blocks (method variant).
 *
 * [NK "RL 训练侧"]: the C4 compressor carries an "overlap transform" that
 * breaks a naive context-parallel split (a shard must first gather its
 * neighbour's tokens).  The pages do not define it.  Reading: entry i covers
 * its own block and the block before it, tokens m(i-1) .. m(i+1)-1, with a
 * bias of 2m rows (row j for token m(i-1)+j):
 *   out[b, i, d] = sum_j softmax_j(gate[b, t_j, d] + bias[j, d]) * x[b, t_j, d]
 * over the tokens t_j >= 0 (entry 0 has only its own block), for every
 * complete block i.  The decode-time state keeps the last 2m tokens in a ring
 * (slot = position mod 2m); the token that completes block i writes entry i.
 *
 *   hsa_compress_overlap: x, gate [B, T, D]; bias [2m, D]; out [B, T/m, D]
 *   hsa_compress_append_overlap: as hsa_compress_append with bias [2m, D] and
 *       ring_x, ring_g [B, 2m, D]
 *   Sizes: 1 <= m <= 4 (HSA_ERR_UNSUPPORTED above); the rest as the plain calls.
 */
int hsa_compress_overlap(int dtype, const void *x, const void *gate, const void *bias, void *out,
                         int32_t B, int32_t T, int32_t D, int32_t m, void *stream);
int hsa_compress_append_overlap(int dtype, const void *x_tok, const void *g_tok, const void *bias,
                                void *ring_x, void *ring_g, const int32_t *pos, void *pool,
                                int32_t B, int32_t D, int32_t m, int32_t S_max, void *stream);

/*
 * hsa_index_topk -- indexer scores and exact top-k select.
 *
 * [KD "Flujo de Inferencia", step "Indexer (TopK)"]: top-k over the
 * compressed-attention candidates; [KD "Arquitectura del Sistema"]: a
 * radix-select reduction replaces a global sort; [LH "Toi uu hoa suy luan
 * voi ShadowRadix va HiSparse"]: C4 keeps the top 512.
 *
 * Scores (score mode, q_idx != NULL):
 *   scores[q, s] = sum_{h<H_I} sum_{e<d_I} q_idx[q, h, e] * k_idx[q_seq[q], s, e]
 * for s < n_cand[q]; entries s >= n_cand[q] are left unspecified.  The sum
 * over heads is formed first in fp32 (it is linear), so each score is one dot
 * product of length d_I with fp32 accumulation (with 64 or more bf16 queries
 * and a select that fits one workgroup, on MFMA with the folded query carried
 * as three bf16 terms); identical key rows of a sequence give
 * bitwise-identical scores.
 *
 * Select (always): candidates s < n_cand[q]; order = score descending, equal
 * scores (IEEE, -0 == +0) by lower index first; NaN ranks below every
 * number.  The first min(k, n_cand[q]) candidates are written to
 * topk_idx[q, :] in ascending index order, followed by -1 padding up to k.
 *
 *   q_idx    : [Nq, H_I, d_I] dtype, or NULL for select-only mode (then
 *              `scores` is an INPUT holding fp32 scores)
 *   k_idx    : [B, S_max, d_I] dtype (ignored in select-only mode, may be NULL)
 *   q_seq    : [Nq] int32 sequence of each query in [0, B), or NULL (query q
 *              reads sequence q; then Nq <= B).  A query whose entry lies
 *              outside [0, B) has no candidates: its scores are not written
 *              and its topk_idx row is all -1.  Ignored in select-only mode.
 *   n_cand   : [Nq] int32 candidate count per query, clamped to [0, S_max]
 *   scores   : [Nq, S_max] fp32, output (score mode) or input (select-only)
 *   topk_idx : [Nq, k] int32 output
 *   Sizes    : Nq >= 1, B >= 1, H_I >= 1, d_I*sizeof(dtype) in {128, 256, 512},
 *              1 <= S_max <= 4,194,304 (HSA_ERR_UNSUPPORTED above), 1 <= k <= 2048.
 *              flags must be 0 (reserved; the weighted/activated head
 *              combination is hsa_index_topk_weighted).
 *   workspace: device memory of hsa_index_topk_workspace_size(Nq, S_max, k)
 *              bytes.  It must be zero-filled before its first use; every
 *              call that completes leaves it zero-filled again.
 */
size_t hsa_index_topk_workspace_size(int32_t Nq, int32_t S_max, int32_t k);
int hsa_index_topk(int dtype, const void *q_idx, const void *k_idx, int32_t B,
                   const int32_t *q_seq, const int32_t *n_cand, float *scores,
                   int32_t *topk_idx, int32_t Nq, int32_t H_I, int32_t d_I, int32_t S_max,
                   int32_t k, uint32_t flags, void *workspace, size_t workspace_bytes,
                   void *stream);

/*
 * hsa_index_topk_weighted -- hsa_index_topk with weighted, activated indexer
 * heads (method variant).
 *
 * [KD "Arquitectura del Sistema"] names a DSA indexer; [NK "RL 训练侧"]
 * likens the attention indexer to an MoE router, whose gate weighs each of
 * its experts.  The pages define no head combination; this variant takes the
 * DSA indexer as published with DeepSeek-V3.2: each head's dot product passes
 * a ReLU and the heads are summed with per-query weights,
 *   scores[q, s] = sum_{h<H_I} head_w[q, h] * max(0, sum_e q_idx[q, h, e] * k_idx[q_seq[q], s, e])
 * (a NaN dot product contributes 0).  Each head's dot product runs on MFMA
 * (bf16 products, fp32 accumulation); identical key rows of a sequence give
 * bitwise-identical scores.  Select, outputs and workspace: as hsa_index_topk.
 *
 *   head_w : [Nq, H_I] fp32 device memory, 4-byte aligned
 *   Sizes  : dtype HSA_BF16, d_I = 128, H_I a multiple of 16 in [16, 64]
 *            (other shapes HSA_ERR_UNSUPPORTED); the rest as hsa_index_topk.
 */
int hsa_index_topk_weighted(int dtype, const void *q_idx, const float *head_w, const void *k_idx,
                            int32_t B, const int32_t *q_seq, const int32_t *n_cand, float *scores,
                            int32_t *topk_idx, int32_t Nq, int32_t H_I, int32_t d_I,
                            int32_t S_max, int32_t k, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * hsa_attn_decode -- one query token per sequence, one joint softmax over the
 * SWA ring plus the selected (sparse) or all (dense) compressed rows.
 *
 * [LH "Tich hop Kernel va Giai ma suy doan"]: SWA and the extra C4/C128
 * attention in one unified kernel call; [LH "Toi uu hoa suy luan..."]: each
 * layer pairs SWA with C4 (sparse top-512) or C128 (dense).
 *
 * Row set of sequence b:
 *   SWA    : ring slots 0 .. swa_len[b]-1 of swa_kv[b] (swa_len clamped to [0, W])
 *   sparse : comp_idx != NULL: rows comp_kv[b, i] for each listed i with
 *            0 <= i < comp_len[b]; other entries (e.g. -1) are skipped
 *   dense  : comp_idx == NULL: rows comp_kv[b, 0 .. comp_len[b]-1]
 *   (comp_len clamped to [0, S_max])
 * For head h:  l_r = scale * <q[b,h,:], row_r[0:d_qk]>;  lse = log sum_r exp(l_r);
 *              out[b,h,:] = sum_r exp(l_r - lse) * row_r[0:d_v]
 * (the value of a latent row is its first d_v channels).  An empty row set
 * gives out = 0 and lse = -inf.
 *
 *   q        : [B, H, d_qk] dtype
 *   swa_kv   : [B, W, d_qk] dtype ring (token t in slot t mod W)
 *   swa_len  : [B] int32
 *   comp_kv  : [B, S_max, d_qk] dtype (may be NULL when S_max == 0)
 *   comp_idx : [B, k] int32 or NULL
 *   comp_len : [B] int32
 *   out      : [B, H, d_v] dtype;  lse: [B, H] fp32 natural log, or NULL
 *   Sizes    : supported (d_qk, d_v): (128, 128) in fp32 and bf16, (576, 512) in
 *              bf16 (other pairs: HSA_ERR_UNSUPPORTED); 1 <= H <= 1024;
 *              1 <= W; 0 <= S_max; k >= 1 in sparse mode.
 *   workspace: hsa_attn_decode_workspace_size(B, H, d_v, max_rows) bytes with
 *              max_rows = W + (sparse ? k : S_max); contents need no init.
 */
size_t hsa_attn_decode_workspace_size(int32_t B, int32_t H, int32_t d_v, int32_t max_rows);
int hsa_attn_decode(int dtype, const void *q, const void *swa_kv, const int32_t *swa_len,
                    const void *comp_kv, const int32_t *comp_idx, const int32_t *comp_len,
                    void *out, float *lse, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                    int32_t W, int32_t S_max, int32_t k, float scale, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * hsa_decode_sparse -- the C4 decode layer-step in one call: indexer scores,
 * exact top-k select and the SWA + selected-row attention, for one query per
 * sequence (query b reads sequence b).
 *
 * [KD "Flujo de Inferencia", step "Indexer (TopK)"] then [LH "Tich hop Kernel
 * va Giai ma suy doan"]: the indexer picks the top-k C4 entries and one
 * attention call covers the window and those entries.
 *
 * Results equal hsa_index_topk(dtype, q_idx, k_idx, B, NULL, n_cand, scores,
 * topk_idx, B, H_I, d_I, S_max, k, 0, ...) followed by hsa_attn_decode(dtype,
 * q, swa_kv, swa_len, comp_kv, topk_idx, comp_len, out, lse, B, H, d_qk, d_v,
 * W, S_max, k, scale, ...): scores and topk_idx identically; out and lse up
 * to rounding, since the attention may sum the selected rows in another
 * order.  For S_max > 12,288 and S_max >= 32 k (and B, H, W, k that split
 * the rows over at least two workgroups per sequence) the scoring launch
 * also leaves, per block of 256..2048 candidates (one per scoring
 * workgroup), a list of those whose top 11 key bits reach that block's own
 * cut (at most 64..256 of them), and the select is
 * finished inside the attention kernel from those lists and the completed
 * first-digit histogram; the scores of a block whose list cannot hold
 * the top-k's threshold bin are read from the score row instead (the whole
 * row when more than 768 blocks are so), with the same result.  The rows are
 * then taken as the selected-above-threshold list followed by the chosen
 * threshold-bin entries, each in index order except that entries of such
 * blocks follow the others.  Other shapes run the two calls above.
 *
 *   Arguments: as in hsa_index_topk (q_idx must not be NULL) and
 *              hsa_attn_decode (sparse mode), same layouts and limits.
 *   workspace: hsa_decode_sparse_workspace_size(B, H, d_v, W, S_max, k)
 *              bytes, zero-filled before its first use.  Every call that
 *              completes leaves it ready for the next call with the same
 *              (B, H, d_v, W, S_max, k) (its histograms zero; other words it
 *              holds are rewritten before they are read), so a buffer reused
 *              with other sizes must be zero-filled again first.  A call that
 *              returns HSA_ERR_HIP after its scoring launch still enqueues the
 *              clearing of the histograms; a caller that cannot tell whether
 *              the queued work ran (e.g. after a device error) zero-fills the
 *              buffer again before reusing it.
 */
size_t hsa_decode_sparse_workspace_size(int32_t B, int32_t H, int32_t d_v, int32_t W,
                                        int32_t S_max, int32_t k);
int hsa_decode_sparse(int dtype, const void *q_idx, const void *k_idx, const int32_t *n_cand,
                      float *scores, int32_t *topk_idx, const void *q, const void *swa_kv,
                      const int32_t *swa_len, const void *comp_kv, const int32_t *comp_len,
                      void *out, float *lse, int32_t B, int32_t H_I, int32_t d_I, int32_t H,
                      int32_t d_qk, int32_t d_v, int32_t W, int32_t S_max, int32_t k,
                      float scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * hsa_decode_sparse_weighted -- hsa_decode_sparse with the weighted,
 * activated indexer heads of hsa_index_topk_weighted (head_w [B, H_I] fp32):
 * results equal hsa_index_topk_weighted followed by hsa_attn_decode, as for
 * hsa_decode_sparse.  Arguments, limits and workspace: as hsa_decode_sparse,
 * with the shape limits of hsa_index_topk_weighted.
 */
int hsa_decode_sparse_weighted(int dtype, const void *q_idx, const float *head_w,
                               const void *k_idx, const int32_t *n_cand, float *scores,
                               int32_t *topk_idx, const void *q, const void *swa_kv,
                               const int32_t *swa_len, const void *comp_kv,
                               const int32_t *comp_len, void *out, float *lse, int32_t B,
                               int32_t H_I, int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v,
                               int32_t W, int32_t S_max, int32_t k, float scale, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * hsa_decode_step -- the C4 decode layer-step with its compression-state
 * update: the new token of every sequence enters its C4 ring (and completes
 * a block every 4th position), then indexer, select and attention run.
 *
 * [NK "DeepSeek V4 的新架构", five state classes]: SWA and C4 pools plus the
 * in-flight C4 block; [KD "Arquitectura del Sistema", Hierarchical
 * Multi-Stream Overlap]: attention preparation overlapped with other work --
 * here the append runs as extra workgroups of the scoring launch.
 *
 * Results equal hsa_compress_append(dtype, x_tok, g_tok, bias, ring_x,
 * ring_g, pos, comp_kv, B, d_qk, 4, S_max) followed by hsa_decode_sparse(...)
 * with the remaining arguments: a block completed by this call's token is in
 * comp_kv before the attention reads it (whether the attention selects it
 * depends on comp_len and n_cand, which the caller sets).
 *
 *   x_tok, g_tok, bias, ring_x, ring_g, pos: as hsa_compress_append with
 *              m = 4, D = d_qk; bias is [4, d_qk].
 *   comp_kv  : [B, S_max, d_qk], the C4 pool: read by the attention, its
 *              completed-block rows written by the append.
 *   Other arguments, workspace and limits: as hsa_decode_sparse.
 */
int hsa_decode_step(int dtype, const void *x_tok, const void *g_tok, const void *bias,
                    void *ring_x, void *ring_g, const int32_t *pos, const void *q_idx,
                    const void *k_idx, const int32_t *n_cand, float *scores, int32_t *topk_idx,
                    const void *q, const void *swa_kv, const int32_t *swa_len, void *comp_kv,
                    const int32_t *comp_len, void *out, float *lse, int32_t B, int32_t H_I,
                    int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v, int32_t W, int32_t S_max,
                    int32_t k, float scale, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * hsa_decode_step_noalloc -- hsa_decode_step for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.
 *
 * Same arguments, results and limits as hsa_decode_step, without the
 * workspace.  Its scratch is a device array of the library itself,
 * HSA_NOALLOC_SCRATCH_BYTES (32 MiB) on each GPU it runs on, held until the
 * process ends; the call allocates nothing (the array's address on a device
 * is looked up once, on the first call that uses that device).  A call whose
 * need, hsa_decode_sparse_workspace_size(B, H, d_v, W, S_max, k), exceeds the
 * array returns HSA_ERR_WORKSPACE and launches nothing (4 sequences x 262,144
 * C4 entries with top-512 need about 22 MB).  Every call first clears, with
 * fill kernels on `stream`, the words of the array that must start at zero,
 * so calls of any sizes may follow one another.  All calls on one GPU share
 * the array: calls that overlap in time on one GPU (for example on two
 * streams) race and give wrong results; the caller orders them.
 */
#define HSA_NOALLOC_SCRATCH_BYTES (32u << 20)
int hsa_decode_step_noalloc(int dtype, const void *x_tok, const void *g_tok, const void *bias,
                            void *ring_x, void *ring_g, const int32_t *pos, const void *q_idx,
                            const void *k_idx, const int32_t *n_cand, float *scores,
                            int32_t *topk_idx, const void *q, const void *swa_kv,
                            const int32_t *swa_len, void *comp_kv, const int32_t *comp_len,
                            void *out, float *lse, int32_t B, int32_t H_I, int32_t d_I, int32_t H,
                            int32_t d_qk, int32_t d_v, int32_t W, int32_t S_max, int32_t k,
                            float scale, void *stream);

/*
 * Paged pools: the shadows of one decode call.
 *
 * [KD "Arquitectura del Sistema", ShadowRadix]: virtual full-token slots are
 * projected onto the physical KV pools (SWA, C4, C128) through one index map
 * per pool, so each pool's lifetime is its own (SWA pages are freed once the
 * window has passed them while the C4 rows stay); the compression-state rings
 * form a pool of their own, reached from the SWA page index by arithmetic.
 * [NK "推理侧优化", shadow radix cache bullet]: one list of virtual addresses
 * per state class; the part of the SWA no longer used is deleted from physical
 * memory and only its index is kept.
 *
 * A paged pool is an array of physical pages of P rows ([pool_pages, P, D]).
 * Row r of sequence b lives at physical page map[b * map_pages + r / P], row
 * r mod P.  A logical page at or past map_pages, or a map entry outside
 * [0, pool_pages) (for example -1 for a freed page), is not resident: its rows
 * do not exist.  SWA rows are indexed by token position; C4 KV and indexer-key
 * rows by C4 entry.  The compression state of token t (its latent and gate
 * logits, while its block is open) is kept in two state pools shaped like the
 * SWA pool, at the physical row of t in the SWA shadow.
 *
 *   swa_map      : [B, swa_map_pages] int32 device memory
 *   swa_page_rows: P of the SWA and state pools, a power of two in [16, 4096]
 *   swa_pool_pages: physical pages of the SWA pool (and of each state pool)
 *   c4_map       : [B, c4_map_pages] int32, shadow of the C4 KV pool
 *   kI_map       : [B, c4_map_pages] int32, shadow of the indexer-key pool (it
 *                  may be the same array as c4_map)
 *   c4_page_rows : P of the C4 KV and indexer-key pools, a power of two in
 *                  [16, 4096]; c4_map_pages * c4_page_rows >= S_max
 *   c4_pool_pages, kI_pool_pages: physical pages of those two pools
 * The struct is read on the host during the call; the maps it points to are
 * read by the kernels.
 */
typedef struct {
    const int32_t *swa_map;
    int32_t swa_map_pages, swa_page_rows, swa_pool_pages;
    const int32_t *c4_map;
    const int32_t *kI_map;
    int32_t c4_map_pages, c4_page_rows, c4_pool_pages, kI_pool_pages;
} hsa_page_maps;

/*
 * hsa_decode_step_paged -- hsa_decode_step (or, with x_tok == NULL,
 * hsa_decode_sparse) on paged pools: the same computation with every row
 * reached through its shadow.
 *
 * For sequence b with p = pos[b] (the position of its query token; p < 0: no
 * token this step):
 *   1. append (x_tok != NULL, p >= 0): the token's latent and gate logits are
 *      stored at its state rows; if p mod 4 == 3 and i = p div 4 < S_max, C4
 *      entry i = sum_j softmax_j(g_j + bias_j) * x_j over tokens p-3 .. p
 *      (their state rows) is written to row i of the C4 pool.  A token whose
 *      SWA row is not resident is not stored; an entry whose C4 row is not
 *      resident is not written.
 *   2. scores[b, s] for s < n_cand[b]: as hsa_index_topk on indexer-key row s
 *      of the kI shadow; a row that is not resident scores NaN (ranks last).
 *   3. top-k select: as hsa_index_topk.
 *   4. attention: as hsa_attn_decode (sparse mode) over the window -- the
 *      n = clamp(swa_len[b], 0, W) tokens p-n+1 .. p, none when p < 0 -- and
 *      the selected C4 rows i < comp_len[b]; rows that are not resident are
 *      skipped.
 * With identity shadows over pools holding the flat layout (and the window
 * ring holding token p-n+1+j in slot j) the results equal hsa_decode_step's
 * bit for bit: only the row addresses differ.
 *
 *   state_x, state_g : [swa_pool_pages, swa_page_rows, d_qk] dtype in/out
 *                      (ignored when x_tok is NULL)
 *   kI_pool  : [kI_pool_pages, c4_page_rows, d_I] dtype
 *   swa_pool : [swa_pool_pages, swa_page_rows, d_qk] dtype (the caller stores
 *              each token's KV latent at its SWA row before the call)
 *   c4_pool  : [c4_pool_pages, c4_page_rows, d_qk] dtype (in/out)
 *   pos      : [B] int32, required
 *   maps     : host pointer to the shadows (above)
 *   Other arguments, limits and workspace: as hsa_decode_step;
 *   HSA_ERR_INVALID_ARG for a bad map description.
 */
int hsa_decode_step_paged(int dtype, const void *x_tok, const void *g_tok, const void *bias,
                          void *state_x, void *state_g, const int32_t *pos, const void *q_idx,
                          const void *kI_pool, const int32_t *n_cand, float *scores,
                          int32_t *topk_idx, const void *q, const void *swa_pool,
                          const int32_t *swa_len, void *c4_pool, const int32_t *comp_len,
                          const hsa_page_maps *maps, void *out, float *lse, int32_t B,
                          int32_t H_I, int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v,
                          int32_t W, int32_t S_max, int32_t k, float scale, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * hsa_attn_prefill -- a chunk of n_q consecutive query positions per
 * sequence, each with its own causal SWA window and its own compressed rows.
 *
 * [KD "Arquitectura del Sistema"]: long prefill; [NK "DeepSeek V4 的新架构"]:
 * a compressed entry exists only once its whole block has arrived.
 *
 * Query i of sequence b sits at position p = q_start + i.  Its row set:
 *   SWA     : tokens max(0, p-W+1) .. p of kv[b]
 *   visible : compressed rows c < min((p+1)/m, S_max)
 *   sparse  : comp_idx != NULL: the listed visible rows of query (b, i)
 *             (row b*n_q + i of comp_idx; other entries skipped)
 *   dense   : comp_idx == NULL: every visible row
 * with the same joint softmax as hsa_attn_decode.
 *
 *   q        : [n_seq, n_q, H, d_qk] dtype
 *   kv       : [n_seq, T, d_qk] dtype (token latents; q_start + n_q <= T)
 *   comp_kv  : [n_seq, S_max, d_qk] dtype
 *   comp_idx : [n_seq*n_q, k] int32 or NULL
 *   out      : [n_seq, n_q, H, d_v] dtype;  lse: [n_seq*n_q, H] fp32 or NULL
 *   Sizes    : as hsa_attn_decode, plus m >= 1 (4 for C4, 128 for C128).
 *   workspace: hsa_attn_prefill_workspace_size(...) bytes (currently 0).
 */
size_t hsa_attn_prefill_workspace_size(int32_t n_seq, int32_t n_q, int32_t H, int32_t d_v);
int hsa_attn_prefill(int dtype, const void *q, const void *kv, const void *comp_kv,
                     const int32_t *comp_idx, void *out, float *lse, int32_t n_seq,
                     int32_t n_q, int32_t q_start, int32_t T, int32_t H, int32_t d_qk,
                     int32_t d_v, int32_t W, int32_t S_max, int32_t k, int32_t m, float scale,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Kernel timing (diagnostics, not on the hot path).
 *
 * hsa_profile_enable arms the kernel families in family_mask (OR of the
 * HSA_PROF_* values; 0 disarms all).  While a family is armed, each launch of
 * it is bracketed by two hipEventRecord calls on the launch stream (up to
 * 8192 launches between reads; later ones go untimed).  hsa_profile_read
 * waits for every recorded launch, adds their durations to per-family totals
 * and returns the total milliseconds and launch count of `family` (a single
 * HSA_PROF_* value); reset != 0 then clears all totals.  Not meant to be
 * called while kernels are being captured into a graph.
 */
enum {
    HSA_PROF_COMPRESS = 1, /* hsa_compress kernel                           */
    HSA_PROF_SCORE = 2,    /* indexer scoring (+ first-digit histogram)     */
    HSA_PROF_SELECT = 4,   /* top-k select kernels                          */
    HSA_PROF_ATTN = 8,     /* attention kernels (decode split / prefill)    */
    HSA_PROF_MERGE = 16,   /* decode split merge                            */
    HSA_PROF_STREAM = 32   /* hsa_stream_read calibration kernel            */
};
int hsa_profile_enable(unsigned family_mask);
int hsa_profile_read(unsigned family, double *total_ms, long long *launches, int reset);

/*
 * Read-bandwidth calibration (diagnostics, not on the hot path): a plain read
 * of `bytes` bytes at src (device memory, 16-byte aligned) by 512 workgroups
 * of 256 threads, workgroup g streaming the g-th of 512 equal contiguous
 * parts with 16-byte non-temporal loads, eight per lane in flight.  That is
 * the launch shape of the decode scoring kernel at the 1M-context workload
 * (512 workgroups, each reading one contiguous 512 KB key slot), so the
 * scoring kernel's duration can be set against what the memory system
 * delivers to the same shape and byte count.  bytes: a positive multiple of
 * 16 MiB (512 x 256 x 8 x 16 bytes).  sink: 4096 bytes of device memory,
 * 16-byte aligned; the kernel stores to it only if the xor of all loaded
 * words equals one fixed 128-bit value (this keeps the loads), so its
 * contents are unspecified.  Timed as family HSA_PROF_STREAM when armed.
 * Returns HSA_ERR_INVALID_ARG for a null or misaligned pointer or a size
 * that is not such a multiple (nothing is launched).
 */
int hsa_stream_read(const void *src, size_t bytes, void *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HSA_ATTN_H */
