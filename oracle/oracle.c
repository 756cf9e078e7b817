/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the hybrid
 * sparse-attention hot path (compressor, indexer scores, top-k select, decode
 * and prefill attention).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file.  It exists so that the GPU library can be checked against
 * something that a reader can verify against the definitions by eye.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * Rules this file keeps:
 *   - every floating-point sum is accumulated in double (fp64), in the order
 *     the definition writes it; no blocking, no fusion, no reordering;
 *   - inputs are read in the element type the caller stored them in
 *     (fp64, fp32 or bf16 bit patterns) and widened exactly to double;
 *   - OpenMP only splits the loop over independent output units (a block, a
 *     query, a sequence/head pair); it never changes the arithmetic of a unit.
 *
 * Pages cited (titles as published; sections named as on the page):
 *   [KD] "DeepSeek-V4: optimizacion de inferencia y RL para modelos con
 *        atencion hibrida y FP4" (kerneldigest.dev)
 *   [LH] "DeepSeek-V4: SGLang va Miles mang den ho tro Day-0 cho suy luan
 *        nhanh va Hoc tang cuong" (lehuy.net)
 *   [NK] "与 SGLang 团队聊 DeepSeek V4:混合注意力的推理与 RL 训练适配"
 *        (nolimitkun.github.io AI-KOL wiki)
 *
 * The pages fix the data flow but print no formula, shape or code.  The
 * definitions below are the plain readings this project adopts; each reading
 * is listed with its reason in the design notes of the repository.
 *
 * All entry points return 0 on success and a positive code on a bad
 * argument (nothing written in that case).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F64 = 0, OR_F32 = 1, OR_BF16 = 2 };

/* Widen element i of an array stored as fp64, fp32 or bf16 to double.
 * bf16 is the upper half of an IEEE binary32, so the widening is exact. */
static double ld(const void *base, int et, size_t i)
{
    if (et == OR_F64) return ((const double *)base)[i];
    if (et == OR_F32) return (double)((const float *)base)[i];
    {
        uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

static int bad_et(int et) { return et != OR_F64 && et != OR_F32 && et != OR_BF16; }

/* ------------------------------------------------------------------------ *
 * Compressor.
 *
 * [NK "推理侧优化", Kernel fusion bullet] the KV compression is a chain
 * read -> add -> softmax -> multiply -> write back; [NK "DeepSeek V4 的新架构"]
 * one entry is produced once every 4 (C4) or 128 (C128) tokens have arrived;
 * [LH "Cac tinh nang chinh"] ratios 4:1 and 128:1.
 *
 * Reading: for sequence b, complete block i (tokens m*i .. m*i+m-1) and
 * channel d,
 *     z_j  = gate[b, m*i+j, d] + bias[j, d]                (add)
 *     w_j  = exp(z_j) / sum_j' exp(z_j')                   (softmax over j)
 *     out[b, i, d] = sum_j w_j * x[b, m*i+j, d]            (multiply, sum)
 * Blocks do not overlap and start at token 0; a trailing partial block
 * (T not a multiple of m) produces nothing.
 *
 * x, gate: [B, T, D]; bias: [m, D]; out: [B, T/m, D] (fp64).
 * The softmax subtracts the block maximum before exp; that is an exact
 * identity of the softmax and only keeps exp in range.
 * ------------------------------------------------------------------------ */
int oracle_compress(int et, const void *x, const void *gate, const void *bias,
                    double *out, int B, int T, int D, int m)
{
    if (bad_et(et) || !x || !gate || !bias || !out) return 1;
    if (B < 0 || T < 0 || D < 1 || m < 1) return 1;
    const int nblk = T / m;
    long units = (long)B * nblk;
#pragma omp parallel for schedule(static)
    for (long u = 0; u < units; ++u) {
        const int b = (int)(u / nblk), i = (int)(u % nblk);
        double *z = (double *)malloc(sizeof(double) * (size_t)m);
        for (int d = 0; d < D; ++d) {
            for (int j = 0; j < m; ++j) {
                size_t t = (size_t)b * T + (size_t)m * i + j;
                z[j] = ld(gate, et, t * D + d) + ld(bias, et, (size_t)j * D + d);
            }
            double zmax = z[0];
            for (int j = 1; j < m; ++j)
                if (z[j] > zmax) zmax = z[j];
            double den = 0.0;
            for (int j = 0; j < m; ++j) den += exp(z[j] - zmax);
            double c = 0.0;
            for (int j = 0; j < m; ++j) {
                size_t t = (size_t)b * T + (size_t)m * i + j;
                c += (exp(z[j] - zmax) / den) * ld(x, et, t * D + d);
            }
            out[((size_t)b * nblk + i) * D + d] = c;
        }
        free(z);
    }
    return 0;
}

/* ------------------------------------------------------------------------ *
 * Compressor with overlapping blocks (method variant).
 *
 * [NK "RL 训练侧"] says the C4 compressor carries an "overlap transform" that
 * makes a naive context-parallel split wrong (each shard has to gather the
 * tokens of its neighbour first).  The pages do not define it.  Reading: each
 * entry covers its own block and the block before it, 2m tokens with stride
 * m, so an entry at a shard boundary needs the previous shard's last block:
 *     tokens t_j = m*(i-1) + j,  j = 0 .. 2m-1   (only those with t_j >= 0)
 *     z_j  = gate[b, t_j, d] + bias[j, d]         bias: [2m, D]
 *     out[b, i, d] = sum_j softmax_j(z) * x[b, t_j, d]
 * for every complete block i (tokens m*i .. m*i+m-1 present); entry 0 has no
 * earlier block, so its softmax runs over its own m tokens (bias rows m..2m-1).
 * ------------------------------------------------------------------------ */
int oracle_compress_overlap(int et, const void *x, const void *gate, const void *bias,
                            double *out, int B, int T, int D, int m)
{
    if (bad_et(et) || !x || !gate || !bias || !out) return 1;
    if (B < 0 || T < 0 || D < 1 || m < 1) return 1;
    const int nblk = T / m;
    long units = (long)B * nblk;
#pragma omp parallel for schedule(static)
    for (long u = 0; u < units; ++u) {
        const int b = (int)(u / nblk), i = (int)(u % nblk);
        const int j0 = i == 0 ? m : 0;  /* first existing token of the window */
        double *z = (double *)malloc(sizeof(double) * (size_t)(2 * m));
        for (int d = 0; d < D; ++d) {
            double zmax = -INFINITY;
            for (int j = j0; j < 2 * m; ++j) {
                size_t t = (size_t)b * T + (size_t)m * (i - 1) + j;
                z[j] = ld(gate, et, t * D + d) + ld(bias, et, (size_t)j * D + d);
                if (z[j] > zmax) zmax = z[j];
            }
            double den = 0.0;
            for (int j = j0; j < 2 * m; ++j) den += exp(z[j] - zmax);
            double c = 0.0;
            for (int j = j0; j < 2 * m; ++j) {
                size_t t = (size_t)b * T + (size_t)m * (i - 1) + j;
                c += (exp(z[j] - zmax) / den) * ld(x, et, t * D + d);
            }
            out[((size_t)b * nblk + i) * D + d] = c;
        }
        free(z);
    }
    return 0;
}

/* ------------------------------------------------------------------------ *
 * Indexer scores.
 *
 * [KD "Flujo de Inferencia", step "Indexer (TopK)"] the indexer ranks the
 * compressed (C4) candidates; [NK "RL 训练侧"] the attention indexer plays the
 * role of a router.  The pages do not say how its heads combine.
 *
 * Reading: score[q, s] = sum_h sum_e q_idx[q, h, e] * k_idx[seq(q), s, e]
 * for s < n_cand[q] (unit-weight sum over heads, no activation, no scale).
 * Entries s >= n_cand[q] are not candidates and are written as NaN.
 *
 * q_idx: [Nq, H_I, d_I]; k_idx: [B, S_max, d_I]; q_seq: [Nq] sequence of
 * each query (NULL: query q reads sequence q); n_cand: [Nq];
 * scores: [Nq, S_max] (fp64).
 * ------------------------------------------------------------------------ */
int oracle_index_scores(int et, const void *q_idx, const void *k_idx,
                        const int32_t *q_seq, const int32_t *n_cand,
                        double *scores, int Nq, int B, int H_I, int d_I, int S_max)
{
    if (bad_et(et) || !q_idx || !k_idx || !n_cand || !scores) return 1;
    if (Nq < 0 || B < 1 || H_I < 1 || d_I < 1 || S_max < 0) return 1;
    for (int q = 0; q < Nq; ++q) {
        int b = q_seq ? q_seq[q] : q;
        if (b < 0 || b >= B) return 2;
        if (n_cand[q] < 0 || n_cand[q] > S_max) return 2;
    }
    long units = (long)Nq * S_max;
#pragma omp parallel for schedule(static)
    for (long u = 0; u < units; ++u) {
        const int q = (int)(u / (S_max ? S_max : 1)), s = (int)(u % (S_max ? S_max : 1));
        const int b = q_seq ? q_seq[q] : q;
        if (s >= n_cand[q]) {
            scores[u] = NAN;
            continue;
        }
        double acc = 0.0;
        for (int h = 0; h < H_I; ++h)
            for (int e = 0; e < d_I; ++e)
                acc += ld(q_idx, et, ((size_t)q * H_I + h) * d_I + e) *
                       ld(k_idx, et, ((size_t)b * S_max + s) * d_I + e);
        scores[u] = acc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ *
 * Indexer scores, weighted and activated heads (method variant).
 *
 * [KD "Arquitectura del Sistema"] names a DSA indexer; [NK "RL 训练侧"]
 * likens the attention indexer to an MoE router, whose gate weighs each of
 * its experts.  The pages define no head combination.  Reading for this
 * variant (the DSA indexer as published with DeepSeek-V3.2): every head's dot
 * product passes a ReLU, and the heads are summed with per-query weights:
 *   score[q, s] = sum_h w[q, h] * max(0, sum_e q_idx[q, h, e] * k_idx[seq(q), s, e])
 * for s < n_cand[q]; other entries NaN.
 *
 * w: [Nq, H_I] fp32; the rest as oracle_index_scores.
 * ------------------------------------------------------------------------ */
int oracle_index_scores_weighted(int et, const void *q_idx, const float *w,
                                 const void *k_idx, const int32_t *q_seq,
                                 const int32_t *n_cand, double *scores, int Nq, int B,
                                 int H_I, int d_I, int S_max)
{
    if (bad_et(et) || !q_idx || !w || !k_idx || !n_cand || !scores) return 1;
    if (Nq < 0 || B < 1 || H_I < 1 || d_I < 1 || S_max < 0) return 1;
    for (int q = 0; q < Nq; ++q) {
        int b = q_seq ? q_seq[q] : q;
        if (b < 0 || b >= B) return 2;
        if (n_cand[q] < 0 || n_cand[q] > S_max) return 2;
    }
    long units = (long)Nq * S_max;
#pragma omp parallel for schedule(static)
    for (long u = 0; u < units; ++u) {
        const int q = (int)(u / (S_max ? S_max : 1)), s = (int)(u % (S_max ? S_max : 1));
        const int b = q_seq ? q_seq[q] : q;
        if (s >= n_cand[q]) {
            scores[u] = NAN;
            continue;
        }
        double acc = 0.0;
        for (int h = 0; h < H_I; ++h) {
            double dot = 0.0;
            for (int e = 0; e < d_I; ++e)
                dot += ld(q_idx, et, ((size_t)q * H_I + h) * d_I + e) *
                       ld(k_idx, et, ((size_t)b * S_max + s) * d_I + e);
            acc += (double)w[(size_t)q * H_I + h] * (dot > 0.0 ? dot : 0.0);
        }
        scores[u] = acc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ *
 * Top-k selection.
 *
 * [KD "Arquitectura del Sistema"] top-k in the indexer picks candidates
 * (the GPU does it by radix select rather than a global sort); [LH "Toi uu
 * hoa suy luan..."] C4 layers keep the top 512.
 *
 * Reading: candidates are s = 0 .. n-1 with n = min(n_cand[q], S_max).
 * Total order: a before c iff score[a] > score[c], or the scores compare
 * equal (IEEE, so -0 == +0) and a < c.  The selection is the first
 * min(k, n) candidates in that order.  Output: their indices sorted
 * ascending, then -1 up to length k.
 *
 * This is written as the plain definition: sort all candidates by the total
 * order with the C library's qsort, keep the head, sort the kept indices.
 * NaN scores are outside the contract (the order above is not total then).
 *
 * scores: [Nq, S_max] fp32; n_cand: [Nq]; out: [Nq, k] int32.
 * ------------------------------------------------------------------------ */
typedef struct { float s; int32_t i; } or_cand;

static int or_cmp_order(const void *pa, const void *pb)
{
    const or_cand *a = (const or_cand *)pa, *c = (const or_cand *)pb;
    if (a->s > c->s) return -1;
    if (a->s < c->s) return 1;
    return (a->i > c->i) - (a->i < c->i);
}

static int or_cmp_int(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, c = *(const int32_t *)pb;
    return (a > c) - (a < c);
}

int oracle_topk(const float *scores, const int32_t *n_cand, int32_t *out,
                int Nq, int S_max, int k)
{
    if (!scores || !n_cand || !out || Nq < 0 || S_max < 0 || k < 1) return 1;
#pragma omp parallel for schedule(dynamic)
    for (int q = 0; q < Nq; ++q) {
        int n = n_cand[q] < 0 ? 0 : (n_cand[q] > S_max ? S_max : n_cand[q]);
        or_cand *all = (or_cand *)malloc(sizeof(or_cand) * (size_t)(n ? n : 1));
        for (int s = 0; s < n; ++s) {
            all[s].s = scores[(size_t)q * S_max + s];
            all[s].i = s;
        }
        qsort(all, (size_t)n, sizeof(or_cand), or_cmp_order);
        int take = n < k ? n : k;
        int32_t *row = out + (size_t)q * k;
        for (int j = 0; j < take; ++j) row[j] = all[j].i;
        qsort(row, (size_t)take, sizeof(int32_t), or_cmp_int);
        for (int j = take; j < k; ++j) row[j] = -1;
        free(all);
    }
    return 0;
}

/* ------------------------------------------------------------------------ *
 * One joint softmax over a list of latent rows, for one query head.
 *
 * [LH "Tich hop Kernel va Giai ma suy doan"] SWA and the extra (C4 or C128)
 * attention are combined in one kernel call; [LH "Toi uu hoa suy luan..."]
 * each layer pairs SWA with one of C4 (sparse top-512) or C128 (dense).
 *
 * Reading: logit_r = scale * sum_{e < d_qk} q[e] * row_r[e];
 *          lse     = log sum_r exp(logit_r);
 *          o[e]    = sum_r exp(logit_r - lse) * row_r[e]   for e < d_v.
 * The value of a row is its first d_v channels (latent K and V share a row).
 * No row list -> o = 0, lse = -inf.
 * ------------------------------------------------------------------------ */
static void or_softmax_rows(int et, const void *qbase, size_t qoff,
                            const void *const *rbase, const size_t *roff, int nrows,
                            int d_qk, int d_v, double scale, double *o, double *lse)
{
    for (int e = 0; e < d_v; ++e) o[e] = 0.0;
    if (nrows == 0) {
        *lse = -INFINITY;
        return;
    }
    double *logit = (double *)malloc(sizeof(double) * (size_t)nrows);
    for (int r = 0; r < nrows; ++r) {
        double acc = 0.0;
        for (int e = 0; e < d_qk; ++e)
            acc += ld(qbase, et, qoff + e) * ld(rbase[r], et, roff[r] + e);
        logit[r] = scale * acc;
    }
    double mx = logit[0];
    for (int r = 1; r < nrows; ++r)
        if (logit[r] > mx) mx = logit[r];
    double z = 0.0;
    for (int r = 0; r < nrows; ++r) z += exp(logit[r] - mx);
    const double l = mx + log(z);
    for (int r = 0; r < nrows; ++r) {
        const double w = exp(logit[r] - l);
        for (int e = 0; e < d_v; ++e) o[e] += w * ld(rbase[r], et, roff[r] + e);
    }
    *lse = l;
    free(logit);
}

/* ------------------------------------------------------------------------ *
 * Decode attention: one query token per sequence.
 *
 * [KD "Flujo de Inferencia", step "Hybrid Attention Kernel"] SWA plus the
 * extra compressed attention in fused kernels; [NK "DeepSeek V4 的新架构"]
 * SWA sees only the most recent tokens, C4 attends to the top-k chosen
 * entries, C128 attends to all of its entries.
 *
 * Row list of sequence b:
 *   SWA   : ring slots 0 .. swa_len[b]-1 of swa_kv[b] (swa_len clamped to
 *           [0, W]); the ring holds token t in slot t mod W, so the valid
 *           slots are exactly these and their order does not matter;
 *   sparse: comp_idx != NULL -> rows comp_kv[b, i] for each listed i with
 *           0 <= i < comp_len[b] (others, including -1 padding, skipped;
 *           no de-duplication);
 *   dense : comp_idx == NULL -> rows comp_kv[b, 0 .. comp_len[b]-1].
 * comp_len is clamped to [0, S_max].
 *
 * q: [B, H, d_qk]; swa_kv: [B, W, d_qk]; comp_kv: [B, S_max, d_qk];
 * comp_idx: [B, k]; out: [B, H, d_v] fp64; lse: [B, H] fp64.
 * ------------------------------------------------------------------------ */
int oracle_attn_decode(int et, const void *q, const void *swa_kv, const int32_t *swa_len,
                       const void *comp_kv, const int32_t *comp_idx, const int32_t *comp_len,
                       double *out, double *lse, int B, int H, int d_qk, int d_v, int W,
                       int S_max, int k, double scale)
{
    if (bad_et(et) || !q || !swa_kv || !swa_len || !comp_len || !out || !lse) return 1;
    if (S_max > 0 && !comp_kv) return 1;
    if (B < 0 || H < 1 || d_qk < 1 || d_v < 1 || d_v > d_qk || W < 1 || S_max < 0) return 1;
    if (comp_idx && k < 1) return 1;
    long units = (long)B * H;
#pragma omp parallel for schedule(dynamic)
    for (long u = 0; u < units; ++u) {
        const int b = (int)(u / H), h = (int)(u % H);
        int ns = swa_len[b] < 0 ? 0 : (swa_len[b] > W ? W : swa_len[b]);
        int nc = comp_len[b] < 0 ? 0 : (comp_len[b] > S_max ? S_max : comp_len[b]);
        int cap = ns + (comp_idx ? k : nc);
        const void **rb = (const void **)malloc(sizeof(void *) * (size_t)(cap ? cap : 1));
        size_t *ro = (size_t *)malloc(sizeof(size_t) * (size_t)(cap ? cap : 1));
        int n = 0;
        for (int s = 0; s < ns; ++s) {
            rb[n] = swa_kv;
            ro[n++] = ((size_t)b * W + s) * d_qk;
        }
        if (comp_idx) {
            for (int j = 0; j < k; ++j) {
                int i = comp_idx[(size_t)b * k + j];
                if (i < 0 || i >= nc) continue;
                rb[n] = comp_kv;
                ro[n++] = ((size_t)b * S_max + i) * d_qk;
            }
        } else {
            for (int i = 0; i < nc; ++i) {
                rb[n] = comp_kv;
                ro[n++] = ((size_t)b * S_max + i) * d_qk;
            }
        }
        or_softmax_rows(et, q, ((size_t)b * H + h) * d_qk, rb, ro, n, d_qk, d_v, scale,
                        out + ((size_t)b * H + h) * d_v, lse + (size_t)b * H + h);
        free(rb);
        free(ro);
    }
    return 0;
}

/* ------------------------------------------------------------------------ *
 * Prefill attention: a chunk of consecutive query positions per sequence.
 *
 * [KD "Arquitectura del Sistema"] long prefill is the context-parallel case;
 * [NK "DeepSeek V4 的新架构"] a compressed entry exists only once its whole
 * block of m tokens has arrived.
 *
 * Query i of sequence b sits at position p = q_start + i.  Its row list:
 *   SWA   : tokens max(0, p-W+1) .. p of kv[b] (causal window, query token
 *           included);
 *   visible compressed rows: i_c < V(p) = min((p+1)/m, S_max) (integer
 *           division: block i_c is complete iff m*i_c + m-1 <= p);
 *   sparse: comp_idx != NULL -> the listed rows of query (b, i) that are
 *           visible (others, including -1, skipped);
 *   dense : comp_idx == NULL -> every visible row.
 * Only the queries listed in sel (flat ids b*n_q + i) are computed; the
 * results go to out[j] / lse[j] for the j-th listed id.
 *
 * q: [n_seq, n_q, H, d_qk]; kv: [n_seq, T, d_qk]; comp_kv: [n_seq, S_max, d_qk];
 * comp_idx: [n_seq*n_q, k]; out: [n_sel, H, d_v] fp64; lse: [n_sel, H] fp64.
 * ------------------------------------------------------------------------ */
int oracle_attn_prefill(int et, const void *q, const void *kv, const void *comp_kv,
                        const int32_t *comp_idx, double *out, double *lse, int n_seq,
                        int n_q, int q_start, int T, int H, int d_qk, int d_v, int W,
                        int S_max, int k, int m, double scale, const int32_t *sel, int n_sel)
{
    if (bad_et(et) || !q || !kv || !out || !lse || !sel) return 1;
    if (S_max > 0 && !comp_kv) return 1;
    if (n_seq < 0 || n_q < 0 || q_start < 0 || q_start + n_q > T || H < 1 || d_qk < 1 ||
        d_v < 1 || d_v > d_qk || W < 1 || S_max < 0 || m < 1 || n_sel < 0)
        return 1;
    if (comp_idx && k < 1) return 1;
    for (int j = 0; j < n_sel; ++j)
        if (sel[j] < 0 || sel[j] >= n_seq * n_q) return 2;
    long units = (long)n_sel * H;
#pragma omp parallel for schedule(dynamic)
    for (long u = 0; u < units; ++u) {
        const int j = (int)(u / H), h = (int)(u % H);
        const int id = sel[j], b = id / n_q, i = id % n_q, p = q_start + i;
        const int t0 = p - W + 1 < 0 ? 0 : p - W + 1;
        int vis = (p + 1) / m;
        if (vis > S_max) vis = S_max;
        int cap = (p - t0 + 1) + (comp_idx ? k : vis);
        const void **rb = (const void **)malloc(sizeof(void *) * (size_t)cap);
        size_t *ro = (size_t *)malloc(sizeof(size_t) * (size_t)cap);
        int n = 0;
        for (int t = t0; t <= p; ++t) {
            rb[n] = kv;
            ro[n++] = ((size_t)b * T + t) * d_qk;
        }
        if (comp_idx) {
            for (int c = 0; c < k; ++c) {
                int r = comp_idx[(size_t)id * k + c];
                if (r < 0 || r >= vis) continue;
                rb[n] = comp_kv;
                ro[n++] = ((size_t)b * S_max + r) * d_qk;
            }
        } else {
            for (int r = 0; r < vis; ++r) {
                rb[n] = comp_kv;
                ro[n++] = ((size_t)b * S_max + r) * d_qk;
            }
        }
        or_softmax_rows(et, q, (((size_t)b * n_q + i) * H + h) * d_qk, rb, ro, n, d_qk,
                        d_v, scale, out + ((size_t)j * H + h) * d_v, lse + (size_t)j * H + h);
        free(rb);
        free(ro);
    }
    return 0;
}
