// index_topk.hip -- indexer scores and exact radix-select top-k for gfx950.
//
// [KD "Flujo de Inferencia", step "Indexer (TopK)"]: the indexer picks the
// top-k compressed (C4) candidates; [KD "Arquitectura del Sistema"]: a
// radix-select reduction instead of a global sort; [NK "推理侧优化",
// Lightning topk bullet]: at 1M-token contexts the selection dominates if it
// is a sort, so it has to be parallel.
//
// Scores.  The score of candidate s for query q is the sum over indexer heads
// of <q_idx[q,h,:], k_idx[s,:]>.  The sum over heads is linear, so each
// workgroup folds the heads once (qsum[e] = sum_h q_idx[q,h,e], fixed order)
// and a score is one fp32 dot product of length d_I.  That turns the
// 64-head contraction into a streaming matrix-vector product: every key row
// is read once with coalesced 16-byte loads (LPR lanes per row) and reduced
// with a fixed lane butterfly, so equal rows give bitwise-equal scores.
//
// Select.  Keys are the order-preserving u32 image of the fp32 scores
// (score_key).  The wanted set is the first min(k, n) candidates under
// (key desc, index asc); it is determined by the k-th key T and by how many
// candidates equal to T are taken (the lowest indices).
//  - n <= kRowSelectCap: one workgroup per query keeps all keys in LDS, runs
//    three LDS histogram passes (11, 11, 10 bits) to find T, then writes the
//    selection in ascending index order with two workgroup prefix sums.
//  - larger n: the scoring kernel also builds the 2048-bin histogram of the
//    top 11 key bits per query (LDS histogram, integer atomics to global).
//    A filter kernel then sends, per segment of 4096 candidates, every
//    candidate above the threshold bin to the segment's "selected" run and
//    every candidate inside it to its short-list run, both in index order
//    at fixed places of the segment (no reservation atomics).  A final
//    kernel, one workgroup per query, gathers the runs, finishes the select
//    on the short list in LDS (two more histogram passes, plus passes over
//    indices when a tie straddles rank k), merges the two ascending lists
//    into the output and zeroes what the call wrote in the workspace.  The
//    kernel boundaries order every hand-off, so no workgroup waits on or
//    fences for another.
#include "compress_append.hpp"
#include "hsa_common.hpp"
#include "hsa_internal.hpp"
#include "select.hpp"

#include <type_traits>

namespace hsa {

namespace {

using namespace sel;

constexpr int kThreads = kSelThreads;
constexpr int kNW = kThreads / kWave;
constexpr int kScoreRowsMulti = 2048;

// The second-digit histogram of a query is built by the filter kernel of the
// same call; the workgroups of the kernel before it (scoring, or the
// select-only histogram) clear it, each its slice, so no later kernel has to.
__device__ inline void clear_hist2_slice(uint8_t* ws, int q, int S_max, int k) {
    const int per = ceil_div(kBins, (int)gridDim.x);
    uint32_t* h2 = ws_of(ws, q, S_max, k).hist2;
    for (int j = (int)threadIdx.x; j < per; j += kThreads) {  // every caller runs kThreads threads
        const int i = (int)blockIdx.x * per + j;
        if (i < kBins) h2[i] = 0;
    }
}

// ---- scoring ---------------------------------------------------------------
// Lanes of a wave are split into row groups of LPR lanes; lane `sub` of a row
// group reads the sub-th 16-byte chunk of a key row.  A lane keeps U = 8 rows
// per batch (one per load), forms its 8 partial dot products, and the row
// group reduces them with a reduce-scatter butterfly: three halving steps
// over the top three lane bits (8 -> 4 -> 2 -> 1 rows per lane) and plain
// xor steps over the remaining bits.  Every row's sum has the same tree over
// the LPR chunk partials (fp add is commutative), so equal rows give equal
// scores wherever they sit.
template <int LPR>
__device__ __forceinline__ float reduce_scatter8(float (&v)[8], int sub) {
    constexpr int LB = (LPR == 8) ? 3 : (LPR == 16 ? 4 : 5);  // log2(LPR)
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "rows are 128, 256 or 512 bytes");
    // step over bit LB-1: 8 -> 4
    {
        const int m = 1 << (LB - 1);
        const bool hi = (sub & m) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float send = hi ? v[i] : v[i + 4];
            const float keep = hi ? v[i + 4] : v[i];
            v[i] = keep + __shfl_xor(send, m, kWave);
        }
    }
    {
        const int m = 1 << (LB - 2);
        const bool hi = (sub & m) != 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float send = hi ? v[i] : v[i + 2];
            const float keep = hi ? v[i + 2] : v[i];
            v[i] = keep + __shfl_xor(send, m, kWave);
        }
    }
    float r;
    {
        const int m = 1 << (LB - 3);
        const bool hi = (sub & m) != 0;
        const float send = hi ? v[0] : v[1];
        const float keep = hi ? v[1] : v[0];
        r = keep + __shfl_xor(send, m, kWave);
    }
#pragma unroll
    for (int b = LB - 4; b >= 0; --b) r += __shfl_xor(r, 1 << b, kWave);
    return r;  // the row (sub >> (LB - 3)) of the batch
}

// SEL: 0 scores only; 1 also the first-digit histogram; 2 (2048-row slots)
// and 3 (256 .. 2048-row slots) also the workgroup's candidate list
// (select.hpp), and grid rows y >= Nq carry the
// decode-time C4 append of `job` (one (sequence, 256-chunk span) per
// workgroup; it touches only the append's own buffers).
// PAGED: k_idx is the paged indexer-key pool of shadow kp (row s of sequence
// b at its physical row; a row that is not resident scores NaN).
// WM = 1: weighted, activated heads, score = sum_h head_w[q, h] * max(0, q_h . k)
// (bf16, 128-wide keys, H_I a multiple of 16 up to 64): per batch each wave
// takes two blocks of 16 key rows as MFMA A operands (lane: row lane % 16,
// channels 8 (lane / 16) + 32 ks), the query's heads are the B operands
// (16 per MFMA column block) held in registers, and v_mfma_f32_16x16x32_bf16
// gives each lane 4 rows x 1 head; the weighted ReLU terms of a lane's heads
// are added in head-block order, then across the 16 lanes of the row group by
// a xor butterfly (quad swaps, half-row and row mirrors), which hands every
// lane the same sum: every row gets one fixed tree, so equal rows score the same.
constexpr int kScorePagesMax = 8192 / 16 + 1;  // logical pages a scoring workgroup spans
constexpr int kWeightedMaxHeads = 64;

// sum over the 16 lanes of a DPP row (xor 1, xor 2, half-row mirror, row
// mirror): every lane of the row receives the bitwise-same value
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false));
    return v;
}

template <typename T, int LPR, int SEL, bool PAGED, int WM>
__global__ __launch_bounds__(kThreads) void score_kernel(
    const T* __restrict__ q_idx, const T* __restrict__ k_idx, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ n_cand, float* __restrict__ scores, uint8_t* __restrict__ ws,
    int B, int H_I, int S_max, int k, int rows_per_wg, int Nq, AppendJob job, PoolMap kp,
    const float* __restrict__ head_w) {
    static_assert(WM == 0 || (LPR == 16 && sizeof(T) == 2), "weighted heads: bf16, 128-wide keys");
    constexpr bool HIST = SEL >= 1;
    constexpr bool LIST = SEL >= 2;
    // log2 of the rows per list slot: fixed at 2048 for SEL 2 (so that the
    // large-pool path compiles with constant slot arithmetic), any of 256 ..
    // 2048 for SEL 3
    const int rows_lg = SEL == 3 ? (int)__builtin_ctz((unsigned)rows_per_wg) : 11;
    constexpr int V = Elem<T>::kPer16B;
    constexpr int DI = LPR * V;            // indexer width
    constexpr int RPL = kWave / LPR;       // rows covered by one wave-wide load
    constexpr int U = 8;                   // loads per lane per batch
    constexpr int RPU = RPL * kNW;         // rows covered by one workgroup-wide load
    constexpr int RPB = RPU * U;           // rows per workgroup batch
    constexpr int NG = kThreads / LPR;     // partial head sums per channel
    constexpr int LB = (LPR == 8) ? 3 : (LPR == 16 ? 4 : 5);
    __shared__ float qpart[WM ? 1 : NG][WM ? 1 : DI];
    __shared__ float qsum[WM ? 1 : DI];
    __shared__ uint32_t hist[HIST ? kBins : 1];
    __shared__ uint32_t scan_tmp[LIST ? kNW + 2 : 1];
    __shared__ uint32_t cut_res;
    __shared__ int spg[PAGED ? kScorePagesMax : 1];  // physical page of each logical page, -1 absent
    extern __shared__ __align__(16) float stage[];  // this workgroup's scores (rows_per_wg)

    if constexpr (LIST) {
        if ((int)blockIdx.y >= Nq) {
            const int spans = (job.D / Elem<T>::kPer16B + kThreads - 1) / kThreads;
            const int j = ((int)blockIdx.y - Nq) * (int)gridDim.x + (int)blockIdx.x;
            if (j < job.B * spans) {
                if (job.swa.map)  // uniform: the paged state pools
                    append_short_chunk_paged<T, 4>(
                        static_cast<const T*>(job.x_tok), static_cast<const T*>(job.g_tok),
                        static_cast<const T*>(job.bias), static_cast<T*>(job.ring_x),
                        static_cast<T*>(job.ring_g), job.pos, static_cast<T*>(job.pool), job.D,
                        job.S_max, job.swa, job.c4, j / spans, (j % spans) * kThreads + threadIdx.x);
                else
                    append_short_chunk<T, 4>(
                        static_cast<const T*>(job.x_tok), static_cast<const T*>(job.g_tok),
                        static_cast<const T*>(job.bias), static_cast<T*>(job.ring_x),
                        static_cast<T*>(job.ring_g), job.pos, static_cast<T*>(job.pool), job.D,
                        job.S_max, j / spans, (j % spans) * kThreads + threadIdx.x);
            }
            return;
        }
    }
    const int q = blockIdx.y;
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int sub = lane % LPR, rs = lane / LPR;
    const int bseq_raw = q_seq ? q_seq[q] : q;
    const int bseq = (bseq_raw < 0 || bseq_raw >= B) ? 0 : bseq_raw;
    // the lane's first channel of a key row: chunk `sub` (unit weights) or the
    // MFMA A-operand chunk 8 (lane / 16) (+ 32 ks per load, weighted)
    const int lane_e = WM ? 8 * (lane >> 4) : sub * V;
    const T* kbase = k_idx + (size_t)bseq * S_max * DI + (size_t)lane_e;
    const int r0 = blockIdx.x * rows_per_wg;
    const int r1m = min(S_max, r0 + rows_per_wg);  // rows that are valid memory
    // paged: the shadow entries of this workgroup's rows (logical pages j0 ..)
    const int j0 = PAGED ? r0 >> kp.lg : 0;
    if constexpr (PAGED) {
        const int np = ((r1m - 1) >> kp.lg) - j0 + 1;
        for (int i = tid; i < np; i += kThreads) {
            const int j = j0 + i;
            const int pg = j < kp.pages ? kp.map[(size_t)bseq * kp.pages + j] : -1;
            spg[i] = (pg >= 0 && pg < kp.pool_pages) ? pg : -1;
        }
        __syncthreads();
    }
    // this lane's chunk of key row r (r < r1m); a row that is not resident reads
    // physical row 0 (its score is replaced by NaN)
    auto krow = [&](int r) -> const T* {
        if constexpr (PAGED) {
            const int pg = spg[(r >> kp.lg) - j0];
            const size_t pr = pg < 0 ? 0 : (((size_t)pg << kp.lg) | (size_t)(r & ((1 << kp.lg) - 1)));
            return k_idx + pr * DI + (size_t)lane_e;
        } else {
            return kbase + (size_t)r * DI;
        }
    };

    // Key rows are read once: nontemporal loads keep them from displacing
    // reusable lines.  Load u of batch bi: unit weights, the 256 lanes read RPU
    // consecutive rows (4 KB), wave w the w-th quarter; weighted, wave w reads
    // rows 32 w .. 32 w + 31 of the batch, load u the 16-row block u / 4 at
    // channels 32 (u % 4) + 8 (lane / 16).  Full batches need no clamp.
    auto urow = [&](int u) {
        return WM ? w * 32 + 16 * (u >> 2) + (lane & 15) : u * RPU + w * RPL + rs;
    };
    auto uoff = [&](int u) { return WM ? 32 * (u & 3) : 0; };
    // (weighted: a load covers half of each of its 16 rows' 128-byte lines and
    // the next load the other half, so these loads keep their lines in L2:
    // plain loads, the second half a hit)
    auto kload = [](const T* p) {
        return WM ? *reinterpret_cast<const u32x4*>(p)
                  : __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    };
    auto load_batch = [&](u32x4 (&buf)[U], int bi, int rlim) {
        const int rb = r0 + bi * RPB;
        if (rb + RPB <= rlim) {
#pragma unroll
            for (int u = 0; u < U; ++u) buf[u] = kload(krow(rb + urow(u)) + uoff(u));
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = rb + urow(u);
                const int rc = r < rlim ? r : rlim - 1;  // stay inside the valid rows
                buf[u] = kload(krow(rc) + uoff(u));
            }
        }
    };

    // The head fold's first round of q_idx loads goes out first and the first
    // key batch right after, so that waiting for the fold (loads retire in
    // issue order) leaves the key batch in flight.  Loads are unconditional
    // (clamped index, value zeroed after) so that none waits on another.
    const int nchunks = H_I * LPR;
    const T* qb = q_idx + (size_t)q * H_I * DI;
    u32x4 f4[4];
    // weighted: the B operands (head 16 hb + lane % 16, channels 32 ks +
    // 8 (lane / 16)) and the lane's head weights; head blocks past H_I are
    // loaded from head block 0 and skipped
    constexpr int NHB = WM ? kWeightedMaxHeads / 16 : 1;
    bf16x8 qf[NHB][4];
    float wl[NHB];
    const int nhb = WM ? H_I / 16 : 0;
    if constexpr (WM == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = tid + j * kThreads;
            f4[j] = *reinterpret_cast<const u32x4*>(qb + (size_t)min(c, nchunks - 1) * V);
        }
    } else {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            const int h = (hb < nhb ? 16 * hb : 0) + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qf[hb][ks] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(qb + (size_t)h * DI + 32 * ks + 8 * (lane >> 4)));
            wl[hb] = head_w[(size_t)q * H_I + h];
        }
    }
    u32x4 cur[U];
    {   // the first batch in the clamped form: no branch, so the loads above
        // keep an exact place in the in-order count
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + urow(u);
            const int rc = r < r1m ? r : r1m - 1;
            cur[u] = kload(krow(rc) + uoff(u));
        }
    }
    if constexpr (HIST) clear_hist2_slice(ws, q, S_max, k);

    int n = clamp_n(n_cand, q, S_max);
    if (bseq_raw < 0 || bseq_raw >= B) n = 0;
    const int r1 = min(n, r0 + rows_per_wg);
    if (r0 >= r1) {  // uniform over the workgroup: no candidate rows here
        __builtin_amdgcn_s_waitcnt(0);  // retire the speculative loads first
        if constexpr (LIST) {  // an empty list that left nothing out, every call
            if (tid == 0) lists_of(ws_of(ws, q, S_max, k), S_max, k, rows_lg).hdr[blockIdx.x] = 0u;
        }
        return;
    }
    const int nb = ceil_div(r1 - r0, RPB);

    // fold the heads: thread t sums the chunks t, t+256, ... of q_idx[q] (all
    // loads issued together), then the NG partials of each channel are added
    // in a fixed order
    if constexpr (WM != 0) {
        if constexpr (HIST)
            for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
        __syncthreads();
    } else {
        const int ec = tid % LPR, grp = tid / LPR;
        float part[V];
#pragma unroll
        for (int e = 0; e < V; ++e) part[e] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 t = (tid + j * kThreads < nchunks) ? f4[j] : u32x4{0u, 0u, 0u, 0u};
            float f[V];
            Elem<T>::unpack(t, f);
#pragma unroll
            for (int e = 0; e < V; ++e) part[e] += f[e];
        }
        if (nchunks > 4 * kThreads) {  // uniform; not taken at 64 heads x 128
            for (int c0 = tid + 4 * kThreads; c0 < nchunks; c0 += 4 * kThreads) {
                u32x4 t4[4];
    #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = c0 + j * kThreads;
                    t4[j] = c < nchunks ? *reinterpret_cast<const u32x4*>(qb + (size_t)c * V)
                                        : u32x4{0u, 0u, 0u, 0u};
                }
    #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float f[V];
                    Elem<T>::unpack(t4[j], f);
    #pragma unroll
                    for (int e = 0; e < V; ++e) part[e] += f[e];
                }
            }
        }
#pragma unroll
        for (int e = 0; e < V; ++e) qpart[grp][ec * V + e] = part[e];
        if constexpr (HIST)
            for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
        __syncthreads();
        for (int e = tid; e < DI; e += kThreads) {
            float acc = 0.f;
            for (int g = 0; g < NG; ++g) acc += qpart[g][e];
            qsum[e] = acc;
        }
        __syncthreads();
    }
    float qv[V];
    if constexpr (WM == 0) {
#pragma unroll
        for (int e = 0; e < V; ++e) qv[e] = qsum[sub * V + e];
    }
    const int my_u = sub >> (LB - 3);

    for (int bi = 0; bi < nb; ++bi) {
        u32x4 nxt[U];
        if (bi + 1 < nb) load_batch(nxt, bi + 1, r1);  // next batch in flight while this one is reduced
        float sc;
        int r;
        bool writer;
        if constexpr (WM == 0) {
            float d[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float kv[V];
                Elem<T>::unpack(cur[u], kv);
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < V; ++e) acc = fmaf(qv[e], kv[e], acc);
                d[u] = acc;
            }
            sc = reduce_scatter8<LPR>(d, sub);
            r = r0 + bi * RPB + my_u * RPU + w * RPL + rs;
            writer = (sub & ((1 << (LB - 3)) - 1)) == 0;
        } else {
            f32x4 tot[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x4 sj = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int hb = 0; hb < NHB; ++hb) {
                    if (hb < nhb) {  // uniform
                        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks)
                            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, cur[4 * j + ks]), qf[hb][ks], c, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < 4; ++i) sj[i] = fmaf(wl[hb], fmaxf(c[i], 0.f), sj[i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sj[i] = row16_sum(sj[i]);
                tot[j] = sj;
            }
            // lane t < 8 of row group g writes row 16 (t / 4) + 4 g + t % 4 of the wave's 32
            const int t = lane & 15, i = t & 3;
            const f32x4 tj = (t >> 2) & 1 ? tot[1] : tot[0];
            sc = i == 0 ? tj[0] : (i == 1 ? tj[1] : (i == 2 ? tj[2] : tj[3]));
            r = r0 + bi * RPB + w * 32 + 16 * ((t >> 2) & 1) + 4 * (lane >> 4) + i;
            writer = t < 8;
        }
        if constexpr (PAGED) {
            if (r < r1 && spg[(r >> kp.lg) - j0] < 0) sc = __builtin_nanf("");
        }
        if (writer && r < r1) {
            stage[r - r0] = sc;
            if constexpr (HIST) atomicAdd(&hist[score_key(sc) >> 21], 1u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
    __syncthreads();
    const int nr = r1 - r0;
    if constexpr (HIST) {
        QWs W = ws_of(ws, q, S_max, k);
        for (int i = tid; i < kBins; i += kThreads) {
            const uint32_t c = hist[i];
            if (c) atomicAdd(&W.hist[i], c);
        }
    }
    if constexpr (LIST) {
        // the cut a: the lowest bin with at most `cap` of this workgroup's
        // candidates at or above it (thread t sums the 8 bins of group
        // 255 - t, so the scan runs from the top bin down)
        const Lists Ls = lists_of(ws_of(ws, q, S_max, k), S_max, k, rows_lg);
        const uint32_t cap = (uint32_t)Ls.cap;
        const int grp = kThreads - 1 - tid;
        uint32_t hb[8], s8 = 0;
#pragma unroll
        for (int h4 = 0; h4 < 2; ++h4) {  // 16-byte LDS reads
            const u32x4 v = reinterpret_cast<const u32x4*>(hist)[2 * grp + h4];
#pragma unroll
            for (int c = 0; c < 4; ++c) { hb[4 * h4 + c] = v[c]; s8 += v[c]; }
        }
        if (tid == 0) cut_res = 0;
        uint32_t all;
        const uint32_t above = block_excl_scan<kThreads>(s8, scan_tmp, &all);
        if (above <= cap && above + s8 > cap) {
            uint32_t cum = above;
#pragma unroll
            for (int j = 7; j >= 0; --j) {
                if (cum + hb[j] > cap) { cut_res = (uint32_t)(grp * 8 + j + 1); break; }
                cum += hb[j];
            }
        }
        __syncthreads();
        const uint32_t a = cut_res;
        // rows rpt t .. rpt t + rpt - 1 of the workgroup (rpt = 1, 2, 4 or 8
        // rows per thread) at or above the cut, in index order
        const int rpt = (1 << rows_lg) / kThreads;
        uint32_t kk[8], m = 0;
        if (rpt == 8) {
            const f32x4 s0 = reinterpret_cast<const f32x4*>(stage)[2 * tid];
            const f32x4 s1 = reinterpret_cast<const f32x4*>(stage)[2 * tid + 1];
#pragma unroll
            for (int c = 0; c < 4; ++c) { kk[c] = score_key(s0[c]); kk[4 + c] = score_key(s1[c]); }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) kk[j] = score_key(stage[min(tid * rpt + j, rows_per_wg - 1)]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = tid * rpt + j;
            if (j < rpt && i < nr && (kk[j] >> 21) >= a) m |= 1u << j;
        }
        uint32_t cnt;
        uint32_t pos = block_excl_scan<kThreads>((uint32_t)__popc(m), scan_tmp, &cnt);
        const uint32_t e0 = (uint32_t)blockIdx.x * cap;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if ((m >> j) & 1u) {
                const uint32_t at = list_pos(e0 + pos);
                Ls.key[at] = kk[j];
                Ls.idx[at] = (uint32_t)(r0 + tid * rpt + j);
                ++pos;
            }
        }
        if (tid == 0) Ls.hdr[blockIdx.x] = cnt | (a << 16);
    }
    // the workgroup's scores leave in one coalesced burst
    float* srow = scores + (size_t)q * S_max + r0;
    for (int i = tid * 4; i < nr; i += kThreads * 4) {
        if (i + 4 <= nr && (((uintptr_t)(srow + i)) & 15u) == 0) {
            __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(stage + i),
                                        reinterpret_cast<f32x4*>(srow + i));
        } else {
            for (int j = i; j < min(nr, i + 4); ++j) srow[j] = stage[j];
        }
    }
}

// top-11-bit histogram of given scores (select-only mode, multi-workgroup path)
__global__ __launch_bounds__(kThreads) void hist_kernel(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ n_cand,
                                                        const int32_t* __restrict__ q_seq, int B,
                                                        uint8_t* __restrict__ ws, int S_max, int k,
                                                        int chunk) {
    __shared__ uint32_t hist[kBins];
    const int q = blockIdx.y, tid = threadIdx.x;
    clear_hist2_slice(ws, q, S_max, k);
    const int n = query_n(n_cand, q_seq, B, q, S_max);
    const int s0 = blockIdx.x * chunk, s1 = min(n, s0 + chunk);
    if (s0 >= s1) return;
    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int s = s0 + tid; s < s1; s += kThreads)
        atomicAdd(&hist[score_key(scores[(size_t)q * S_max + s]) >> 21], 1u);
    __syncthreads();
    QWs W = ws_of(ws, q, S_max, k);
    for (int i = tid; i < kBins; i += kThreads) {
        const uint32_t c = hist[i];
        if (c) atomicAdd(&W.hist[i], c);
    }
}

// ---- many queries per sequence: scores as a matrix product on MFMA ----------
//
// With many queries routed to the same sequence (prefill: every query
// position of a chunk), the scores of a sequence are one matrix product
// qsum[q,:] . k_idx[b,s,:].  A workgroup takes 32 consecutive queries: it
// folds their heads in fp32 (h = 0, 1, ... in order) and splits each folded
// value exactly into three bf16 terms (hi + mid + lo, residual below 2^-26
// of the value), so that the bf16 MFMA products carry the folded query at
// better than fp32 precision.  Keys are staged in LDS 128 rows at a time and
// every wave produces 16 queries x 64 keys with v_mfma_f32_16x16x32_bf16
// (the three terms accumulated lo, mid, hi per step).  Queries of one
// workgroup that belong to different sequences are served by one pass per
// distinct sequence.  Equal key rows of a sequence give bitwise-equal scores.
constexpr int kGemmQ = 32;       // queries per workgroup
constexpr int kGemmK = 128;      // key rows per LDS block
constexpr int kGemmMinQueries = 64;  // fewer queries: the streaming kernel

__device__ __forceinline__ uint16_t bf16_bits_rn(float f) { return f32_to_bf16(f); }
__device__ __forceinline__ float bf16_value(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <int D>
__global__ __launch_bounds__(kThreads) void score_gemm_kernel(
    const bf16_t* __restrict__ q_idx, const bf16_t* __restrict__ k_idx,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ n_cand,
    float* __restrict__ scores, int B, int Nq, int H_I, int S_max) {
    constexpr int NKS = D / 32;      // MFMA steps over the key width
    constexpr int CPR = D / 8;       // 16-byte chunks per key row
    constexpr int SK = D + 8;        // LDS row stride (elements): rows land on distinct banks
    static_assert(D % 32 == 0 && kThreads == 256, "layout");
    __shared__ __align__(16) uint16_t kb[kGemmK][SK];
    __shared__ __align__(16) uint16_t qs[3][kGemmQ][SK];
    __shared__ int s_seq[kGemmQ], s_n[kGemmQ];
    __shared__ int s_list[kGemmQ], s_lmax[kGemmQ], s_nl;
    __shared__ __align__(16) float so[kGemmQ][kGemmK + 4];  // scores of a block, by query

    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int hl = lane & 15, quad = lane >> 4;
    const int q0 = blockIdx.x * kGemmQ;
    if (tid < kGemmQ) {
        const int q = q0 + tid;
        int b = -1, n = 0;
        if (q < Nq) {
            b = q_seq ? q_seq[q] : q;
            if (b < 0 || b >= B) b = -1;
            else n = clamp_n(n_cand, q, S_max);
        }
        s_seq[tid] = b;
        s_n[tid] = n;
    }
    // fold + exact three-term split: thread pair (query, 16-byte chunk)
    for (int p = tid; p < kGemmQ * CPR; p += kThreads) {
        const int qq = p / CPR, c = p % CPR, q = q0 + qq;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        if (q < Nq) {
            const bf16_t* src = q_idx + (size_t)q * H_I * D + (size_t)c * 8;
            int h = 0;
            for (; h + 8 <= H_I; h += 8) {
                u32x4 v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const u32x4*>(src + (size_t)(h + j) * D);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float f[8];
                    Elem<bf16_t>::unpack(v[j], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += f[e];
                }
            }
            for (; h < H_I; ++h) {
                float f[8];
                Elem<bf16_t>::load16(src + (size_t)h * D, f);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += f[e];
            }
        }
        u32x4 hi, mid, lo;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            uint32_t wh = 0, wm = 0, wl = 0;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const float v = acc[2 * e2 + s];
                const uint16_t bh = bf16_bits_rn(v);
                const float r1 = v - bf16_value(bh);
                const uint16_t bm = bf16_bits_rn(r1);
                const float r2 = r1 - bf16_value(bm);
                const uint16_t bl = bf16_bits_rn(r2);
                wh |= (uint32_t)bh << (16 * s);
                wm |= (uint32_t)bm << (16 * s);
                wl |= (uint32_t)bl << (16 * s);
            }
            hi[e2] = wh; mid[e2] = wm; lo[e2] = wl;
        }
        *reinterpret_cast<u32x4*>(&qs[0][qq][c * 8]) = hi;
        *reinterpret_cast<u32x4*>(&qs[1][qq][c * 8]) = mid;
        *reinterpret_cast<u32x4*>(&qs[2][qq][c * 8]) = lo;
    }
    __syncthreads();
    if (tid == 0) {  // distinct sequences of the workgroup, with their longest candidate range
        int nl = 0;
        for (int i = 0; i < kGemmQ; ++i) {
            const int b = s_seq[i];
            if (b < 0 || s_n[i] == 0) continue;
            int j = 0;
            while (j < nl && s_list[j] != b) ++j;
            if (j == nl) {
                s_list[nl] = b;
                s_lmax[nl] = 0;
                ++nl;
            }
            s_lmax[j] = max(s_lmax[j], s_n[i]);
        }
        s_nl = nl;
    }
    // wave w: queries 16*(w & 1) + hl, keys 64*(w >> 1) .. +63 of each block
    const int qb = w & 1, kh = w >> 1;
    bf16x8 bq[3][NKS];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            bq[t][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&qs[t][16 * qb + hl][32 * ks + 8 * quad]));
    __syncthreads();
    const int my_q = 16 * qb + hl;
    const bool vec_ok = (S_max & 3) == 0;
    const int nl = s_nl;
    // key block staging: thread moves chunks p = tid + j*256 (row p / CPR), the
    // next block's chunks in flight while a block is computed
    constexpr int KPT = kGemmK * CPR / kThreads;
    static_assert(kGemmK * CPR % kThreads == 0, "staging map");
    u32x4 kreg[KPT];
    auto load_block = [&](const bf16_t* kseq, int k0) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int p = tid + j * kThreads, r = p / CPR, c = p % CPR, key = k0 + r;
            kreg[j] = key < S_max ? *reinterpret_cast<const u32x4*>(kseq + (size_t)key * D + c * 8)
                                  : u32x4{0u, 0u, 0u, 0u};
        }
    };
    for (int li = 0; li < nl; ++li) {
        const int bs = s_list[li], nmax = s_lmax[li];
        const bf16_t* kseq = k_idx + (size_t)bs * S_max * D;
        load_block(kseq, 0);
        for (int k0 = 0; k0 < nmax; k0 += kGemmK) {
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const int p = tid + j * kThreads;
                *reinterpret_cast<u32x4*>(&kb[p / CPR][(p % CPR) * 8]) = kreg[j];
            }
            __syncthreads();
            if (k0 + kGemmK < nmax) load_block(kseq, k0 + kGemmK);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const int kr = 64 * kh + 16 * kt;
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8 af = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&kb[kr + hl][32 * ks + 8 * quad]));
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bq[2][ks], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bq[1][ks], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bq[0][ks], acc, 0, 0, 0);
                }
                // acc[r] = score of key k0 + kr + 4*quad + r for query my_q
                *reinterpret_cast<f32x4*>(&so[my_q][kr + 4 * quad]) = acc;
            }
            __syncthreads();
            // the block's scores leave as whole runs of each query's row
            for (int p = tid; p < kGemmQ * (kGemmK / 4); p += kThreads) {
                const int qq = p / (kGemmK / 4), key0 = k0 + (p % (kGemmK / 4)) * 4;
                if (s_seq[qq] != bs) continue;
                const int nq = s_n[qq];
                float* row = scores + (size_t)(q0 + qq) * S_max;
                const f32x4 v = *reinterpret_cast<const f32x4*>(&so[qq][key0 - k0]);
                if (vec_ok && key0 + 4 <= nq) {
                    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(row + key0));
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (key0 + r < nq) row[key0 + r] = v[r];
                }
            }
        }
    }
}

// ---- one workgroup per query, all keys in LDS ---------------------------------
// The row histograms keep two 16-bit bin counts per LDS word (bin b in half
// b & 1 of word b >> 1; a row has at most 12,288 keys, so no half carries
// into the other): 4 KB instead of 8 for 2048 bins, which lets four
// 8,192-key rows share a CU.
__device__ __forceinline__ void hist16_add(uint32_t* hp, uint32_t b) {
    atomicAdd(&hp[b >> 1], 1u << ((b & 1u) << 4));
}

// The bin d of packed counts hp[0..NB/2) such that (members in bins above d)
// < need <= (members above d) + count(d).  Returns d; *rem = need minus the
// members above d, *cnt = count(d), both read before the closing barrier so
// the caller may reuse hp right away.  Every thread calls it.
template <int NB>
__device__ int row_crossing(const uint32_t* hp, int need, uint32_t* tmp, int* rem, int* cnt) {
    constexpr int BPT = NB / kThreads;  // bins per thread
    static_assert(BPT == 8 || BPT == 4, "one 16- or 8-byte LDS read of packed bins per thread");
    __shared__ int res[3];
    const int tid = threadIdx.x;
    const int grp = kThreads - 1 - tid;  // thread 0 owns the top bins
    if (tid == 0) {
        res[0] = 0;
        res[1] = 1;
        res[2] = 0;
    }
    uint32_t c[BPT];
    if constexpr (BPT == 8) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(hp + grp * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            c[2 * j] = v[j] & 0xffffu;
            c[2 * j + 1] = v[j] >> 16;
        }
    } else {
        const uint32_t v0 = hp[grp * 2], v1 = hp[grp * 2 + 1];
        c[0] = v0 & 0xffffu;
        c[1] = v0 >> 16;
        c[2] = v1 & 0xffffu;
        c[3] = v1 >> 16;
    }
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) sum += c[j];
    uint32_t tot;
    const uint32_t above = block_excl_scan<kThreads>(sum, tmp, &tot);
    if (above < (uint32_t)need && (uint32_t)need <= above + sum) {
        uint32_t cum = above;
        bool found = false;
#pragma unroll
        for (int j = BPT - 1; j >= 0; --j) {
            if (!found && cum + c[j] >= (uint32_t)need) {
                res[0] = grp * BPT + j;
                res[1] = need - (int)cum;
                res[2] = (int)c[j];
                found = true;
            }
            cum += c[j];
        }
    }
    __syncthreads();
    const int d = res[0];
    *rem = res[1];
    *cnt = res[2];
    __syncthreads();
    return d;
}

// Histogram of digit (key >> shift) & (NB-1) over the keys matching pref under
// pmask, reading the LDS keys 16 bytes at a time; then the crossing bin.
template <int NB>
__device__ int row_digit(const uint32_t* keys, int n, uint32_t pmask, uint32_t pref, int shift,
                         int need, uint32_t* hp, uint32_t* tmp, int* rem) {
    const int tid = threadIdx.x;
    for (int i = tid; i < NB / 2; i += kThreads) hp[i] = 0;
    __syncthreads();
    const int n4 = n / 4;
    for (int i4 = tid; i4 < n4; i4 += kThreads) {
        const u32x4 kk = *reinterpret_cast<const u32x4*>(keys + 4 * i4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if ((kk[j] & pmask) == pref) hist16_add(hp, (kk[j] >> shift) & (NB - 1));
    }
    for (int i = 4 * n4 + tid; i < n; i += kThreads) {
        const uint32_t kk = keys[i];
        if ((kk & pmask) == pref) hist16_add(hp, (kk >> shift) & (NB - 1));
    }
    __syncthreads();
    int cnt;
    return row_crossing<NB>(hp, need, tmp, rem, &cnt);
}

constexpr int kRowListCap = 4096;  // short list of the row select (entries at or above bin d1)

// Rows of at least 6,144 key words keep the short list's indices (kRowListCap
// uint16) in key words [4096, 6144): the compacted list overwrites only words
// below 4096, and every key is in registers before it is written.  Shorter
// rows put them after the keys.
__host__ __device__ constexpr bool row_lidx_in_keys(int S_max) {
    return 4 * ((S_max + 3) / 4) >= kRowListCap + kRowListCap / 2;
}
__host__ __device__ constexpr size_t row_lds_bytes(int S_max) {
    return (size_t)4 * (4 * ((S_max + 3) / 4)) + (row_lidx_in_keys(S_max) ? 0 : (size_t)kRowListCap * 2);
}

// Ordered compaction of the selected keys of list (lk, li?) of length n: the
// first min(k, ...) under (key desc, index asc) given the k-th key T and the
// number `need` of keys equal to T to take; writes ascending indices.
__device__ void row_write(const uint32_t* lk, const uint16_t* li, int n, uint32_t T, int need,
                          uint32_t* tmp, int32_t* o) {
    const int tid = threadIdx.x;
    const int E = 4 * ceil_div(n, 4 * kThreads);
    const int s0 = min(n, tid * E), s1 = min(n, s0 + E);
    uint32_t gt = 0, eq = 0;
    int s = s0;
    for (; s + 4 <= s1; s += 4) {
        const u32x4 kk = *reinterpret_cast<const u32x4*>(lk + s);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            gt += kk[j] > T;
            eq += kk[j] == T;
        }
    }
    for (; s < s1; ++s) {
        gt += lk[s] > T;
        eq += lk[s] == T;
    }
    // one paired scan: the equal keys taken before this thread's range are the
    // first min(eq_base, need) of them (they are taken in index order)
    uint32_t gt_base, eq_base, gt_tot, eq_tot;
    block_excl_scan2<kThreads>(gt, eq, tmp, &gt_base, &eq_base, &gt_tot, &eq_tot);
    const int eq_take = max(0, min((int)eq, need - (int)eq_base));
    const uint32_t pos0 = gt_base + min(eq_base, (uint32_t)max(need, 0));
    if (gt + (uint32_t)eq_take == 0) return;
    int pos = (int)pos0, e = 0;
    for (s = s0; s < s1; ++s) {
        const uint32_t kk = lk[s];
        const int idx = li ? (int)li[s] : s;
        if (kk > T) {
            o[pos++] = idx;
        } else if (kk == T) {
            if (e < eq_take) o[pos++] = idx;
            ++e;
        }
    }
}

__global__ __launch_bounds__(kThreads) void topk_row_kernel(const float* __restrict__ scores,
                                                            const int32_t* __restrict__ n_cand,
                                                            const int32_t* __restrict__ q_seq,
                                                            int B, int32_t* __restrict__ out,
                                                            int S_max, int k) {
    // dynamic LDS: the row's keys (S_max rounded up to 4) and the short list's
    // indices (kRowListCap uint16, inside the key words for long rows)
    extern __shared__ __align__(16) uint32_t keys[];
    uint16_t* lidx = reinterpret_cast<uint16_t*>(
        keys + (row_lidx_in_keys(S_max) ? kRowListCap : 4 * ceil_div(S_max, 4)));
    __shared__ __align__(16) uint32_t h[kBins / 2];  // packed 16-bit counts
    __shared__ uint32_t tmp[2 * kNW + 2];
    const int q = blockIdx.x, tid = threadIdx.x;
    const int n = query_n(n_cand, q_seq, B, q, S_max);
    const int take = min(k, n);
    int32_t* o = out + (size_t)q * k;
    if (take == n) {  // every candidate is selected
        for (int i = tid; i < k; i += kThreads) o[i] = i < n ? i : -1;
        return;
    }
    // the row's scores -> keys in LDS (8 loads in flight per thread, 16-byte
    // loads when the row is 16-byte aligned) and the histogram of their top
    // 11 bits on the way
    for (int i = tid; i < kBins / 2; i += kThreads) h[i] = 0;
    __syncthreads();
    const float* src = scores + (size_t)q * S_max;
    int i0 = 0;
    if ((S_max & 3) == 0) {
        const int n4 = n / 4;
        constexpr int U = 8;
        for (int b0 = 0; b0 < n4; b0 += U * kThreads) {
            // unconditional loads (clamped index; chunks past the row are
            // skipped below): a load inside a branch is followed by a wait
            // there, which made the eight loads eight round trips
            f32x4 v[U];
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const int i4 = min(b0 + j * kThreads + tid, n4 - 1);
                v[j] = *reinterpret_cast<const f32x4*>(src + 4 * i4);
            }
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const int i4 = b0 + j * kThreads + tid;
                if (i4 < n4) {
                    const u32x4 kk = u32x4{score_key(v[j][0]), score_key(v[j][1]), score_key(v[j][2]),
                                           score_key(v[j][3])};
                    *reinterpret_cast<u32x4*>(keys + 4 * i4) = kk;
#pragma unroll
                    for (int e = 0; e < 4; ++e) hist16_add(h, kk[e] >> 21);
                }
            }
        }
        i0 = 4 * n4;
    }
    for (int b0 = i0; b0 < n; b0 += 8 * kThreads) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = src[min(b0 + j * kThreads + tid, n - 1)];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = b0 + j * kThreads + tid;
            if (i < n) {
                const uint32_t kk = score_key(v[j]);
                keys[i] = kk;
                hist16_add(h, kk >> 21);
            }
        }
    }
    __syncthreads();
    int need = take, rem, hc;
    const int d1 = row_crossing<kBins>(h, need, tmp, &rem, &hc);
    const int m = (take - rem) + hc;  // entries with bin >= d1
    need = rem;
    const uint32_t lo1 = (uint32_t)d1 << 21;
    // short list: the entries at or above bin d1, compacted in index order in
    // place (every thread holds its range in registers before any write)
    int nl = n;
    const uint16_t* li = nullptr;
    if (m <= kRowListCap) {
        // wave w takes keys [w P, w P + P) (P a multiple of 256), and in chunk j
        // lane l the four keys w P + 256 j + 4 l .. + 3: one 16-byte LDS read
        // per lane covers 256 consecutive keys without bank conflicts, and a
        // wave prefix sum of the per-lane counts keeps index order.  Every key
        // is in registers before the barrier, so the compacted list can
        // overwrite the keys in place afterwards.
        constexpr int JMAX = kRowSelectCap / (4 * kThreads);  // chunks per wave at most (12)
        const int lane = lane_id(), w = tid / kWave;
        const int P = ceil_div(n, 4 * kThreads) * (4 * kWave);
        const int wb = w * P;
        u32x4 r[JMAX];
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < JMAX; ++j) {
            // chunks past the wave's range count nothing (their zeros would
            // pass the test below when lo1 is 0: a crossing at bin 0)
            const bool in = 4 * kWave * j < P;
            const int s = wb + 4 * kWave * j + 4 * lane;
            r[j] = (in && s < n) ? *reinterpret_cast<const u32x4*>(keys + s) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 4; ++e) cnt += (in && s + e < n && r[j][e] >= lo1) ? 1u : 0u;
        }
        const uint32_t wcnt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(cnt), kWave - 1);
        if (lane == 0) tmp[w] = wcnt;
        __syncthreads();  // every key read
        uint32_t run = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < kNW; ++i) {
            run += i < w ? tmp[i] : 0u;
            tot += tmp[i];
        }
#pragma unroll
        for (int j = 0; j < JMAX; ++j) {
            if (4 * kWave * j >= P) break;  // wave-uniform
            const int s = wb + 4 * kWave * j + 4 * lane;
            bool t[4];
            uint32_t c = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                t[e] = s + e < n && r[j][e] >= lo1;
                c += t[e] ? 1u : 0u;
            }
            const uint32_t inc = wave_incl_scan(c);
            uint32_t p = run + inc - c;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (t[e]) {
                    keys[p] = r[j][e];
                    lidx[p] = (uint16_t)(s + e);
                    ++p;
                }
            }
            run += (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
        }
        __syncthreads();
        nl = (int)tot;
        li = lidx;
    }
    const int d2 = row_digit<kBins>(keys, nl, 0xffe00000u, lo1, 10, need, h, tmp, &rem);
    need = rem;
    const uint32_t pref = lo1 | ((uint32_t)d2 << 10);
    const int d3 = row_digit<1024>(keys, nl, 0xfffffc00u, pref, 0, need, h, tmp, &rem);
    need = rem;  // how many keys equal to T are taken (the lowest indices)
    const uint32_t T = pref | (uint32_t)d3;
    row_write(keys, li, nl, T, need, tmp, o);
    for (int i = take + tid; i < k; i += kThreads) o[i] = -1;
}

// ---- multi-workgroup path: filter + final select ---------------------------------
constexpr int kPerThread = kFilterChunk / kThreads;  // consecutive scores per thread (16)
static_assert(kPerThread == 16, "per-thread masks and counts are 16 bits wide");

// One workgroup per segment of 4096 candidates: thread t classifies the 16
// consecutive candidates 16t..16t+15 of the segment against the threshold
// bin, so one block prefix sum over (selected, short) counts places every
// entry in index order.  Segment g's short list goes to cand_[4096 g ...),
// its selected indices right after it, and its two counts to seg[g].
__global__ __launch_bounds__(kThreads) void topk_filter_kernel(const float* __restrict__ scores,
                                                               const int32_t* __restrict__ n_cand,
                                                               const int32_t* __restrict__ q_seq,
                                                               int B, uint8_t* __restrict__ ws,
                                                               int S_max, int k) {
    __shared__ __align__(16) uint32_t h[kBins];
    __shared__ uint32_t tmp[kNW + 2];
    static_assert(kBins == 8 * kThreads, "two 16-byte histogram loads per thread");

    const int q = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
    QWs W = ws_of(ws, q, S_max, k);
    const int n = query_n(n_cand, q_seq, B, q, S_max);
    const int take = min(k, n);
    const int s0 = g * kFilterChunk;
    if (s0 >= n) {  // uniform: nothing here; the count is written every call
        if (tid == 0) W.seg[g] = 0;
        return;
    }
    const int sb = s0 + tid * kPerThread;

    // 1. the completed first-digit histogram (two 16-byte loads per thread)
    //    and this thread's scores, all loads in flight together; then the
    //    threshold bin
    const bool partial = take < n;
    u32x4 h0 = u32x4{0u, 0u, 0u, 0u}, h1 = u32x4{0u, 0u, 0u, 0u};
    if (partial) {
        const u32x4* hs = reinterpret_cast<const u32x4*>(W.hist);
        h0 = hs[tid];
        h1 = hs[tid + kThreads];
    }
    float v[kPerThread];
    const float* src = scores + (size_t)q * S_max + sb;
    if (sb + kPerThread <= n && (((uintptr_t)src) & 15u) == 0) {
#pragma unroll
        for (int j = 0; j < kPerThread / 4; ++j) {
            const f32x4 t4 = reinterpret_cast<const f32x4*>(src)[j];
            v[4 * j] = t4[0]; v[4 * j + 1] = t4[1]; v[4 * j + 2] = t4[2]; v[4 * j + 3] = t4[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) v[i] = sb + i < n ? src[i] : 0.f;
    }
    int t1 = -1;  // -1: every candidate is selected
    if (partial) {
        reinterpret_cast<u32x4*>(h)[tid] = h0;
        reinterpret_cast<u32x4*>(h)[tid + kThreads] = h1;
        __syncthreads();
        int rem;
        t1 = find_crossing<kBins>(h, take, tmp, &rem);
    }

    // 2. route: above the threshold bin -> selected, inside it -> short list
    uint32_t selm = 0, candm = 0, keys[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        keys[i] = score_key(v[i]);
        const int bin = (int)(keys[i] >> 21);
        const bool ok = sb + i < n;
        if (ok && bin > t1) selm |= 1u << i;
        if (ok && bin == t1) candm |= 1u << i;
    }
    const uint32_t packed = ((uint32_t)__popc(selm) << 16) | (uint32_t)__popc(candm);
    uint32_t tot;
    const uint32_t off = block_excl_scan<kThreads>(packed, tmp, &tot);
    const uint32_t n_short = tot & 0xffffu;
    uint32_t pc = (uint32_t)s0 + (off & 0xffffu);
    uint32_t ps = (uint32_t)s0 + n_short + (off >> 16);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const uint32_t sidx = (uint32_t)(sb + i);
        if (candm & (1u << i)) {
            W.cand_key[pc] = keys[i];
            W.cand_idx[pc] = sidx;
            ++pc;
            atomicAdd(&W.hist2[(keys[i] >> 10) & (kBins - 1)], 1u);
        }
        if (selm & (1u << i)) W.cand_idx[ps++] = sidx;
    }
    if (tid == 0) W.seg[g] = tot;
}

// Final select, one workgroup per query, after every filter workgroup of the
// query has finished (kernel boundary): the steps of select.hpp, the merge of
// the two ascending lists into the output, and the zeroing of the query's
// workspace.
__global__ __launch_bounds__(kThreads) void topk_final_kernel(const int32_t* __restrict__ n_cand,
                                                              const int32_t* __restrict__ q_seq,
                                                              int B, int32_t* __restrict__ out,
                                                              uint8_t* __restrict__ ws, int S_max,
                                                              int k) {
    __shared__ uint32_t h[kBins];
    __shared__ uint32_t tmp[2 * kNW + 2];
    __shared__ uint32_t segc[kMaxSeg], sbase[kMaxSeg], lbase[kMaxSeg];
    __shared__ uint32_t ck[kCandCap], ci[kCandCap];
    __shared__ int32_t selv[kTopkMaxK], chs[kTopkMaxK];
    __shared__ uint32_t misc[4];
    __shared__ uint32_t mem[3 * kThreads];
    __shared__ uint8_t flag[kCandCap];

    const int q = blockIdx.x;
    QWs W = ws_of(ws, q, S_max, k);
    const SelLds L = {h, tmp, segc, sbase, lbase, ck, ci, selv, chs, misc, mem, flag, nullptr};
    const SelResult R = select_query(W, query_n(n_cand, q_seq, B, q, S_max), S_max, k, k, L);
    select_write_sorted(L, R, out + (size_t)q * k, k);
    __syncthreads();
    select_zero<kThreads>(W, S_max, segc, tmp);
}

template <typename T, int LPR, int SEL, int WM>
void launch_score_wm(dim3 grid, size_t lds, hipStream_t st, const void* q_idx, const void* k_idx,
                     const int32_t* q_seq, const int32_t* n_cand, float* scores, uint8_t* ws,
                     int B, int H_I, int S_max, int k, int rows, int Nq, const AppendJob& aj,
                     const PoolMap* kp, const float* head_w) {
    if (kp && kp->map)
        hipLaunchKernelGGL((score_kernel<T, LPR, SEL, true, WM>), grid, dim3(kThreads), lds, st,
                           (const T*)q_idx, (const T*)k_idx, q_seq, n_cand, scores, ws, B, H_I,
                           S_max, k, rows, Nq, aj, *kp, head_w);
    else
        hipLaunchKernelGGL((score_kernel<T, LPR, SEL, false, WM>), grid, dim3(kThreads), lds, st,
                           (const T*)q_idx, (const T*)k_idx, q_seq, n_cand, scores, ws, B, H_I,
                           S_max, k, rows, Nq, aj, PoolMap{}, head_w);
}

template <typename T, int LPR, int SEL>
void launch_score_sel(dim3 grid, size_t lds, hipStream_t st, const void* q_idx, const void* k_idx,
                      const int32_t* q_seq, const int32_t* n_cand, float* scores, uint8_t* ws,
                      int B, int H_I, int S_max, int k, int rows, int Nq, const AppendJob& aj,
                      const PoolMap* kp, const float* head_w) {
    if constexpr (std::is_same<T, bf16_t>::value && LPR == 16) {
        if (head_w) {  // the caller checked the weighted shape (bf16, 128-wide, H_I % 16 == 0, <= 64)
            launch_score_wm<T, LPR, SEL, 1>(grid, lds, st, q_idx, k_idx, q_seq, n_cand, scores, ws, B,
                                            H_I, S_max, k, rows, Nq, aj, kp, head_w);
            return;
        }
    }
    launch_score_wm<T, LPR, SEL, 0>(grid, lds, st, q_idx, k_idx, q_seq, n_cand, scores, ws, B, H_I,
                                    S_max, k, rows, Nq, aj, kp, nullptr);
}

template <typename T, int LPR>
hipError_t launch_score(const void* q_idx, const void* k_idx, int B, const int32_t* q_seq,
                        const int32_t* n_cand, float* scores, uint8_t* ws, int Nq, int H_I,
                        int S_max, int k, int sel, const AppendJob* job, hipStream_t st,
                        const PoolMap* kp, const float* head_w) {
    const int rows_lg = list_rows_log2(S_max, Nq);
    if (sel == 2 && rows_lg != 11) sel = 3;  // smaller slots: the variable-slot instantiation
    const int rows = sel >= 2 ? (1 << rows_lg) : sel ? kScoreRowsMulti : min(S_max, 8192);
    dim3 grid((unsigned)ceil_div(S_max, rows), (unsigned)Nq);
    if (sel >= 2 && job) {  // append rows after the query rows
        const int units = job->B * ((job->D / Elem<T>::kPer16B + kThreads - 1) / kThreads);
        grid.y += (unsigned)ceil_div(units, (int)grid.x);
    }
    const AppendJob none{};
    const AppendJob& aj = job ? *job : none;
    const size_t lds = (size_t)rows * sizeof(float);  // staged scores
    ProfScope prof(kProfScore, st);
    if (sel == 3)
        launch_score_sel<T, LPR, 3>(grid, lds, st, q_idx, k_idx, q_seq, n_cand, scores, ws, B, H_I, S_max, k, rows, Nq, aj, kp, head_w);
    else if (sel == 2)
        launch_score_sel<T, LPR, 2>(grid, lds, st, q_idx, k_idx, q_seq, n_cand, scores, ws, B, H_I, S_max, k, rows, Nq, aj, kp, head_w);
    else if (sel == 1)
        launch_score_sel<T, LPR, 1>(grid, lds, st, q_idx, k_idx, q_seq, n_cand, scores, ws, B, H_I, S_max, k, rows, Nq, aj, kp, head_w);
    else
        launch_score_sel<T, LPR, 0>(grid, lds, st, q_idx, k_idx, q_seq, n_cand, scores, ws, B, H_I, S_max, k, rows, Nq, aj, kp, head_w);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_score_t(int d_I, const void* q_idx, const void* k_idx, int B,
                          const int32_t* q_seq, const int32_t* n_cand, float* scores, uint8_t* ws,
                          int Nq, int H_I, int S_max, int k, int sel, const AppendJob* job,
                          hipStream_t st, const PoolMap* kp, const float* head_w) {
    const int lpr = d_I * (int)sizeof(T) / 16;
    if (lpr == 8)
        return launch_score<T, 8>(q_idx, k_idx, B, q_seq, n_cand, scores, ws, Nq, H_I, S_max, k, sel, job, st, kp, head_w);
    if (lpr == 16)
        return launch_score<T, 16>(q_idx, k_idx, B, q_seq, n_cand, scores, ws, Nq, H_I, S_max, k, sel, job, st, kp, head_w);
    return launch_score<T, 32>(q_idx, k_idx, B, q_seq, n_cand, scores, ws, Nq, H_I, S_max, k, sel, job, st, kp, head_w);
}

// Zero the first-digit histogram of every query (a scoring launch whose select
// never ran leaves it counted).
__global__ __launch_bounds__(kThreads) void clear_hist_kernel(uint8_t* __restrict__ ws, int S_max,
                                                              int k) {
    uint32_t* h = ws_of(ws, (int)blockIdx.x, S_max, k).hist;
    for (int i = (int)threadIdx.x; i < kBins; i += kThreads) h[i] = 0;
}

// Zero `words` 32-bit words from p (16-byte aligned), grid-stride with 16-byte stores.
__global__ __launch_bounds__(kThreads) void zero_words_kernel(uint32_t* __restrict__ p,
                                                              size_t words) {
    const size_t n4 = words / 4;
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride)
        reinterpret_cast<u32x4*>(p)[i] = u32x4{0u, 0u, 0u, 0u};
    for (size_t i = n4 * 4 + (size_t)blockIdx.x * kThreads + threadIdx.x; i < words; i += stride)
        p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_words(void* p, size_t words, hipStream_t st) {
    if (words == 0) return hipSuccess;
    const size_t blocks = (words / 4 + kThreads - 1) / kThreads;
    const unsigned grid = (unsigned)(blocks < 1024 ? (blocks < 1 ? 1 : blocks) : 1024);
    hipLaunchKernelGGL(zero_words_kernel, dim3(grid), dim3(kThreads), 0, st,
                       static_cast<uint32_t*>(p), words);
    return hipGetLastError();
}

hipError_t launch_clear_select_hist(void* ws, int Nq, int S_max, int k, hipStream_t st) {
    hipLaunchKernelGGL(clear_hist_kernel, dim3((unsigned)Nq), dim3(kThreads), 0, st,
                       static_cast<uint8_t*>(ws), S_max, k);
    return hipGetLastError();
}

size_t topk_workspace_bytes(int Nq, int S_max, int k) {
    if (S_max <= kRowSelectCap) return 0;
    return (size_t)Nq * ws_per_query(S_max, k);
}

// Scores, first-digit histogram and per-workgroup candidate lists (the fused
// decode select reads them), with the decode-time C4 append of `job` (may be
// null) in the same launch.
bool index_lists_apply(int S_max, int k, int Nq) { return lists_apply(S_max, k, Nq); }

hipError_t launch_index_lists(int dtype, const void* q_idx, const void* k_idx, int B,
                              const int32_t* n_cand, float* scores, int Nq, int H_I, int d_I,
                              int S_max, int k, void* ws, const AppendJob* job, hipStream_t st,
                              const PoolMap* kI, const float* head_w) {
    uint8_t* w = static_cast<uint8_t*>(ws);
    return dtype == kF32 ? launch_score_t<float>(d_I, q_idx, k_idx, B, nullptr, n_cand, scores, w,
                                                  Nq, H_I, S_max, k, 2, job, st, kI, head_w)
                         : launch_score_t<bf16_t>(d_I, q_idx, k_idx, B, nullptr, n_cand, scores, w,
                                                   Nq, H_I, S_max, k, 2, job, st, kI, head_w);
}

hipError_t launch_index_topk(int dtype, const void* q_idx, const void* k_idx, int B,
                             const int32_t* q_seq, const int32_t* n_cand, float* scores,
                             int32_t* topk_idx, int Nq, int H_I, int d_I, int S_max, int k,
                             void* ws, hipStream_t st, const PoolMap* kI, const float* head_w) {
    const bool paged = kI && kI->map;
    const bool multi = S_max > kRowSelectCap;
    uint8_t* w = static_cast<uint8_t*>(ws);
    hipError_t e = hipSuccess;
    // the select treats a query routed outside [0, B) as one without candidates
    // (select-only mode has no key sequences: q_seq is ignored there)
    const int32_t* sel_seq = q_idx ? q_seq : nullptr;
    if (q_idx && !multi && !paged && !head_w && dtype == kBF16 && Nq >= kGemmMinQueries &&
        (d_I == 64 || d_I == 128 || d_I == 256)) {
        ProfScope prof(kProfScore, st);
        const dim3 grid((unsigned)ceil_div(Nq, kGemmQ));
        const bf16_t* qp = static_cast<const bf16_t*>(q_idx);
        const bf16_t* kp = static_cast<const bf16_t*>(k_idx);
        if (d_I == 64)
            hipLaunchKernelGGL(score_gemm_kernel<64>, grid, dim3(kThreads), 0, st, qp, kp, q_seq,
                               n_cand, scores, B, Nq, H_I, S_max);
        else if (d_I == 128)
            hipLaunchKernelGGL(score_gemm_kernel<128>, grid, dim3(kThreads), 0, st, qp, kp, q_seq,
                               n_cand, scores, B, Nq, H_I, S_max);
        else
            hipLaunchKernelGGL(score_gemm_kernel<256>, grid, dim3(kThreads), 0, st, qp, kp, q_seq,
                               n_cand, scores, B, Nq, H_I, S_max);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (q_idx) {
        e = dtype == kF32 ? launch_score_t<float>(d_I, q_idx, k_idx, B, q_seq, n_cand, scores, w,
                                                   Nq, H_I, S_max, k, multi ? 1 : 0, nullptr, st, kI, head_w)
                          : launch_score_t<bf16_t>(d_I, q_idx, k_idx, B, q_seq, n_cand, scores,
                                                   w, Nq, H_I, S_max, k, multi ? 1 : 0, nullptr, st, kI, head_w);
        if (e != hipSuccess) return e;
    } else if (multi) {
        dim3 grid((unsigned)ceil_div(S_max, kFilterChunk), (unsigned)Nq);
        ProfScope prof(kProfSelect, st);
        hipLaunchKernelGGL(hist_kernel, grid, dim3(kThreads), 0, st, scores, n_cand, sel_seq, B, w,
                           S_max, k, kFilterChunk);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    ProfScope prof(kProfSelect, st);
    if (!multi) {
        // LDS for S_max keys (and the short list's indices) only, so that short
        // rows fit more workgroups per CU
        const size_t lds = row_lds_bytes(S_max);
        hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)Nq), dim3(kThreads), lds, st, scores,
                           n_cand, sel_seq, B, topk_idx, S_max, k);
    } else {
        const int G = ceil_div(S_max, kFilterChunk);
        hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)G, (unsigned)Nq), dim3(kThreads), 0,
                           st, scores, n_cand, sel_seq, B, w, S_max, k);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL(topk_final_kernel, dim3((unsigned)Nq), dim3(kThreads), 0, st, n_cand,
                           sel_seq, B, topk_idx, w, S_max, k);
    }
    return hipGetLastError();
}

}  // namespace hsa
