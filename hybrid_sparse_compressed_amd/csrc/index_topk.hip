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
//    A filter kernel then sends every candidate above the threshold bin to
//    the "selected" list and every candidate inside it to a short list; the
//    last filter workgroup of each query finishes the select on that short
//    list in LDS (two more histogram passes, plus a pass over indices when
//    a tie straddles rank k), sorts the result ascending and zeroes its
//    part of the workspace for the next call.
#include "hsa_common.hpp"
#include "hsa_internal.hpp"

namespace hsa {

namespace {

constexpr int kThreads = 256;
constexpr int kNW = kThreads / kWave;
constexpr int kBins = 2048;         // first digit: key bits 31..21
constexpr int kFilterChunk = 4096;  // scores per filter workgroup
constexpr int kCandCap = 4096;      // short-list entries the final select keeps in LDS
constexpr int kScoreRowsMulti = 2048;

// ---- workspace (multi-workgroup path), per query -------------------------
//   hist[2048] u32 | ctr[16] u32 (0: short-list size, 1: selected size,
//   2: finished filter workgroups) | cand_key[S_max] | cand_idx[S_max] | sel[k]
__host__ __device__ inline size_t ws_per_query(int S_max, int k) {
    size_t b = (size_t)kBins * 4 + 64 + (size_t)S_max * 8 + (size_t)k * 4;
    return (b + 255) & ~(size_t)255;
}

struct QWs {
    uint32_t* hist;
    uint32_t* ctr;
    uint32_t* cand_key;
    uint32_t* cand_idx;
    int32_t* sel;
};

__device__ inline QWs ws_of(uint8_t* ws, int q, int S_max, int k) {
    uint8_t* base = ws + (size_t)q * ws_per_query(S_max, k);
    QWs w;
    w.hist = reinterpret_cast<uint32_t*>(base);
    w.ctr = w.hist + kBins;
    w.cand_key = w.ctr + 16;
    w.cand_idx = w.cand_key + S_max;
    w.sel = reinterpret_cast<int32_t*>(w.cand_idx + S_max);
    return w;
}

// Counters that other workgroups of the same launch update with atomics.
__device__ inline uint32_t counter_load(const uint32_t* p) {
    return __atomic_load_n(p, __ATOMIC_RELAXED);
}

__device__ inline int clamp_n(const int32_t* n_cand, int q, int S_max) {
    int n = n_cand[q];
    return n < 0 ? 0 : (n > S_max ? S_max : n);
}

template <typename T> __device__ inline float widen(const T* p, size_t i);
template <> __device__ inline float widen<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ inline float widen<bf16_t>(const bf16_t* p, size_t i) {
    return __uint_as_float((uint32_t)p[i].bits << 16);
}

// ---- scoring ---------------------------------------------------------------
template <typename T, int LPR, bool HIST>
__global__ __launch_bounds__(kThreads) void score_kernel(
    const T* __restrict__ q_idx, const T* __restrict__ k_idx, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ n_cand, float* __restrict__ scores, uint8_t* __restrict__ ws,
    int B, int H_I, int S_max, int k, int rows_per_wg) {
    constexpr int V = Elem<T>::kPer16B;
    constexpr int DI = LPR * V;          // indexer width
    constexpr int RPL = kWave / LPR;     // rows covered by one wave-wide load
    constexpr int UNROLL = 8;
    __shared__ float qsum[DI];
    __shared__ uint32_t hist[HIST ? kBins : 1];

    const int q = blockIdx.y;
    const int bseq = q_seq ? q_seq[q] : q;
    int n = clamp_n(n_cand, q, S_max);
    if (bseq < 0 || bseq >= B) n = 0;
    const int r0 = blockIdx.x * rows_per_wg;
    const int r1 = min(n, r0 + rows_per_wg);
    if (r0 >= r1) return;  // uniform over the workgroup

    const int tid = threadIdx.x;
    for (int e = tid; e < DI; e += kThreads) {
        float s = 0.f;
        for (int h = 0; h < H_I; ++h) s += widen<T>(q_idx, ((size_t)q * H_I + h) * DI + e);
        qsum[e] = s;
    }
    if constexpr (HIST)
        for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
    __syncthreads();

    const int lane = lane_id(), w = tid / kWave;
    const int sub = lane % LPR, rs = lane / LPR;
    float qv[V];
#pragma unroll
    for (int e = 0; e < V; ++e) qv[e] = qsum[sub * V + e];
    const T* kbase = k_idx + (size_t)bseq * S_max * DI + (size_t)sub * V;
    float* srow = scores + (size_t)q * S_max;

    const int nit = ceil_div(r1 - r0, kNW * RPL);
    for (int it0 = 0; it0 < nit; it0 += UNROLL) {
        u32x4 buf[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int r = r0 + ((it0 + u) * kNW + w) * RPL + rs;
            const int rc = r < r1 ? r : r1 - 1;  // stay inside this query's rows
            buf[u] = *reinterpret_cast<const u32x4*>(kbase + (size_t)rc * DI);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int r = r0 + ((it0 + u) * kNW + w) * RPL + rs;
            float kv[V];
            Elem<T>::unpack(buf[u], kv);
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < V; ++e) d = fmaf(qv[e], kv[e], d);
#pragma unroll
            for (int o = 1; o < LPR; o <<= 1) d += __shfl_xor(d, o, kWave);
            if (sub == 0 && r < r1) {
                srow[r] = d;
                if constexpr (HIST) atomicAdd(&hist[score_key(d) >> 21], 1u);
            }
        }
    }
    if constexpr (HIST) {
        __syncthreads();
        QWs W = ws_of(ws, q, S_max, k);
        for (int i = tid; i < kBins; i += kThreads) {
            const uint32_t c = hist[i];
            if (c) atomicAdd(&W.hist[i], c);
        }
    }
}

// top-11-bit histogram of given scores (select-only mode, multi-workgroup path)
__global__ __launch_bounds__(kThreads) void hist_kernel(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ n_cand,
                                                        uint8_t* __restrict__ ws, int S_max, int k,
                                                        int chunk) {
    __shared__ uint32_t hist[kBins];
    const int q = blockIdx.y, tid = threadIdx.x;
    const int n = clamp_n(n_cand, q, S_max);
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

// ---- LDS radix machinery -------------------------------------------------------
// Given bin counts h[0..NB), find the bin d such that (members in bins above d)
// < need <= (members in bins above d) + h[d].  Returns d; *rem = need minus the
// members above d.  Every thread calls it (it has barriers).
template <int NB>
__device__ int find_crossing(const uint32_t* h, int need, uint32_t* tmp, int* rem) {
    static_assert(NB % kThreads == 0, "bins must be a multiple of the workgroup size");
    constexpr int BPT = NB / kThreads;
    __shared__ int res[2];
    const int tid = threadIdx.x;
    const int grp = kThreads - 1 - tid;  // thread 0 owns the top bins
    if (tid == 0) { res[0] = 0; res[1] = 1; }
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) s += h[grp * BPT + j];
    uint32_t tot;
    const uint32_t above = block_excl_scan<kThreads>(s, tmp, &tot);
    if (above < (uint32_t)need && (uint32_t)need <= above + s) {
        uint32_t cum = above;
        for (int j = BPT - 1; j >= 0; --j) {
            const uint32_t c = h[grp * BPT + j];
            if (cum + c >= (uint32_t)need) {
                res[0] = grp * BPT + j;
                res[1] = need - (int)cum;
                break;
            }
            cum += c;
        }
    }
    __syncthreads();
    const int d = res[0];
    *rem = res[1];
    __syncthreads();
    return d;
}

// Histogram of digit (key >> shift) & (NB-1) over the members i < n
// (member: (key & pmask) == pref, and, if eq_key != nullptr, eq_key[i] == eq_val),
// then find_crossing.
template <int NB>
__device__ int radix_digit(const uint32_t* keys, int n, uint32_t pmask, uint32_t pref, int shift,
                           const uint32_t* eq_key, uint32_t eq_val, int need, uint32_t* h,
                           uint32_t* tmp, int* rem) {
    const int tid = threadIdx.x;
    for (int i = tid; i < NB; i += kThreads) h[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
        const uint32_t kk = keys[i];
        if ((kk & pmask) == pref && (eq_key == nullptr || eq_key[i] == eq_val))
            atomicAdd(&h[(kk >> shift) & (NB - 1)], 1u);
    }
    __syncthreads();
    return find_crossing<NB>(h, need, tmp, rem);
}

// ---- one workgroup per query, all keys in LDS ---------------------------------
__global__ __launch_bounds__(kThreads) void topk_row_kernel(const float* __restrict__ scores,
                                                            const int32_t* __restrict__ n_cand,
                                                            int32_t* __restrict__ out, int S_max,
                                                            int k) {
    __shared__ uint32_t keys[kRowSelectCap];
    __shared__ uint32_t h[kBins];
    __shared__ uint32_t tmp[kNW + 2];
    const int q = blockIdx.x, tid = threadIdx.x;
    const int n = clamp_n(n_cand, q, S_max);
    const int take = min(k, n);
    int32_t* o = out + (size_t)q * k;
    if (take == n) {  // every candidate is selected
        for (int i = tid; i < k; i += kThreads) o[i] = i < n ? i : -1;
        return;
    }
    for (int i = tid; i < n; i += kThreads) keys[i] = score_key(scores[(size_t)q * S_max + i]);
    __syncthreads();
    int need = take, rem;
    const int d1 = radix_digit<kBins>(keys, n, 0u, 0u, 21, nullptr, 0u, need, h, tmp, &rem);
    need = rem;
    uint32_t pref = (uint32_t)d1 << 21;
    const int d2 = radix_digit<kBins>(keys, n, 0xffe00000u, pref, 10, nullptr, 0u, need, h, tmp, &rem);
    need = rem;
    pref |= (uint32_t)d2 << 10;
    const int d3 = radix_digit<1024>(keys, n, 0xfffffc00u, pref, 0, nullptr, 0u, need, h, tmp, &rem);
    need = rem;  // how many keys equal to T are taken (the lowest indices)
    const uint32_t T = pref | (uint32_t)d3;

    // ordered compaction over contiguous per-thread ranges
    const int E = ceil_div(n, kThreads);
    const int s0 = min(n, tid * E), s1 = min(n, s0 + E);
    uint32_t gt = 0, eq = 0;
    for (int s = s0; s < s1; ++s) {
        const uint32_t kk = keys[s];
        gt += kk > T;
        eq += kk == T;
    }
    uint32_t tot;
    const uint32_t eq_base = block_excl_scan<kThreads>(eq, tmp, &tot);
    const int eq_take = max(0, min((int)eq, need - (int)eq_base));
    const uint32_t pos0 = block_excl_scan<kThreads>(gt + (uint32_t)eq_take, tmp, &tot);
    int pos = (int)pos0, e = 0;
    for (int s = s0; s < s1; ++s) {
        const uint32_t kk = keys[s];
        if (kk > T) {
            o[pos++] = s;
        } else if (kk == T) {
            if (e < eq_take) o[pos++] = s;
            ++e;
        }
    }
    for (int i = take + tid; i < k; i += kThreads) o[i] = -1;
}

// ---- multi-workgroup path: filter + final select ---------------------------------
__device__ inline void wave_append(bool pred, uint32_t* counter, uint32_t cap, uint32_t* dst0,
                                   uint32_t v0, uint32_t* dst1, uint32_t v1) {
    const uint64_t mask = __ballot(pred);
    if (mask == 0) return;
    const int lane = lane_id();
    const int leader = __ffsll((long long)mask) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
    base = __shfl(base, leader, kWave);
    if (pred) {
        const uint32_t pos = base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
        if (pos < cap) {
            dst0[pos] = v0;
            if (dst1) dst1[pos] = v1;
        }
    }
}

__global__ __launch_bounds__(kThreads) void topk_filter_kernel(const float* __restrict__ scores,
                                                               const int32_t* __restrict__ n_cand,
                                                               int32_t* __restrict__ out,
                                                               uint8_t* __restrict__ ws, int S_max,
                                                               int k, int G) {
    __shared__ uint32_t h[kBins];
    __shared__ uint32_t tmp[kNW + 2];
    __shared__ uint32_t ck[kCandCap], ci[kCandCap];
    __shared__ int32_t sel[kTopkMaxK];
    __shared__ uint32_t nsel_lds;
    __shared__ int is_last;

    const int q = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
    QWs W = ws_of(ws, q, S_max, k);
    const int n = clamp_n(n_cand, q, S_max);
    const int take = min(k, n);

    // 1. threshold bin of the first digit from the completed histogram
    int t1 = -1;  // -1: every candidate is selected
    if (take < n) {
        for (int i = tid; i < kBins; i += kThreads) h[i] = W.hist[i];
        __syncthreads();
        int rem;
        t1 = find_crossing<kBins>(h, take, tmp, &rem);
    }

    // 2. route this chunk's candidates
    const int s0 = g * kFilterChunk, s1 = min(n, s0 + kFilterChunk);
    for (int base = s0; base < s1; base += kThreads) {
        const int s = base + tid;
        const bool in = s < s1;
        const uint32_t key = in ? score_key(scores[(size_t)q * S_max + s]) : 0u;
        const int bin = (int)(key >> 21);
        wave_append(in && bin > t1, &W.ctr[1], (uint32_t)k, reinterpret_cast<uint32_t*>(W.sel),
                    (uint32_t)s, nullptr, 0u);
        wave_append(in && bin == t1, &W.ctr[0], (uint32_t)S_max, W.cand_key, key, W.cand_idx,
                    (uint32_t)s);
    }

    // 3. the last workgroup of this query finishes
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = (atomicAdd(&W.ctr[2], 1u) == (uint32_t)(G - 1));
    __syncthreads();
    if (!is_last) return;
    __threadfence();

    // counters read once and broadcast, so every branch below is uniform
    __shared__ int cnt[2], cnt_raw[2];
    if (tid == 0) {
        const uint32_t a = counter_load(&W.ctr[1]), b = counter_load(&W.ctr[0]);
        cnt[0] = min((int)min(a, (uint32_t)take), take);
        cnt[1] = (int)min(b, (uint32_t)S_max);
        cnt_raw[0] = (int)min(a, (uint32_t)k);      // entries written to sel (capacity k)
        cnt_raw[1] = (int)min(b, (uint32_t)S_max);  // entries written to the short list
    }
    __syncthreads();
    const int nsel0 = cnt[0];
    const int nc = cnt[1];
    for (int i = tid; i < nsel0; i += kThreads) sel[i] = W.sel[i];
    if (tid == 0) nsel_lds = (uint32_t)nsel0;
    __syncthreads();
    int need = take - nsel0;
    if (need > 0 && nc > 0) {
        const uint32_t* key = W.cand_key;
        const uint32_t* idx = W.cand_idx;
        if (nc <= kCandCap) {
            for (int i = tid; i < nc; i += kThreads) {
                ck[i] = W.cand_key[i];
                ci[i] = W.cand_idx[i];
            }
            __syncthreads();
            key = ck;
            idx = ci;
        }
        const uint32_t p1 = (uint32_t)t1 << 21;
        int rem;
        const int d2 = radix_digit<kBins>(key, nc, 0xffe00000u, p1, 10, nullptr, 0u, need, h, tmp, &rem);
        need = rem;
        const uint32_t p2 = p1 | ((uint32_t)d2 << 10);
        const int d3 = radix_digit<1024>(key, nc, 0xfffffc00u, p2, 0, nullptr, 0u, need, h, tmp, &rem);
        need = rem;
        const uint32_t T = p2 | (uint32_t)d3;
        // how many candidates equal T?
        uint32_t eq = 0;
        for (int i = tid; i < nc; i += kThreads) eq += key[i] == T;
        uint32_t eq_all;
        block_excl_scan<kThreads>(eq, tmp, &eq_all);
        // the need lowest indices among the T-valued: select on ~idx
        uint32_t imax = 0xffffffffu;  // take every T-valued candidate
        if ((int)eq_all > need) {
            // ~idx of the need-th smallest index, found digit by digit
            // digits of ~idx, highest first, among the T-valued candidates
            int r = need;
            uint32_t pr = 0, pm = 0;
            const int shifts[3] = {21, 10, 0};
            const int widths[3] = {11, 11, 10};
            for (int pass = 0; pass < 3; ++pass) {
                const int nb = 1 << widths[pass];
                for (int i = tid; i < kBins; i += kThreads) h[i] = 0;
                __syncthreads();
                for (int i = tid; i < nc; i += kThreads) {
                    if (key[i] != T) continue;
                    const uint32_t ni = ~idx[i];
                    if ((ni & pm) == pr) atomicAdd(&h[(ni >> shifts[pass]) & (nb - 1)], 1u);
                }
                __syncthreads();
                const int d = (nb == kBins) ? find_crossing<kBins>(h, r, tmp, &rem)
                                            : find_crossing<1024>(h, r, tmp, &rem);
                r = rem;
                pr |= (uint32_t)d << shifts[pass];
                pm |= (uint32_t)(nb - 1) << shifts[pass];
            }
            imax = ~pr;  // indices <= imax among the T-valued are taken
        }
        for (int i = tid; i < nc; i += kThreads) {
            const uint32_t kk = key[i];
            if (kk > T || (kk == T && idx[i] <= imax)) {
                const uint32_t pos = atomicAdd(&nsel_lds, 1u);
                if (pos < (uint32_t)take) sel[pos] = (int32_t)idx[i];
            }
        }
    }
    __syncthreads();
    // bitonic sort of sel[0..take) ascending (padded to a power of two)
    int N = 1;
    while (N < take) N <<= 1;
    const int filled = min((int)nsel_lds, take);
    for (int i = filled + tid; i < N; i += kThreads) sel[i] = 0x7fffffff;
    __syncthreads();
    for (int size = 2; size <= N; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (N >> 1); i += kThreads) {
                const int lo = 2 * stride * (i / stride) + (i % stride);
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const int32_t a = sel[lo], c = sel[hi];
                if ((a > c) == up) { sel[lo] = c; sel[hi] = a; }
            }
            __syncthreads();
        }
    }
    int32_t* o = out + (size_t)q * k;
    for (int i = tid; i < k; i += kThreads) o[i] = (i < filled) ? sel[i] : -1;
    // Leave every word this call wrote for this query zeroed again (histogram,
    // counters, short list, selected list), so the whole workspace is zero
    // whatever layout the next call uses.
    __syncthreads();
    for (int i = tid; i < kBins; i += kThreads) W.hist[i] = 0;
    for (int i = tid; i < cnt_raw[1]; i += kThreads) { W.cand_key[i] = 0; W.cand_idx[i] = 0; }
    for (int i = tid; i < cnt_raw[0]; i += kThreads) W.sel[i] = 0;
    if (tid < 16) W.ctr[tid] = 0;
}

template <typename T, int LPR>
hipError_t launch_score(const void* q_idx, const void* k_idx, int B, const int32_t* q_seq,
                        const int32_t* n_cand, float* scores, uint8_t* ws, int Nq, int H_I,
                        int S_max, int k, bool hist, hipStream_t st) {
    const int rows = hist ? kScoreRowsMulti : min(S_max, 8192);
    dim3 grid((unsigned)ceil_div(S_max, rows), (unsigned)Nq);
    ProfScope prof(kProfScore, st);
    if (hist)
        hipLaunchKernelGGL((score_kernel<T, LPR, true>), grid, dim3(kThreads), 0, st,
                           (const T*)q_idx, (const T*)k_idx, q_seq, n_cand, scores, ws, B, H_I,
                           S_max, k, rows);
    else
        hipLaunchKernelGGL((score_kernel<T, LPR, false>), grid, dim3(kThreads), 0, st,
                           (const T*)q_idx, (const T*)k_idx, q_seq, n_cand, scores, ws, B, H_I,
                           S_max, k, rows);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_score_t(int d_I, const void* q_idx, const void* k_idx, int B,
                          const int32_t* q_seq, const int32_t* n_cand, float* scores, uint8_t* ws,
                          int Nq, int H_I, int S_max, int k, bool hist, hipStream_t st) {
    const int lpr = d_I * (int)sizeof(T) / 16;
    if (lpr == 8)
        return launch_score<T, 8>(q_idx, k_idx, B, q_seq, n_cand, scores, ws, Nq, H_I, S_max, k, hist, st);
    if (lpr == 16)
        return launch_score<T, 16>(q_idx, k_idx, B, q_seq, n_cand, scores, ws, Nq, H_I, S_max, k, hist, st);
    return launch_score<T, 32>(q_idx, k_idx, B, q_seq, n_cand, scores, ws, Nq, H_I, S_max, k, hist, st);
}

}  // namespace

size_t topk_workspace_bytes(int Nq, int S_max, int k) {
    if (S_max <= kRowSelectCap) return 0;
    return (size_t)Nq * ws_per_query(S_max, k);
}

hipError_t launch_index_topk(int dtype, const void* q_idx, const void* k_idx, int B,
                             const int32_t* q_seq, const int32_t* n_cand, float* scores,
                             int32_t* topk_idx, int Nq, int H_I, int d_I, int S_max, int k,
                             void* ws, hipStream_t st) {
    const bool multi = S_max > kRowSelectCap;
    uint8_t* w = static_cast<uint8_t*>(ws);
    hipError_t e = hipSuccess;
    if (q_idx) {
        e = dtype == kF32 ? launch_score_t<float>(d_I, q_idx, k_idx, B, q_seq, n_cand, scores, w,
                                                   Nq, H_I, S_max, k, multi, st)
                          : launch_score_t<bf16_t>(d_I, q_idx, k_idx, B, q_seq, n_cand, scores,
                                                   w, Nq, H_I, S_max, k, multi, st);
        if (e != hipSuccess) return e;
    } else if (multi) {
        dim3 grid((unsigned)ceil_div(S_max, kFilterChunk), (unsigned)Nq);
        ProfScope prof(kProfSelect, st);
        hipLaunchKernelGGL(hist_kernel, grid, dim3(kThreads), 0, st, scores, n_cand, w, S_max, k,
                           kFilterChunk);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    ProfScope prof(kProfSelect, st);
    if (!multi) {
        hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)Nq), dim3(kThreads), 0, st, scores,
                           n_cand, topk_idx, S_max, k);
    } else {
        const int G = ceil_div(S_max, kFilterChunk);
        hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)G, (unsigned)Nq), dim3(kThreads), 0,
                           st, scores, n_cand, topk_idx, w, S_max, k, G);
    }
    return hipGetLastError();
}

}  // namespace hsa
