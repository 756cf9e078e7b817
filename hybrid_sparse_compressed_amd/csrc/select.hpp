// select.hpp -- workspace layout and device steps of the multi-workgroup
// exact top-k, shared by the final select kernel (index_topk.hip) and the
// fused sparse-decode attention kernel (attention.hip).
//
// [KD "Arquitectura del Sistema"] and [NK "推理侧优化", Lightning topk
// bullet]: the C4 top-k is a radix select.  Order: score descending, equal
// scores by lower index; keys are the order-preserving u32 images of the
// fp32 scores (score_key).  The scoring kernel builds the histogram of the
// top 11 key bits, the filter kernel writes per segment of 4096 candidates
// the candidates above the threshold bin ("selected") and inside it ("short
// list"), both in index order, and the steps here finish the select for one
// query inside one workgroup of 256 threads.
#pragma once

#include "hsa_common.hpp"
#include "hsa_internal.hpp"

namespace hsa {
namespace sel {

constexpr int kSelThreads = 256;
constexpr int kSelNW = kSelThreads / kWave;
constexpr int kBins = 2048;         // first digit: key bits 31..21
constexpr int kFilterChunk = 4096;  // candidates per filter segment
constexpr int kCandCap = 4096;      // short-list entries kept in LDS
constexpr int kMaxSeg = kTopkMaxSegments;

// ---- workspace (multi-workgroup path), per query -------------------------
//   hist[2048] u32 (key bits 31..21 of every candidate) | hist2[2048] u32
//   (key bits 20..10 of the short list) | ctr[16] u32 (reserved) |
//   seg[nseg] u32 (per filter segment: short-list count | selected count << 16)
//   | cand_key[S_max] | cand_idx[S_max] (segment g owns [4096 g, 4096 g + 4096):
//   its short-list (key, index) pairs first, then its selected indices) |
//   flat_key[S_max] | flat_idx[S_max] (the whole short list in one run, used
//   only when it does not fit in LDS)
__host__ __device__ inline int n_segments(int S_max) { return (S_max + kFilterChunk - 1) / kFilterChunk; }
__host__ __device__ inline size_t ws_per_query(int S_max, int k) {
    (void)k;
    size_t b = (size_t)kBins * 8 + 64 + (size_t)n_segments(S_max) * 4 + (size_t)S_max * 16;
    return (b + 255) & ~(size_t)255;
}

struct QWs {
    uint32_t* hist;
    uint32_t* hist2;
    uint32_t* ctr;
    uint32_t* seg;
    uint32_t* cand_key;
    uint32_t* cand_idx;
    uint32_t* flat_key;
    uint32_t* flat_idx;
};

__device__ inline QWs ws_of(uint8_t* ws, int q, int S_max, int k) {
    uint8_t* base = ws + (size_t)q * ws_per_query(S_max, k);
    QWs w;
    w.hist = reinterpret_cast<uint32_t*>(base);
    w.hist2 = w.hist + kBins;
    w.ctr = w.hist2 + kBins;
    w.seg = w.ctr + 16;
    w.cand_key = w.seg + n_segments(S_max);
    w.cand_idx = w.cand_key + S_max;
    w.flat_key = w.cand_idx + S_max;
    w.flat_idx = w.flat_key + S_max;
    return w;
}

__device__ inline int clamp_n(const int32_t* n_cand, int q, int S_max) {
    int n = n_cand[q];
    return n < 0 ? 0 : (n > S_max ? S_max : n);
}

// Candidates of query q: n_cand[q] clamped to [0, S_max], or none when q_seq
// (may be null) sends the query to a sequence outside [0, B).
__device__ inline int query_n(const int32_t* n_cand, const int32_t* q_seq, int B, int q, int S_max) {
    if (q_seq) {
        const int b = q_seq[q];
        if (b < 0 || b >= B) return 0;
    }
    return clamp_n(n_cand, q, S_max);
}

// ---- LDS radix machinery -------------------------------------------------------
// Given bin counts h[0..NB), find the bin d such that (members in bins above d)
// < need <= (members in bins above d) + h[d].  Returns d; *rem = need minus the
// members above d.  Every thread calls it (it has barriers).
template <int NB>
__device__ int find_crossing(const uint32_t* h, int need, uint32_t* tmp, int* rem) {
    static_assert(NB % kSelThreads == 0, "bins must be a multiple of the workgroup size");
    constexpr int BPT = NB / kSelThreads;
    __shared__ int res[2];
    const int tid = threadIdx.x;
    const int grp = kSelThreads - 1 - tid;  // thread 0 owns the top bins
    if (tid == 0) { res[0] = 0; res[1] = 1; }
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) s += h[grp * BPT + j];
    uint32_t tot;
    const uint32_t above = block_excl_scan<kSelThreads>(s, tmp, &tot);
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
    for (int i = tid; i < NB; i += kSelThreads) h[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
        const uint32_t kk = keys[i];
        if ((kk & pmask) == pref && (eq_key == nullptr || eq_key[i] == eq_val))
            atomicAdd(&h[(kk >> shift) & (NB - 1)], 1u);
    }
    __syncthreads();
    return find_crossing<NB>(h, need, tmp, rem);
}

// lower bound of v in the ascending LDS list a[0..n)
__device__ __forceinline__ uint32_t lower_bound_lds(const int32_t* a, uint32_t n, int32_t v) {
    uint32_t lo = 0, hi = n;
    while (lo < hi) {
        const uint32_t mid = (lo + hi) >> 1;
        if (a[mid] < v) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// ---- one query's select inside one workgroup ---------------------------------
// LDS working set (any LDS the caller owns; nothing else may use it meanwhile).
struct SelLds {
    uint32_t* h;      // [kBins]
    uint32_t* tmp;    // [2 * kSelNW + 2]
    uint32_t* segc;   // [kMaxSeg] per segment: short count | selected count << 16
    uint32_t* sbase;  // [kMaxSeg] first short-list position of the segment
    uint32_t* lbase;  // [kMaxSeg] first selected-list position of the segment
    uint32_t* ck;     // [kCandCap] short-list keys   (when it fits)
    uint32_t* ci;     // [kCandCap] short-list indices
    int32_t* sel;     // [kTopkMaxK] selected indices, ascending
    int32_t* chs;     // [kTopkMaxK] chosen short-list indices, ascending
    uint32_t* misc;   // [4]
    uint32_t* mem;    // [3 * kSelThreads] crossing-bucket members: position, key, index
    uint8_t* flag;    // [kCandCap] chosen flags of crossing-bucket members
    u32x4* stage;     // [kSelThreads * 16] list entries of one read round (select_query_lists)
};

struct SelResult {
    int nseg;    // filter segments
    int take;    // min(k, n)
    int nc;      // short-list length
    int nsel;    // selected-list length (<= take)
    int nch;     // chosen short-list entries (nsel + nch = take)
    int T_s;     // threads per segment in the gather / zero mapping
    bool unordered;  // select_query_lists: the lists are not in index order (see there)
};

// The steps after the runs are placed.  L.h holds the second-digit
// histogram (key bits 20..10) of the short list, whose members all share the
// threshold bin; the short list is in L.ck / L.ci (small) or in W.flat_key /
// W.flat_idx; R.nc and R.nsel are set and `need` = R.take - R.nsel > 0 of the
// short list are to be chosen.  Leaves the chosen entries in L.chs, ascending,
// and sets R.nch.  Every thread calls it.
// SMALL (the short list is in LDS) is a template argument so that the list
// pointers are known to be LDS or global: a pointer that may be either makes
// every access a flat one.
template <bool SMALL>
__device__ inline void select_finish_t(const QWs& W, SelResult& R, int need, const SelLds& L) {
    const int tid = threadIdx.x;
    constexpr bool small = SMALL;
    // 3. the crossing bucket of the second digit and how much of it is taken
    const uint32_t* key = SMALL ? L.ck : W.flat_key;
    const uint32_t* idx = SMALL ? L.ci : W.flat_idx;
    const int nc = R.nc;
    uint32_t* h = L.h;
    bool whole, direct = false;
    uint32_t p2, T, imax = 0xffffffffu;
    {
        const uint32_t p1 = key[0] & 0xffe00000u;  // the threshold bin's 11 bits
        int rem;
        const int d2 = find_crossing<kBins>(h, need, L.tmp, &rem);
        p2 = p1 | ((uint32_t)d2 << 10);
        // read by all before h is reused
        const uint32_t members = h[d2];
        whole = (int)members == rem;
        if (tid == 0) L.misc[1] = 0;
        __syncthreads();
        need = rem;
        T = p2;
        if (!whole && small && members <= (uint32_t)kSelThreads) {
            // rank the bucket's members directly: (key desc, index asc)
            direct = true;
            uint32_t* mpos = L.mem;
            uint32_t* mkey = L.mem + kSelThreads;
            uint32_t* midx = L.mem + 2 * kSelThreads;
            for (int i = tid; i < nc; i += kSelThreads) {
                const uint32_t kk = key[i];
                if ((kk & 0xfffffc00u) == p2) {
                    const uint32_t slot = atomicAdd(&L.misc[1], 1u);
                    mpos[slot] = (uint32_t)i;
                    mkey[slot] = kk;
                    midx[slot] = idx[i];
                }
            }
            __syncthreads();
            if (tid < (int)members) {
                const uint32_t mk = mkey[tid], mi = midx[tid];
                uint32_t rank = 0;
                for (uint32_t j = 0; j < members; ++j) {
                    const uint32_t kj = mkey[j];
                    rank += (kj > mk) || (kj == mk && midx[j] < mi);
                }
                L.flag[mpos[tid]] = rank < (uint32_t)need ? 1 : 0;
            }
            __syncthreads();
        } else if (!whole) {
            const int d3 = radix_digit<1024>(key, nc, 0xfffffc00u, p2, 0, nullptr, 0u, need, h, L.tmp, &rem);
            need = rem;
            T = p2 | (uint32_t)d3;
            uint32_t eq = 0;
            for (int i = tid; i < nc; i += kSelThreads) eq += key[i] == T;
            uint32_t eq_all;
            block_excl_scan<kSelThreads>(eq, L.tmp, &eq_all);
            if ((int)eq_all > need) {
                // the need lowest indices among the T-valued: digits of ~idx, highest first
                int rr = need;
                uint32_t pr = 0, pm = 0;
                const int shifts[3] = {21, 10, 0};
                const int widths[3] = {11, 11, 10};
                for (int pass = 0; pass < 3; ++pass) {
                    const int nb = 1 << widths[pass];
                    for (int i = tid; i < kBins; i += kSelThreads) h[i] = 0;
                    __syncthreads();
                    for (int i = tid; i < nc; i += kSelThreads) {
                        if (key[i] != T) continue;
                        const uint32_t ni = ~idx[i];
                        if ((ni & pm) == pr) atomicAdd(&h[(ni >> shifts[pass]) & (nb - 1)], 1u);
                    }
                    __syncthreads();
                    const int d = (nb == kBins) ? find_crossing<kBins>(h, rr, L.tmp, &rem)
                                                : find_crossing<1024>(h, rr, L.tmp, &rem);
                    rr = rem;
                    pr |= (uint32_t)d << shifts[pass];
                    pm |= (uint32_t)(nb - 1) << shifts[pass];
                }
                imax = ~pr;  // indices <= imax among the T-valued are taken
            }
        }
    }

    // 4. chosen short-list entries, compacted in order (contiguous ranges per thread)
    {
        const int E = ceil_div(nc, kSelThreads);
        const int i0 = min(nc, tid * E), i1 = min(nc, i0 + E);
        auto chosen = [&](int i) {
            const uint32_t kk = key[i];
            if (whole) return kk >= p2;
            if (direct) return kk >= p2 + 1024u || ((kk & 0xfffffc00u) == p2 && L.flag[i] != 0);
            return kk > T || (kk == T && idx[i] <= imax);
        };
        // short list in LDS: at most kCandCap / kSelThreads = 16 entries per
        // thread, whose chosen flags are read once (all reads in flight) into
        // a mask; the flat copy keeps the two plain passes
        constexpr int EMAX = kCandCap / kSelThreads;
        static_assert(EMAX <= 32, "chosen mask is 32 bits");
        uint32_t mask = 0, cnt = 0;
        if (small) {
#pragma unroll
            for (int j = 0; j < EMAX; ++j) {
                const int i = i0 + j;
                if (i < i1 && chosen(i)) mask |= 1u << j;
            }
            cnt = (uint32_t)__popc(mask);
        } else {
            for (int i = i0; i < i1; ++i) cnt += chosen(i);
        }
        uint32_t all;
        uint32_t pos = block_excl_scan<kSelThreads>(cnt, L.tmp, &all);
        if (small) {
            while (mask) {
                const int j = __ffs(mask) - 1;
                mask &= mask - 1;
                if (pos < (uint32_t)kTopkMaxK) L.chs[pos] = (int32_t)idx[i0 + j];
                ++pos;
            }
        } else {
            for (int i = i0; i < i1; ++i)
                if (chosen(i)) {
                    if (pos < (uint32_t)kTopkMaxK) L.chs[pos] = (int32_t)idx[i];
                    ++pos;
                }
        }
        if (tid == 0) L.misc[0] = all;
        __syncthreads();
        R.nch = min((int)L.misc[0], R.take - R.nsel);
    }
}

__device__ inline void select_finish(const QWs& W, SelResult& R, int need, bool small,
                                     const SelLds& L) {
    if (small) select_finish_t<true>(W, R, need, L);
    else select_finish_t<false>(W, R, need, L);
}

// Gathers the selected list (ascending, all of it) and, when positions past
// it are needed (j_need > its length), the short list, then resolves the
// short list from the second-digit histogram: buckets above the crossing
// bucket are taken, and the crossing bucket is taken whole, or its members
// (at most kSelThreads of them, short list in LDS) are ranked directly under
// (key desc, index asc), or else one 10-bit pass gives the k-th key and three
// passes over complemented indices settle a tie that straddles rank k.  The
// chosen short-list entries are then compacted in order.  The result lists
// are L.sel[0..nsel) and
// L.chs[0..nch), both ascending; the first take = nsel + nch entries of the
// query's top-k are their union.  Short lists longer than kCandCap go through
// W.flat_key / W.flat_idx (every caller that reaches that path writes the
// same values).  Every thread calls it.
__device__ inline SelResult select_query(const QWs& W, int n, int S_max, int k, int j_need,
                                        const SelLds& L) {
    const int tid = threadIdx.x;
    SelResult R;
    R.nseg = n_segments(S_max);
    R.take = min(k, n);
    R.unordered = false;

    // 1. segment counts, the second-digit histogram and the first entries of
    //    every segment's runs, all loads in flight together: T_s threads per
    //    segment, thread r of a segment takes entries r, r + T_s, ... and the
    //    first kSpec of them are read before their count is known (they lie
    //    inside the segment's slots, so reading them is always in bounds)
    constexpr int SPT = kMaxSeg / kSelThreads;  // segments per thread in the scan (contiguous)
    constexpr int kSpec = 12;
    int T_s = 1;
    while (T_s * 2 * R.nseg <= kSelThreads) T_s *= 2;
    R.T_s = T_s;
    const int par = kSelThreads / T_s, r = tid % T_s, g0 = tid / T_s;
    uint32_t c[SPT], hv[kBins / kSelThreads], kk[kSpec], ii[kSpec];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        const int gg = tid * SPT + j;
        c[j] = gg < R.nseg ? W.seg[gg] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kBins / kSelThreads; ++j) hv[j] = W.hist2[tid + j * kSelThreads];
    if (g0 < R.nseg) {
        const uint32_t base = (uint32_t)g0 * kFilterChunk;
        const uint32_t room = (uint32_t)min(kFilterChunk, S_max - g0 * kFilterChunk);  // slots of the segment
#pragma unroll
        for (int u = 0; u < kSpec; ++u) {
            const uint32_t j = (uint32_t)(r + u * T_s);
            ii[u] = j < room ? W.cand_idx[base + j] : 0u;
            kk[u] = j < room ? W.cand_key[base + j] : 0u;
        }
    }
    uint32_t s_short = 0, s_sel = 0;
#pragma unroll
    for (int j = 0; j < SPT; ++j) { s_short += c[j] & 0xffffu; s_sel += c[j] >> 16; }
    uint32_t nc_all, nsel_all;
    uint32_t b_short, b_sel;
    block_excl_scan2<kSelThreads>(s_short, s_sel, L.tmp, &b_short, &b_sel, &nc_all, &nsel_all);
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        const int gg = tid * SPT + j;
        if (gg < R.nseg) { L.segc[gg] = c[j]; L.sbase[gg] = b_short; L.lbase[gg] = b_sel; }
        b_short += c[j] & 0xffffu;
        b_sel += c[j] >> 16;
    }
#pragma unroll
    for (int j = 0; j < kBins / kSelThreads; ++j) L.h[tid + j * kSelThreads] = hv[j];
    __syncthreads();
    R.nc = (int)nc_all;
    R.nsel = min((int)nsel_all, R.take);
    const bool small = R.nc <= kCandCap;
    int need = R.take - R.nsel;
    const bool refine = need > 0 && R.nc > 0 && j_need > R.nsel;  // uniform

    // 2. place the runs: the speculative entries first, then whatever lies past them
    auto place = [&](int gg, uint32_t j, uint32_t kv, uint32_t iv) {
        const uint32_t cs = L.segc[gg] & 0xffffu, cnt = cs + (L.segc[gg] >> 16);
        if (j < cs) {
            if (refine) {
                const uint32_t d = L.sbase[gg] + j;
                if (small) { L.ck[d] = kv; L.ci[d] = iv; }
                else { W.flat_key[d] = kv; W.flat_idx[d] = iv; }
            }
        } else if (j < cnt) {
            const uint32_t d = L.lbase[gg] + (j - cs);
            if (d < (uint32_t)kTopkMaxK) L.sel[d] = (int32_t)iv;
        }
    };
    if (g0 < R.nseg) {
#pragma unroll
        for (int u = 0; u < kSpec; ++u) place(g0, (uint32_t)(r + u * T_s), kk[u], ii[u]);
    }
    for (int gg = g0; gg < R.nseg; gg += par) {
        const uint32_t cs = L.segc[gg] & 0xffffu, cnt = cs + (L.segc[gg] >> 16);
        const uint32_t base = (uint32_t)gg * kFilterChunk;
        const uint32_t jstart = (uint32_t)r + (gg == g0 ? (uint32_t)(kSpec * T_s) : 0u);
        for (uint32_t j0 = jstart; j0 < cnt; j0 += 8u * (uint32_t)T_s) {
            uint32_t k8[8], i8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t j = j0 + (uint32_t)(u * T_s);
                i8[u] = j < cnt ? W.cand_idx[base + j] : 0u;
                k8[u] = (refine && j < cs) ? W.cand_key[base + j] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) place(gg, j0 + (uint32_t)(u * T_s), k8[u], i8[u]);
        }
    }
    __syncthreads();
    R.nch = 0;
    if (!refine) return R;

    select_finish(W, R, need, small, L);
    return R;
}

// ---- per-workgroup candidate lists (fused decode select) ----------------------
// Scoring workgroup g covers rows [2048 g, 2048 g + 2048) of its query.  Next
// to the first-digit histogram it leaves a list, in index order, of its
// candidates whose first digit (key bits 31..21) is at least a_g, the lowest
// bin that has at most `cap` of its candidates at or above it, and records
// a_g: candidates it left out have first digits below a_g.  If the query's
// threshold bin t1 (the bin where the top-k crosses, from the completed
// histogram) is at least every a_g, the lists hold every candidate in t1 or
// above, which is all the select reads; the filter pass over the whole score
// row is then not needed.  When some a_g exceeds t1 (a workgroup holds more
// than `cap` candidates at or above t1: far more than its share on typical
// rows, but possible for adversarial or tied scores) the select falls back to
// passes over the score row itself, with the same result.
constexpr int kListRows = 2048;   // most rows per scoring workgroup (slot)
constexpr int kListEPT = 32;      // list entries per thread per read round

// log2 of the rows per slot: 2048, halved while the Nq queries would give
// fewer than 512 scoring workgroups (two per compute unit), down to 256
__host__ __device__ inline int list_rows_log2(int S_max, int Nq) {
    int lg = 11;
    while (lg > 8 && (long long)Nq * ((S_max + (1 << lg) - 1) >> lg) < 512) --lg;
    return lg;
}
__host__ __device__ inline int list_slots(int S_max, int rows_lg) {
    return (S_max + (1 << rows_lg) - 1) >> rows_lg;
}

// log2 of the list capacity per slot: the smallest power of two in [64, 256]
// that is at least four times a slot's even share of the top-k,
// 4 k rows / S_max (compared by products: no division on the device)
__host__ __device__ inline int list_cap_log2(int S_max, int k, int rows_lg) {
    const long long need = ((long long)4 * k) << rows_lg;
    int lg = 6;
    while (lg < 8 && ((long long)S_max << lg) < need) ++lg;
    return lg;
}

// words of the list area: headers, alignment pad, keys and indices in whole
// rounds of 8192
__host__ __device__ inline long long list_words(int S_max, int k, int rows_lg) {
    const long long slots = list_slots(S_max, rows_lg);
    const long long ent = ((slots << list_cap_log2(S_max, k, rows_lg)) + 8191) & ~8191LL;
    return slots + 3 + 2 * ent;
}

// the lists are used when that capacity covers four even shares, every
// header is read in one pass and the lists fit the candidate area
__host__ __device__ inline bool lists_apply(int S_max, int k, int Nq) {
    const int rl = list_rows_log2(S_max, Nq);
    return S_max > kRowSelectCap && (((long long)4 * k) << rl) <= 256LL * S_max &&
           list_slots(S_max, rl) <= 2048 && list_words(S_max, k, rl) <= 2LL * S_max;
}

// Lists live in the query's candidate area (cand_key / cand_idx, 2 S_max
// words): hdr[nslot] (count | a_g << 16), then key[] and idx[] (16-byte
// aligned), nslot * cap words each rounded up to whole rounds of 8192 (at
// most S_max / 2 + 16384 words in all, within 2 S_max for S_max > 12288).
// Entry j of slot g has the flat number
// e = g * cap + j; the reader takes rounds of 8192 entries, thread t the 32
// consecutive entries 32t .. 32t + 31 of a round in eight 16-byte loads, and
// the words are stored so that load u of every thread of the workgroup is
// one contiguous 4 KB run: e sits at list_pos(e), with entries 4u .. 4u + 3
// of thread t at words 1024 u + 4 t .. + 3 of the round.
__host__ __device__ inline uint32_t list_pos(uint32_t e) {
    return (e & ~8191u) | (((e >> 2) & 7u) << 10) | (((e >> 5) & 255u) << 2) | (e & 3u);
}
static_assert(kListEPT == 32 && kSelThreads == 256, "list_pos assumes 256 readers x 32 entries");

struct Lists {
    uint32_t* hdr;
    uint32_t* key;
    uint32_t* idx;
    int nslot, cap, cap_lg, rows_lg;
};
// rows_lg: list_rows_log2(S_max, Nq), which the host passes down
__device__ inline Lists lists_of(const QWs& W, int S_max, int k, int rows_lg) {
    Lists l;
    l.rows_lg = rows_lg;
    l.nslot = list_slots(S_max, l.rows_lg);
    l.cap_lg = list_cap_log2(S_max, k, l.rows_lg);
    l.cap = 1 << l.cap_lg;
    l.hdr = W.cand_key;
    // 16-byte alignment by an index offset (a pointer rebuilt from an integer
    // would lose its global address space and turn the loads into flat ones)
    const int pad = (int)((0u - (uint32_t)(reinterpret_cast<uintptr_t>(l.hdr + l.nslot) >> 2)) & 3u);
    l.key = l.hdr + l.nslot + pad;
    // list_pos spreads a round over 8192 words: whole rounds are reserved
    l.idx = l.key + ((((size_t)l.nslot << l.cap_lg) + 8191) & ~(size_t)8191);
    return l;
}

// f(i, key) for every candidate i < n (n >= 1) of a score row, all threads:
// sixteen coalesced loads per thread in flight at once (clamped indices past
// the row are loaded and skipped)
template <typename F>
__device__ __forceinline__ void for_each_key(const float* srow, int n, F&& f) {
    constexpr int U = 16;
    for (int i0 = (int)threadIdx.x; i0 < n; i0 += U * kSelThreads) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = srow[min(i0 + u * kSelThreads, n - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kSelThreads;
            if (i < n) f(i, score_key(v[u]));
        }
    }
}

// Exact select by passes over the query's score row (the lists' fallback):
// t1 / rem1 are the threshold bin and how many of it are taken (take < n).
// Leaves the whole selection in L.sel[0..take), ascending (R.nch = 0).
__device__ inline void select_scan(const float* srow, int n, int S_max, int t1, int rem1,
                                   const SelLds& L, SelResult& R) {
    const int tid = threadIdx.x;
    (void)S_max;
    uint32_t* h = L.h;
    uint32_t pref = (uint32_t)t1 << 21, pmask = 0xffe00000u;
    int need = rem1, rem;
    uint32_t eq = 0;  // candidates equal to the k-th key
    // second digit (bits 20..10) and third digit (bits 9..0) of the threshold
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 10 : 0;
        const uint32_t nbm = pass == 0 ? (uint32_t)(kBins - 1) : 1023u;
        for (int i = tid; i < kBins; i += kSelThreads) h[i] = 0;
        __syncthreads();
        for_each_key(srow, n, [&](int, uint32_t kk) {
            if ((kk & pmask) == pref) atomicAdd(&h[(kk >> shift) & nbm], 1u);
        });
        __syncthreads();
        const int d = pass == 0 ? find_crossing<kBins>(h, need, L.tmp, &rem)
                                : find_crossing<1024>(h, need, L.tmp, &rem);
        if (pass == 1) eq = h[d];
        __syncthreads();  // h read by all before the next pass clears it
        need = rem;
        pref |= (uint32_t)d << shift;
        pmask |= nbm << shift;
    }
    const uint32_t T = pref;
    uint32_t imax = 0xffffffffu;
    if (eq > (uint32_t)need) {
        // the `need` lowest indices among those equal to T: digits of ~index
        int rr = need;
        uint32_t pr = 0, pm = 0;
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);  // 11, 11, 10 bits
            const uint32_t nbm = pass == 2 ? 1023u : (uint32_t)(kBins - 1);
            for (int i = tid; i < kBins; i += kSelThreads) h[i] = 0;
            __syncthreads();
            for_each_key(srow, n, [&](int i, uint32_t kk) {
                const uint32_t ni = ~(uint32_t)i;
                if (kk == T && (ni & pm) == pr) atomicAdd(&h[(ni >> shift) & nbm], 1u);
            });
            __syncthreads();
            const int d = pass < 2 ? find_crossing<kBins>(h, rr, L.tmp, &rem)
                                   : find_crossing<1024>(h, rr, L.tmp, &rem);
            rr = rem;
            pr |= (uint32_t)d << shift;
            pm |= nbm << shift;
        }
        imax = ~pr;
    }
    // every chosen candidate in index order, 16 consecutive per thread and
    // round; the next round's scores are loaded before this round's scan
    constexpr int E = 16;
    uint32_t base = 0;
    float v[E];
    auto load = [&](int r0) {
        const int i0 = r0 + tid * E;
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = srow[min(i0 + j, n - 1)];  // clamped, unconditional
    };
    load(0);
#pragma unroll 1
    for (int r0 = 0; r0 < n; r0 += E * kSelThreads) {
        const int i0 = r0 + tid * E;
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const int i = i0 + j;
            const uint32_t kk = score_key(v[j]);
            if (i < n && (kk > T || (kk == T && (uint32_t)i <= imax))) m |= 1u << j;
        }
        if (r0 + E * kSelThreads < n) load(r0 + E * kSelThreads);
        uint32_t all;
        uint32_t pos = base + block_excl_scan<kSelThreads>((uint32_t)__popc(m), L.tmp, &all);
        while (m) {
            const int j = __ffs(m) - 1;
            m &= m - 1;
            if (pos < (uint32_t)kTopkMaxK) L.sel[pos] = i0 + j;
            ++pos;
        }
        base += all;
    }
    __syncthreads();
    R.nsel = R.take;
    R.nc = 0;
    R.nch = 0;
}

// One query's select inside one workgroup from the scoring workgroups' lists
// (the fused decode path): the completed first-digit histogram gives the
// threshold bin t1; the lists' candidates above it form the selected list and
// those inside it the short list (both ascending), whose second-digit
// histogram is built here; then as select_query.  Positions below j_need of
// the result are what the caller needs (the short list is resolved only if
// they reach past the selected list).  srow: the query's scores (fallback).
//   after_loads(): called once every thread's first list loads are issued
//   (the caller's own loads that the select does not wait for go there)
template <typename F>
__device__ inline SelResult select_query_lists(const QWs& W, const float* srow, int n, int S_max,
                                               int k, int rows_lg, int j_need, const SelLds& L,
                                               F&& after_loads) {
    const int tid = threadIdx.x;
    SelResult R;
    R.nseg = 0;
    R.T_s = 1;
    R.unordered = false;
    R.take = min(k, n);
    R.nc = 0;
    R.nsel = 0;
    R.nch = 0;
    if (R.take == n) {  // every candidate is taken (also n = 0)
        after_loads();
        for (int i = tid; i < n; i += kSelThreads) L.sel[i] = i;
        __syncthreads();
        R.nsel = n;
        return R;
    }
    const Lists Ls = lists_of(W, S_max, k, rows_lg);
    const int total = Ls.nslot << Ls.cap_lg;
    const int rounds = (total + kListEPT * kSelThreads - 1) >> 13;
    static_assert(kListEPT * kSelThreads == 8192, "rounds of 8192 entries");

    // 1. histogram, every list header and the first round of list entries,
    //    all loads in flight together (entries past the lists are clamped in
    //    bounds and ignored)
    u32x4 h0, h1;
    {
        const u32x4* hs = reinterpret_cast<const u32x4*>(W.hist);
        h0 = hs[tid];
        h1 = hs[tid + kSelThreads];
    }
    // Loads are unconditional (clamped indices, values past the end masked
    // afterwards): a load inside a branch gets its use scheduled inside the
    // branch too, and that wait would hold back every load issued after it.
    constexpr int kHdrPT = 8;  // headers per thread per pass (2048 slots in one pass)
    uint32_t hv[kHdrPT];
#pragma unroll
    for (int j = 0; j < kHdrPT; ++j) hv[j] = Ls.hdr[min(tid + j * kSelThreads, Ls.nslot - 1)];
    // (lists_apply keeps nslot <= kHdrPT * kSelThreads = 2048)
    u32x4 kq[kListEPT / 4], iq[kListEPT / 4];
    uint32_t own_hdr;
    // a thread past the lists reads its round's first entries (in bounds:
    // rounds are reserved whole) and ignores them
    auto load_round = [&](int rd) {
        const int e0 = rd * kListEPT * kSelThreads + tid * kListEPT;
        const bool in = e0 < total;
        own_hdr = Ls.hdr[min(e0 >> Ls.cap_lg, Ls.nslot - 1)];  // unconditional; masked by `in` below
        const int rb = rd * kListEPT * kSelThreads;
        const int t = in ? tid : 0;
#pragma unroll
        for (int j = 0; j < kListEPT / 4; ++j) {
            const int w = rb + j * 4 * kSelThreads + 4 * t;
            kq[j] = *reinterpret_cast<const u32x4*>(Ls.key + w);
            iq[j] = *reinterpret_cast<const u32x4*>(Ls.idx + w);
        }
    };
    load_round(0);
    after_loads();

    // 2. threshold bin and the check that no list left out a candidate in it or above
    reinterpret_cast<u32x4*>(L.h)[tid] = h0;
    reinterpret_cast<u32x4*>(L.h)[tid + kSelThreads] = h1;
    __syncthreads();
    int rem1;
    const int t1 = find_crossing<kBins>(L.h, R.take, L.tmp, &rem1);
    const uint32_t nc = L.h[t1];
    // slots whose list was cut above t1 ("short" slots: their lists may miss
    // candidates of bin t1 or above), listed in L.mem in (thread, pass) order
    uint32_t badm = 0;
#pragma unroll
    for (int j = 0; j < kHdrPT; ++j)
        if (tid + j * kSelThreads < Ls.nslot && (int)(hv[j] >> 16) > t1) badm |= 1u << j;
    uint32_t nbad;
    uint32_t bpos = block_excl_scan<kSelThreads>((uint32_t)__popc(badm), L.tmp, &nbad);  // barriers: L.h read by all
    if (nbad > (uint32_t)(3 * kSelThreads)) {  // uniform: too many to list, select from the score row
        select_scan(srow, n, S_max, t1, rem1, L, R);
        return R;
    }
#pragma unroll
    for (int j = 0; j < kHdrPT; ++j)
        if ((badm >> j) & 1u) L.mem[bpos++] = (uint32_t)(tid + j * kSelThreads);
    R.unordered = nbad > 0;
    R.nc = (int)nc;
    R.nsel = R.take - rem1;
    const int need = rem1;
    const bool refine = j_need > R.nsel;  // uniform; need >= 1 and nc >= need here
    const bool small = R.nc <= kCandCap;
    if (refine)
        for (int i = tid; i < kBins; i += kSelThreads) L.h[i] = 0;
    __syncthreads();

    // 3. route each round's entries: above t1 -> selected list, t1 -> short list
    uint32_t bsel = 0, bsh = 0;
#pragma unroll 1
    for (int rd = 0; rd < rounds; ++rd) {
        if (rd > 0) load_round(rd);
        const int e0 = rd * kListEPT * kSelThreads + tid * kListEPT;
        // valid entries here (own_hdr is a clamped slot's past the lists); a
        // short slot's list is skipped: its rows are read below
        const int cnt = (e0 < total && (int)(own_hdr >> 16) <= t1)
                            ? (int)(own_hdr & 0xffffu) - (e0 & (Ls.cap - 1)) : 0;
        uint32_t selm = 0, shm = 0;
#pragma unroll
        for (int j = 0; j < kListEPT; ++j) {
            const uint32_t kk = kq[j / 4][j % 4];
            const int bin = (int)(kk >> 21);
            if (j < cnt && bin > t1) selm |= 1u << j;
            if (j < cnt && bin == t1) shm |= 1u << j;
        }
        if (!refine) shm = 0;
        // the thread's 32 keys and indices go to its own 256 bytes of LDS
        // (chunk c at slot c ^ (t & 15): the 16 lanes of an LDS pass hit 16
        // different columns), so the few set bits below are visited with
        // dynamic indices that stay out of scratch memory
        u32x4* st = L.stage + tid * 16;
        const int sw = tid & 15;
#pragma unroll
        for (int j = 0; j < kListEPT / 4; ++j) {
            st[j ^ sw] = kq[j];
            st[(8 + j) ^ sw] = iq[j];
        }
        uint32_t ps, pc, ts, tc;
        block_excl_scan2<kSelThreads>((uint32_t)__popc(selm), (uint32_t)__popc(shm), L.tmp, &ps, &pc,
                                      &ts, &tc);
        ps += bsel;
        pc += bsh;
        const uint32_t* sw32 = reinterpret_cast<const uint32_t*>(st);
        auto stage_at = [&](int c, int j) { return sw32[((c ^ sw) << 2) | (j & 3)]; };
        while (selm) {
            const int j = __ffs(selm) - 1;
            selm &= selm - 1;
            if (ps < (uint32_t)kTopkMaxK) L.sel[ps] = (int32_t)stage_at(8 + (j >> 2), j);
            ++ps;
        }
        while (shm) {
            const int j = __ffs(shm) - 1;
            shm &= shm - 1;
            const uint32_t kk = stage_at(j >> 2, j), ii = stage_at(8 + (j >> 2), j);
            if (small) {
                if (pc < (uint32_t)kCandCap) { L.ck[pc] = kk; L.ci[pc] = ii; }
            } else if (pc < (uint32_t)S_max) {
                // a short list too long for LDS goes to the query's flat area;
                // every workgroup of the sequence computes the same list, so
                // their concurrent writes to these words store identical values
                W.flat_key[pc] = kk;
                W.flat_idx[pc] = ii;
            }
            atomicAdd(&L.h[(kk >> 10) & (kBins - 1)], 1u);
            ++pc;
        }
        __syncthreads();  // the next round reuses the stage
        bsel += ts;
        bsh += tc;
    }
    // 4. short slots: their rows straight from the score row (up to 8 per
    //    thread), routed like the list entries and appended after them
    const int rpt = (1 << Ls.rows_lg) / kSelThreads;  // rows per thread: 1, 2, 4 or 8
#pragma unroll 1
    for (uint32_t qb = 0; qb < nbad; ++qb) {
        const int r0 = ((int)L.mem[qb] << Ls.rows_lg) + tid * rpt;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = srow[min(r0 + j, n - 1)];  // clamped, unconditional; j >= rpt unused
        uint32_t selm = 0, shm = 0, kk8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            kk8[j] = score_key(v[j]);
            const int bin = (int)(kk8[j] >> 21);
            const bool ok = j < rpt && r0 + j < n;
            if (ok && bin > t1) selm |= 1u << j;
            if (ok && bin == t1 && refine) shm |= 1u << j;
        }
        uint32_t ps, pc, ts, tc;
        block_excl_scan2<kSelThreads>((uint32_t)__popc(selm), (uint32_t)__popc(shm), L.tmp, &ps, &pc,
                                      &ts, &tc);
        ps += bsel;
        pc += bsh;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if ((selm >> j) & 1u) {
                if (ps < (uint32_t)kTopkMaxK) L.sel[ps] = r0 + j;
                ++ps;
            }
            if ((shm >> j) & 1u) {
                if (small) {
                    if (pc < (uint32_t)kCandCap) { L.ck[pc] = kk8[j]; L.ci[pc] = (uint32_t)(r0 + j); }
                } else if (pc < (uint32_t)S_max) {
                    W.flat_key[pc] = kk8[j];
                    W.flat_idx[pc] = (uint32_t)(r0 + j);
                }
                atomicAdd(&L.h[(kk8[j] >> 10) & (kBins - 1)], 1u);
                ++pc;
            }
        }
        bsel += ts;
        bsh += tc;
    }
    __syncthreads();
    if (!refine) return R;
    select_finish(W, R, need, small, L);
    return R;
}

// The query's top-k in ascending index order when the two lists are not
// (select_query_lists with short slots): both lists sorted together in LDS
// (bitonic, in `buf`, at least 2048 words), -1 padded.
__device__ inline void select_write_sorted_any(const SelLds& L, const SelResult& R, int32_t* o, int k,
                                               uint32_t* buf) {
    const int tid = threadIdx.x;
    const int take = R.nsel + R.nch;
    int P = 1;
    while (P < take) P <<= 1;
    for (int i = tid; i < P; i += kSelThreads)
        buf[i] = i < R.nsel ? (uint32_t)L.sel[i] : (i < take ? (uint32_t)L.chs[i - R.nsel] : 0xffffffffu);
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < P / 2; t += kSelThreads) {
                const int lo = 2 * t - (t & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const uint32_t a = buf[lo], b = buf[hi];
                if ((a > b) == up) { buf[lo] = b; buf[hi] = a; }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < k; i += kSelThreads) o[i] = i < take ? (int32_t)buf[i] : -1;
}

// The query's top-k in ascending index order: the merge of the two ascending
// lists (output position = own rank + rank in the other list), -1 padded.
__device__ inline void select_write_sorted(const SelLds& L, const SelResult& R, int32_t* o, int k) {
    const int tid = threadIdx.x;
    for (int i = tid; i < R.nsel; i += kSelThreads) {
        const int32_t v = L.sel[i];
        o[i + (int)lower_bound_lds(L.chs, (uint32_t)R.nch, v)] = v;
    }
    for (int j = tid; j < R.nch; j += kSelThreads) {
        const int32_t v = L.chs[j];
        o[j + (int)lower_bound_lds(L.sel, (uint32_t)R.nsel, v)] = v;
    }
    for (int i = R.nsel + R.nch + tid; i < k; i += kSelThreads) o[i] = -1;
}

// Zero every workspace word a call wrote for one query (one workgroup of NT
// threads, after every reader of the query's workspace has finished).
// segc: LDS [kMaxSeg], tmp: LDS [NT / 64 + 2].
template <int NT>
__device__ inline void select_zero(const QWs& W, int S_max, uint32_t* segc, uint32_t* tmp) {
    const int tid = threadIdx.x;
    const int nseg = n_segments(S_max);
    uint32_t mine = 0;
    for (int gg = tid; gg < nseg; gg += NT) {
        const uint32_t v = W.seg[gg];
        segc[gg] = v;
        mine += v & 0xffffu;
    }
    for (int i = tid; i < kBins; i += NT) { W.hist[i] = 0; W.hist2[i] = 0; }
    if (tid < 16) W.ctr[tid] = 0;
    uint32_t nc;  // short-list length (decides whether the flat copy was written)
    block_excl_scan<NT>(mine, tmp, &nc);  // its barriers publish segc
    int T_s = 1;
    while (T_s * 2 * nseg <= NT) T_s *= 2;
    const int par = NT / T_s, r = tid % T_s;
    for (int gg = tid / T_s; gg < nseg; gg += par) {
        const uint32_t cs = segc[gg] & 0xffffu, cnt = cs + (segc[gg] >> 16);
        const uint32_t base = (uint32_t)gg * kFilterChunk;
        for (uint32_t j = (uint32_t)r; j < cnt; j += (uint32_t)T_s) {
            W.cand_idx[base + j] = 0;
            if (j < cs) W.cand_key[base + j] = 0;
        }
    }
    if (nc > (uint32_t)kCandCap)
        for (uint32_t i = (uint32_t)tid; i < nc; i += NT) { W.flat_key[i] = 0; W.flat_idx[i] = 0; }
    for (int gg = tid; gg < nseg; gg += NT) W.seg[gg] = 0;  // every count was read above
}

}  // namespace sel
}  // namespace hsa
