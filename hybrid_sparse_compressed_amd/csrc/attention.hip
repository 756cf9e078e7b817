// attention.hip -- fused SWA + compressed-row attention for gfx950.
//
// [LH "Tich hop Kernel va Giai ma suy doan"]: SWA and the extra C4/C128
// attention are combined in a single kernel call; [LH "Toi uu hoa suy luan
// voi ShadowRadix va HiSparse"]: a layer pairs SWA with C4 (sparse top-512)
// or C128 (dense).  One softmax runs over the union of the window rows and
// the compressed rows; the value of a latent row is its first d_v channels.
//
// Layout of the work.  A workgroup (4 waves) owns 16 query heads (one MFMA
// column block) and a range of "virtual rows": rows 0..W-1 are the window
// (ring slots for decode, causal tokens for prefill), rows W.. are the
// compressed candidates (the index list in sparse mode, 0..len-1 in dense
// mode).  Rows are processed in tiles of 64:
//   1. gather: the 64 latent rows are copied into LDS with 16-byte loads,
//      row-major for the QK product and transposed (first d_v channels) for
//      the PV product; rows that are not valid are zero-filled and masked;
//   2. S^T = K_tile * Q^T on MFMA 16x16 tiles: wave w takes rows
//      16w..16w+15 (rows on M, heads on N), so a lane owns one head and 4
//      rows;
//   3. online softmax per head in base 2: each wave reduces its 16 rows, the
//      four (max, sum) pairs meet in LDS and every wave derives the same
//      running statistics; P^T goes to LDS in bf16 (fp32 for fp32 inputs);
//   4. O^T += V^T * P^T on MFMA over the 64 rows, wave w owning value
//      channels [w*d_v/4, (w+1)*d_v/4), accumulating O^T in fp32.
// The rows of the next tile are loaded into registers while the current
// tile is computed.  Decode splits the rows of a sequence over several
// workgroups and merges their (max, sum, O) partials in a second kernel, in a
// fixed order; prefill gives each (query position, head block) its own
// workgroup, the head blocks of a query dispatched back to back on one XCD so
// that they gather the same rows through one L2.  For the 64-head bf16
// latent-576 shape, prefill64_kernel instead gives a query's 64 heads one
// 8-wave workgroup that gathers each tile once.
//
// Fused sparse decode (the whole C4 layer-step after the scoring launch): a
// workgroup with compressed rows first finishes its sequence's top-k select
// itself from the scoring workgroups' candidate lists and the first-digit
// histogram (select.hpp, in the LDS its tiles use later) and takes its rows
// from the selected list followed by the chosen short-list entries, so no
// filter pass, separate select kernel, index round trip or sort sits on the
// attention's critical path.  One extra workgroup per sequence writes the
// ascending top-k indices; the merge kernel clears the histogram.
#include "hsa_common.hpp"
#include "hsa_internal.hpp"
#include "select.hpp"

namespace hsa {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kNW = kAttnThreads / kWave;  // waves per workgroup
constexpr int kHeadsPerWG = 16;
constexpr int kTile = 16 * kNW;            // rows per tile: 16 per wave in the QK product
constexpr int kChunkRows = 256;            // rows whose list is built at once (one per thread)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// MFMA 16x16 traits.  Operand lane layout (both dtypes): lane l supplies row
// (A) or column (B) l%16, and the k-slots of lane group l/16; the result tile
// gives lane l the elements (4*(l/16) + r, l%16), r = 0..3.
template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
    static constexpr int kK = 32;  // contraction length of one instruction
    typedef bf16x8 frag;
    __device__ static __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<float> {
    static constexpr int kK = 4;
    typedef float frag;
    __device__ static __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// fp32 tiles: a store of the x-th elements of two rows (consecutive in the
// transposed tile) as one 2-element write.
template <typename T> struct Pair;
template <> struct Pair<float> {
    __device__ static __forceinline__ void put(float* dst, const u32x4& a, const u32x4& b, int x) {
        *reinterpret_cast<uint2*>(dst) = uint2{a[x], b[x]};
    }
};

struct AttnArgs {
    const void* q;
    uint8_t* sel_ws;      // fused decode: top-k workspace (histogram, candidate lists)
    const float* scores;  // fused decode: [B, S_max] indexer scores (the select's fallback)
    const int32_t* n_cand;
    int32_t* topk_out;    // fused decode: [B, k] ascending top-k indices
    const void* win;      // decode: swa ring [B, W, d_qk]; prefill: token kv [n_seq, T, d_qk]
    const int32_t* swa_len;
    const void* comp;     // [n_seq, S_max, d_qk]
    const int32_t* comp_idx;
    const int32_t* comp_len;
    void* out;
    float* lse;
    float* part_ml;       // decode partials: (max, sum) [B][n_split][H][2]
    float* part_o;        //                  outputs    [B][n_split][H][d_v]
    int H, W, S_max, k, m, T_len, n_q, q_start;
    int rows_per_split, n_split, max_rows;
    int hblocks, n_queries;  // prefill: head blocks per query, queries in the grid
    int list_rows_lg;     // fused decode: log2 of the candidate rows per list slot
    float scale_log2;     // scale * log2(e)
    // paged decode (pg_swa.map != nullptr): win and comp are the paged SWA and
    // C4 pools; window row vr of sequence b is token pos[b] - n_swa + 1 + vr
    PoolMap pg_swa, pg_c4;
    const int32_t* pos;
    // dense 64-head decode with splits planned on the device from comp_len
    // (n_seq sequences): workgroup g takes split g of the plan
    int dense_plan, n_seq;
    int* dense_seq_plan;  // [n_seq]: first split | split count << 16, for the merge
};

// LDS footprint of one tile, in elements of T: K row-major, V^T (one row per
// value channel; fp32 only), P^T (one row per head).  Every row carries a
// 32-byte skew so that the 16 rows one MFMA operand reads fall on distinct
// banks.  bf16 tiles keep no V^T: the PV product reads the value columns out
// of the row-major K rows with transposing LDS loads (kTr).
template <typename T, int DQK, int DV> struct TileLds {
    static constexpr bool kTr = sizeof(T) == 2;
    static constexpr int kSkew = 32 / (int)sizeof(T);  // 32 bytes (16 bytes measured 0.3 us slower per step)
    static constexpr int kStrideK = DQK + kSkew;
    static constexpr int kStrideT = kTile + kSkew;   // V^T and P^T rows
    static constexpr size_t kOffV = (size_t)kTile * kStrideK;
    static constexpr size_t kOffP = kOffV + (kTr ? (size_t)0 : (size_t)DV * kStrideT);
    static constexpr size_t kBytes = (kOffP + (size_t)kHeadsPerWG * kStrideT) * sizeof(T);
};

// bf16 PV operands.  Step ks of the PV product contracts tile rows 32 ks ..
// 32 ks + 31; k-slot 8 q + j of lane group q stands for row
// 32 ks + 4 q + j (j < 4) or 32 ks + 16 + 4 q + (j - 4) (j >= 4), so that each
// half of a lane's V^T fragment is one transposing read of 4 consecutive rows,
// and the 8 rows that two lane groups read together sit 36 banks apart.  P^T
// is stored in the same order: tile row R goes to position p_pos(R).
__device__ __forceinline__ int p_pos(int R) {
    return (R & ~31) + 8 * ((R >> 2) & 3) + 4 * ((R >> 4) & 1) + (R & 3);
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane
// groups of one head column) with gfx950's row swaps: v_permlane16_swap
// pairs 16-lane rows 0-1 and 2-3, v_permlane32_swap the two 32-lane halves;
// each hands every lane its partner's value without an LDS round trip, and
// both lanes of a pair combine the same two values (bitwise-equal results).
__device__ __forceinline__ float quad4_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x for the softmax weights on the hardware base-2 exponential: every
// argument is a difference from a running maximum (<= 0, or -inf for a
// masked row: 0), so the library function's range reduction is not needed; a
// weight below 2^-126 comes out as 0, far below the resolution of the sum it
// joins, which holds the maximum row's weight 1.
__device__ __forceinline__ float exp2_le0(float x) { return __builtin_amdgcn_exp2f(x); }

// four P values -> bf16 with the hardware conversion (round to nearest even)
__device__ __forceinline__ uint2 pack_p4(float a, float b, float c, float d) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 lo = {(__bf16)a, (__bf16)b}, hi = {(__bf16)c, (__bf16)d};
    return uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Rows of the PV contraction.  bf16: step ks takes tile rows 32*ks..32*ks+31,
// lane group q the 8 rows 32*ks + 8*q + j.  fp32: step ks takes 4 rows, lane
// group q row 16*q + ks, so a lane's rows over the 16 steps are contiguous.
// V^T and P^T are both stored in natural row order, which these maps read
// with 16-byte loads.
static_assert(kTile == 64, "the fp32 PV map assumes 16 steps of 4 rows");

// kModeFused: 2048-row list slots (constant slot arithmetic, the large-pool
// case); kModeFusedVar: list slots of 256 .. 2048 rows (a.list_rows_lg)
constexpr int kModeDecode = 0, kModePrefill = 1, kModeFused = 2, kModeFusedVar = 3;

// LDS the select prologue of the fused mode carves out of the tile buffers
constexpr size_t kSelLdsBytes = (size_t)sel::kBins * 4 + (2 * sel::kSelNW + 2) * 4 + 3 * (size_t)sel::kMaxSeg * 4 +
                                2 * (size_t)sel::kCandCap * 4 + 2 * (size_t)kTopkMaxK * 4 + 16 +
                                3 * (size_t)sel::kSelThreads * 4 + (size_t)sel::kCandCap;
// LDS of the list entries one read round of the fused select stages (after the above)
constexpr size_t kSelStageOff = (kSelLdsBytes + 15) & ~(size_t)15;
constexpr size_t kSelStageBytes = (size_t)sel::kSelThreads * 16 * 16;
__device__ inline sel::SelLds sel_lds_at(unsigned char* base) {
    sel::SelLds L;
    uint32_t* p = reinterpret_cast<uint32_t*>(base);
    L.h = p; p += sel::kBins;
    L.segc = p; p += sel::kMaxSeg;
    L.sbase = p; p += sel::kMaxSeg;
    L.lbase = p; p += sel::kMaxSeg;
    L.ck = p; p += sel::kCandCap;
    L.ci = p; p += sel::kCandCap;
    L.sel = reinterpret_cast<int32_t*>(p); p += kTopkMaxK;
    L.chs = reinterpret_cast<int32_t*>(p); p += kTopkMaxK;
    L.misc = p; p += 4;
    L.mem = p; p += 3 * sel::kSelThreads;
    L.tmp = p; p += 2 * sel::kSelNW + 2;
    L.flag = reinterpret_cast<uint8_t*>(p);
    L.stage = reinterpret_cast<u32x4*>(base + kSelStageOff);
    return L;
}

template <typename T, int DQK, int DV, int MODE>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnArgs a) {
    constexpr bool PREFILL = MODE == kModePrefill;
    constexpr bool FUSED = MODE == kModeFused || MODE == kModeFusedVar;
    const int list_rows_lg = MODE == kModeFusedVar ? a.list_rows_lg : 11;
    typedef TileLds<T, DQK, DV> L;
    typedef Mma<T> M;
    constexpr int V16 = Elem<T>::kPer16B;          // elements per 16-byte chunk
    constexpr int CPR = DQK / V16;                 // 16-byte chunks per row
    constexpr int NKK = DQK / M::kK;               // MFMA steps of the QK product
    constexpr int DW = DV / kNW;                   // value channels per wave
    constexpr int NMT = DW / 16;                   // O^T row tiles per wave
    static_assert(DQK % M::kK == 0 && DV % (16 * kNW) == 0 && DV <= DQK && DV <= 512,
                  "unsupported head dims");
    static_assert(kChunkRows % kTile == 0 && kChunkRows == kAttnThreads, "row list layout");

    extern __shared__ __align__(16) unsigned char lds_raw[];
    T* Ks = reinterpret_cast<T*>(lds_raw);
    T* Vt = Ks + L::kOffV;
    T* Pt = Ks + L::kOffP;
    __shared__ long long row_off[kChunkRows];  // element offset of the row in its source, -1 invalid
    __shared__ int row_src[kChunkRows];        // 0: window source, 1: compressed pool
    __shared__ int tile_any[kChunkRows / kTile];
    __shared__ float red_m[kNW][kHeadsPerWG], red_s[kNW][kHeadsPerWG];
    __shared__ int32_t fidx[FUSED ? kChunkRows : 1];  // fused: this workgroup's selected indices

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int hl = lane & 15, quad = lane >> 4;
    int hb = blockIdx.z;
    int pq = 0;  // prefill: query (sequence-major)
    if constexpr (PREFILL) {
        // Workgroup L runs on XCD L % 8.  Among one XCD's workgroups the head
        // blocks of a query come one after another, and consecutive queries
        // of that XCD are 8 positions apart: rows shared by them (the head
        // blocks' whole lists, neighbouring windows) meet in one L2.
        const int L = (int)blockIdx.x, s8 = L / 8;
        hb = s8 % a.hblocks;
        pq = (s8 / a.hblocks) * 8 + L % 8;
        if (pq >= a.n_queries) return;
    }
    const int head = hb * kHeadsPerWG + hl;
    const bool head_ok = head < a.H;

    // sequence / query identity and row range
    int b, qpos = 0, qid = 0, vr0, vr1;
    if constexpr (PREFILL) {
        const int i = pq % a.n_q;
        b = pq / a.n_q;
        qid = pq;
        qpos = a.q_start + i;
        vr0 = 0;
        vr1 = a.max_rows;
    } else {
        b = blockIdx.y;
        vr0 = blockIdx.x * a.rows_per_split;
        vr1 = min(a.max_rows, vr0 + a.rows_per_split);
    }
    int n_swa, n_comp, n_fc = 0;  // n_fc (fused): the sequence's candidates, clamped to [0, S_max]
    if constexpr (PREFILL) {
        n_swa = 0;
        int vis = (qpos + 1) / a.m;
        n_comp = vis < a.S_max ? vis : a.S_max;
    } else {
        // The sequence's counts are read together, in one memory round trip
        // ahead of the select (the asm statement uses all four, so none of the
        // loads is moved behind the wait for another).
        int sw = a.swa_len[b];
        int cl = a.comp_len[b];
        int ps = (a.pg_swa.map ? a.pos : a.swa_len)[b];  // paged: the query token's position
        int nc = FUSED ? a.n_cand[b] : 0;
        asm volatile("" : "+s"(sw), "+s"(cl), "+s"(ps), "+s"(nc));
        n_swa = sw < 0 ? 0 : (sw > a.W ? a.W : sw);
        if (a.pg_swa.map && ps < 0) n_swa = 0;  // paged: no query token, no window
        n_comp = cl < 0 ? 0 : (cl > a.S_max ? a.S_max : cl);
        n_fc = nc < 0 ? 0 : (nc > a.S_max ? a.S_max : nc);
    }

    // Fused: finish the sequence's select and keep this workgroup's list
    // positions [f_j0, f_j0 + f_jn) in fidx (the host keeps a split within
    // one row chunk).
    int f_j0 = 0, f_jn = 0;
    if constexpr (FUSED) {
        const sel::QWs Wq = sel::ws_of(a.sel_ws, b, a.S_max, a.k);
        const sel::SelLds SL = sel_lds_at(lds_raw);
        const int n = n_fc;
        if ((int)blockIdx.x == a.n_split) {  // the sequence's ascending top-k output
            if (hb != 0) return;
            const sel::SelResult R = sel::select_query_lists(
                Wq, a.scores + (size_t)b * a.S_max, n, a.S_max, a.k, list_rows_lg, a.k, SL, [] {});
            if (R.unordered)  // uniform
                sel::select_write_sorted_any(SL, R, a.topk_out + (size_t)b * a.k, a.k, SL.ck);
            else
                sel::select_write_sorted(SL, R, a.topk_out + (size_t)b * a.k, a.k);
            return;
        }
    }

    // Row list entry of virtual row vr (chunk end c1): element offset of the
    // latent row in its source (-1: not a row of this query) and the source.
    auto row_entry = [&](int vr, int c1, long long& off, int& src) {
        off = -1;
        src = 0;
        if (vr >= c1) return;
        if (vr < a.W) {
            if constexpr (PREFILL) {
                const int tok = qpos - a.W + 1 + vr;
                if (tok >= 0) off = ((long long)b * a.T_len + tok) * DQK;
            } else if (vr < n_swa) {
                if (a.pg_swa.map) {
                    const long long pr = paged_row(a.pg_swa, b, (long long)a.pos[b] - n_swa + 1 + vr);
                    if (pr >= 0) off = pr * DQK;
                } else {
                    off = ((long long)b * a.W + vr) * DQK;
                }
            }
        } else {
            const int j = vr - a.W;
            int ci = -1;
            if constexpr (FUSED) {
                const int t = j - f_j0;
                ci = (t >= 0 && t < f_jn) ? fidx[t] : -1;
            } else if (a.comp_idx) {
                if (j < a.k) {
                    const long long row = PREFILL ? (long long)qid : (long long)b;
                    ci = a.comp_idx[row * a.k + j];
                }
            } else {
                ci = j;
            }
            if (ci >= 0 && ci < n_comp) {
                if (!PREFILL && a.pg_c4.map) {
                    const long long pr = paged_row(a.pg_c4, b, ci);
                    if (pr >= 0) {
                        off = pr * DQK;
                        src = 1;
                    }
                } else {
                    off = ((long long)b * a.S_max + ci) * DQK;
                    src = 1;
                }
            }
        }
    };
    // the first chunk's index loads go out before the Q loads, so waiting for
    // them does not wait for Q (the vector-memory counter retires in order)
    long long first_off;
    int first_src;
    if constexpr (!FUSED) row_entry(vr0 + tid, min(vr1, vr0 + kChunkRows), first_off, first_src);

    // Q fragments for this lane's head: k-slots of lane group `quad` (every
    // wave holds the same 16 heads)
    typename M::frag qf[NKK];
    auto load_q = [&]() {
        const T* qrow;
        if constexpr (PREFILL)
            qrow = reinterpret_cast<const T*>(a.q) + ((size_t)qid * a.H + (head_ok ? head : 0)) * DQK;
        else
            qrow = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.H + (head_ok ? head : 0)) * DQK;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            // unconditional loads (row clamped to head 0), zeroed after: a
            // load inside a branch would get a wait for every load before it
            if constexpr (sizeof(T) == 2) {
                u32x4 v = *reinterpret_cast<const u32x4*>(qrow + kk * M::kK + quad * 8);
                if (!head_ok) v = u32x4{0u, 0u, 0u, 0u};
                qf[kk] = __builtin_bit_cast(bf16x8, v);
            } else {
                const float v = reinterpret_cast<const float*>(qrow)[kk * M::kK + quad];
                qf[kk] = head_ok ? v : 0.f;
            }
        }
    };
    // fused: Q is loaded inside the select, behind its first loads (the
    // vector-memory counter retires in order), or right away if there is none
    if constexpr (!FUSED) load_q();

    if constexpr (FUSED) {
        const sel::QWs Wq = sel::ws_of(a.sel_ws, b, a.S_max, a.k);
        const sel::SelLds SL = sel_lds_at(lds_raw);
        const int n = n_fc;
        if (vr1 > a.W) {  // uniform: this workgroup has compressed rows
            f_j0 = max(0, vr0 - a.W);
            const int j1 = min(a.k, vr1 - a.W);
            // Q goes out right behind the select's first loads: the select
            // never waits for it, and it arrives during the select
            const sel::SelResult R = sel::select_query_lists(
                Wq, a.scores + (size_t)b * a.S_max, n, a.S_max, a.k, list_rows_lg, j1, SL, load_q);
            f_jn = j1 - f_j0;
            for (int t = tid; t < f_jn; t += kAttnThreads) {
                const int j = f_j0 + t;
                fidx[t] = j < R.nsel ? SL.sel[j] : (j - R.nsel < R.nch ? SL.chs[j - R.nsel] : -1);
            }
            __syncthreads();  // fidx published; the select LDS goes back to the tiles
        }
    }
    if constexpr (FUSED) {
        if (vr1 <= a.W) load_q();  // uniform: a window-only split runs no select
        row_entry(vr0 + tid, min(vr1, vr0 + kChunkRows), first_off, first_src);
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[NMT];
#pragma unroll
    for (int t = 0; t < NMT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const T* win = reinterpret_cast<const T*>(a.win);
    const T* comp = reinterpret_cast<const T*>(a.comp);

    // gather registers; the next tile's rows are loaded while this one is
    // computed.  bf16: thread t moves chunks (t & 7) + 8 i of rows t / 8 and
    // t / 8 + 32 (one instruction of a wave covers eight 128-byte runs),
    // stored row-major.  fp32: chunk `ch` of the row pair (2rp, 2rp+1),
    // stored row-major and transposed.
    constexpr bool TR = L::kTr;
    static_assert(!TR || (CPR % 8 == 0 && kTile == 2 * (kAttnThreads / 8)), "bf16 gather map");
    constexpr int kUnits = TR ? kTile * CPR : (kTile / 2) * CPR;
    constexpr int kIter = (kUnits + kAttnThreads - 1) / kAttnThreads;
    u32x4 ga[kIter], gb[TR ? 1 : kIter];
    auto issue = [&](int tb) {
        if constexpr (TR) {
            constexpr int NC = CPR / 8;  // chunks per row and thread
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = (tid >> 3) + 32 * h;
                const long long o = row_off[tb + row];
                const T* src = (row_src[tb + row] ? comp : win) + (o >= 0 ? o : 0) + (tid & 7) * V16;
#pragma unroll
                for (int i = 0; i < NC; ++i)
                    ga[h * NC + i] = o >= 0 ? *reinterpret_cast<const u32x4*>(src + 8 * i * V16)
                                            : u32x4{0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int it = 0; it < kIter; ++it) {
                const int u = tid + it * kAttnThreads;
                const int rp = u % (kTile / 2), ch = u / (kTile / 2);
                ga[it] = gb[it] = u32x4{0u, 0u, 0u, 0u};
                if (u < kUnits) {
                    const long long oa = row_off[tb + 2 * rp], ob = row_off[tb + 2 * rp + 1];
                    if (oa >= 0)
                        ga[it] = *reinterpret_cast<const u32x4*>((row_src[tb + 2 * rp] ? comp : win) + oa + (long long)ch * V16);
                    if (ob >= 0)
                        gb[it] = *reinterpret_cast<const u32x4*>((row_src[tb + 2 * rp + 1] ? comp : win) + ob + (long long)ch * V16);
                }
            }
        }
    };

    for (int c0 = vr0; c0 < vr1; c0 += kChunkRows) {
        const int c1 = min(vr1, c0 + kChunkRows);
        // ---- row list of this chunk: one thread per virtual row
        {
            long long off = first_off;
            int src = first_src;
            if (c0 != vr0) row_entry(c0 + tid, c1, off, src);
            row_off[tid] = off;
            row_src[tid] = src;
        }
        if (tid < kChunkRows / kTile) tile_any[tid] = 0;
        __syncthreads();
        if (row_off[tid] >= 0) tile_any[tid / kTile] = 1;  // benign race: all write 1
        __syncthreads();

    int pre = -1;  // tile (offset in the chunk) whose rows are in flight in ga/gb
    for (int t0 = c0; t0 < c1; t0 += kTile) {
        const int tb = t0 - c0;
        if (!tile_any[tb / kTile]) continue;  // uniform: nothing valid in this tile
        // ---- gather: K goes row-major, V transposed with the two rows packed
        // in one write (consecutive lanes -> consecutive words: no bank conflicts)
        if (pre != tb) issue(tb);
#pragma unroll
        for (int it = 0; it < kIter; ++it) {
            const int u = tid + it * kAttnThreads;
            if constexpr (TR) {
                constexpr int NC = CPR / 8;
                const int row = (tid >> 3) + 32 * (it / NC), ch = (tid & 7) + 8 * (it % NC);
                *reinterpret_cast<u32x4*>(Ks + (size_t)row * L::kStrideK + ch * V16) = ga[it];
            } else {
                const int rp = u % (kTile / 2), ch = u / (kTile / 2);
                if (u < kUnits) {
                    *reinterpret_cast<u32x4*>(Ks + (size_t)(2 * rp) * L::kStrideK + ch * V16) = ga[it];
                    *reinterpret_cast<u32x4*>(Ks + (size_t)(2 * rp + 1) * L::kStrideK + ch * V16) = gb[it];
                    if (ch * V16 < DV) {
#pragma unroll
                        for (int x = 0; x < V16; ++x)
                            Pair<T>::put(Vt + (size_t)(ch * V16 + x) * L::kStrideT + 2 * rp, ga[it], gb[it], x);
                    }
                }
            }
        }
        __syncthreads();
        // the next tile of this chunk with valid rows goes out now (prefill,
        // whose workgroups walk many tiles; a decode split is mostly one tile,
        // and the registers held through the tile would cost more there)
        if constexpr (PREFILL) {
            pre = -1;
            for (int nb = tb + kTile; nb < c1 - c0; nb += kTile) {
                if (tile_any[nb / kTile]) {
                    issue(nb);
                    pre = nb;
                    break;
                }
            }
        }

        // ---- S^T for this wave's rows 16*wave + 4*quad + r, head `hl`; two
        // accumulation chains (even / odd steps) halve the dependent latency
        f32x4 s;
        {
            f32x4 c0v = f32x4{0.f, 0.f, 0.f, 0.f}, c1v = f32x4{0.f, 0.f, 0.f, 0.f};
            const T* krow = Ks + (size_t)(wave * 16 + hl) * L::kStrideK;
            // K fragments are read from LDS a group at a time, all reads of a
            // group in flight before its MFMAs
            constexpr int KG = NKK % 6 == 0 ? 6 : (NKK % 4 == 0 ? 4 : 1);
#pragma unroll
            for (int g0 = 0; g0 < NKK; g0 += KG) {
                typename M::frag af[KG];
#pragma unroll
                for (int j = 0; j < KG; ++j) {
                    const int kk = g0 + j;
                    if constexpr (sizeof(T) == 2) {
                        u32x4 v = *reinterpret_cast<const u32x4*>(krow + kk * M::kK + quad * 8);
                        af[j] = __builtin_bit_cast(bf16x8, v);
                    } else {
                        af[j] = reinterpret_cast<const float*>(krow)[kk * M::kK + quad];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);  // keep the group's reads ahead of its MFMAs
#pragma unroll
                for (int j = 0; j < KG; ++j) {
                    const int kk = g0 + j;
                    if (kk & 1)
                        c1v = M::mma(af[j], qf[kk], c1v);
                    else
                        c0v = M::mma(af[j], qf[kk], c0v);
                }
            }
            s = c0v + c1v;
        }

        // ---- online softmax (base 2); masked rows -> -inf.  Each wave
        // reduces its 16 rows to (max, sum relative to that max) per head.
        float x[4];
        float wmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wave * 16 + quad * 4 + r;
            const float v = row_off[tb + row] >= 0 ? s[r] * a.scale_log2 : -INFINITY;
            x[r] = v;
            wmax = fmaxf(wmax, v);
        }
        wmax = quad4_max(wmax);
        float p[4];
        float wsum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = wmax == -INFINITY ? 0.f : exp2_le0(x[r] - wmax);
            wsum += p[r];
        }
        wsum = quad4_sum(wsum);
        if (quad == 0) {
            red_m[wave][hl] = wmax;
            red_s[wave][hl] = wsum;
        }
        __syncthreads();
        // The reference max only moves when a logit exceeds it by more than
        // 2^8 (p stays <= 256, no overflow); the rescale of the accumulator is
        // skipped unless some lane of the wave moved a nonzero accumulator.
        float tmax = -INFINITY;
#pragma unroll
        for (int w = 0; w < kNW; ++w) tmax = fmaxf(tmax, red_m[w][hl]);
        const bool move = tmax > m_run + 8.f;
        const float m_new = move ? tmax : m_run;
        const float alpha = move ? exp2_le0(m_run - m_new) : 1.f;  // 0 when m_run = -inf
        float tsum = 0.f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
            const float mw = red_m[w][hl];
            if (mw != -INFINITY) tsum += red_s[w][hl] * exp2_le0(mw - m_new);
        }
        const float sc = wmax == -INFINITY ? 0.f : exp2_le0(wmax - m_new);
        // P^T rows of this wave (bf16: in the PV k-slot order, p_pos; fp32: natural)
        if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<uint2*>(Pt + (size_t)hl * L::kStrideT + p_pos(wave * 16 + quad * 4)) =
                pack_p4(p[0] * sc, p[1] * sc, p[2] * sc, p[3] * sc);
        } else {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(Pt) + (size_t)hl * L::kStrideT + wave * 16 + quad * 4) =
                f32x4{p[0] * sc, p[1] * sc, p[2] * sc, p[3] * sc};
        }
        if (__ballot(move && l_run > 0.f)) {
#pragma unroll
            for (int t = 0; t < NMT; ++t) acc[t] *= alpha;
        }
        l_run = l_run * alpha + tsum;
        m_run = m_new;
        __syncthreads();

        // ---- O^T[wave's channels] += V^T * P^T
        const T* pbase = Pt + (size_t)hl * L::kStrideT;
        if constexpr (sizeof(T) == 2) {
            // V^T fragment of channel block t: two transposing reads of the K
            // rows (rows 4 quad + (lane & 15) / 4 and 16 more, channels
            // 16 t + 4 (lane & 3) of the wave's range), in p_pos order
            const T* vtr = Ks + (size_t)(4 * quad + ((lane & 15) >> 2)) * L::kStrideK + wave * DW + 4 * (lane & 3);
#pragma unroll
            for (int ks = 0; ks < kTile / 32; ++ks) {
                // the step's P^T and V^T fragments are all read before its MFMAs
                const bf16x8 pf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(pbase + ks * 32 + quad * 8));
                u32x4 vv[NMT];
#pragma unroll
                for (int t = 0; t < NMT; ++t) {
                    const T* pa = vtr + (size_t)(32 * ks) * L::kStrideK + 16 * t;
                    const uint2 lo = lds_read_tr16x4(pa);
                    const uint2 hi = lds_read_tr16x4(pa + (size_t)16 * L::kStrideK);
                    vv[t] = u32x4{lo.x, lo.y, hi.x, hi.y};
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < NMT; ++t) acc[t] = M::mma(__builtin_bit_cast(bf16x8, vv[t]), pf, acc[t]);
            }
        } else {
            const T* vbase = Vt + (size_t)(wave * DW + hl) * L::kStrideT;
            // lane group q contracts rows 16q..16q+15 (one per step): 4 vector reads per operand
            const float* pf = reinterpret_cast<const float*>(pbase) + quad * 16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 pv = *reinterpret_cast<const f32x4*>(pf + 4 * j);
#pragma unroll
                for (int t = 0; t < NMT; ++t) {
                    const f32x4 vv = *reinterpret_cast<const f32x4*>(
                        reinterpret_cast<const float*>(vbase) + (size_t)t * 16 * L::kStrideT + quad * 16 + 4 * j);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[t] = M::mma(vv[e], pv[e], acc[t]);
                }
            }
        }
        __syncthreads();  // LDS tile is rewritten by the next iteration
    }
    }

    // ---- epilogue.  acc[t][r] = O^T[wave*DW + 16*t + 4*quad + r][head]
    if constexpr (!PREFILL) {
        if (a.n_split > 1) {
            // Split partials go out through LDS (the tile buffers are free: the
            // tile loop ends on a barrier), so that each store instruction
            // writes whole runs of one head's row.
            constexpr int OS = DW + 4;                          // LDS row stride (floats)
            constexpr int CPRW = DW / 4;                        // 16-byte chunks per row and wave
            constexpr int NCH = kHeadsPerWG * CPRW / kWave;     // chunks per lane
            static_assert((size_t)kNW * kHeadsPerWG * OS * sizeof(float) <= L::kBytes,
                          "partial staging must fit in the tile buffers");
            float* ob = reinterpret_cast<float*>(lds_raw) + (size_t)wave * kHeadsPerWG * OS;
            const int h0 = hb * kHeadsPerWG;
            const size_t prow0 = ((size_t)b * a.n_split + blockIdx.x) * a.H + h0;
            if (wave == 0 && head_ok && quad == 0)
                *reinterpret_cast<float2*>(a.part_ml + (prow0 + hl) * 2) = float2{m_run, l_run};
#pragma unroll
            for (int t = 0; t < NMT; ++t)
                *reinterpret_cast<f32x4*>(ob + hl * OS + t * 16 + quad * 4) = acc[t];
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int c = lane + j * kWave;
                const int row = c / CPRW, col = (c % CPRW) * 4;
                if (h0 + row < a.H)  // streamed past the L2: only the merge kernel reads it
                    __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(ob + row * OS + col),
                                                reinterpret_cast<f32x4*>(a.part_o + (prow0 + row) * DV + wave * DW + col));
            }
            return;
        }
    }
    if (!head_ok) return;
    const size_t orow = PREFILL ? ((size_t)qid * a.H + head) : ((size_t)b * a.H + head);
    T* o = reinterpret_cast<T*>(a.out) + orow * DV + wave * DW;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int t = 0; t < NMT; ++t) {
        if constexpr (sizeof(T) == 2) {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16(acc[t][0] * inv) | ((uint32_t)f32_to_bf16(acc[t][1] * inv) << 16);
            pk.y = (uint32_t)f32_to_bf16(acc[t][2] * inv) | ((uint32_t)f32_to_bf16(acc[t][3] * inv) << 16);
            *reinterpret_cast<uint2*>(o + t * 16 + quad * 4) = pk;
        } else {
            *reinterpret_cast<f32x4*>(o + t * 16 + quad * 4) = acc[t] * inv;
        }
    }
    if (a.lse && wave == 0 && quad == 0)
        a.lse[orow] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

// 64-head kernel shape (prefill64_kernel, below)
constexpr int kP64Threads = 512;
constexpr int kP64Waves = kP64Threads / kWave;
constexpr int kP64Heads = 64;
constexpr int kP64Rows = 64;                    // rows per tile
constexpr int kP64Chunk = 2 * kP64Threads;      // rows listed at once (two per thread)

// ---- dense decode splits planned on the device --------------------------------
// Sequence b has t_b = ceil((W + comp_len[b]) / 64) tiles (comp_len clamped to
// [0, S_max]).  With R tiles per split, the smallest R that keeps the total
// number of splits at most kDenseTarget (plus at most one partial split per
// sequence) and every sequence at most kMaxSplit splits, sequence b gets
// n_b = ceil(t_b / R) splits, numbered after the splits of sequences 0 .. b-1.
// Every workgroup derives the same plan from the lengths, one lane per
// sequence, and a sequence's first split hands (first, n_b) to the merge: a
// short sequence no longer waits on the longest one's split length, and the
// merge reads only the splits a sequence has.
constexpr int kDenseTarget = 256;  // about one workgroup per compute unit
constexpr int kMaxSplit = 128;

__device__ inline int dense_tiles(const AttnArgs& a, int i) {
    int n = a.comp_len[i];
    n = n < 0 ? 0 : (n > a.S_max ? a.S_max : n);
    return ceil_div(a.W + n, kP64Rows);
}

__device__ inline int dense_tiles_per_split(const AttnArgs& a) {
    int sum = 0, mx = 0;
    for (int i = lane_id(); i < a.n_seq; i += kWave) {
        const int t = dense_tiles(a, i);
        sum += t;
        mx = max(mx, t);
    }
    for (int o = kWave / 2; o > 0; o >>= 1) {
        sum += __shfl_xor(sum, o, kWave);
        mx = max(mx, __shfl_xor(mx, o, kWave));
    }
    return max(1, max(ceil_div(sum, kDenseTarget), ceil_div(mx, kMaxSplit)));
}

// Up to one wave of sequences: lane i reads sequence i's two lengths (both
// loads in one round trip), and the plan, the search for split g and that
// split's own lengths all come from the lanes, with no further memory read.
// Same plan as dense_tiles_per_split + dense_locate.  False past the last
// split; otherwise *b, *split, *first, *R, *count (the sequence's splits),
// *comp (its comp_len, clamped) and *swa (its swa_len, unclamped).
struct DenseSplit { int b, split, first, R, count, comp, swa; };
__device__ inline bool dense_locate_wave(const AttnArgs& a, int g, DenseSplit* d) {
    const int lane = lane_id();
    const int i = min(lane, a.n_seq - 1);  // unconditional loads: no wait between them
    int cl = a.comp_len[i];
    int sl = a.swa_len[i];
    asm volatile("" : "+v"(cl), "+v"(sl));  // both used here: the swa load is not sunk to its late use
    const int cc = cl < 0 ? 0 : (cl > a.S_max ? a.S_max : cl);
    const int t = lane < a.n_seq ? ceil_div(a.W + cc, kP64Rows) : 0;
    int sum = t, mx = t;
    for (int o = kWave / 2; o > 0; o >>= 1) {
        sum += __shfl_xor(sum, o, kWave);
        mx = max(mx, __shfl_xor(mx, o, kWave));
    }
    const int R = max(1, max(ceil_div(sum, kDenseTarget), ceil_div(mx, kMaxSplit)));
    const int n = ceil_div(t, R);
    const int incl = (int)wave_incl_scan((uint32_t)n);
    const int excl = incl - n;
    const unsigned long long hit = __ballot(n > 0 && excl <= g && g < incl);
    if (!hit) return false;
    const int src = (int)__ffsll(hit) - 1;
    d->b = src;
    d->first = __shfl(excl, src, kWave);
    d->split = g - d->first;
    d->R = R;
    d->count = __shfl(n, src, kWave);
    d->comp = __shfl(cc, src, kWave);
    d->swa = __shfl(sl, src, kWave);
    return true;
}

// the sequence and split of split g; false past the last split
__device__ inline bool dense_locate(const AttnArgs& a, int R, int g, int* b, int* split, int* first) {
    int base = 0;
    for (int i0 = 0; i0 < a.n_seq; i0 += kWave) {
        const int i = i0 + lane_id();
        const int n = i < a.n_seq ? ceil_div(dense_tiles(a, i), R) : 0;
        const int incl = base + (int)wave_incl_scan((uint32_t)n);
        const int excl = incl - n;
        const unsigned long long hit = __ballot(n > 0 && excl <= g && g < incl);
        if (hit) {
            const int src = (int)__ffsll(hit) - 1;
            *b = i0 + src;
            *first = __shfl(excl, src, kWave);
            *split = g - *first;
            return true;
        }
        base = __shfl(incl, kWave - 1, kWave);
    }
    return false;
}

// ---- prefill with all heads of a query in one workgroup --------------------
//
// bf16, latent 576 / value 512, 64 heads.  A workgroup (8 waves) owns one
// query position and every head, so each 64-row tile is gathered into LDS
// once for all 64 heads.  Wave w takes head block w % 4 (16 heads, one MFMA
// column block) and half w / 4 of the work: tile rows 32*half..+31 in the QK
// product and value channels 256*half..+255 in the PV product.  The two waves
// of a head block meet in LDS for the per-head (max, sum) of the tile; the
// operand layouts are those of attn_kernel.  Rows are listed 1024 at a time
// as device addresses (0: not a row of this query).  Two tile buffers: tile
// j + 1 is stored into the free one while tile j is computed, and tile
// j + 2 is loaded into registers during tile j's PV product.

// A row of zeros (never written): the gather reads it for a missing row.
constexpr int kP64ZeroRow = 1024;  // bf16 elements
__device__ __align__(16) uint16_t g_p64_zero_row[kP64ZeroRow];

// Two buffers of K rows (row-major; the PV product reads the value columns
// out of them with transposing LDS loads, and P^T, one row per head in p_pos
// order, goes into the columns past DV of the buffer's first 64 rows).
template <int DQK, int DV> struct P64Lds {
    // row stride of 296 words (8 mod 32): a K-row skew of 16 bf16 (32 bytes)
    // instead of 8 took the prefill_32k call from 3.25 to 2.90 ms in same-box
    // runs (strides of 4, 12 or 20 words mod 32 measured like 8 elements, 8
    // or 24 mod 32 like 16)
    static constexpr int kSkew = 16;
    static constexpr int kStrideK = DQK + kSkew;
    static constexpr size_t kOffB = (size_t)kP64Rows * kStrideK;  // second buffer
    static constexpr size_t kBytes = 2 * kOffB * sizeof(bf16_t);
};

template <int DQK, int DV, bool DEC>
__global__ __launch_bounds__(kP64Threads) void prefill64_kernel(AttnArgs a) {
    typedef bf16_t T;
    typedef P64Lds<DQK, DV> L;
    typedef Mma<T> M;
    constexpr int V16 = 8;                          // bf16 per 16-byte chunk
    constexpr int CPR = DQK / V16;                  // chunks per row
    constexpr int NKK = DQK / M::kK;                // MFMA steps of the QK product
    constexpr int DW = DV / 2;                      // value channels per wave
    constexpr int NMT = DW / 16;                    // O^T row tiles per wave
    static_assert(DQK % M::kK == 0 && DV % 32 == 0 && DV <= DQK, "unsupported head dims");
    static_assert(kP64Waves == 8 && kP64Heads == 4 * 16, "wave split");

    extern __shared__ __align__(16) unsigned char lds_raw[];
    T* Ks = reinterpret_cast<T*>(lds_raw);
    __shared__ const T* row_ptr[kP64Chunk];        // row address, nullptr: no row
    __shared__ unsigned long long tile_mask[kP64Chunk / kP64Rows];  // valid rows of each tile
    __shared__ float red_m[2][kP64Heads], red_s[2][kP64Heads];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int hb = wave & 3, half = wave >> 2;
    const int hl = lane & 15, quad = lane >> 4;
    const int head = hb * 16 + hl;
    const bool head_ok = head < a.H;

    // The zero row's address is read from the global offset table.  Decode
    // splits gather a tile or two: they take it here, beside the kernel
    // arguments, instead of in front of their first gather.
    const T* zrow = reinterpret_cast<const T*>(g_p64_zero_row);
    if constexpr (DEC) asm volatile("" : "+s"(zrow));

    int b, pq = 0, qpos = 0, n_comp, n_swa = 0, vr0 = 0, vr1 = a.max_rows;
    int part = 0;  // decode: this split's partial slot
    if constexpr (DEC) {
        bool have_len = false;
        if (a.dense_plan) {
            // split g of the device plan: R tiles of sequence b from tile R * split
            int R, split, first, count;
            if (a.n_seq <= kWave) {
                DenseSplit d;
                if (!dense_locate_wave(a, (int)blockIdx.x, &d)) return;  // uniform
                b = d.b;
                split = d.split;
                first = d.first;
                R = d.R;
                count = d.count;
                n_comp = d.comp;
                n_swa = d.swa;
                have_len = true;
            } else {
                R = dense_tiles_per_split(a);
                if (!dense_locate(a, R, (int)blockIdx.x, &b, &split, &first)) return;  // uniform
                count = ceil_div(dense_tiles(a, b), R);
            }
            // uniform values: scalar registers (the vector ones are all taken by the tiles)
            b = __builtin_amdgcn_readfirstlane(b);
            split = __builtin_amdgcn_readfirstlane(split);
            first = __builtin_amdgcn_readfirstlane(first);
            R = __builtin_amdgcn_readfirstlane(R);
            vr0 = split * R * kP64Rows;
            vr1 = vr0 + R * kP64Rows;
            part = first + split;
            // the sequence's first split hands its (first, count) to the merge
            if (split == 0 && tid == 0) a.dense_seq_plan[b] = first | (count << 16);
        } else {
            // decode split: workgroup (split x, sequence y) takes rows [vr0, vr1)
            b = blockIdx.y;
            vr0 = (int)blockIdx.x * a.rows_per_split;
            vr1 = min(a.max_rows, vr0 + a.rows_per_split);
            part = b * a.n_split + (int)blockIdx.x;
        }
        if (!have_len) {
            n_swa = a.swa_len[b];
            n_comp = a.comp_len[b];
        }
        n_swa = __builtin_amdgcn_readfirstlane(n_swa);
        n_swa = n_swa < 0 ? 0 : (n_swa > a.W ? a.W : n_swa);
        n_comp = __builtin_amdgcn_readfirstlane(n_comp);
        n_comp = n_comp < 0 ? 0 : (n_comp > a.S_max ? a.S_max : n_comp);
    } else {
        // queries go to XCDs in contiguous ranges (workgroup L runs on XCD L % 8),
        // so the windows of neighbouring positions meet in one L2
        const int nq8 = ceil_div(a.n_queries, 8);
        pq = ((int)blockIdx.x % 8) * nq8 + (int)blockIdx.x / 8;
        if (pq >= a.n_queries) return;
        b = pq / a.n_q;
        qpos = a.q_start + pq % a.n_q;
        n_comp = (qpos + 1) / a.m;
        n_comp = n_comp < a.S_max ? n_comp : a.S_max;
    }

    const T* win = reinterpret_cast<const T*>(a.win);
    const T* comp = reinterpret_cast<const T*>(a.comp);
    auto row_at = [&](int vr) -> const T* {
        if (vr >= vr1) return nullptr;
        if (vr < a.W) {
            if constexpr (DEC) {
                return vr < n_swa ? win + ((size_t)b * a.W + vr) * DQK : nullptr;
            } else {
                const int tok = qpos - a.W + 1 + vr;
                return tok >= 0 ? win + ((size_t)b * a.T_len + tok) * DQK : nullptr;
            }
        }
        const int j = vr - a.W;
        int ci;
        if (a.comp_idx)
            ci = j < a.k ? a.comp_idx[(size_t)(DEC ? b : pq) * a.k + j] : -1;
        else
            ci = j;
        return (ci >= 0 && ci < n_comp) ? comp + ((size_t)b * a.S_max + ci) * DQK : nullptr;
    };
    // index loads before the Q loads (decode mode: the first row of each
    // thread only, its other registers leave less room)
    constexpr int kFirst = DEC ? 1 : kP64Chunk / kP64Threads;
    const T* first_row[kFirst];
#pragma unroll
    for (int i = 0; i < kFirst; ++i) first_row[i] = row_at(vr0 + i * kP64Threads + tid);

    typename M::frag qf[NKK];
    {
        const T* qrow = reinterpret_cast<const T*>(a.q) + ((size_t)(DEC ? b : pq) * a.H + (head_ok ? head : 0)) * DQK;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            u32x4 v = head_ok ? *reinterpret_cast<const u32x4*>(qrow + kk * M::kK + quad * 8)
                              : u32x4{0u, 0u, 0u, 0u};
            qf[kk] = __builtin_bit_cast(bf16x8, v);
        }
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[NMT];
#pragma unroll
    for (int t = 0; t < NMT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // gather: thread t moves chunks (t & 7) + 8 i of row t / 8 of a tile (one
    // instruction of a wave covers eight 128-byte runs), stored row-major
    static_assert(CPR % 8 == 0 && kP64Rows * 8 == kP64Threads, "gather map");
    constexpr int kIter = CPR / 8;
    u32x4 ga[kIter];
    // loads it0 .. it1 - 1 of this thread's row pr (nullptr: the zero row).
    // Global (not flat) loads with no select on the data: a flat load also
    // counts against the LDS wait counter, and a select would wait for it.
    static_assert(DQK <= kP64ZeroRow, "zero row");
    typedef const __attribute__((address_space(1))) u32x4 gu32x4;
    auto issue_part = [&](const T* pr, int it0, int it1) {
        const T* z = DEC ? zrow : reinterpret_cast<const T*>(g_p64_zero_row);
        const T* src = (pr ? pr : z) + (tid & 7) * V16;
#pragma unroll
        for (int it = it0; it < it1; ++it)
            ga[it] = *(gu32x4*)(src + 8 * it * V16);
    };
    auto issue = [&](int tb) { issue_part(row_ptr[tb + (tid >> 3)], 0, kIter); };
    auto store = [&](T* buf) {
#pragma unroll
        for (int it = 0; it < kIter; ++it)
            *reinterpret_cast<u32x4*>(buf + (size_t)(tid >> 3) * L::kStrideK + ((tid & 7) + 8 * it) * V16) = ga[it];
    };

    // Two K buffers: tile j is computed from buffer j mod 2 while tile j + 1,
    // loaded into registers during tile j - 1, is stored into the other one
    // between the tile's two barriers (its last reader, the PV product of
    // tile j - 1, has finished everywhere by the first).  Once the QK product
    // is done the K columns past DV are free and hold P^T of the tile.
    static_assert(DQK - DV >= kP64Rows && kP64Heads <= kP64Rows, "P^T in the rope columns");
    int cur = 0;
    for (int c0 = vr0; c0 < vr1; c0 += kP64Chunk) {
        const int c1 = min(vr1, c0 + kP64Chunk);
        const int ntile = ceil_div(c1 - c0, kP64Rows);
#pragma unroll
        for (int i = 0; i < kP64Chunk / kP64Threads; ++i) {
            const int r = i * kP64Threads + tid;
            const T* p_row = c0 == vr0 && i < kFirst ? first_row[i < kFirst ? i : 0] : row_at(c0 + r);
            row_ptr[r] = p_row;
            // wave w's 64 threads hold the 64 rows of tile 8 i + w of the chunk
            static_assert(kP64Rows == kWave, "one tile per wave");
            const unsigned long long m = __ballot(p_row != nullptr);
            if (lane == 0) tile_mask[i * kP64Waves + wave] = m;
        }
        __syncthreads();
        // the chunk's tiles with a row, one bit each (uniform)
        static_assert(kP64Chunk / kP64Rows <= kWave, "tile bits");
        const unsigned long long live = __ballot(lane < ntile && tile_mask[lane < ntile ? lane : 0] != 0ull);
        auto next_tile = [&](int j) -> int {  // first live tile >= j, or -1
            const unsigned long long r = j < 64 ? live >> j : 0ull;
            return r ? j + (int)__builtin_ctzll(r) : -1;
        };
        int tj = next_tile(0);
        if (tj < 0) continue;  // uniform
        issue(tj * kP64Rows);
        store(Ks + (size_t)cur * L::kOffB);
        __syncthreads();
        int nj = next_tile(tj + 1);
        if (nj >= 0) issue(nj * kP64Rows);

        for (; tj >= 0; cur ^= 1) {
            T* Kc = Ks + (size_t)cur * L::kOffB;
            // the tile's row mask, uniform: in scalar registers
            const unsigned long long tm0 = tile_mask[tj];
            const unsigned long long tm =
                ((unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(tm0 >> 32)) << 32) |
                (unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)tm0);

            // ---- S^T for rows 32*half + 16*rb + 4*quad + r, head hl
            f32x4 s[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                f32x4 e0 = f32x4{0.f, 0.f, 0.f, 0.f}, e1 = f32x4{0.f, 0.f, 0.f, 0.f};
                const T* krow = Kc + (size_t)(32 * half + 16 * rb + hl) * L::kStrideK;
                // K fragments read a group ahead (decode mode: groups of 3, its
                // workgroups' other registers leave less room)
                constexpr int KG = DEC ? (NKK % 3 == 0 ? 3 : 1) : (NKK % 6 == 0 ? 6 : 1);
#pragma unroll
                for (int g0 = 0; g0 < NKK; g0 += KG) {
                    u32x4 v[KG];
#pragma unroll
                    for (int j = 0; j < KG; ++j)
                        v[j] = *reinterpret_cast<const u32x4*>(krow + (g0 + j) * M::kK + quad * 8);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < KG; ++j) {
                        const int kk = g0 + j;
                        if (kk & 1)
                            e1 = M::mma(__builtin_bit_cast(bf16x8, v[j]), qf[kk], e1);
                        else
                            e0 = M::mma(__builtin_bit_cast(bf16x8, v[j]), qf[kk], e0);
                    }
                }
                s[rb] = e0 + e1;
            }

            // ---- online softmax (base 2) over this wave's 32 rows, then the
            // two halves of the head block meet in LDS
            float x[8];
            float wmax = -INFINITY;
            // bit 16 rb + r: row 32 half + 16 rb + 4 quad + r of the tile
            const uint32_t tmr = (uint32_t)(tm >> (32 * half + 4 * quad));
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = (tmr >> (16 * rb + r)) & 1u ? s[rb][r] * a.scale_log2 : -INFINITY;
                    x[4 * rb + r] = v;
                    wmax = fmaxf(wmax, v);
                }
            }
            wmax = quad4_max(wmax);
            float p[8];
            float wsum = 0.f;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                p[r] = wmax == -INFINITY ? 0.f : exp2_le0(x[r] - wmax);
                wsum += p[r];
            }
            wsum = quad4_sum(wsum);
            if (quad == 0) {
                red_m[half][head] = wmax;
                red_s[half][head] = wsum;
            }
            __syncthreads();
            float rm[2], rs[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                rm[h2] = red_m[h2][head];
                rs[h2] = red_s[h2][head];
            }
            // the next tile into the other buffer, and the one after it into registers
            // the next tile into the other buffer; the tile after it is
            // loaded into registers during the PV product below, a load per
            // group of MFMAs, so that the vector memory unit (about 16 cycles
            // per 1 KB wave load) works under the MFMAs instead of holding up
            // this phase
            int nn = -1;
            const T* nn_row = nullptr;
            if (nj >= 0) {
                store(Ks + (size_t)(cur ^ 1) * L::kOffB);
                nn = next_tile(nj + 1);
                if (nn >= 0) nn_row = row_ptr[nn * kP64Rows + (tid >> 3)];
            }
            const float tmax = fmaxf(rm[0], rm[1]);
            const bool move = tmax > m_run + 8.f;   // lazy rescale, p stays <= 2^8
            const float m_new = move ? tmax : m_run;
            const float alpha = move ? exp2_le0(m_run - m_new) : 1.f;
            float tsum = 0.f;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
                if (rm[h2] != -INFINITY) tsum += rs[h2] * exp2_le0(rm[h2] - m_new);
            const float sc = wmax == -INFINITY ? 0.f : exp2_le0(wmax - m_new);
            T* pbase = Kc + (size_t)head * L::kStrideK + DV;  // P^T row of this head
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {  // P^T in the PV k-slot order (p_pos)
                *reinterpret_cast<uint2*>(pbase + p_pos(32 * half + 16 * rb + 4 * quad)) =
                    pack_p4(p[4 * rb] * sc, p[4 * rb + 1] * sc, p[4 * rb + 2] * sc, p[4 * rb + 3] * sc);
            }
            if (__ballot(move && l_run > 0.f)) {
#pragma unroll
                for (int t = 0; t < NMT; ++t) acc[t] *= alpha;
            }
            l_run = l_run * alpha + tsum;
            m_run = m_new;
            __syncthreads();

            // ---- O^T[channels 256*half + 16t.., head] += V^T * P^T; V^T
            // fragments by transposing reads of the K rows (as attn_kernel)
            const T* vtr = Kc + (size_t)(4 * quad + ((lane & 15) >> 2)) * L::kStrideK + half * DW + 4 * (lane & 3);
#pragma unroll
            for (int ks = 0; ks < kP64Rows / 32; ++ks) {
                const bf16x8 pf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(pbase + ks * 32 + quad * 8));
                constexpr int VG = 4;  // V^T fragments read a group ahead of their MFMAs
#pragma unroll
                for (int t0 = 0; t0 < NMT; t0 += VG) {
                    u32x4 vv[VG];
#pragma unroll
                    for (int j = 0; j < VG; ++j) {
                        const T* pa = vtr + (size_t)(32 * ks) * L::kStrideK + 16 * (t0 + j);
                        const uint2 lo = lds_read_tr16x4(pa);
                        const uint2 hi = lds_read_tr16x4(pa + (size_t)16 * L::kStrideK);
                        vv[j] = u32x4{lo.x, lo.y, hi.x, hi.y};
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < VG; ++j)
                        acc[t0 + j] = M::mma(__builtin_bit_cast(bf16x8, vv[j]), pf, acc[t0 + j]);
                    // group g of the PV product issues loads [kIter g / G, kIter (g + 1) / G)
                    constexpr int G = (kP64Rows / 32) * (NMT / VG);
                    const int g = ks * (NMT / VG) + t0 / VG;
                    if (nn >= 0) issue_part(nn_row, kIter * g / G, kIter * (g + 1) / G);  // uniform
                }
            }
            tj = nj;
            nj = nn;
        }
    }

    // ---- epilogue.  acc[t][r] = O^T[256*half + 16t + 4quad + r][head]
    if (!head_ok) return;
    if constexpr (DEC) {
        if (a.n_split > 1 || a.dense_plan) {  // unnormalised partials for the merge kernel
            const size_t prow = (size_t)part * a.H + head;
            if (half == 0 && quad == 0)
                *reinterpret_cast<float2*>(a.part_ml + prow * 2) = float2{m_run, l_run};
            float* po = a.part_o + prow * DV + half * DW;
#pragma unroll
            for (int t = 0; t < NMT; ++t)  // streamed past the L2: only the merge kernel reads it
                __builtin_nontemporal_store(acc[t], reinterpret_cast<f32x4*>(po + t * 16 + quad * 4));
            return;
        }
    }
    const size_t orow = (size_t)(DEC ? b : pq) * a.H + head;
    T* o = reinterpret_cast<T*>(a.out) + orow * DV + half * DW;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int t = 0; t < NMT; ++t)  // hardware conversion (nearest-even, NaN stays NaN): two per instruction
        *reinterpret_cast<uint2*>(o + t * 16 + quad * 4) =
            pack_p4(acc[t][0] * inv, acc[t][1] * inv, acc[t][2] * inv, acc[t][3] * inv);
    if (a.lse && half == 0 && quad == 0)
        a.lse[orow] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

// Merge the split partials of one (sequence, head) in a fixed split order.
// All (max, sum) pairs are loaded at once, the weights go through LDS, and
// each thread then issues the loads of its 4 channels for every split before
// combining them.  With a device plan (plan.dense_plan) the sequence's splits
// are the ones the attention launch recorded for it.

template <typename T, int DV, int kBatch>
__global__ __launch_bounds__(128) void attn_merge_kernel(const float* __restrict__ part_ml,
                                                         const float* __restrict__ part_o,
                                                         void* __restrict__ out,
                                                         float* __restrict__ lse, int H,
                                                         int n_split, uint8_t* __restrict__ sel_ws,
                                                         int S_max, int k, AttnArgs plan) {
    // kBatch: split partials loaded per round (the launch picks the
    // smallest of 4, 8, 12, 16 that covers the splits, or 16)
    auto load4 = [&](size_t i) -> f32x4 { return *reinterpret_cast<const f32x4*>(part_o + i); };
    __shared__ float wsp[kMaxSplit], lsp[kMaxSplit];
    __shared__ float stat[2];
    const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
    int first = b * n_split;
    if (plan.dense_plan) {  // written by the attention launch's first split of the sequence
        const int v = plan.dense_seq_plan[b];
        first = v & 0xffff;
        n_split = v >> 16;
    }
    const size_t p0 = ((size_t)first * H + h) * DV;  // element index of split 0
    const size_t sstride = (size_t)H * DV;
    const int d = tid * 4;           // this thread's 4 channels (DV <= 512)
    const bool has_d = d < DV;
    const int dc = has_d ? d : 0;    // loads stay in bounds; results of !has_d are not stored
    // first round of output partials in flight with the (max, sum) loads; the
    // loads are unconditional (a slot past n_split reloads the last split and
    // is not accumulated), so none of them waits for another
    f32x4 pv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) pv[j] = load4(p0 + (size_t)min(j, n_split - 1) * sstride + dc);
    float ms = -INFINITY, ls = 0.f;
    if (tid < n_split) {
        const float2 v = *reinterpret_cast<const float2*>(part_ml + (((size_t)first + tid) * H + h) * 2);
        ms = v.x;
        ls = v.y;
    }
    wsp[tid] = ms;
    __syncthreads();
    if (tid == 0) {
        float mx = -INFINITY;
        for (int s = 0; s < n_split; ++s) mx = fmaxf(mx, wsp[s]);
        stat[0] = mx;
    }
    __syncthreads();
    const float mx = stat[0];
    const float wgt = (tid < n_split && ms != -INFINITY) ? exp2_le0(ms - mx) : 0.f;
    __syncthreads();
    wsp[tid] = wgt;
    lsp[tid] = ls * wgt;
    __syncthreads();
    if (tid == 0) {
        float L = 0.f;
        for (int s = 0; s < n_split; ++s) L += lsp[s];
        stat[1] = L;
    }
    __syncthreads();
    const float L = stat[1];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_split; s0 += kBatch) {
        if (s0 > 0) {
#pragma unroll
            for (int j = 0; j < kBatch; ++j) pv[j] = load4(p0 + (size_t)min(s0 + j, n_split - 1) * sstride + dc);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int s = s0 + j;
            if (s < n_split) {
                const float wj = wsp[s];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(pv[j][e], wj, acc[e]);
            }
        }
    }
    if (has_d) {  // the thread's 4 channels in one store
        T* o = reinterpret_cast<T*>(out) + ((size_t)b * H + h) * DV + d;
        if constexpr (sizeof(T) == 2) {
            const uint2 pk{(uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16),
                           (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16)};
            *reinterpret_cast<uint2*>(o) = pk;
        } else {
            *reinterpret_cast<f32x4*>(o) = acc * inv;
        }
    }
    if (lse && tid == 0) lse[(size_t)b * H + h] = L > 0.f ? (mx + log2f(L)) * kLn2 : -INFINITY;
    // fused decode: every reader of the sequence's first-digit histogram (the
    // attention workgroups) has finished; clear it for the next call's scoring
    if (sel_ws && h == 0) {
        uint32_t* hist = sel::ws_of(sel_ws, b, S_max, k).hist;
        for (int i = tid; i < sel::kBins; i += 128) hist[i] = 0;
    }
}

template <typename T, int DQK, int DV, int MODE>
hipError_t launch_attn_kernel(const AttnArgs& a, dim3 grid, hipStream_t st) {
    size_t lds = TileLds<T, DQK, DV>::kBytes;
    if ((MODE == kModeFused || MODE == kModeFusedVar) && lds < kSelStageOff + kSelStageBytes)
        lds = kSelStageOff + kSelStageBytes;
    static bool attr_set = false;  // raise the dynamic-LDS limit once per instantiation
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&attn_kernel<T, DQK, DV, MODE>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    ProfScope prof(kProfAttn, st);
    hipLaunchKernelGGL((attn_kernel<T, DQK, DV, MODE>), grid, dim3(kAttnThreads), lds, st, a);
    return hipGetLastError();
}

template <int MODE>
hipError_t dispatch_attn(int dtype, int d_qk, int d_v, const AttnArgs& a, dim3 grid,
                         hipStream_t st) {
    (void)d_v;
    if (dtype == kBF16) {
        if (d_qk == 576) return launch_attn_kernel<bf16_t, 576, 512, MODE>(a, grid, st);
        return launch_attn_kernel<bf16_t, 128, 128, MODE>(a, grid, st);
    }
    return launch_attn_kernel<float, 128, 128, MODE>(a, grid, st);
}

}  // namespace

bool attn_shape_supported(int dtype, int d_qk, int d_v) {
    if (d_qk == 128 && d_v == 128) return true;
    return dtype == kBF16 && d_qk == 576 && d_v == 512;  // fp32 at 576 would spill registers
}

template <bool DEC>
hipError_t launch_p64(const AttnArgs& a, dim3 grid, hipStream_t st) {
    constexpr size_t lds = P64Lds<576, 512>::kBytes;
    static bool attr_set = false;  // raise the dynamic-LDS limit once per instantiation
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill64_kernel<576, 512, DEC>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    ProfScope prof(kProfAttn, st);
    hipLaunchKernelGGL((prefill64_kernel<576, 512, DEC>), grid, dim3(kP64Threads), lds, st, a);
    return hipGetLastError();
}

// Dense decode with 64 bf16 heads over a 576/512 latent goes to the 64-head
// kernel when its workgroups (one per split and sequence) fill the GPU.
bool decode64_applies(int B, int H, int d_v, int max_rows, bool dense) {
    return dense && H == kP64Heads && d_v == 512 && (long long)B * ceil_div(max_rows, kP64Rows) >= 256;
}

// the 64-head dense decode plans its splits on the device: at most
// kDenseTarget + B partial slots (partials of slot g at [g][H][...])
static int dense_parts(int B) { return kDenseTarget + B; }

DecodePlan plan_decode(int B, int H, int max_rows) {
    DecodePlan p;
    p.max_rows = max_rows;
    const int hblocks = ceil_div(H, kHeadsPerWG);
    const int tiles = ceil_div(max_rows, kTile);
    // about one workgroup per compute unit; a workgroup's tiles run one after
    // another, so small batches get one tile per split
    int n_split = ceil_div(256, B * hblocks);
    if (n_split > tiles) n_split = tiles;
    if (n_split > kMaxSplit) n_split = kMaxSplit;
    if (n_split < 1) n_split = 1;
    const int tiles_per = ceil_div(tiles, n_split);
    p.rows_per_split = tiles_per * kTile;
    p.n_split = ceil_div(max_rows, p.rows_per_split);
    if (p.n_split < 1) p.n_split = 1;
    return p;
}

// decode partials: (max, sum) pairs [B][n_split][H][2], then the unnormalised
// outputs [B][n_split][H][d_v] (16-byte aligned rows)
static size_t ml_bytes(int B, int n_split, int H) {
    return (((size_t)B * n_split * H * 2 * sizeof(float)) + 255) & ~(size_t)255;
}

size_t decode_workspace_bytes(int B, int H, int d_v, int max_rows, bool dense) {
    // enough for either plan (the 64-head one, dense only, is chosen at launch, by shape)
    const DecodePlan p = plan_decode(B, H, max_rows);
    size_t bytes = p.n_split <= 1 ? 0 : ml_bytes(B, p.n_split, H) + (size_t)B * p.n_split * H * d_v * sizeof(float);
    if (decode64_applies(B, H, d_v, max_rows, dense)) {
        const int P = dense_parts(B);
        const size_t b64 = ml_bytes(P, 1, H) + (size_t)P * H * d_v * sizeof(float) + (size_t)B * 4;
        bytes = b64 > bytes ? b64 : bytes;
    }
    return bytes;
}

template <int NB>
static void launch_merge_nb(int dtype, int d_v, const AttnArgs& a, int B, int H, int n_split,
                            int S_max, int k, hipStream_t st) {
    dim3 mg((unsigned)H, (unsigned)B);
    if (dtype == kBF16) {
        if (d_v == 512)
            hipLaunchKernelGGL((attn_merge_kernel<bf16_t, 512, NB>), mg, dim3(128), 0, st, a.part_ml,
                               a.part_o, a.out, a.lse, H, n_split, a.sel_ws, S_max, k, a);
        else
            hipLaunchKernelGGL((attn_merge_kernel<bf16_t, 128, NB>), mg, dim3(128), 0, st, a.part_ml,
                               a.part_o, a.out, a.lse, H, n_split, a.sel_ws, S_max, k, a);
    } else {
        hipLaunchKernelGGL((attn_merge_kernel<float, 128, NB>), mg, dim3(128), 0, st, a.part_ml,
                           a.part_o, a.out, a.lse, H, n_split, a.sel_ws, S_max, k, a);
    }
}

static hipError_t launch_merge(int dtype, int d_v, const AttnArgs& a, int B, int H, int n_split,
                               int S_max, int k, hipStream_t st) {
    ProfScope prof(kProfMerge, st);
    if (n_split <= 4) launch_merge_nb<4>(dtype, d_v, a, B, H, n_split, S_max, k, st);
    else if (n_split <= 8) launch_merge_nb<8>(dtype, d_v, a, B, H, n_split, S_max, k, st);
    else if (n_split <= 12) launch_merge_nb<12>(dtype, d_v, a, B, H, n_split, S_max, k, st);
    else launch_merge_nb<16>(dtype, d_v, a, B, H, n_split, S_max, k, st);
    return hipGetLastError();
}

hipError_t launch_attn_decode(int dtype, const void* q, const void* swa_kv,
                              const int32_t* swa_len, const void* comp_kv,
                              const int32_t* comp_idx, const int32_t* comp_len, void* out,
                              float* lse, int B, int H, int d_qk, int d_v, int W, int S_max,
                              int k, float scale, void* ws, hipStream_t st, const Paging* pg) {
    AttnArgs a = {};
    if (pg) {
        if (!comp_idx) return hipErrorInvalidValue;  // paged: sparse mode only
        a.pg_swa = pg->swa;
        a.pg_c4 = pg->c4;
        a.pos = pg->pos;
    }
    a.q = q;
    a.win = swa_kv;
    a.swa_len = swa_len;
    a.comp = comp_kv;
    a.comp_idx = comp_idx;
    a.comp_len = comp_len;
    a.out = out;
    a.lse = lse;
    a.part_ml = static_cast<float*>(ws);
    a.H = H;
    a.W = W;
    a.S_max = S_max;
    a.k = k;
    a.m = 1;
    const int max_rows = W + (comp_idx ? k : S_max);
    a.max_rows = max_rows;
    a.scale_log2 = scale * kLog2e;
    if (dtype == kBF16 && d_qk == 576 && decode64_applies(B, H, d_v, max_rows, comp_idx == nullptr)) {
        // splits planned on the device from comp_len (dense_locate / dense_seq)
        if (!ws) return hipErrorInvalidValue;
        const int P = dense_parts(B);
        a.dense_plan = 1;
        a.n_seq = B;
        a.n_split = kMaxSplit;  // the merge takes each sequence's split count from the plan
        a.part_o = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + ml_bytes(P, 1, H));
        a.dense_seq_plan = reinterpret_cast<int*>(a.part_o + (size_t)P * H * d_v);
        hipError_t e = launch_p64<true>(a, dim3((unsigned)P, 1u, 1u), st);
        if (e != hipSuccess) return e;
        return launch_merge(dtype, d_v, a, B, H, 8, S_max, k, st);
    }
    const DecodePlan p = plan_decode(B, H, max_rows);
    a.rows_per_split = p.rows_per_split;
    a.n_split = p.n_split;
    a.part_o = ws ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + ml_bytes(B, p.n_split, H))
                  : nullptr;
    dim3 grid((unsigned)p.n_split, (unsigned)B, (unsigned)ceil_div(H, kHeadsPerWG));
    hipError_t e = dispatch_attn<kModeDecode>(dtype, d_qk, d_v, a, grid, st);
    if (e != hipSuccess || p.n_split <= 1) return e;
    return launch_merge(dtype, d_v, a, B, H, p.n_split, S_max, k, st);
}

bool fused_decode_supported(int B, int H, int W, int k) {
    const DecodePlan p = plan_decode(B, H, W + k);
    return p.n_split >= 2 && p.rows_per_split <= kChunkRows;
}

hipError_t launch_attn_decode_fused(int dtype, const void* q, const void* swa_kv,
                                    const int32_t* swa_len, const void* comp_kv,
                                    const int32_t* comp_len, const int32_t* n_cand, void* sel_ws,
                                    const float* scores, int32_t* topk_out, void* out, float* lse, int B, int H,
                                    int d_qk, int d_v, int W, int S_max, int k, float scale,
                                    void* ws, hipStream_t st, const Paging* pg) {
    AttnArgs a = {};
    if (pg) {
        a.pg_swa = pg->swa;
        a.pg_c4 = pg->c4;
        a.pos = pg->pos;
    }
    a.q = q;
    a.win = swa_kv;
    a.swa_len = swa_len;
    a.comp = comp_kv;
    a.comp_idx = nullptr;
    a.comp_len = comp_len;
    a.sel_ws = static_cast<uint8_t*>(sel_ws);
    a.scores = scores;
    a.list_rows_lg = sel::list_rows_log2(S_max, B);
    a.n_cand = n_cand;
    a.topk_out = topk_out;
    a.out = out;
    a.lse = lse;
    a.part_ml = static_cast<float*>(ws);
    a.H = H;
    a.W = W;
    a.S_max = S_max;
    a.k = k;
    a.m = 1;
    const int max_rows = W + k;
    const DecodePlan p = plan_decode(B, H, max_rows);
    if (p.n_split < 2 || p.rows_per_split > kChunkRows) return hipErrorNotSupported;
    a.max_rows = max_rows;
    a.rows_per_split = p.rows_per_split;
    a.n_split = p.n_split;
    a.part_o = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + ml_bytes(B, p.n_split, H));
    a.scale_log2 = scale * kLog2e;
    // one more workgroup column per sequence writes the ascending top-k
    dim3 grid((unsigned)p.n_split + 1u, (unsigned)B, (unsigned)ceil_div(H, kHeadsPerWG));
    hipError_t e = a.list_rows_lg == 11 ? dispatch_attn<kModeFused>(dtype, d_qk, d_v, a, grid, st)
                                        : dispatch_attn<kModeFusedVar>(dtype, d_qk, d_v, a, grid, st);
    if (e != hipSuccess) return e;
    return launch_merge(dtype, d_v, a, B, H, p.n_split, S_max, k, st);
}

hipError_t launch_attn_prefill(int dtype, const void* q, const void* kv, const void* comp_kv,
                               const int32_t* comp_idx, void* out, float* lse, int n_seq,
                               int n_q, int q_start, int T_len, int H, int d_qk, int d_v, int W,
                               int S_max, int k, int m, float scale, hipStream_t st) {
    AttnArgs a = {};
    a.q = q;
    a.win = kv;
    a.comp = comp_kv;
    a.comp_idx = comp_idx;
    a.out = out;
    a.lse = lse;
    a.H = H;
    a.W = W;
    a.S_max = S_max;
    a.k = k;
    a.m = m;
    a.T_len = T_len;
    a.n_q = n_q;
    a.q_start = q_start;
    a.max_rows = W + (comp_idx ? k : S_max);
    a.rows_per_split = a.max_rows;
    a.n_split = 1;
    a.scale_log2 = scale * kLog2e;
    if ((long long)n_seq * n_q > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    a.hblocks = ceil_div(H, kHeadsPerWG);
    a.n_queries = n_seq * n_q;
    if (dtype == kBF16 && d_qk == 576 && d_v == 512 && H == kP64Heads) {
        const long long nwg = (long long)ceil_div(a.n_queries, 8) * 8;
        if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        return launch_p64<false>(a, dim3((unsigned)nwg), st);
    }
    const long long nwg = (long long)ceil_div(a.n_queries, 8) * 8 * a.hblocks;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)nwg, 1u, 1u);
    return dispatch_attn<kModePrefill>(dtype, d_qk, d_v, a, grid, st);
}

}  // namespace hsa
