// attention.hip -- fused SWA + compressed-row attention for gfx950.
//
// [LH "Tich hop Kernel va Giai ma suy doan"]: SWA and the extra C4/C128
// attention are combined in a single kernel call; [LH "Toi uu hoa suy luan
// voi ShadowRadix va HiSparse"]: a layer pairs SWA with C4 (sparse top-512)
// or C128 (dense).  One softmax runs over the union of the window rows and
// the compressed rows; the value of a latent row is its first d_v channels.
//
// Layout of the work.  A workgroup (4 waves) owns up to 64 query heads, 16
// per wave, and a range of "virtual rows": rows 0..W-1 are the window (ring
// slots for decode, causal tokens for prefill), rows W.. are the compressed
// candidates (the index list in sparse mode, 0..len-1 in dense mode).
// Rows are processed in tiles of 32:
//   1. gather: the 32 latent rows are copied into LDS with 16-byte loads,
//      row-major for the QK product and transposed (first d_v channels) for
//      the PV product; rows that are not valid are zero-filled and masked;
//   2. S^T = K_tile * Q^T on MFMA 16x16 tiles (rows on M, heads on N), so a
//      lane owns one head and 8 rows of the tile;
//   3. online softmax per head in base 2 (running max and sum per lane);
//   4. O^T += V^T * P^T on MFMA, P^T taken straight from the S^T registers
//      (the row order inside the contraction is permuted identically in both
//      operands, which leaves the sum unchanged), accumulating O^T in fp32.
// Decode splits the rows of a sequence over several workgroups and merges
// their (max, sum, O) partials in a second kernel, in a fixed order; prefill
// gives each query position its own workgroup.
#include "hsa_common.hpp"
#include "hsa_internal.hpp"

namespace hsa {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = 64;
constexpr int kTile = 32;
constexpr int kChunkRows = 256;  // rows whose list is built at once (one per thread)
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

// Position of tile row r inside a transposed V row: the 8 rows that lane
// group q contracts in one bf16 MFMA step (4q..4q+3 and 16+4q..16+4q+3, the
// rows its S^T registers hold) become contiguous, as do the 4 rows of one fp32
// step (16*mt + 4q .. +3 at 8q + 4mt).
__device__ __forceinline__ int vt_pos(int r) { return 8 * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3); }

// Element x of a 16-byte chunk, and a store of the x-th elements of two rows
// (consecutive in the transposed tile) as one 2-element write.
template <typename T> struct Pair;
template <> struct Pair<bf16_t> {
    __device__ static __forceinline__ void put(bf16_t* dst, const u32x4& a, const u32x4& b, int x) {
        const uint32_t lo = (a[x >> 1] >> (16 * (x & 1))) & 0xffffu;
        const uint32_t hi = (b[x >> 1] >> (16 * (x & 1))) & 0xffffu;
        *reinterpret_cast<uint32_t*>(dst) = lo | (hi << 16);
    }
};
template <> struct Pair<float> {
    __device__ static __forceinline__ void put(float* dst, const u32x4& a, const u32x4& b, int x) {
        *reinterpret_cast<uint2*>(dst) = uint2{a[x], b[x]};
    }
};

struct AttnArgs {
    const void* q;
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
    float scale_log2;     // scale * log2(e)
};

// LDS footprint of one tile, in elements of T
template <typename T, int DQK, int DV> struct TileLds {
    static constexpr int kPadK = 16 / (int)sizeof(T);   // one 16-byte pad per K row
    static constexpr int kStrideK = DQK + kPadK;
    static constexpr int kPadV = 8;  // transposed rows stay 16-byte aligned
    static constexpr int kStrideV = kTile + kPadV;
    static constexpr size_t kBytes = (size_t)kTile * kStrideK * sizeof(T) +
                                     (size_t)DV * kStrideV * sizeof(T);
};

template <typename T, int DQK, int DV, bool PREFILL>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnArgs a) {
    typedef TileLds<T, DQK, DV> L;
    typedef Mma<T> M;
    constexpr int V16 = Elem<T>::kPer16B;          // elements per 16-byte chunk
    constexpr int CPR = DQK / V16;                 // 16-byte chunks per row
    constexpr int NKK = DQK / M::kK;               // MFMA steps of the QK product
    constexpr int NMT = DV / 16;                   // O^T row tiles
    static_assert(DQK % M::kK == 0 && DV % 16 == 0 && DV <= DQK && DV <= 512, "unsupported head dims");

    extern __shared__ __align__(16) unsigned char lds_raw[];
    T* Ks = reinterpret_cast<T*>(lds_raw);
    T* Vt = Ks + (size_t)kTile * L::kStrideK;
    __shared__ long long row_off[kChunkRows];  // element offset of the row in its source, -1 invalid
    __shared__ int row_src[kChunkRows];        // 0: window source, 1: compressed pool
    __shared__ int tile_any[kChunkRows / kTile];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int hl = lane & 15, quad = lane >> 4;
    const int hb = blockIdx.z;
    const int head = hb * kHeadsPerWG + wave * kHeadsPerWave + hl;
    const bool head_ok = head < a.H;

    // sequence / query identity and row range
    int b, qpos = 0, qid = 0, vr0, vr1;
    if constexpr (PREFILL) {
        const int i = blockIdx.x;
        b = blockIdx.y;
        qid = b * a.n_q + i;
        qpos = a.q_start + i;
        vr0 = 0;
        vr1 = a.max_rows;
    } else {
        b = blockIdx.y;
        vr0 = blockIdx.x * a.rows_per_split;
        vr1 = min(a.max_rows, vr0 + a.rows_per_split);
    }
    int n_swa, n_comp;
    if constexpr (PREFILL) {
        n_swa = 0;
        int vis = (qpos + 1) / a.m;
        n_comp = vis < a.S_max ? vis : a.S_max;
    } else {
        n_swa = a.swa_len[b];
        n_swa = n_swa < 0 ? 0 : (n_swa > a.W ? a.W : n_swa);
        n_comp = a.comp_len[b];
        n_comp = n_comp < 0 ? 0 : (n_comp > a.S_max ? a.S_max : n_comp);
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
            } else {
                if (vr < n_swa) off = ((long long)b * a.W + vr) * DQK;
            }
        } else {
            const int j = vr - a.W;
            int ci = -1;
            if (a.comp_idx) {
                if (j < a.k) {
                    const long long row = PREFILL ? (long long)qid : (long long)b;
                    ci = a.comp_idx[row * a.k + j];
                }
            } else {
                ci = j;
            }
            if (ci >= 0 && ci < n_comp) {
                off = ((long long)b * a.S_max + ci) * DQK;
                src = 1;
            }
        }
    };
    // the first chunk's index loads go out before the Q loads, so waiting for
    // them does not wait for Q (the vector-memory counter retires in order)
    long long first_off;
    int first_src;
    row_entry(vr0 + tid, min(vr1, vr0 + kChunkRows), first_off, first_src);

    // Q fragments for this lane's head: k-slots of lane group `quad`
    typename M::frag qf[NKK];
    {
        const T* qrow;
        if constexpr (PREFILL)
            qrow = reinterpret_cast<const T*>(a.q) + ((size_t)qid * a.H + (head_ok ? head : 0)) * DQK;
        else
            qrow = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.H + (head_ok ? head : 0)) * DQK;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if constexpr (sizeof(T) == 2) {
                u32x4 v = head_ok ? *reinterpret_cast<const u32x4*>(qrow + kk * M::kK + quad * 8)
                                  : u32x4{0u, 0u, 0u, 0u};
                qf[kk] = __builtin_bit_cast(bf16x8, v);
            } else {
                qf[kk] = head_ok ? reinterpret_cast<const float*>(qrow)[kk * M::kK + quad] : 0.f;
            }
        }
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[NMT];
#pragma unroll
    for (int t = 0; t < NMT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const T* win = reinterpret_cast<const T*>(a.win);
    const T* comp = reinterpret_cast<const T*>(a.comp);

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

    for (int t0 = c0; t0 < c1; t0 += kTile) {
        const int tb = t0 - c0;
        if (!tile_any[tb / kTile]) continue;  // uniform: nothing valid in this tile
        // ---- gather: a thread moves chunk `ch` of the row pair (2rp, 2rp+1);
        // K goes row-major, V transposed with the two rows packed in one write
        // (consecutive lanes -> consecutive words: no bank conflicts)
        constexpr int kUnits = (kTile / 2) * CPR;
        constexpr int kIter = (kUnits + kAttnThreads - 1) / kAttnThreads;
        u32x4 ga[kIter], gb[kIter];
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
#pragma unroll
        for (int it = 0; it < kIter; ++it) {
            const int u = tid + it * kAttnThreads;
            const int rp = u % (kTile / 2), ch = u / (kTile / 2);
            if (u < kUnits) {
                *reinterpret_cast<u32x4*>(Ks + (size_t)(2 * rp) * L::kStrideK + ch * V16) = ga[it];
                *reinterpret_cast<u32x4*>(Ks + (size_t)(2 * rp + 1) * L::kStrideK + ch * V16) = gb[it];
                if (ch * V16 < DV) {
#pragma unroll
                    for (int x = 0; x < V16; ++x)
                        Pair<T>::put(Vt + (size_t)(ch * V16 + x) * L::kStrideV + vt_pos(2 * rp), ga[it], gb[it], x);
                }
            }
        }
        __syncthreads();

        // ---- S^T tile: rows 16*mt + 4*quad + r, head `hl`
        f32x4 s[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
            const T* krow = Ks + (size_t)(mt * 16 + hl) * L::kStrideK;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                typename M::frag af;
                if constexpr (sizeof(T) == 2) {
                    u32x4 v = *reinterpret_cast<const u32x4*>(krow + kk * M::kK + quad * 8);
                    af = __builtin_bit_cast(bf16x8, v);
                } else {
                    af = reinterpret_cast<const float*>(krow)[kk * M::kK + quad];
                }
                c = M::mma(af, qf[kk], c);
            }
            s[mt] = c;
        }

        // ---- online softmax (base 2); masked rows -> -inf
        float x[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = mt * 16 + quad * 4 + r;
                const float v = row_off[tb + row] >= 0 ? s[mt][r] * a.scale_log2 : -INFINITY;
                x[mt * 4 + r] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
        // The reference max only moves when a logit exceeds it by more than
        // 2^8 (p stays <= 256, no overflow); the rescale of the accumulator is
        // skipped unless some lane of the wave moved a nonzero accumulator.
        const bool move = tmax > m_run + 8.f;
        const float m_new = move ? tmax : m_run;
        const float alpha = move ? exp2f(m_run - m_new) : 1.f;  // 0 when m_run = -inf
        float p[8];
        float psum = 0.f;
        if (m_new == -INFINITY) {
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = 0.f;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                p[j] = exp2f(x[j] - m_new);
                psum += p[j];
            }
        }
        psum += __shfl_xor(psum, 16, kWave);
        psum += __shfl_xor(psum, 32, kWave);
        if (__ballot(move && l_run > 0.f)) {
#pragma unroll
            for (int t = 0; t < NMT; ++t) acc[t] *= alpha;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;

        // ---- O^T += V^T * P^T
        if constexpr (sizeof(T) == 2) {
            // k-slot j of lane group `quad` <-> tile row (j<4 ? 4*quad+j : 16+4*quad+j-4)
            u32x4 pb;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                pb[w] = (uint32_t)f32_to_bf16(p[2 * w]) | ((uint32_t)f32_to_bf16(p[2 * w + 1]) << 16);
            const bf16x8 pf = __builtin_bit_cast(bf16x8, pb);
#pragma unroll
            for (int t = 0; t < NMT; ++t) {
                const T* vrow = Vt + (size_t)(t * 16 + hl) * L::kStrideV;
                const u32x4 vv = *reinterpret_cast<const u32x4*>(vrow + quad * 8);
                acc[t] = M::mma(__builtin_bit_cast(bf16x8, vv), pf, acc[t]);
            }
        } else {
            // one instruction per (row tile mt, register r): k-slot of group
            // `quad` <-> tile row 16*mt + 4*quad + r
#pragma unroll
            for (int t = 0; t < NMT; ++t) {
                const float* vrow = reinterpret_cast<const float*>(Vt) + (size_t)(t * 16 + hl) * L::kStrideV;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const f32x4 vv = *reinterpret_cast<const f32x4*>(vrow + quad * 8 + mt * 4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[t] = M::mma(vv[r], p[mt * 4 + r], acc[t]);
                }
            }
        }
        __syncthreads();  // LDS tile is rewritten by the next iteration
    }
    }

    // ---- epilogue.  acc[t][r] = O^T[16*t + 4*quad + r][head]
    if (!head_ok) return;
    if constexpr (!PREFILL) {
        if (a.n_split > 1) {
            const size_t prow = ((size_t)b * a.n_split + blockIdx.x) * a.H + head;
            if (quad == 0) *reinterpret_cast<float2*>(a.part_ml + prow * 2) = float2{m_run, l_run};
            float* pb = a.part_o + prow * DV;
#pragma unroll
            for (int t = 0; t < NMT; ++t)
                *reinterpret_cast<f32x4*>(pb + t * 16 + quad * 4) = acc[t];
            return;
        }
    }
    const size_t orow = PREFILL ? ((size_t)qid * a.H + head) : ((size_t)b * a.H + head);
    T* o = reinterpret_cast<T*>(a.out) + orow * DV;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int t = 0; t < NMT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) Elem<T>::store(o, t * 16 + quad * 4 + r, acc[t][r] * inv);
    if (a.lse && quad == 0)
        a.lse[orow] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

// Merge the split partials of one (sequence, head) in a fixed split order.
// All (max, sum) pairs are loaded at once, the weights go through LDS, and
// each thread then issues the loads of its 4 channels for every split before
// combining them.
constexpr int kMaxSplit = 128;

template <typename T, int DV>
__global__ __launch_bounds__(128) void attn_merge_kernel(const float* __restrict__ part_ml,
                                                         const float* __restrict__ part_o,
                                                         void* __restrict__ out,
                                                         float* __restrict__ lse, int H,
                                                         int n_split) {
    constexpr int kBatch = 32;  // split partials loaded per round
    auto load4 = [](const float* p) -> f32x4 { return *reinterpret_cast<const f32x4*>(p); };
    __shared__ float wsp[kMaxSplit], lsp[kMaxSplit];
    __shared__ float stat[2];
    const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
    const float* p0 = part_o + ((size_t)b * n_split * H + h) * DV;
    const size_t sstride = (size_t)H * DV;
    const int d = tid * 4;           // this thread's 4 channels (DV <= 512)
    const bool has_d = d < DV;
    // first round of output partials in flight with the (max, sum) loads
    f32x4 pv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
        pv[j] = (has_d && j < n_split) ? load4(p0 + j * sstride + d) : f32x4{0.f, 0.f, 0.f, 0.f};
    float ms = -INFINITY, ls = 0.f;
    if (tid < n_split) {
        const float2 v = *reinterpret_cast<const float2*>(part_ml + (((size_t)b * n_split + tid) * H + h) * 2);
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
    const float wgt = (tid < n_split && ms != -INFINITY) ? exp2f(ms - mx) : 0.f;
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
            for (int j = 0; j < kBatch; ++j) {
                const int s = s0 + j;
                pv[j] = (has_d && s < n_split) ? load4(p0 + s * sstride + d) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
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
    if (has_d) {
        T* o = reinterpret_cast<T*>(out) + ((size_t)b * H + h) * DV;
#pragma unroll
        for (int e = 0; e < 4; ++e) Elem<T>::store(o, d + e, acc[e] * inv);
    }
    if (lse && tid == 0) lse[(size_t)b * H + h] = L > 0.f ? (mx + log2f(L)) * kLn2 : -INFINITY;
}

template <typename T, int DQK, int DV, bool PREFILL>
hipError_t launch_attn_kernel(const AttnArgs& a, dim3 grid, hipStream_t st) {
    const size_t lds = TileLds<T, DQK, DV>::kBytes;
    static bool attr_set = false;  // raise the dynamic-LDS limit once per instantiation
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&attn_kernel<T, DQK, DV, PREFILL>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    ProfScope prof(kProfAttn, st);
    hipLaunchKernelGGL((attn_kernel<T, DQK, DV, PREFILL>), grid, dim3(kAttnThreads), lds, st, a);
    return hipGetLastError();
}

template <bool PREFILL>
hipError_t dispatch_attn(int dtype, int d_qk, int d_v, const AttnArgs& a, dim3 grid,
                         hipStream_t st) {
    (void)d_v;
    if (dtype == kBF16) {
        if (d_qk == 576) return launch_attn_kernel<bf16_t, 576, 512, PREFILL>(a, grid, st);
        return launch_attn_kernel<bf16_t, 128, 128, PREFILL>(a, grid, st);
    }
    return launch_attn_kernel<float, 128, 128, PREFILL>(a, grid, st);
}

}  // namespace

bool attn_shape_supported(int dtype, int d_qk, int d_v) {
    if (d_qk == 128 && d_v == 128) return true;
    return dtype == kBF16 && d_qk == 576 && d_v == 512;  // fp32 at 576 would spill registers
}

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

size_t decode_workspace_bytes(int B, int H, int d_v, int max_rows) {
    const DecodePlan p = plan_decode(B, H, max_rows);
    if (p.n_split <= 1) return 0;
    return ml_bytes(B, p.n_split, H) + (size_t)B * p.n_split * H * d_v * sizeof(float);
}

hipError_t launch_attn_decode(int dtype, const void* q, const void* swa_kv,
                              const int32_t* swa_len, const void* comp_kv,
                              const int32_t* comp_idx, const int32_t* comp_len, void* out,
                              float* lse, int B, int H, int d_qk, int d_v, int W, int S_max,
                              int k, float scale, void* ws, hipStream_t st) {
    AttnArgs a = {};
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
    const DecodePlan p = plan_decode(B, H, max_rows);
    a.max_rows = max_rows;
    a.rows_per_split = p.rows_per_split;
    a.n_split = p.n_split;
    a.part_o = ws ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + ml_bytes(B, p.n_split, H))
                  : nullptr;
    a.scale_log2 = scale * kLog2e;
    dim3 grid((unsigned)p.n_split, (unsigned)B, (unsigned)ceil_div(H, kHeadsPerWG));
    hipError_t e = dispatch_attn<false>(dtype, d_qk, d_v, a, grid, st);
    if (e != hipSuccess || p.n_split <= 1) return e;
    dim3 mg((unsigned)H, (unsigned)B);
    ProfScope prof(kProfMerge, st);
    if (dtype == kBF16) {
        if (d_v == 512)
            hipLaunchKernelGGL((attn_merge_kernel<bf16_t, 512>), mg, dim3(128), 0, st, a.part_ml, a.part_o, out, lse, H, p.n_split);
        else
            hipLaunchKernelGGL((attn_merge_kernel<bf16_t, 128>), mg, dim3(128), 0, st, a.part_ml, a.part_o, out, lse, H, p.n_split);
    } else {
        hipLaunchKernelGGL((attn_merge_kernel<float, 128>), mg, dim3(128), 0, st, a.part_ml, a.part_o, out, lse, H, p.n_split);
    }
    return hipGetLastError();
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
    dim3 grid((unsigned)n_q, (unsigned)n_seq, (unsigned)ceil_div(H, kHeadsPerWG));
    return dispatch_attn<true>(dtype, d_qk, d_v, a, grid, st);
}

}  // namespace hsa
