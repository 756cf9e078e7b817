// compress.hip -- one-pass block KV compressor for gfx950.
//
// [NK "推理侧优化", Kernel fusion bullet]: the compression chain reads the
// block, adds the bias to the gate logits, takes a softmax, multiplies with
// the latents and writes back; the middle three steps are fused so the block
// is read once and the entry written once ([KD "Arquitectura del Sistema"],
// Flash Compressor).  Here the whole chain is one kernel: x and gate are
// streamed once with 16-byte loads, the softmax runs online in registers
// (running max, running sum, running weighted sum, all fp32, base-2
// exponentials), and each entry is written once.
//
// Work unit = (sequence b, block i, 16-byte channel chunk c).
//  * m <= 4 (the C4 case): one thread owns a unit.  Workgroups stay resident
//    (as many as fit at once) and walk the units tile by tile with the next
//    tile's rows in flight; a thread keeps its chunk from tile to tile, so its
//    bias words are loaded once.
//  * larger m (C128): P = 4 threads split a block's rows into contiguous
//    ranges (32 rows each at m = 128), each walking its range four rows at a
//    time with the next four in flight (4 threads per unit measured faster
//    than 2, 8 or 16, and four rows per step faster than two or three); the partial (max, sum, weighted sum) triples are merged in LDS
//    in a fixed order, every thread merging some (unit, channel) pairs.
// The short-block kernel keeps its registers at <= 128 per lane (four waves
// per SIMD; the C128 kernel's four rows in flight take 163, three waves):
// the latents stay packed until their product is taken, and entries leave as
// one 16-byte store per chunk.
#include "compress_append.hpp"
#include "hsa_common.hpp"
#include "hsa_internal.hpp"

#include <algorithm>
#include <mutex>
#include <numeric>

namespace hsa {

namespace {

constexpr int kCompressThreads = 256;

// Softmax weights 2^(z - max) on the hardware base-2 exponential: every
// argument is <= 0, or -inf for a padded row (weight 0), so the library
// function's range reduction is not needed; a weight below 2^-126 comes out
// as 0, far below the fp32 resolution of the sum it joins (which holds the
// maximum row's weight 1).
__device__ __forceinline__ float exp2_le0(float x) { return __builtin_amdgcn_exp2f(x); }
// a / s with the hardware reciprocal (within about 1 ulp); s >= 1 here
__device__ __forceinline__ float div_ge1(float a, float s) { return a * __builtin_amdgcn_rcpf(s); }

// G rows of one chunk, as loaded: gate and latent words (the short-block
// kernel holds its bias words apart), and gate, bias and latent words.
template <int G> struct RowGroup {
    u32x4 g[G], x[G];
};
template <int G> struct RowGroupB {
    u32x4 g[G], b[G], x[G];
};

template <typename T, int P, int G>
__global__ __launch_bounds__(kCompressThreads) void compress_kernel(
    const T* __restrict__ x, const T* __restrict__ gate, const T* __restrict__ bias,
    T* __restrict__ out, int B, int T_len, int D, int m) {
    constexpr int V = Elem<T>::kPer16B;
    constexpr int U = kCompressThreads / P;  // units per workgroup
    const int u = (int)threadIdx.x % U;
    const int part = (int)threadIdx.x / U;
    const int nchunk = D / V;
    const int nblk = T_len / m;
    const long long unit = (long long)blockIdx.x * U + u;
    const long long nunits = (long long)B * nblk * nchunk;
    const bool active = unit < nunits;

    float M[V], S[V], A[V];
#pragma unroll
    for (int e = 0; e < V; ++e) { M[e] = -INFINITY; S[e] = 0.f; A[e] = 0.f; }

    int b = 0, i = 0, c = 0;
    if (active) {
        c = (int)(unit % nchunk);
        const long long bi = unit / nchunk;
        i = (int)(bi % nblk);
        b = (int)(bi / nblk);
        const int rp = (m + P - 1) / P;
        const int j0 = part * rp;
        const int j1 = min(m, j0 + rp);
        const size_t row0 = (size_t)b * T_len + (size_t)m * i;
        // the G rows from j on.  Every load is issued (a row past the part's
        // range reloads the part's last row, which is still cached, and is
        // masked below): a load under a branch would make the compiler wait
        // for the next group's loads too before this group's arithmetic.
        auto load = [&](RowGroupB<G>& rg, int j) {
#pragma unroll
            for (int r = 0; r < G; ++r) {
                const int jr = min(j + r, j1 - 1);
                const size_t off = (row0 + jr) * (size_t)D + (size_t)c * V;
                rg.g[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gate + off));
                rg.x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + off));
                rg.b[r] = *reinterpret_cast<const u32x4*>(bias + (size_t)jr * D + (size_t)c * V);
            }
        };
        RowGroupB<G> cur;
        load(cur, j0);
        for (int j = j0; j < j1; j += G) {
            RowGroupB<G> nxt;
            load(nxt, j + G);  // next group in flight during this one
            float z[G][V];
            const int g = min(G, j1 - j);
#pragma unroll
            for (int r = 0; r < G; ++r) {
                if (r < g) {
                    float gv[V], bv[V];
                    Elem<T>::unpack(cur.g[r], gv);
                    Elem<T>::unpack(cur.b[r], bv);
#pragma unroll
                    for (int e = 0; e < V; ++e) z[r][e] = (gv[e] + bv[e]) * kLog2e;
                } else {
#pragma unroll
                    for (int e = 0; e < V; ++e) z[r][e] = -INFINITY;
                }
            }
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float gm = z[0][e];
#pragma unroll
                for (int r = 1; r < G; ++r) gm = fmaxf(gm, z[r][e]);
                const float mn = fmaxf(M[e], gm);
                const float sc = exp2_le0(M[e] - mn);  // 0 on the first group (M = -inf)
                float s = 0.f, a = 0.f;
#pragma unroll
                for (int r = 0; r < G; ++r) {
                    const float w = exp2_le0(z[r][e] - mn);  // 0 for padded rows
                    s += w;
                    if (r < g) a = fmaf(w, chunk_elem<T>(cur.x[r], e), a);
                }
                S[e] = fmaf(S[e], sc, s);
                A[e] = fmaf(A[e], sc, a);
                M[e] = mn;
            }
            cur = nxt;
        }
    }

    if constexpr (P > 1) {
        // partial (max, sum, weighted sum) triples meet in LDS; every thread
        // then merges (unit, element) pairs over the P parts in a fixed order
        __shared__ float sm[P][U][V], ss[P][U][V], sa[P][U][V];
        __shared__ float res[U][V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            sm[part][u][e] = M[e];
            ss[part][u][e] = S[e];
            sa[part][u][e] = A[e];
        }
        __syncthreads();
        for (int idx = (int)threadIdx.x; idx < U * V; idx += kCompressThreads) {
            const int uu = idx / V, e = idx % V;
            float mx = sm[0][uu][e];
            for (int p = 1; p < P; ++p) mx = fmaxf(mx, sm[p][uu][e]);
            float s = 0.f, a = 0.f;
            for (int p = 0; p < P; ++p) {
                const float mp = sm[p][uu][e];
                const float w = (mp == -INFINITY) ? 0.f : exp2_le0(mp - mx);
                s = fmaf(ss[p][uu][e], w, s);
                a = fmaf(sa[p][uu][e], w, a);
            }
            res[uu][e] = div_ge1(a, s);
        }
        __syncthreads();
        if (part != 0 || !active) return;
        float r[V];
#pragma unroll
        for (int e = 0; e < V; ++e) r[e] = res[u][e];
        const size_t o = ((size_t)b * nblk + i) * (size_t)D + (size_t)c * V;
        *reinterpret_cast<u32x4*>(out + o) = pack16<T>(r);
        return;
    }
    if (!active) return;
    float r[V];
#pragma unroll
    for (int e = 0; e < V; ++e) r[e] = div_ge1(A[e], S[e]);
    const size_t o = ((size_t)b * nblk + i) * (size_t)D + (size_t)c * V;
    *reinterpret_cast<u32x4*>(out + o) = pack16<T>(r);
}

// Division by a divisor fixed for the launch, for dividends below 2^31: one
// high multiply and a shift with a precomputed multiplier (the round-up
// method of Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994: l = ceil(log2 d), mul = floor(2^32 (2^l - d) / d) + 1,
// n / d = (mulhi(mul, n) + n) >> l; the sum stays below 2^32 for n < 2^31).
struct MagicDiv {
    uint32_t d, mul;
    int shift;
};
inline MagicDiv make_magic(uint32_t d) {
    int l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t mul = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return MagicDiv{d, (uint32_t)mul, l};
}
__device__ __forceinline__ uint32_t magic_div(uint32_t n, const MagicDiv& m) {
    return (__umulhi(n, m.mul) + n) >> m.shift;
}

// Short blocks (m <= G): one thread owns a unit (b, i, c); a tile is
// kCompressThreads consecutive units.  Unit numbers below 2^31 (W64 false)
// are split into (chunk, block) with the magic divisions above (64-bit
// divisions cost more than the rest of a unit's work) and every workgroup
// takes one tile.  Larger inputs (W64) keep as many workgroups as fit at once
// walking the tiles, the next tile's rows in flight during this one; when the
// grid's unit stride is a multiple of the chunk count a thread keeps its
// chunk, so its bias words are loaded (and scaled by log2 e) once.
template <typename T, int G, bool W64>
__global__ __launch_bounds__(kCompressThreads) void compress_short_kernel(
    const T* __restrict__ x, const T* __restrict__ gate, const T* __restrict__ bias,
    T* __restrict__ out, int B, int T_len, int D, int m, int fixed_chunk, MagicDiv div_chunk,
    MagicDiv div_blk) {
    constexpr int V = Elem<T>::kPer16B;
    const int nchunk = D / V;
    const int nblk = T_len / m;
    const long long nunits = (long long)B * nblk * nchunk;
    const long long ntiles = (nunits + kCompressThreads - 1) / kCompressThreads;
    const long long stride = gridDim.x;
    // unit -> its chunk, its block number b * nblk + i and the block's first row
    auto split = [&](long long unit, int& c, long long& bi, size_t& row0) {
        if constexpr (W64) {
            c = (int)(unit % nchunk);
            bi = unit / nchunk;
            row0 = (size_t)(bi / nblk) * T_len + (size_t)m * (bi % nblk);
        } else {
            const uint32_t u = (uint32_t)unit;
            const uint32_t q = magic_div(u, div_chunk);
            const uint32_t b = magic_div(q, div_blk);
            c = (int)(u - q * (uint32_t)nchunk);
            bi = q;
            row0 = (size_t)b * T_len + (size_t)m * (q - b * (uint32_t)nblk);
        }
    };
    // Every load is issued, from a clamped unit and row (a unit past the end
    // reloads the last unit, a row past m the block's last row; neither is
    // used): a load under a branch would make the compiler wait for the next
    // tile's loads too before this tile's arithmetic.
    auto load = [&](RowGroup<G>& rg, long long t) {
        int c;
        long long bi;
        size_t row0;
        split(min(t * kCompressThreads + (long long)threadIdx.x, nunits - 1), c, bi, row0);
#pragma unroll
        for (int r = 0; r < G; ++r) {
            const size_t off = (row0 + min(r, m - 1)) * (size_t)D + (size_t)c * V;
            rg.g[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gate + off));
            rg.x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + off));
        }
    };
    u32x4 bw[G];
    float bl[G][V];  // bias * log2 e
    auto load_bias = [&](long long unit) {
        int c;
        long long bi;
        size_t row0;
        split(min(unit, nunits - 1), c, bi, row0);
#pragma unroll
        for (int r = 0; r < G; ++r)
            bw[r] = *reinterpret_cast<const u32x4*>(bias + (size_t)min(r, m - 1) * D + (size_t)c * V);
    };
    auto scale_bias = [&]() {
#pragma unroll
        for (int r = 0; r < G; ++r) {
            float bv[V];
            Elem<T>::unpack(bw[r], bv);
#pragma unroll
            for (int e = 0; e < V; ++e) bl[r][e] = bv[e] * kLog2e;
        }
    };
    // the tile's entries from its rows (cur) and the scaled bias (bl)
    auto tile = [&](long long t, const RowGroup<G>& cur) {
        const long long unit = t * kCompressThreads + threadIdx.x;
        if (unit >= nunits) return;
        int c;
        long long bi;
        size_t row0;
        split(unit, c, bi, row0);
        // z = (g + bias) log2 e as one fma per element
        float z[G][V];
#pragma unroll
        for (int r = 0; r < G; ++r) {
            if (r < m) {
                float gv[V];
                Elem<T>::unpack(cur.g[r], gv);
#pragma unroll
                for (int e = 0; e < V; ++e) z[r][e] = fmaf(gv[e], kLog2e, bl[r][e]);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) z[r][e] = -INFINITY;
            }
        }
        float res[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float gm = z[0][e];
#pragma unroll
            for (int r = 1; r < G; ++r) gm = fmaxf(gm, z[r][e]);
            float s = 0.f, a = 0.f;
#pragma unroll
            for (int r = 0; r < G; ++r) {
                const float w = exp2_le0(z[r][e] - gm);  // 0 for padded rows
                s += w;
                if (r < m) a = fmaf(w, chunk_elem<T>(cur.x[r], e), a);
            }
            res[e] = div_ge1(a, s);
        }
        *reinterpret_cast<u32x4*>(out + (size_t)bi * D + (size_t)c * V) = pack16<T>(res);
    };
    long long t = blockIdx.x;
    if constexpr (!W64) {
        // one tile per workgroup (the launch covers every tile): its rows and
        // bias go out together, and the hardware keeps each CU's share of the
        // grid in flight
        RowGroup<G> cur;
        load(cur, t);
        load_bias(t * kCompressThreads + threadIdx.x);
        scale_bias();
        tile(t, cur);
    } else {
        // resident workgroups walk the tiles, the next tile's rows in flight
        if (fixed_chunk) {
            load_bias(t * kCompressThreads + threadIdx.x);
            scale_bias();
        }
        RowGroup<G> cur;
        load(cur, t);
        for (; t < ntiles; t += stride) {
            // a thread whose chunk changes from tile to tile loads this tile's
            // bias words before the next tile's rows (the count retires in order)
            if (!fixed_chunk) load_bias(t * kCompressThreads + threadIdx.x);
            RowGroup<G> nxt;
            load(nxt, min(t + stride, ntiles - 1));
            if (!fixed_chunk) scale_bias();
            tile(t, cur);
            cur = nxt;
        }
    }
}

// resident workgroups of compress_short_kernel<T, G, true> on the current device
template <typename T, int G>
int short_kernel_capacity() {
    static std::mutex mu;
    static int cap[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lk(mu);
    if (cap[dev] == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(&compress_short_kernel<T, G, true>),
                kCompressThreads, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cap[dev] = std::max(1, per_cu) * std::max(1, cus);
    }
    return cap[dev];
}

template <typename T, int G>
hipError_t launch_compress_short(const void* x, const void* g, const void* bias, void* out, int B,
                                 int T_len, int D, int m, hipStream_t st) {
    const int nchunk = D / Elem<T>::kPer16B;
    const long long nunits = (long long)B * (T_len / m) * nchunk;
    const long long ntiles = (nunits + kCompressThreads - 1) / kCompressThreads;
    if (ntiles <= 0) return hipSuccess;
    const MagicDiv dc = make_magic((uint32_t)nchunk), db = make_magic((uint32_t)std::max(1, T_len / m));
    if ((ntiles + 1) * kCompressThreads < (1ll << 31)) {
        // unit numbers (clamped ones included) below 2^31: the 32-bit split and
        // one tile per workgroup (faster than the resident walk below once the
        // kernel's arithmetic stopped bounding it: 112 against 121 us for the
        // prefill_32k C4 call)
        ProfScope prof(kProfCompress, st);
        hipLaunchKernelGGL((compress_short_kernel<T, G, false>), dim3((unsigned)ntiles),
                           dim3(kCompressThreads), 0, st, (const T*)x, (const T*)g, (const T*)bias,
                           (T*)out, B, T_len, D, m, 0, dc, db);
        return hipGetLastError();
    }
    const int cap = short_kernel_capacity<T, G>();
    if (cap <= 0) return hipErrorInvalidDevice;
    long long grid = std::min<long long>(ntiles, cap);
    // a grid whose unit stride is a multiple of nchunk keeps every thread on one chunk
    const long long q = nchunk / std::gcd(nchunk, kCompressThreads);
    int fixed = 0;
    if (grid >= q && grid < ntiles) {
        grid -= grid % q;
        fixed = 1;
    } else if (grid == ntiles && ntiles <= 1) {
        fixed = 1;  // one tile: nothing to keep across tiles
    }
    ProfScope prof(kProfCompress, st);
    hipLaunchKernelGGL((compress_short_kernel<T, G, true>), dim3((unsigned)grid),
                       dim3(kCompressThreads), 0, st, (const T*)x, (const T*)g, (const T*)bias,
                       (T*)out, B, T_len, D, m, fixed, dc, db);
    return hipGetLastError();
}

template <typename T, int P, int G>
hipError_t launch_compress_p(const void* x, const void* g, const void* bias, void* out, int B,
                             int T_len, int D, int m, hipStream_t st) {
    constexpr int U = kCompressThreads / P;
    const long long nunits = (long long)B * (T_len / m) * (D / Elem<T>::kPer16B);
    const long long nwg = (nunits + U - 1) / U;
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    ProfScope prof(kProfCompress, st);
    hipLaunchKernelGGL((compress_kernel<T, P, G>), dim3((unsigned)nwg), dim3(kCompressThreads), 0, st,
                       (const T*)x, (const T*)g, (const T*)bias, (T*)out, B, T_len, D, m);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_compress_t(const void* x, const void* g, const void* bias, void* out, int B,
                             int T_len, int D, int m, hipStream_t st) {
    if (m <= 4) return launch_compress_short<T, 4>(x, g, bias, out, B, T_len, D, m, st);
    return launch_compress_p<T, 4, 4>(x, g, bias, out, B, T_len, D, m, st);
}

// ---- decode-time compression state ----
// [NK "DeepSeek V4 的新架构", five state classes] and [KD "Arquitectura del
// Sistema", compression-state ring buffers]: between block boundaries a
// sequence's newest tokens wait in a ring of m slots; the token that fills
// the last slot completes the block and its entry is formed.
//
// Workgroup (b, y) owns kAppendThreads / P consecutive chunks of sequence b;
// thread (part j, chunk c).  Part-0 threads store the token's chunks into
// slot pos mod m.  When the token completes its block, part j folds rows
// j, j+P, j+2P, ... (kAppendRows of them in flight at a time) into a running
// (max, sum, weighted sum) per channel, the completing row read from the
// token itself, and the P partials of a chunk are merged in LDS in part order.
// Different workgroups touch disjoint chunks, so nothing is shared between them.
constexpr int kAppendThreads = 256;
constexpr int kAppendRows = 4;

template <typename T>
__global__ __launch_bounds__(kAppendThreads) void compress_append_kernel(
    const T* __restrict__ x_tok, const T* __restrict__ g_tok, const T* __restrict__ bias,
    T* __restrict__ ring_x, T* __restrict__ ring_g, const int32_t* __restrict__ pos,
    T* __restrict__ pool, int D, int m, int S_max, int parts) {
    constexpr int V = Elem<T>::kPer16B;
    __shared__ float part_max[V * kAppendThreads], part_sum[V * kAppendThreads],
        part_acc[V * kAppendThreads];
    const int b = blockIdx.x;
    const int p = pos[b];
    if (p < 0) return;  // idle sequence: takes no token
    const int cw = kAppendThreads / parts;
    const int part = threadIdx.x / cw;
    const int cl = threadIdx.x - part * cw;
    const int c = blockIdx.y * cw + cl;
    const bool live = c < D / V;
    const int s = p % m;
    const size_t tok = (size_t)b * D + (size_t)c * V;
    const size_t ring = (size_t)b * m * D + (size_t)c * V;
    if (live && part == 0) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(x_tok + tok);
        const u32x4 gv = *reinterpret_cast<const u32x4*>(g_tok + tok);
        *reinterpret_cast<u32x4*>(ring_x + ring + (size_t)s * D) = xv;
        *reinterpret_cast<u32x4*>(ring_g + ring + (size_t)s * D) = gv;
    }
    const int blk = p / m;
    if (s != m - 1 || blk >= S_max) return;  // block still open, or past the pool

    float mx[V], sm[V], acc[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        mx[e] = -INFINITY;
        sm[e] = 0.f;
        acc[e] = 0.f;
    }
    if (live) {
        for (int r0 = part; r0 < m; r0 += kAppendRows * parts) {
            u32x4 gw[kAppendRows], bw[kAppendRows], xw[kAppendRows];
#pragma unroll
            for (int k = 0; k < kAppendRows; ++k) {
                const int r = r0 + k * parts;
                if (r < m) {
                    const bool own = r == s;  // the completing row is this call's token
                    gw[k] = *reinterpret_cast<const u32x4*>(
                        own ? g_tok + tok : ring_g + ring + (size_t)r * D);
                    xw[k] = *reinterpret_cast<const u32x4*>(
                        own ? x_tok + tok : ring_x + ring + (size_t)r * D);
                    bw[k] = *reinterpret_cast<const u32x4*>(bias + (size_t)r * D + (size_t)c * V);
                }
            }
            float z[kAppendRows][V];
#pragma unroll
            for (int k = 0; k < kAppendRows; ++k) {
                if (r0 + k * parts < m) {
                    float gv[V], bv[V];
                    Elem<T>::unpack(gw[k], gv);
                    Elem<T>::unpack(bw[k], bv);
#pragma unroll
                    for (int e = 0; e < V; ++e) z[k][e] = (gv[e] + bv[e]) * kLog2e;
                } else {
#pragma unroll
                    for (int e = 0; e < V; ++e) z[k][e] = -INFINITY;
                }
            }
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float gm = mx[e];
#pragma unroll
                for (int k = 0; k < kAppendRows; ++k) gm = fmaxf(gm, z[k][e]);
                const float sc = exp2f(mx[e] - gm);  // 0 on the first group
                float s_e = sm[e] * sc, a_e = acc[e] * sc;
#pragma unroll
                for (int k = 0; k < kAppendRows; ++k) {
                    const float w = exp2f(z[k][e] - gm);  // 0 for rows past m
                    s_e += w;
                    if (r0 + k * parts < m) a_e = fmaf(w, chunk_elem<T>(xw[k], e), a_e);
                }
                mx[e] = gm;
                sm[e] = s_e;
                acc[e] = a_e;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
        part_max[e * kAppendThreads + threadIdx.x] = mx[e];
        part_sum[e * kAppendThreads + threadIdx.x] = sm[e];
        part_acc[e * kAppendThreads + threadIdx.x] = acc[e];
    }
    __syncthreads();
    // merge: one (channel element, chunk) pair per thread per pass, parts in order;
    // the result overwrites part 0's weighted-sum slot
    for (int q = threadIdx.x; q < V * cw; q += kAppendThreads) {
        const int e = q / cw, ql = q - e * cw;
        const int base = e * kAppendThreads + ql;
        float gm = part_max[base];
        for (int j = 1; j < parts; ++j) gm = fmaxf(gm, part_max[base + j * cw]);
        float s_e = 0.f, a_e = 0.f;
        for (int j = 0; j < parts; ++j) {
            const float w = exp2f(part_max[base + j * cw] - gm);
            s_e = fmaf(part_sum[base + j * cw], w, s_e);
            a_e = fmaf(part_acc[base + j * cw], w, a_e);
        }
        part_max[base] = a_e / s_e;  // slot (e, part 0, ql) is read by its own thread only
    }
    __syncthreads();
    if (live && part == 0) {
        float res[V];
#pragma unroll
        for (int e = 0; e < V; ++e) res[e] = part_max[e * kAppendThreads + cl];
        *reinterpret_cast<u32x4*>(pool + ((size_t)b * S_max + blk) * D + (size_t)c * V) =
            pack16<T>(res);
    }
}

// m = M <= 4 (the C4 case): one thread per chunk, the whole block in its
// registers (append_short_chunk).
template <typename T, int M>
__global__ __launch_bounds__(kAppendThreads) void compress_append_short_kernel(
    const T* x_tok, const T* g_tok, const T* bias, T* ring_x, T* ring_g, const int32_t* pos,
    T* pool, int D, int S_max) {
    append_short_chunk<T, M>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, D, S_max, blockIdx.x,
                             blockIdx.y * kAppendThreads + threadIdx.x);
}

template <typename T, int M>
hipError_t launch_append_short(const void* x_tok, const void* g_tok, const void* bias,
                               void* ring_x, void* ring_g, const int32_t* pos, void* pool, int B,
                               int D, int S_max, hipStream_t st) {
    const int nchunk = D / Elem<T>::kPer16B;
    const int gy = (nchunk + kAppendThreads - 1) / kAppendThreads;
    ProfScope prof(kProfCompress, st);
    hipLaunchKernelGGL((compress_append_short_kernel<T, M>), dim3((unsigned)B, (unsigned)gy),
                       dim3(kAppendThreads), 0, st, (const T*)x_tok, (const T*)g_tok,
                       (const T*)bias, (T*)ring_x, (T*)ring_g, pos, (T*)pool, D, S_max);
    return hipGetLastError();
}

// Overlapping blocks (method variant; [NK "RL 训练侧"], overlap transform):
// entry i over the 2M tokens of blocks i-1 and i, bias [2M, D], entry 0 over
// its own block.  One thread per (sequence, entry, 16-byte chunk), units in
// chunk-major order, so the two entries that read a block run in neighbouring
// workgroups and the second read of a block is served from L2 (plain loads).
template <typename T, int M>
__global__ __launch_bounds__(kCompressThreads) void compress_overlap_kernel(
    const T* __restrict__ x, const T* __restrict__ gate, const T* __restrict__ bias,
    T* __restrict__ out, int B, int T_len, int D) {
    constexpr int V = Elem<T>::kPer16B;
    constexpr int W2 = 2 * M;
    const int nchunk = D / V;
    const int nblk = T_len / M;
    const long long unit = (long long)blockIdx.x * kCompressThreads + threadIdx.x;
    if (unit >= (long long)B * nblk * nchunk) return;
    const int c = (int)(unit % nchunk);
    const long long bi = unit / nchunk;
    const int i = (int)(bi % nblk);
    const size_t row0 = (size_t)(bi / nblk) * T_len + (size_t)M * i;  // the block's first token
    const int jlo = i == 0 ? M : 0;
    u32x4 gw[W2], xw[W2], bw[W2];
#pragma unroll
    for (int j = 0; j < W2; ++j) {
        const size_t t = j < jlo ? row0 : row0 - M + j;  // missing tokens: a valid row, unused
        gw[j] = *reinterpret_cast<const u32x4*>(gate + t * D + (size_t)c * V);
        xw[j] = *reinterpret_cast<const u32x4*>(x + t * D + (size_t)c * V);
        bw[j] = *reinterpret_cast<const u32x4*>(bias + (size_t)j * D + (size_t)c * V);
    }
    float res[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        float z[W2];
        float gm = -INFINITY;
#pragma unroll
        for (int j = 0; j < W2; ++j) {
            z[j] = j < jlo ? -INFINITY : (chunk_elem<T>(gw[j], e) + chunk_elem<T>(bw[j], e)) * kLog2e;
            gm = fmaxf(gm, z[j]);
        }
        float sm = 0.f, acc = 0.f;
#pragma unroll
        for (int j = 0; j < W2; ++j) {
            if (j < jlo) continue;
            const float w = exp2f(z[j] - gm);
            sm += w;
            acc = fmaf(w, chunk_elem<T>(xw[j], e), acc);
        }
        res[e] = acc / sm;
    }
    *reinterpret_cast<u32x4*>(out + (size_t)bi * D + (size_t)c * V) = pack16<T>(res);
}

template <typename T, int M>
__global__ __launch_bounds__(kAppendThreads) void compress_append_overlap_kernel(
    const T* x_tok, const T* g_tok, const T* bias, T* ring_x, T* ring_g, const int32_t* pos,
    T* pool, int D, int S_max) {
    append_overlap_chunk<T, M>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, D, S_max, blockIdx.x,
                               blockIdx.y * kAppendThreads + threadIdx.x);
}

template <typename T, int M>
hipError_t launch_overlap_m(const void* x, const void* g, const void* bias, void* out, int B,
                            int T_len, int D, hipStream_t st) {
    const long long nunits = (long long)B * (T_len / M) * (D / Elem<T>::kPer16B);
    const long long nwg = (nunits + kCompressThreads - 1) / kCompressThreads;
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    ProfScope prof(kProfCompress, st);
    hipLaunchKernelGGL((compress_overlap_kernel<T, M>), dim3((unsigned)nwg), dim3(kCompressThreads), 0,
                       st, (const T*)x, (const T*)g, (const T*)bias, (T*)out, B, T_len, D);
    return hipGetLastError();
}

template <typename T, int M>
hipError_t launch_append_overlap_m(const void* x_tok, const void* g_tok, const void* bias,
                                   void* ring_x, void* ring_g, const int32_t* pos, void* pool, int B,
                                   int D, int S_max, hipStream_t st) {
    const int nchunk = D / Elem<T>::kPer16B;
    const int gy = (nchunk + kAppendThreads - 1) / kAppendThreads;
    ProfScope prof(kProfCompress, st);
    hipLaunchKernelGGL((compress_append_overlap_kernel<T, M>), dim3((unsigned)B, (unsigned)gy),
                       dim3(kAppendThreads), 0, st, (const T*)x_tok, (const T*)g_tok,
                       (const T*)bias, (T*)ring_x, (T*)ring_g, pos, (T*)pool, D, S_max);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_overlap_t(const void* x, const void* g, const void* bias, void* out, int B,
                            int T_len, int D, int m, hipStream_t st) {
    switch (m) {
        case 1: return launch_overlap_m<T, 1>(x, g, bias, out, B, T_len, D, st);
        case 2: return launch_overlap_m<T, 2>(x, g, bias, out, B, T_len, D, st);
        case 3: return launch_overlap_m<T, 3>(x, g, bias, out, B, T_len, D, st);
        default: return launch_overlap_m<T, 4>(x, g, bias, out, B, T_len, D, st);
    }
}

template <typename T>
hipError_t launch_append_overlap_t(const void* x_tok, const void* g_tok, const void* bias,
                                   void* ring_x, void* ring_g, const int32_t* pos, void* pool,
                                   int B, int D, int m, int S_max, hipStream_t st) {
    switch (m) {
        case 1: return launch_append_overlap_m<T, 1>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B, D, S_max, st);
        case 2: return launch_append_overlap_m<T, 2>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B, D, S_max, st);
        case 3: return launch_append_overlap_m<T, 3>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B, D, S_max, st);
        default: return launch_append_overlap_m<T, 4>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B, D, S_max, st);
    }
}

// the paged C4 append (append_short_chunk_paged), one thread per chunk
template <typename T>
__global__ __launch_bounds__(kAppendThreads) void compress_append_paged_kernel(AppendJob job) {
    append_short_chunk_paged<T, 4>(
        static_cast<const T*>(job.x_tok), static_cast<const T*>(job.g_tok),
        static_cast<const T*>(job.bias), static_cast<T*>(job.ring_x), static_cast<T*>(job.ring_g),
        job.pos, static_cast<T*>(job.pool), job.D, job.S_max, job.swa, job.c4, blockIdx.x,
        blockIdx.y * kAppendThreads + threadIdx.x);
}

// rows folded per thread: enough parts that each holds about kAppendRows rows
int append_parts(int m) {
    int want = std::min(32, (m + kAppendRows - 1) / kAppendRows);
    int p = 1;
    while (p * 2 <= want) p *= 2;
    return p;
}

template <typename T>
hipError_t launch_compress_append_t(const void* x_tok, const void* g_tok, const void* bias,
                                    void* ring_x, void* ring_g, const int32_t* pos, void* pool,
                                    int B, int D, int m, int S_max, hipStream_t st) {
    switch (m) {
        case 1: return launch_append_short<T, 1>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B, D, S_max, st);
        case 2: return launch_append_short<T, 2>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B, D, S_max, st);
        case 3: return launch_append_short<T, 3>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B, D, S_max, st);
        case 4: return launch_append_short<T, 4>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B, D, S_max, st);
        default: break;
    }
    const int nchunk = D / Elem<T>::kPer16B;
    const int parts = append_parts(m);
    const int cw = kAppendThreads / parts;
    const int gy = (nchunk + cw - 1) / cw;
    ProfScope prof(kProfCompress, st);
    hipLaunchKernelGGL((compress_append_kernel<T>), dim3((unsigned)B, (unsigned)gy),
                       dim3(kAppendThreads), 0, st, (const T*)x_tok, (const T*)g_tok,
                       (const T*)bias, (T*)ring_x, (T*)ring_g, pos, (T*)pool, D, m, S_max, parts);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_compress_append(int dtype, const void* x_tok, const void* g_tok,
                                  const void* bias, void* ring_x, void* ring_g,
                                  const int32_t* pos, void* pool, int B, int D, int m, int S_max,
                                  hipStream_t st) {
    if (dtype == kF32)
        return launch_compress_append_t<float>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B,
                                               D, m, S_max, st);
    return launch_compress_append_t<bf16_t>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B, D,
                                            m, S_max, st);
}

hipError_t launch_compress_overlap(int dtype, const void* x, const void* g, const void* bias,
                                   void* out, int B, int T_len, int D, int m, hipStream_t st) {
    if (dtype == kF32) return launch_overlap_t<float>(x, g, bias, out, B, T_len, D, m, st);
    return launch_overlap_t<bf16_t>(x, g, bias, out, B, T_len, D, m, st);
}

hipError_t launch_compress_append_overlap(int dtype, const void* x_tok, const void* g_tok,
                                          const void* bias, void* ring_x, void* ring_g,
                                          const int32_t* pos, void* pool, int B, int D, int m,
                                          int S_max, hipStream_t st) {
    if (dtype == kF32)
        return launch_append_overlap_t<float>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B, D, m, S_max, st);
    return launch_append_overlap_t<bf16_t>(x_tok, g_tok, bias, ring_x, ring_g, pos, pool, B, D, m, S_max, st);
}

hipError_t launch_compress_append_paged(int dtype, const AppendJob& job, hipStream_t st) {
    const int nchunk = job.D * (dtype == kF32 ? 4 : 2) / 16;
    const dim3 grid((unsigned)job.B, (unsigned)((nchunk + kAppendThreads - 1) / kAppendThreads));
    ProfScope prof(kProfCompress, st);
    if (dtype == kF32)
        hipLaunchKernelGGL(compress_append_paged_kernel<float>, grid, dim3(kAppendThreads), 0, st, job);
    else
        hipLaunchKernelGGL(compress_append_paged_kernel<bf16_t>, grid, dim3(kAppendThreads), 0, st, job);
    return hipGetLastError();
}

hipError_t launch_compress(int dtype, const void* x, const void* g, const void* bias, void* out,
                           int B, int T_len, int D, int m, hipStream_t st) {
    if (dtype == kF32) return launch_compress_t<float>(x, g, bias, out, B, T_len, D, m, st);
    return launch_compress_t<bf16_t>(x, g, bias, out, B, T_len, D, m, st);
}

}  // namespace hsa
