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
//  * larger m (C128): P = 8 threads split a block's rows into contiguous
//    ranges, each walking its range two rows at a time with the next two in
//    flight; the partial (max, sum, weighted sum) triples are merged in LDS
//    in a fixed order, every thread merging some (unit, channel) pairs.
// Registers are kept at <= 128 per lane (four waves per SIMD): the latents
// stay packed until their product is taken, and entries leave as one
// 16-byte store per chunk.
#include "hsa_common.hpp"
#include "hsa_internal.hpp"

#include <algorithm>
#include <mutex>
#include <numeric>

namespace hsa {

namespace {

constexpr int kCompressThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// V floats -> the 16 bytes of one chunk in the storage dtype
template <typename T> __device__ __forceinline__ u32x4 pack16(const float* v);
template <> __device__ __forceinline__ u32x4 pack16<float>(const float* v) {
    return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                 __float_as_uint(v[3])};
}
template <> __device__ __forceinline__ u32x4 pack16<bf16_t>(const float* v) {
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        r[w] = (uint32_t)f32_to_bf16(v[2 * w]) | ((uint32_t)f32_to_bf16(v[2 * w + 1]) << 16);
    return r;
}

// element e of a raw 16-byte chunk, widened to fp32
template <typename T> __device__ __forceinline__ float chunk_elem(const u32x4& t, int e);
template <> __device__ __forceinline__ float chunk_elem<float>(const u32x4& t, int e) {
    return __uint_as_float(t[e]);
}
template <> __device__ __forceinline__ float chunk_elem<bf16_t>(const u32x4& t, int e) {
    return (e & 1) ? __uint_as_float(t[e >> 1] & 0xffff0000u) : __uint_as_float(t[e >> 1] << 16);
}

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
        // the G rows from j on (rows past j1 are not loaded)
        auto load = [&](RowGroupB<G>& rg, int j) {
#pragma unroll
            for (int r = 0; r < G; ++r) {
                if (j + r < j1) {
                    const size_t off = (row0 + j + r) * (size_t)D + (size_t)c * V;
                    rg.g[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gate + off));
                    rg.x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + off));
                    rg.b[r] = *reinterpret_cast<const u32x4*>(bias + (size_t)(j + r) * D + (size_t)c * V);
                }
            }
        };
        RowGroupB<G> cur;
        if (j0 < j1) load(cur, j0);
        for (int j = j0; j < j1; j += G) {
            RowGroupB<G> nxt;
            if (j + G < j1) load(nxt, j + G);  // next group in flight during this one
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
                const float sc = exp2f(M[e] - mn);  // 0 on the first group (M = -inf)
                float s = 0.f, a = 0.f;
#pragma unroll
                for (int r = 0; r < G; ++r) {
                    const float w = exp2f(z[r][e] - mn);  // 0 for padded rows
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
                const float w = (mp == -INFINITY) ? 0.f : exp2f(mp - mx);
                s = fmaf(ss[p][uu][e], w, s);
                a = fmaf(sa[p][uu][e], w, a);
            }
            res[uu][e] = a / s;
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
    for (int e = 0; e < V; ++e) r[e] = A[e] / S[e];
    const size_t o = ((size_t)b * nblk + i) * (size_t)D + (size_t)c * V;
    *reinterpret_cast<u32x4*>(out + o) = pack16<T>(r);
}

// Short blocks (m <= G): one thread owns a unit (b, i, c); the workgroups stay
// resident and walk the units tile by tile (a tile = kCompressThreads
// consecutive units), the next tile's rows in flight during this one.  When
// the grid's unit stride is a multiple of the chunk count a thread keeps its
// chunk, so its bias words are loaded once.
template <typename T, int G>
__global__ __launch_bounds__(kCompressThreads) void compress_short_kernel(
    const T* __restrict__ x, const T* __restrict__ gate, const T* __restrict__ bias,
    T* __restrict__ out, int B, int T_len, int D, int m, int fixed_chunk) {
    constexpr int V = Elem<T>::kPer16B;
    const int nchunk = D / V;
    const int nblk = T_len / m;
    const long long nunits = (long long)B * nblk * nchunk;
    const long long ntiles = (nunits + kCompressThreads - 1) / kCompressThreads;
    const long long stride = gridDim.x;
    auto load = [&](RowGroup<G>& rg, long long t) {
        const long long unit = t * kCompressThreads + threadIdx.x;
        if (unit >= nunits) return;
        const int c = (int)(unit % nchunk);
        const long long bi = unit / nchunk;
        const size_t row0 = (size_t)(bi / nblk) * T_len + (size_t)m * (bi % nblk);
#pragma unroll
        for (int r = 0; r < G; ++r) {
            if (r < m) {
                const size_t off = (row0 + r) * (size_t)D + (size_t)c * V;
                rg.g[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gate + off));
                rg.x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + off));
            }
        }
    };
    u32x4 bw[G];
    auto load_bias = [&](int c) {
#pragma unroll
        for (int r = 0; r < G; ++r)
            if (r < m) bw[r] = *reinterpret_cast<const u32x4*>(bias + (size_t)r * D + (size_t)c * V);
    };
    long long t = blockIdx.x;
    if (fixed_chunk) load_bias((int)((t * kCompressThreads + threadIdx.x) % nchunk));
    RowGroup<G> cur;
    if (t < ntiles) load(cur, t);
    for (; t < ntiles; t += stride) {
        RowGroup<G> nxt;
        if (t + stride < ntiles) load(nxt, t + stride);
        const long long unit = t * kCompressThreads + threadIdx.x;
        if (unit < nunits) {
            const int c = (int)(unit % nchunk);
            if (!fixed_chunk) load_bias(c);
            float z[G][V];
#pragma unroll
            for (int r = 0; r < G; ++r) {
                if (r < m) {
                    float gv[V], bv[V];
                    Elem<T>::unpack(cur.g[r], gv);
                    Elem<T>::unpack(bw[r], bv);
#pragma unroll
                    for (int e = 0; e < V; ++e) z[r][e] = (gv[e] + bv[e]) * kLog2e;
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
                    const float w = exp2f(z[r][e] - gm);  // 0 for padded rows
                    s += w;
                    if (r < m) a = fmaf(w, chunk_elem<T>(cur.x[r], e), a);
                }
                res[e] = a / s;
            }
            *reinterpret_cast<u32x4*>(out + (size_t)(unit / nchunk) * D + (size_t)c * V) =
                pack16<T>(res);
        }
        cur = nxt;
    }
}

// resident workgroups of compress_short_kernel<T, G> on the current device
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
                &per_cu, reinterpret_cast<const void*>(&compress_short_kernel<T, G>),
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
    hipLaunchKernelGGL((compress_short_kernel<T, G>), dim3((unsigned)grid), dim3(kCompressThreads),
                       0, st, (const T*)x, (const T*)g, (const T*)bias, (T*)out, B, T_len, D, m,
                       fixed);
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
    return launch_compress_p<T, 8, 2>(x, g, bias, out, B, T_len, D, m, st);
}

}  // namespace

hipError_t launch_compress(int dtype, const void* x, const void* g, const void* bias, void* out,
                           int B, int T_len, int D, int m, hipStream_t st) {
    if (dtype == kF32) return launch_compress_t<float>(x, g, bias, out, B, T_len, D, m, st);
    return launch_compress_t<bf16_t>(x, g, bias, out, B, T_len, D, m, st);
}

}  // namespace hsa
