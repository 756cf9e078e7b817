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
// Work unit = (sequence b, block i, 16-byte channel chunk c).  For m <= 16
// one thread owns a unit; for larger m, P threads of the same workgroup split
// the block's rows into contiguous ranges and their partial (max, sum,
// weighted sum) triples are merged in LDS in a fixed order.
#include "hsa_common.hpp"
#include "hsa_internal.hpp"

namespace hsa {

namespace {

constexpr int kCompressThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int P>
__global__ __launch_bounds__(kCompressThreads) void compress_kernel(
    const T* __restrict__ x, const T* __restrict__ gate, const T* __restrict__ bias,
    T* __restrict__ out, int B, int T_len, int D, int m) {
    constexpr int V = Elem<T>::kPer16B;
    constexpr int U = kCompressThreads / P;  // units per workgroup
    constexpr int G = 4;                     // rows loaded per group
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
        for (int j = j0; j < j1; j += G) {
            float z[G][V], xv[G][V];
            const int g = min(G, j1 - j);
#pragma unroll
            for (int r = 0; r < G; ++r) {
                if (r < g) {
                    const size_t off = (row0 + j + r) * (size_t)D + (size_t)c * V;
                    float gv[V], bv[V];
                    Elem<T>::load16(gate + off, gv);
                    Elem<T>::load16(bias + (size_t)(j + r) * D + (size_t)c * V, bv);
                    Elem<T>::load16(x + off, xv[r]);
#pragma unroll
                    for (int e = 0; e < V; ++e) z[r][e] = (gv[e] + bv[e]) * kLog2e;
                } else {
#pragma unroll
                    for (int e = 0; e < V; ++e) { z[r][e] = -INFINITY; xv[r][e] = 0.f; }
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
                    a = fmaf(w, xv[r][e], a);
                }
                S[e] = fmaf(S[e], sc, s);
                A[e] = fmaf(A[e], sc, a);
                M[e] = mn;
            }
        }
    }

    if constexpr (P > 1) {
        __shared__ float sm[P][U][V], ss[P][U][V], sa[P][U][V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            sm[part][u][e] = M[e];
            ss[part][u][e] = S[e];
            sa[part][u][e] = A[e];
        }
        __syncthreads();
        if (part != 0 || !active) return;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float mx = sm[0][u][e];
            for (int p = 1; p < P; ++p) mx = fmaxf(mx, sm[p][u][e]);
            float s = 0.f, a = 0.f;
            for (int p = 0; p < P; ++p) {
                const float mp = sm[p][u][e];
                const float w = (mp == -INFINITY) ? 0.f : exp2f(mp - mx);
                s = fmaf(ss[p][u][e], w, s);
                a = fmaf(sa[p][u][e], w, a);
            }
            S[e] = s;
            A[e] = a;
        }
    }
    if (!active) return;
    const size_t o = ((size_t)b * nblk + i) * (size_t)D + (size_t)c * V;
#pragma unroll
    for (int e = 0; e < V; ++e) Elem<T>::store(out, o + e, A[e] / S[e]);
}

template <typename T, int P>
hipError_t launch_compress_p(const void* x, const void* g, const void* bias, void* out, int B,
                             int T_len, int D, int m, hipStream_t st) {
    constexpr int U = kCompressThreads / P;
    const long long nunits = (long long)B * (T_len / m) * (D / Elem<T>::kPer16B);
    const long long nwg = (nunits + U - 1) / U;
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    ProfScope prof(kProfCompress, st);
    hipLaunchKernelGGL((compress_kernel<T, P>), dim3((unsigned)nwg), dim3(kCompressThreads), 0, st,
                       (const T*)x, (const T*)g, (const T*)bias, (T*)out, B, T_len, D, m);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_compress_t(const void* x, const void* g, const void* bias, void* out, int B,
                             int T_len, int D, int m, hipStream_t st) {
    if (m <= 16) return launch_compress_p<T, 1>(x, g, bias, out, B, T_len, D, m, st);
    if (m <= 64) return launch_compress_p<T, 4>(x, g, bias, out, B, T_len, D, m, st);
    return launch_compress_p<T, 8>(x, g, bias, out, B, T_len, D, m, st);
}

}  // namespace

hipError_t launch_compress(int dtype, const void* x, const void* g, const void* bias, void* out,
                           int B, int T_len, int D, int m, hipStream_t st) {
    if (dtype == kF32) return launch_compress_t<float>(x, g, bias, out, B, T_len, D, m, st);
    return launch_compress_t<bf16_t>(x, g, bias, out, B, T_len, D, m, st);
}

}  // namespace hsa
