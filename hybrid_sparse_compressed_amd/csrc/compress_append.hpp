// compress_append.hpp -- compressor helpers shared by compress.hip and the
// decode layer-step kernels: chunk packing/widening and the short-block
// decode-time append of one (sequence, 16-byte channel chunk).
#pragma once

#include "hsa_common.hpp"
#include "hsa_internal.hpp"

namespace hsa {

constexpr float kLog2e = 1.4426950408889634f;

// V floats -> the 16 bytes of one chunk in the storage dtype
template <typename T> __device__ __forceinline__ u32x4 pack16(const float* v);
template <> __device__ __forceinline__ u32x4 pack16<float>(const float* v) {
    return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                 __float_as_uint(v[3])};
}
// bf16: gfx950's paired conversion (round to nearest even, NaN kept quiet),
// two elements per instruction
template <> __device__ __forceinline__ u32x4 pack16<bf16_t>(const float* v) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const bf16x2 p = {(__bf16)v[2 * w], (__bf16)v[2 * w + 1]};
        r[w] = __builtin_bit_cast(uint32_t, p);
    }
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

// Decode-time compression state, block length M <= 4 (the C4 case), for chunk
// c of sequence b ([NK "DeepSeek V4 的新架构", five state classes]; [KD
// "Arquitectura del Sistema", compression-state ring buffers]).  The token at
// position p = pos[b] goes to ring slot p mod M; when it is the block's last
// token the block's entry, sum_j softmax_j(g_j + bias_j) * x_j per channel
// (fp32, base-2 exponentials), is written to pool row p div M if that row
// exists.  p < 0: nothing.
//
// One thread holds the whole block.  No load address depends on the position:
// the token, the ring's first M-1 rows (the completing token is always row
// M-1) and the bias are requested together with pos[b], so a call costs one
// memory round trip; when the token does not complete its block the ring and
// bias words are dropped.  The empty asm with a memory clobber keeps those
// loads in front of the position test (otherwise the compiler issues pos[b]
// first and moves the other loads behind the branch on it); for that the
// pointers must not be __restrict__, whose loads the compiler moves past any
// barrier.
template <typename T, int M>
__device__ __forceinline__ void append_short_chunk(const T* x_tok, const T* g_tok, const T* bias,
                                                   T* ring_x, T* ring_g, const int32_t* pos,
                                                   T* pool, int D, int S_max, int b, int c) {
    constexpr int V = Elem<T>::kPer16B;
    if (c >= D / V) return;  // a chunk past the row
    const size_t tok = (size_t)b * D + (size_t)c * V;
    const size_t ring = (size_t)b * M * D + (size_t)c * V;
    u32x4 xw[M], gw[M], bw[M];  // row M-1 is the token
#pragma unroll
    for (int r = 0; r < M; ++r) {
        const T* sg = r == M - 1 ? g_tok + tok : ring_g + ring + (size_t)r * D;
        const T* sx = r == M - 1 ? x_tok + tok : ring_x + ring + (size_t)r * D;
        gw[r] = *reinterpret_cast<const u32x4*>(sg);
        xw[r] = *reinterpret_cast<const u32x4*>(sx);
        bw[r] = *reinterpret_cast<const u32x4*>(bias + (size_t)r * D + (size_t)c * V);
    }
    asm volatile("" ::: "memory");
    const int p = pos[b];
    if (p < 0) return;  // idle sequence
    const int s = p % M;
    *reinterpret_cast<u32x4*>(ring_x + ring + (size_t)s * D) = xw[M - 1];
    *reinterpret_cast<u32x4*>(ring_g + ring + (size_t)s * D) = gw[M - 1];
    const int blk = p / M;
    if (s != M - 1 || blk >= S_max) return;
    float res[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        float z[M];
#pragma unroll
        for (int r = 0; r < M; ++r)
            z[r] = (chunk_elem<T>(gw[r], e) + chunk_elem<T>(bw[r], e)) * kLog2e;
        float gm = z[0];
#pragma unroll
        for (int r = 1; r < M; ++r) gm = fmaxf(gm, z[r]);
        float sm = 0.f, acc = 0.f;
#pragma unroll
        for (int r = 0; r < M; ++r) {
            const float w = exp2f(z[r] - gm);
            sm += w;
            acc = fmaf(w, chunk_elem<T>(xw[r], e), acc);
        }
        res[e] = acc / sm;
    }
    *reinterpret_cast<u32x4*>(pool + ((size_t)b * S_max + blk) * D + (size_t)c * V) =
        pack16<T>(res);
}

// Decode-time state of the overlapping compressor (method variant: entry i
// covers blocks i-1 and i, bias [2M, D]; [NK "RL 训练侧"], overlap transform).
// The ring keeps the last 2M tokens, slot = position mod 2M.  The token at
// p = pos[b] goes to slot p mod 2M; when it completes block i = p div M
// (i < S_max) the entry over tokens M(i-1) .. p (those >= 0) is written to
// pool row i.  Token M(i-1) + j sits in slot (M(i-1) + j) mod 2M, which is
// slot j or slot (j + M) mod 2M depending on the parity of i - 1: the ring is
// loaded before the position is known and its halves swapped by a select.
template <typename T, int M>
__device__ __forceinline__ void append_overlap_chunk(const T* x_tok, const T* g_tok, const T* bias,
                                                     T* ring_x, T* ring_g, const int32_t* pos,
                                                     T* pool, int D, int S_max, int b, int c) {
    constexpr int V = Elem<T>::kPer16B;
    constexpr int W2 = 2 * M;
    if (c >= D / V) return;
    const size_t tok = (size_t)b * D + (size_t)c * V;
    const size_t ring = (size_t)b * W2 * D + (size_t)c * V;
    u32x4 xr[W2], gr[W2], bw[W2];
    const u32x4 xt = *reinterpret_cast<const u32x4*>(x_tok + tok);
    const u32x4 gt = *reinterpret_cast<const u32x4*>(g_tok + tok);
#pragma unroll
    for (int r = 0; r < W2; ++r) {
        xr[r] = *reinterpret_cast<const u32x4*>(ring_x + ring + (size_t)r * D);
        gr[r] = *reinterpret_cast<const u32x4*>(ring_g + ring + (size_t)r * D);
        bw[r] = *reinterpret_cast<const u32x4*>(bias + (size_t)r * D + (size_t)c * V);
    }
    asm volatile("" ::: "memory");
    const int p = pos[b];
    if (p < 0) return;  // idle sequence
    const int s = p % W2;
    *reinterpret_cast<u32x4*>(ring_x + ring + (size_t)s * D) = xt;
    *reinterpret_cast<u32x4*>(ring_g + ring + (size_t)s * D) = gt;
    const int blk = p / M;
    if (p % M != M - 1 || blk >= S_max) return;
    const bool swap = ((blk - 1) & 1) != 0;  // token M(blk-1) sits in slot M
    const int jlo = blk == 0 ? M : 0;        // entry 0 has no earlier block
    float res[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        float z[W2], xv[W2];
        float gm = -INFINITY;
#pragma unroll
        for (int j = 0; j < W2; ++j) {
            const u32x4& gj = j == W2 - 1 ? gt : (swap ? gr[(j + M) % W2] : gr[j]);
            const u32x4& xj = j == W2 - 1 ? xt : (swap ? xr[(j + M) % W2] : xr[j]);
            z[j] = j < jlo ? -INFINITY : (chunk_elem<T>(gj, e) + chunk_elem<T>(bw[j], e)) * kLog2e;
            xv[j] = chunk_elem<T>(xj, e);
            gm = fmaxf(gm, z[j]);
        }
        float sm = 0.f, acc = 0.f;
#pragma unroll
        for (int j = 0; j < W2; ++j) {
            if (j < jlo) continue;
            const float w = exp2f(z[j] - gm);
            sm += w;
            acc = fmaf(w, xv[j], acc);
        }
        res[e] = acc / sm;
    }
    *reinterpret_cast<u32x4*>(pool + ((size_t)b * S_max + blk) * D + (size_t)c * V) = pack16<T>(res);
}

// The same append on paged pools ([KD "Arquitectura del Sistema",
// ShadowRadix]: the compression-state rings form a pool of their own, reached
// from the SWA page by an arithmetic second-level map).  Token t's latent and
// gate logits are state rows of the SWA row of t (physical row of t in the SWA
// shadow `swa`); since 4 divides the page size a block's M <= 4 tokens share
// one page.  The token at position p = pos[b] is stored at its row; when it
// completes block i = p div M, the entry formed from the rows of tokens
// p-M+1 .. p goes to row i of the C4 shadow `c4` if i < S_max.  Rows that are
// not resident are neither read nor written (the token or entry is dropped).
template <typename T, int M>
__device__ __forceinline__ void append_short_chunk_paged(const T* x_tok, const T* g_tok,
                                                         const T* bias, T* state_x, T* state_g,
                                                         const int32_t* pos, T* pool, int D,
                                                         int S_max, const PoolMap& swa,
                                                         const PoolMap& c4, int b, int c) {
    constexpr int V = Elem<T>::kPer16B;
    if (c >= D / V) return;  // a chunk past the row
    const size_t tok = (size_t)b * D + (size_t)c * V;
    const u32x4 xt = *reinterpret_cast<const u32x4*>(x_tok + tok);
    const u32x4 gt = *reinterpret_cast<const u32x4*>(g_tok + tok);
    const int p = pos[b];
    if (p < 0) return;  // idle sequence
    const long long sr = paged_row(swa, b, p);
    if (sr < 0) return;
    *reinterpret_cast<u32x4*>(state_x + (size_t)sr * D + (size_t)c * V) = xt;
    *reinterpret_cast<u32x4*>(state_g + (size_t)sr * D + (size_t)c * V) = gt;
    const int blk = p / M;
    if (p % M != M - 1 || blk >= S_max) return;
    const long long er = paged_row(c4, b, blk);
    if (er < 0) return;
    u32x4 xw[M], gw[M], bw[M];  // row M-1 is the token; rows before it are sr-M+1 .. sr-1
#pragma unroll
    for (int r = 0; r < M; ++r) {
        const size_t row = (size_t)(sr - (M - 1) + r) * D + (size_t)c * V;
        gw[r] = r == M - 1 ? gt : *reinterpret_cast<const u32x4*>(state_g + row);
        xw[r] = r == M - 1 ? xt : *reinterpret_cast<const u32x4*>(state_x + row);
        bw[r] = *reinterpret_cast<const u32x4*>(bias + (size_t)r * D + (size_t)c * V);
    }
    float res[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        float z[M];
#pragma unroll
        for (int r = 0; r < M; ++r)
            z[r] = (chunk_elem<T>(gw[r], e) + chunk_elem<T>(bw[r], e)) * kLog2e;
        float gm = z[0];
#pragma unroll
        for (int r = 1; r < M; ++r) gm = fmaxf(gm, z[r]);
        float sm = 0.f, acc = 0.f;
#pragma unroll
        for (int r = 0; r < M; ++r) {
            const float w = exp2f(z[r] - gm);
            sm += w;
            acc = fmaf(w, chunk_elem<T>(xw[r], e), acc);
        }
        res[e] = acc / sm;
    }
    *reinterpret_cast<u32x4*>(pool + (size_t)er * D + (size_t)c * V) = pack16<T>(res);
}

}  // namespace hsa
