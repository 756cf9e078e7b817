// hsa_common.hpp -- device helpers shared by the gfx950 kernels of
// libhsa_attn.so: element widening/rounding, 16-byte vector loads, wave and
// workgroup scans, and the order-preserving key used by the radix select.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsa {

constexpr int kWave = 64;  // CDNA wavefront width

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane b passes the address of 4 consecutive 16-bit elements
// B_b[0..3]; lane l of the group receives B_{4m + l/4}[l % 4] for m = 0..3.
// Pointing lane b at M[r0 + b/4][c0 + 4 (b % 4)] of a row-major 16-bit matrix
// M therefore hands lane l the column c0 + l % 16 over rows r0 .. r0 + 3.
__device__ __forceinline__ uint2 lds_read_tr16x4(const void* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(const __attribute__((address_space(3))) void*)p);
    return __builtin_bit_cast(uint2, v);
}

// Storage tag for bf16 (raw 16-bit pattern); fp32 is stored as float.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kPer16B = 4;
    // widen the 16 bytes at p into kPer16B floats
    __device__ static __forceinline__ void load16(const void* p, float* v) {
        f32x4 t = *reinterpret_cast<const f32x4*>(p);
        v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
    }
    __device__ static __forceinline__ void unpack(const u32x4& t, float* v) {
        v[0] = __uint_as_float(t[0]); v[1] = __uint_as_float(t[1]);
        v[2] = __uint_as_float(t[2]); v[3] = __uint_as_float(t[3]);
    }
    __device__ static __forceinline__ void store(void* base, size_t i, float f) {
        reinterpret_cast<float*>(base)[i] = f;
    }
};
template <> struct Elem<bf16_t> {
    static constexpr int kPer16B = 8;
    __device__ static __forceinline__ void unpack(const u32x4& t, float* v) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            v[2 * w] = __uint_as_float(t[w] << 16);
            v[2 * w + 1] = __uint_as_float(t[w] & 0xffff0000u);
        }
    }
    __device__ static __forceinline__ void load16(const void* p, float* v) {
        unpack(*reinterpret_cast<const u32x4*>(p), v);
    }
    __device__ static __forceinline__ void store(void* base, size_t i, float f) {
        reinterpret_cast<uint16_t*>(base)[i] = f32_to_bf16(f);
    }
};

// ---- wave / workgroup primitives ------------------------------------------

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Inclusive prefix sum over the 64 lanes of a wave, on DPP lane moves (no
// LDS round trips): shifts by 1, 2, 4 and 8 lanes within each row of 16
// (lanes without a source read 0), then the last lane of row 0 is added to
// rows 1 and 3 and the last lane of row 1 (rows 0-1 total) to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false); // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false); // row_bcast:31 -> rows 2, 3
    return (uint32_t)x;
}

// Exclusive prefix sum over a workgroup of NT threads (NT multiple of 64).
// `tmp` must hold NT/64 + 1 words of LDS; the total is returned in *total.
// Every thread of the workgroup must call it (it contains barriers).
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
    constexpr int NW = NT / kWave;
    const int w = (int)threadIdx.x / kWave;
    uint32_t inc = wave_incl_scan(v);
    if (lane_id() == kWave - 1) tmp[w] = inc;
    __syncthreads();
    uint32_t base = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        uint32_t t = tmp[i];
        base += (i < w) ? t : 0u;
        all += t;
    }
    __syncthreads();
    *total = all;
    return base + inc - v;
}

// Two exclusive prefix sums over a workgroup of NT threads in one pass (one
// barrier pair).  `tmp` must hold 2 * (NT/64) words of LDS.
template <int NT>
__device__ __forceinline__ void block_excl_scan2(uint32_t a, uint32_t b, uint32_t* tmp,
                                                 uint32_t* base_a, uint32_t* base_b,
                                                 uint32_t* total_a, uint32_t* total_b) {
    constexpr int NW = NT / kWave;
    const int w = (int)threadIdx.x / kWave;
    const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
    if (lane_id() == kWave - 1) { tmp[w] = ia; tmp[NW + w] = ib; }
    __syncthreads();
    uint32_t pa = 0, pb = 0, ta = 0, tb = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t xa = tmp[i], xb = tmp[NW + i];
        pa += (i < w) ? xa : 0u;
        pb += (i < w) ? xb : 0u;
        ta += xa;
        tb += xb;
    }
    __syncthreads();
    *base_a = pa + ia - a;
    *base_b = pb + ib - b;
    *total_a = ta;
    *total_b = tb;
}

// ---- radix-select key -------------------------------------------------------
// Order-preserving map fp32 -> u32: a > b (IEEE) iff key(a) > key(b); -0 and
// +0 share one key; every NaN maps to 0, below -inf (0x007fffff).
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN
    if (u == 0x80000000u) u = 0u;                      // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace hsa
