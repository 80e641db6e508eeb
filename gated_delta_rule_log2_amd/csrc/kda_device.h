// kda_device.h -- gfx950 device helpers shared by the KDA kernels.
//
// Wave64 lane layouts used throughout (CDNA 16x16 MFMA tiles):
//   "row fragment"  lane l holds row (l & 15) of a 16-row block and, for every
//                   32-column step kk, the 8 contiguous columns 32*kk + 8*(l >> 4) + i.
//                   This is the A-operand layout of a 16x16x32 MFMA (and, for the
//                   right-hand factor of A*B^T, the B-operand layout).
//   "acc layout"    lane l holds the 16x16 fp32 result rows 4*(l >> 4) + j (j < 4),
//                   column (l & 15).
// The contraction index a lane supplies (8*(l >> 4) + i inside a 32-step) is the
// same for both operands, which is all an MFMA contraction needs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even (v_cvt_pk_bf16_f32)
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

template <typename T> struct Store;  // storage type traits: float or uint16_t (bf16 bits)
template <> struct Store<float> {
    static __device__ __forceinline__ float to(float x) { return x; }
    static __device__ __forceinline__ float from(float x) { return x; }
};
template <> struct Store<uint16_t> {
    static __device__ __forceinline__ uint16_t to(float x) { return f2bf(x); }
    static __device__ __forceinline__ float from(uint16_t x) { return bf2f(x); }
};

// 8 contiguous elements -> fp32
__device__ __forceinline__ void load8(const float *p, float (&o)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t *p, float (&o)[8]) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
// 8 contiguous fp32 values -> storage
__device__ __forceinline__ void store8(float *p, const float (&x)[8]) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void store8(uint16_t *p, const float (&x)[8]) {
    uint4 u;
    u.x = (uint32_t)f2bf(x[0]) | ((uint32_t)f2bf(x[1]) << 16);
    u.y = (uint32_t)f2bf(x[2]) | ((uint32_t)f2bf(x[3]) << 16);
    u.z = (uint32_t)f2bf(x[4]) | ((uint32_t)f2bf(x[5]) << 16);
    u.w = (uint32_t)f2bf(x[6]) | ((uint32_t)f2bf(x[7]) << 16);
    *reinterpret_cast<uint4 *>(p) = u;
}
// 4 contiguous values (acc-layout column of a 16x16 tile, transposed store)
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(uint16_t *p, float a, float b, float c, float d) {
    uint2 u;
    u.x = (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
    u.y = (uint32_t)f2bf(c) | ((uint32_t)f2bf(d) << 16);
    *reinterpret_cast<uint2 *>(p) = u;
}

// 16-byte load / store with the non-temporal hint, for data used exactly once (the gate
// and value inputs, the output): it keeps them from displacing the per-chunk
// intermediates that the recurrence reads back from the memory-side cache.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_once(const void *ptr) {
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(ptr));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store16_once(void *ptr, uint4 x) {
    const u32x4_nt v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_nt *>(ptr));
}

// Scalar load of one element of either storage type.
__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t *p) { return bf2f(*p); }

// ---------------------------------------------------------------------- MFMA
// 16x16 tile, contraction 32: acc += A(16x32) * B(32x16).  a[i], b[i] are the
// lane's 8 contraction elements.  F32 selects fp32 matrix cores (8 x 16x16x4)
// instead of one bf16 16x16x32 instruction.
template <bool F32>
__device__ __forceinline__ f32x4 mma32(f32x4 acc, const float (&a)[8], const float (&b)[8]) {
    if constexpr (F32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
        return acc;
    } else {
        bf16x8 x, y;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = (__bf16)a[i];
            y[i] = (__bf16)b[i];
        }
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
    }
}

// Operands already in bf16 storage (16 bytes each).
__device__ __forceinline__ f32x4 mma32_bf16(f32x4 acc, uint4 a, uint4 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ------------------------------------------------------------- lane exchange
// Value of lane (l - n) within the same 16-lane row, 0 when that lane is outside
// the row (DPP row_shr; `old` = 0 covers both bound-control conventions).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x110 + N, 0xf, 0xf, false));
}
// Inclusive prefix sum over the 16 lanes of each DPP row (Hillis-Steele).
__device__ __forceinline__ float row_scan16(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}

__device__ __forceinline__ float shfl(float x, int src) { return __shfl(x, src, 64); }
__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// Sum over the four lanes that share (l & 15): the four column groups of a row.
__device__ __forceinline__ float sum_col_groups(float x) {
    x += shfl_xor(x, 16);
    x += shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

}  // namespace kda
