// Device building blocks shared by the kernels: format decoders, dot
// products and fixed-order cross-lane sums for 64-wide wavefronts (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qg {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- decoders

// Two E2M1 codes held in byte B of w (low nibble = lower element) -> two bf16
// values.  Every E2M1 value is exact in bf16.  Uses gfx950's packed FP4
// conversion with a unit scale.
template <int B>
__device__ __forceinline__ bf16x2 e2m1x2_to_bf16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B);
}

// E4M3 byte B of w -> fp32 (exact; gfx950 converts the OCP E4M3 encoding).
template <int B>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_f32_fp8(int(w), B);
}

// E4M3 bytes 2W and 2W+1 of w -> two bf16 (lower byte first).  Every E4M3
// value, subnormals included, is exact in bf16; NaN stays NaN.  gfx950's
// packed FP8 conversion with a unit scale.
template <int W>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, W != 0);
}

// IEEE binary16 bits -> fp32 (exact, subnormals included).
__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
    return float(__builtin_bit_cast(_Float16, uint16_t(bits)));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

__device__ __forceinline__ float bf16x2_lo(bf16x2 v) { return float(v.x); }
__device__ __forceinline__ float bf16x2_hi(bf16x2 v) { return float(v.y); }

// One dword of a Q4_0 block (packed layout): lo = elements 4q..4q+3 (low
// nibbles), hi = elements 16+4q..16+4q+3 (high nibbles), one unsigned code
// per byte.
__device__ __forceinline__ void q4_unpack(uint32_t c, uint32_t& lo, uint32_t& hi) {
    lo = c & 0x0F0F0F0Fu;
    hi = (c >> 4) & 0x0F0F0F0Fu;
}

// Signed byte B of c as fp32 (Q8_0 codes).
template <int B>
__device__ __forceinline__ float i8_to_f32(uint32_t c) {
    return float(int32_t(c << (24 - 8 * B)) >> 24);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// ---------------------------------------------------------------- products

// c + a.lo * b.lo + a.hi * b.hi, with b a pair of bf16 bit patterns.
__device__ __forceinline__ float dot2_bf16(bf16x2 a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b), c, false);
}

// c + sum of four signed int8 products (exact int32).
__device__ __forceinline__ int dot4_i8(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(int(a), int(b), c, false);
}

// ---------------------------------------------------------------- lane sums

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of G lanes (G a power of two, 1..64).  Every lane of
// a group ends with the same value, computed in a fixed butterfly order that
// depends only on G (commutative pairings give bitwise-identical values in
// all lanes of a group).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (G >= 4) v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (G >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror: quads 0 <-> 1
    if constexpr (G >= 16) v += dpp_mov<0x140>(v); // row_mirror: half-rows 0 <-> 1
    if constexpr (G >= 32)                          // lane ^ 16 inside 32-lane halves
        v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
    if constexpr (G >= 64) {
        float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
        float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
        v = lo + hi;
    }
    return v;
}

__device__ __forceinline__ int lane_id() { return int(threadIdx.x) & (kWave - 1); }

// ---------------------------------------------------------------- loads

template <typename T>
__device__ __forceinline__ T ld(const void* p) {
    return *reinterpret_cast<const T*>(p);
}

// Streaming (read-once) load of 16 bytes: weights are touched exactly once per
// call, so mark them non-temporal to keep activations resident in the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld_stream16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Branch-free predicated loads: the load is always issued (callers pass an
// address that is valid either way) and the value is replaced by zero when
// ok is false.  Keeping loads out of branches lets the compiler count
// outstanding loads exactly, so later loads stay in flight while earlier
// data is used.
__device__ __forceinline__ u32x4 zero_unless(bool ok, const u32x4& v) {
    return u32x4{ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u};
}

}  // namespace qg
