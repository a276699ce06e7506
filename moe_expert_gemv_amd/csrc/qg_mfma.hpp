// NVFP4 x bf16 matrix-core building blocks shared by the prefill GEMMs:
// weight decode into bf16 MFMA fragments, the MFMA itself, the weight-slab
// register stage and an LDS-only workgroup barrier.
#pragma once

#include <hip/hip_runtime.h>

#include "qg_device.hpp"

namespace qg {

constexpr int KW = 128;  // k per wave per stage: one slab

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4 mfma_16x16x32_bf16(const u32x4& a, const u32x4& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Eight E2M1 codes (one dword, low nibble first) times the fp32 block scale s,
// as eight bf16 (exact: at most 6 significant bits).
template <int B>
__device__ __forceinline__ uint32_t decode2_scaled(uint32_t codes, float s) {
    f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, B);  // byte B: two codes
    f = f * s;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

__device__ __forceinline__ u32x4 decode8_scaled(uint32_t codes, float s) {
    return u32x4{decode2_scaled<0>(codes, s), decode2_scaled<1>(codes, s), decode2_scaled<2>(codes, s),
                 decode2_scaled<3>(codes, s)};
}

// Workgroup barrier that publishes LDS only: waits for this wave's LDS
// accesses (not its global loads, so weight prefetches stay in flight), then
// s_barrier.  __syncthreads() would also wait for every outstanding global
// load.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One stage of one wave's W rows: codes and scales of its NB row blocks.
template <int NB>
struct WStage {
    uint32_t c[NB][4];
    uint32_t s[NB];  // the two scale bytes in the low half
};

}  // namespace qg
