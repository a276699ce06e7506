// Verification dequantizer: writes every weight of a packed matrix as fp32,
// using the same device decoders as the GEMV kernels (qg_device.hpp), so a
// bit-exact comparison with the oracle checks the decode path itself.
#include <hip/hip_runtime.h>

#include "qg_device.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"

namespace qg {

namespace {

constexpr int kBlock = 256;

// One thread per 16-byte code chunk; writes fp32 weight values.
__global__ __launch_bounds__(kBlock) void k_dequant_nvfp4(const uint8_t* __restrict__ w,
                                                          int64_t soff, float s_t, int64_t n,
                                                          int k, float* __restrict__ out) {
    const int64_t idx = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    const int nch = k / 32;
    if (idx >= n * nch) return;
    const int64_t r = idx / nch;
    const int j = int(idx % nch);
    const u32x4 c = ld16(w + r * (k / 2) + 16 * j);
    const uint32_t sc = ld<uint16_t>(w + soff + r * (k / 16) + 2 * j);
    const float s[2] = {e4m3_to_f32<0>(sc), e4m3_to_f32<1>(sc)};
    float* o = out + r * k + 32 * j;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bf16x2 p[4] = {e2m1x2_to_bf16x2<0>(c[q]), e2m1x2_to_bf16x2<1>(c[q]),
                             e2m1x2_to_bf16x2<2>(c[q]), e2m1x2_to_bf16x2<3>(c[q])};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float bs = s[q / 2];
            o[8 * q + 2 * b] = (bf16x2_lo(p[b]) * bs) * s_t;
            o[8 * q + 2 * b + 1] = (bf16x2_hi(p[b]) * bs) * s_t;
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_dequant_q4_0(const uint8_t* __restrict__ w, int64_t soff,
                                                         int64_t n, int k, float* __restrict__ out) {
    const int64_t idx = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    const int nb = k / 32;
    if (idx >= n * nb) return;
    const int64_t r = idx / nb;
    const int j = int(idx % nb);
    const u32x4 c = ld16(w + r * (k / 2) + 16 * j);
    const float d = f16_to_f32(ld<uint16_t>(w + soff + r * nb * 2 + 2 * j));
    float* o = out + r * k + 32 * j;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t lo, hi;
        q4_unpack(c[q], lo, hi);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            o[4 * q + b] = float(int((lo >> (8 * b)) & 0xff) - 8) * d;
            o[16 + 4 * q + b] = float(int((hi >> (8 * b)) & 0xff) - 8) * d;
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_dequant_q8_0(const uint8_t* __restrict__ w, int64_t soff,
                                                         int64_t n, int k, float* __restrict__ out) {
    const int64_t idx = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    const int nch = k / 16;
    if (idx >= n * nch) return;
    const int64_t r = idx / nch;
    const int j = int(idx % nch);
    const u32x4 c = ld16(w + r * k + 16 * j);
    const float d = f16_to_f32(ld<uint16_t>(w + soff + r * (k / 32) * 2 + 2 * (j >> 1)));
    float* o = out + r * k + 16 * j;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        o[4 * q + 0] = i8_to_f32<0>(c[q]) * d;
        o[4 * q + 1] = i8_to_f32<1>(c[q]) * d;
        o[4 * q + 2] = i8_to_f32<2>(c[q]) * d;
        o[4 * q + 3] = i8_to_f32<3>(c[q]) * d;
    }
}

}  // namespace

hipError_t launch_dequant(int fmt, const uint8_t* w, float s_t, int64_t n, int64_t k, float* out,
                          hipStream_t s) {
    const int64_t soff = scale_plane_offset(fmt, n, k);
    const int64_t per_row = fmt == QG_Q8_0 ? k / 16 : k / 32;
    const dim3 grid(unsigned((n * per_row + kBlock - 1) / kBlock));
    if (fmt == QG_NVFP4)
        hipLaunchKernelGGL(k_dequant_nvfp4, grid, dim3(kBlock), 0, s, w, soff, s_t, n, int(k), out);
    else if (fmt == QG_Q4_0)
        hipLaunchKernelGGL(k_dequant_q4_0, grid, dim3(kBlock), 0, s, w, soff, n, int(k), out);
    else
        hipLaunchKernelGGL(k_dequant_q8_0, grid, dim3(kBlock), 0, s, w, soff, n, int(k), out);
    return hipGetLastError();
}

}  // namespace qg
