// Achievable-peak probes: what one MI355X actually delivers for the two
// resources the path is bound by, measured with the same instructions the
// kernels use.  The pages keep standalone bandwidth and tensor-core peak
// microbenchmarks beside their kernels (bw24 README, crate table: the probe
// crate; memra README, research notes: microbenched peaks) so that a kernel's
// speed can be read against what the machine reaches, not only against the
// data-sheet figure.
//
//  * k_probe_read: a streaming read of a device buffer with 16-byte
//    non-temporal loads, eight in flight per lane, every wave-wide load 1 KB
//    contiguous, WG_PER_CU four-wave workgroups per CU looping over the buffer.
//  * k_probe_mfma: v_mfma_f32_16x16x32_bf16 with sixteen independent
//    accumulators per wave, two waves per SIMD, no memory traffic.
// Both fold their results into a value that is stored only if it equals a
// key the caller never produces, so nothing is optimised away.
#include <hip/hip_runtime.h>

#include "qg_device.hpp"
#include "qg_internal.hpp"
#include "qg_mfma.hpp"

namespace qg {

namespace {

constexpr int kProbeBlock = 256;
constexpr int kProbeInFlight = 8;

__global__ __launch_bounds__(kProbeBlock) void k_probe_read(const u32x4* __restrict__ p, int64_t n16,
                                                            uint32_t* __restrict__ sink, uint32_t key) {
    const int64_t stride = int64_t(gridDim.x) * kProbeBlock;
    int64_t i = int64_t(blockIdx.x) * kProbeBlock + threadIdx.x;
    uint32_t acc = 0;
    // whole rounds of kProbeInFlight loads, all issued before any is used
    for (; i + (kProbeInFlight - 1) * stride < n16; i += kProbeInFlight * stride) {
        u32x4 v[kProbeInFlight];
#pragma unroll
        for (int j = 0; j < kProbeInFlight; ++j) v[j] = ld_stream16(p + i + j * stride);
#pragma unroll
        for (int j = 0; j < kProbeInFlight; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (; i < n16; i += stride) {  // the tail
        const u32x4 v = ld_stream16(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == key) sink[0] = acc;
}

constexpr int kMfmaBlock = 512;  // eight waves: two per SIMD
constexpr int kMfmaAcc = 16;

__global__ __launch_bounds__(kMfmaBlock) void k_probe_mfma(int64_t iters, float* __restrict__ sink, float key) {
    const uint32_t lane = threadIdx.x & 63u;
    const u32x4 a = {0x3F803F80u ^ lane, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u ^ (lane << 16)};
    const u32x4 b = {0x3F003F00u, 0x3F003F00u ^ lane, 0x3F003F00u, 0x3F003F00u};
    floatx4 acc[kMfmaAcc];
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kMfmaAcc; ++j) acc[j] = mfma_16x16x32_bf16(a, b, acc[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (s == key) sink[0] = s;
}

}  // namespace

hipError_t launch_probe_read(const void* buf, int64_t bytes, uint32_t* sink, int wg_per_cu, hipStream_t s) {
    int cus = 0;
    if (hipError_t e = device_cu_count(&cus); e != hipSuccess) return e;
    hipLaunchKernelGGL(k_probe_read, dim3(unsigned(cus * wg_per_cu)), dim3(kProbeBlock), 0, s,
                       static_cast<const u32x4*>(buf), bytes / 16, sink, 0x9E3779B9u);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int64_t iters, float* sink, hipStream_t s, int64_t* flops) {
    int cus = 0;
    if (hipError_t e = device_cu_count(&cus); e != hipSuccess) return e;
    // one 16x16x32 MFMA is 2 * 16 * 16 * 32 flops
    *flops = int64_t(cus) * (kMfmaBlock / kWave) * iters * kMfmaAcc * (2 * 16 * 16 * 32);
    hipLaunchKernelGGL(k_probe_mfma, dim3(unsigned(cus)), dim3(kMfmaBlock), 0, s, iters, sink, -1.0f);
    return hipGetLastError();
}

}  // namespace qg
