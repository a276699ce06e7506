// Small-M prefill GEMM over packed NVFP4 weights on gfx950 matrix cores.
//
// Y[t][r] = bf16_rne(s_t * sum_c D[r][c] * X[t][c]), D = e2m1 * e4m3 (exact in
// bf16).  This is the one place on the path that is a dense contraction, so it
// runs on MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  The pages keep
// prefill at bf16-activation numerics instead of W4A4 (memra README, known
// gaps), which is why the block-scaled FP4 MFMA of gfx950 is not used: its
// E8M0-per-32 scales and low-precision activations would change the result.
//
// Workgroup tile: 64 tokens x 64 weight rows, k-step 64, 4 waves in a 2x2
// arrangement, each wave a 32x32 sub-tile (2x2 MFMA tiles).  Per k-step the
// workgroup stages the X tile (bf16) and the decoded W tile (bf16) in LDS.
#include <hip/hip_runtime.h>

#include "qg_device.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"

namespace qg {

namespace {

constexpr int kBlock = 256;
constexpr int BM = 64, BN = 64, BK = 64;
constexpr int kPad = 8;  // bf16 elements of padding per LDS row

__device__ __forceinline__ floatx4 mfma_16x16x32_bf16(const u32x4& a, const u32x4& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__global__ __launch_bounds__(kBlock) void k_prefill(const uint8_t* __restrict__ w, int64_t soff,
                                                    float s_t, int n, int k,
                                                    const uint16_t* __restrict__ x, int m,
                                                    uint16_t* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint16_t Xs[BM][BK + kPad];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[BN][BK + kPad];

    const int tid = int(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = int(blockIdx.y) * BM, n0 = int(blockIdx.x) * BN;
    // loader role: one row and one 16-element segment of each tile
    const int lr = tid >> 2, lc = tid & 3;
    const bool x_ok = m0 + lr < m, w_ok = n0 + lr < n;
    const uint16_t* xrow = x + int64_t(x_ok ? m0 + lr : 0) * k;
    const uint8_t* crow = w + int64_t(w_ok ? n0 + lr : 0) * (k / 2);
    const uint8_t* srow = w + soff + int64_t(w_ok ? n0 + lr : 0) * (k / 16);

    floatx4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < k; k0 += BK) {
        const int kc = k0 + 16 * lc;  // first element of this thread's segment
        const bool k_ok = kc < k;
        u32x4 xa = {0, 0, 0, 0}, xb = {0, 0, 0, 0};
        if (x_ok && k_ok) {
            xa = ld16(xrow + kc);
            xb = ld16(xrow + kc + 8);
        }
        u32x4 wa = {0, 0, 0, 0}, wb = {0, 0, 0, 0};
        if (w_ok && k_ok) {
            const u32x2 c = *reinterpret_cast<const u32x2*>(crow + kc / 2);
            const float s = e4m3_to_f32<0>(srow[kc / 16]);
            uint32_t o[8];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const bf16x2 p[4] = {e2m1x2_to_bf16x2<0>(c[q]), e2m1x2_to_bf16x2<1>(c[q]),
                                     e2m1x2_to_bf16x2<2>(c[q]), e2m1x2_to_bf16x2<3>(c[q])};
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    // e2m1 * e4m3 has at most 6 significant bits: exact in bf16
                    const uint32_t lo = f32_to_bf16_rne(bf16x2_lo(p[b]) * s);
                    const uint32_t hi = f32_to_bf16_rne(bf16x2_hi(p[b]) * s);
                    o[4 * q + b] = lo | (hi << 16);
                }
            }
            wa = u32x4{o[0], o[1], o[2], o[3]};
            wb = u32x4{o[4], o[5], o[6], o[7]};
        }
        __syncthreads();  // previous k-step's fragment reads are done
        *reinterpret_cast<u32x4*>(&Xs[lr][16 * lc]) = xa;
        *reinterpret_cast<u32x4*>(&Xs[lr][16 * lc + 8]) = xb;
        *reinterpret_cast<u32x4*>(&Ws[lr][16 * lc]) = wa;
        *reinterpret_cast<u32x4*>(&Ws[lr][16 * lc + 8]) = wb;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            u32x4 af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const u32x4*>(&Xs[wm * 32 + i * 16 + (lane & 15)][kk + 8 * (lane >> 4)]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[j] = *reinterpret_cast<const u32x4*>(&Ws[wn * 32 + j * 16 + (lane & 15)][kk + 8 * (lane >> 4)]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma_16x16x32_bf16(af[i], bf[j], acc[i][j]);
        }
    }
    // D[i][j] of a 16x16 tile: lane holds rows 4*(lane/16)+v, column lane%16
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + v;
                const int col = n0 + wn * 32 + j * 16 + (lane & 15);
                if (row < m && col < n)
                    y[int64_t(row) * n + col] = uint16_t(f32_to_bf16_rne(acc[i][j][v] * s_t));
            }
}

}  // namespace

hipError_t launch_prefill(const uint8_t* w, float s_t, int64_t n, int64_t k, const uint16_t* x,
                          int64_t m, uint16_t* y, hipStream_t s) {
    const int64_t soff = scale_plane_offset(QG_NVFP4, n, k);
    const dim3 grid(unsigned((n + BN - 1) / BN), unsigned((m + BM - 1) / BM));
    hipLaunchKernelGGL(k_prefill, grid, dim3(kBlock), 0, s, w, soff, s_t, int(n), int(k), x, int(m), y);
    return hipGetLastError();
}

}  // namespace qg
