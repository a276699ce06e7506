// The NVFP4 row-dot core shared by the dense and the MoE GEMV kernels.
#pragma once

#include "qg_device.hpp"

namespace qg {

// Add this lane's share of R rows x up to MT tokens into acc.  Chunk j of a
// row is 32 elements: 16 code bytes at codes[r] + 16j and the two E4M3 block
// scales at scales[r] + 2j.  x[t] points at token t's bf16 activations.
template <int R, int MT, int G>
__device__ __forceinline__ void nvfp4_partial(const uint8_t* const (&codes)[R],
                                              const uint8_t* const (&scales)[R],
                                              const uint16_t* const (&x)[MT], int m, int nchunks,
                                              int l, float (&acc)[R][MT]) {
    for (int j = l; j < nchunks; j += G) {
        u32x4 c[R];
        uint32_t sc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            c[r] = ld_stream16(codes[r] + 16 * j);
            sc[r] = ld<uint16_t>(scales[r] + 2 * j);
        }
        bf16x2 d[R][16];
        float s0[R], s1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                d[r][4 * q + 0] = e2m1x2_to_bf16x2<0>(c[r][q]);
                d[r][4 * q + 1] = e2m1x2_to_bf16x2<1>(c[r][q]);
                d[r][4 * q + 2] = e2m1x2_to_bf16x2<2>(c[r][q]);
                d[r][4 * q + 3] = e2m1x2_to_bf16x2<3>(c[r][q]);
            }
            s0[r] = e4m3_to_f32<0>(sc[r]);
            s1[r] = e4m3_to_f32<1>(sc[r]);
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < m) {
                u32x4 xv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[i] = ld16(x[t] + 32 * j + 8 * i);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float b0 = 0.f, b1 = 0.f;
#pragma unroll
                    for (int p = 0; p < 8; ++p) b0 = dot2_bf16(d[r][p], xv[p / 4][p % 4], b0);
#pragma unroll
                    for (int p = 8; p < 16; ++p) b1 = dot2_bf16(d[r][p], xv[p / 4][p % 4], b1);
                    acc[r][t] = fmaf(s0[r], b0, acc[r][t]);
                    acc[r][t] = fmaf(s1[r], b1, acc[r][t]);
                }
            }
        }
    }
}

}  // namespace qg
