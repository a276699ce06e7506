// Q8_0 x fp32 GEMV for gfx950 (wave64).
//
// Same streaming shape as the NVFP4 kernel: a group of G lanes owns R rows,
// lane l loads the 16-byte code chunks c*G + l (16 int8 codes, half of a
// 32-element block) of each row, all loads issued up front.  Each chunk's
// products are summed in fp32 and scaled once by the block's fp16 scale.
#include <hip/hip_runtime.h>

#include "qg_device.hpp"
#include "qg_gemv_core.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"

namespace qg {

namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ float q8_chunk_dot(const u32x4& c, float d, const float (&xf)[16], float acc) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        s = fmaf(i8_to_f32<0>(c[q]), xf[4 * q + 0], s);
        s = fmaf(i8_to_f32<1>(c[q]), xf[4 * q + 1], s);
        s = fmaf(i8_to_f32<2>(c[q]), xf[4 * q + 2], s);
        s = fmaf(i8_to_f32<3>(c[q]), xf[4 * q + 3], s);
    }
    return fmaf(d, s, acc);
}

// 16 activations at p (always a valid address); zeros when !ok.
__device__ __forceinline__ void load_x16(const float* p, bool ok, float (&xf)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 v = ld<float4>(p + 4 * i);
        xf[4 * i] = ok ? v.x : 0.f;
        xf[4 * i + 1] = ok ? v.y : 0.f;
        xf[4 * i + 2] = ok ? v.z : 0.f;
        xf[4 * i + 3] = ok ? v.w : 0.f;
    }
}

// Chunk j of a row: 16 int8 codes at codes + 16j, block scale (fp16) j/2.
template <int R, int MT, int G, int C>
__global__ __launch_bounds__(kBlock) void k_gemv_q8_0(const uint8_t* __restrict__ w, int64_t soff,
                                                      int n, int k, const float* __restrict__ x,
                                                      int m, float* __restrict__ y) {
    constexpr int kGroups = kWave / G;
    const int lane = lane_id();
    const int grp = lane / G, l = lane % G;
    const int wave = int(blockIdx.x) * (kBlock / kWave) + int(threadIdx.x) / kWave;
    const int unit = wave * kGroups + grp;
    const int64_t srow = (k / 32) * 2;
    const int nchunks = k / 16;

    const uint8_t* codes[R];
    const uint8_t* scales[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(unit * R + r, n - 1);
        codes[r] = w + int64_t(row) * k;
        scales[r] = w + soff + row * srow;
    }
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = 0.f;

    if constexpr (C > 0) {
        u32x4 cw[C][R];
        float d[C][R];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int j = c * G + l;
            const bool ok = j < nchunks;
            const int js = ok ? j : 0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                cw[c][r] = zero_unless(ok, ld_stream16(codes[r] + 16 * js));
                const float dv = f16_to_f32(ld<uint16_t>(scales[r] + 2 * (js >> 1)));
                d[c][r] = ok ? dv : 0.f;
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int j = c * G + l;
            const bool ok = j < nchunks;
            const int js = ok ? j : 0;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < m) {
                    float xf[16];
                    load_x16(x + int64_t(t) * k + 16 * js, ok, xf);
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[r][t] = q8_chunk_dot(cw[c][r], d[c][r], xf, acc[r][t]);
                }
            }
        }
    } else {
        for (int j = l; j < nchunks; j += G) {
            u32x4 cw[R];
            float d[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                cw[r] = ld_stream16(codes[r] + 16 * j);
                d[r] = f16_to_f32(ld<uint16_t>(scales[r] + 2 * (j >> 1)));
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < m) {
                    float xf[16];
                    load_x16(x + int64_t(t) * k + 16 * j, true, xf);
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[r][t] = q8_chunk_dot(cw[r], d[r], xf, acc[r][t]);
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = group_sum<G>(acc[r][t]);
    if (l != 0) return;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = unit * R + r;
        if (row >= n) break;
#pragma unroll
        for (int t = 0; t < MT; ++t)
            if (t < m) y[int64_t(t) * n + row] = acc[r][t];
    }
}

struct Args {
    const uint8_t* w;
    int64_t soff;
    int n, k;
    const float* x;
    int m;
    float* y;
};

// Small matrices: one row per group so that the grid still covers the GPU.
constexpr int64_t kFewRows = 4096;

template <int G, int C, int MT>
hipError_t go(const Args& A, hipStream_t s) {
    constexpr int R = rows_per_group(C, MT);
    const int64_t per_block = (kBlock / kWave) * (kWave / G);
    if (A.n <= kFewRows) {
        const dim3 grid(unsigned((A.n + per_block - 1) / per_block));
        hipLaunchKernelGGL((k_gemv_q8_0<1, MT, G, C>), grid, dim3(kBlock), 0, s, A.w, A.soff, A.n, A.k, A.x,
                           A.m, A.y);
    } else {
        const int64_t units = (int64_t(A.n) + R - 1) / R;
        const dim3 grid(unsigned((units + per_block - 1) / per_block));
        hipLaunchKernelGGL((k_gemv_q8_0<R, MT, G, C>), grid, dim3(kBlock), 0, s, A.w, A.soff, A.n, A.k, A.x,
                           A.m, A.y);
    }
    return hipGetLastError();
}

template <int G, int MT>
hipError_t by_chunks(const Args& A, hipStream_t s) {
    const int C = chunks_per_lane(A.k / 16, G);
    if constexpr (G == 16) {
        switch (C) {
            case 1: return go<16, 1, MT>(A, s);
            case 2: return go<16, 2, MT>(A, s);
            case 3: return go<16, 3, MT>(A, s);
            default: return go<16, 4, MT>(A, s);
        }
    } else {
        switch (C) {
            case 1: return go<64, 1, MT>(A, s);
            case 2: return go<64, 2, MT>(A, s);
            case 3: return go<64, 3, MT>(A, s);
            case 4: return go<64, 4, MT>(A, s);
            case 6: return go<64, 6, MT>(A, s);
            case 8: return go<64, 8, MT>(A, s);
            default: return go<64, 0, MT>(A, s);
        }
    }
}

}  // namespace

hipError_t launch_gemv_q8_0(const uint8_t* w, int64_t n, int64_t k, const float* x, int m, float* y,
                            hipStream_t s) {
    const Args A{w, scale_plane_offset(QG_Q8_0, n, k), int(n), int(k), x, m, y};
    const bool wide = lanes_per_row(k / 16) == 64;
    switch (token_class(m)) {
        case 1: return wide ? by_chunks<64, 1>(A, s) : by_chunks<16, 1>(A, s);
        case 4: return wide ? by_chunks<64, 4>(A, s) : by_chunks<16, 4>(A, s);
        default: return wide ? by_chunks<64, 16>(A, s) : by_chunks<16, 16>(A, s);
    }
}

}  // namespace qg
