// FP8 (E4M3) x bf16 GEMV for gfx950 (wave64).
//
// The LumenLLM README runs its 9B model with native FP8 weights (model table
// and feature list); the memra README loads the "block-128" FP8 checkpoints
// (loaders entry).  Weights are one E4M3 byte each with fp32 scales, one per
// tensor or one per 128 x 128 tile.  The kernel has the shape of the NVFP4
// streaming GEMV:
//  * a group of G lanes (64, or 16 for rows under 1024 elements) owns R rows;
//    lane l loads the 16-byte code chunks c*G + l, c < C (16 weights each), so
//    one wave-wide load reads 1 KB of a row contiguously (non-temporal);
//  * every code load of the R*C chunks (and, for tiles, the chunk's scale) is
//    issued before any arithmetic;
//  * E4M3 pairs are widened to bf16 by v_cvt_scalef32_pk_bf16_fp8 (exact) and
//    multiplied into fp32 by v_dot2_f32_bf16; a chunk's sum is added into the
//    row sum as fma(s, sum, acc) with its tile's scale (a chunk never straddles
//    a tile: 16 divides 128), or the row sum is scaled once by the tensor
//    scale;
//  * per-lane sums are combined by the fixed DPP/swizzle butterfly.
// The chunk-to-lane mapping and every summation order depend on k only, so a
// token's result does not depend on m, the grid or the schedule.
#include <hip/hip_runtime.h>

#include "qg_device.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"

namespace qg {

namespace {

constexpr int kBlock = 256;

// Sum over one 16-weight chunk (4 dwords of codes) times the bf16 activations
// xv (2 x 16 bytes), in a fixed order.
__device__ __forceinline__ float fp8_chunk_sum(const u32x4& c, const u32x4 (&xv)[2]) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        s = dot2_bf16(e4m3x2_to_bf16x2<0>(c[q]), xv[q / 2][2 * (q % 2)], s);
        s = dot2_bf16(e4m3x2_to_bf16x2<1>(c[q]), xv[q / 2][2 * (q % 2) + 1], s);
    }
    return s;
}

// Chunks per lane as a compile-time count (0: runtime loop).
inline constexpr int fp8_chunks_per_lane(int64_t nch, int G) {
    const int64_t c = (nch + G - 1) / G;
    return c <= 4 ? int(c) : c <= 6 ? 6 : c <= 8 ? 8 : c <= 12 ? 12 : c <= 16 ? 16 : 0;
}
// Rows per group: about 8 KB of weight loads in flight per wave.
inline constexpr int fp8_rows(int C, int MT) {
    const int c = C == 0 ? 8 : C;
    int r = 8 / c;
    if (MT >= 16 && r > 2) r = 2;
    return r >= 4 ? 4 : r >= 2 ? 2 : 1;
}

template <int R, int MT, int G, int C, bool TILE>
__global__ __launch_bounds__(kBlock) void k_gemv_fp8(const uint8_t* __restrict__ w, int64_t soff, int n, int k,
                                                     const uint16_t* __restrict__ x, int m,
                                                     float* __restrict__ y) {
    constexpr int kGroups = kWave / G;
    const int lane = lane_id();
    const int grp = G == kWave ? 0 : lane / G;
    const int l = G == kWave ? lane : lane % G;
    const int wave = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * (kBlock / kWave) + int(threadIdx.x) / kWave);
    const int unit = wave * kGroups + grp;
    const int nch = k / 16;
    const float* sp = reinterpret_cast<const float*>(w + soff);
    // R divides 128 and unit * R is a multiple of R, so the R rows of a unit
    // share one row of scale tiles
    const int r0 = min(unit * R, n - 1);
    const float* stile = sp + int64_t(r0 / 128) * ((k + 127) / 128);

    const uint8_t* codes[R];
#pragma unroll
    for (int r = 0; r < R; ++r) codes[r] = w + int64_t(min(unit * R + r, n - 1)) * k;
    const uint16_t* xp[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xp[t] = x + int64_t(t < m ? t : 0) * k;

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = 0.f;

    if constexpr (C > 0) {
        // lanes whose chunk lies past the row load chunk 0 (a valid address)
        // and drop the result
        bool okc[C];
        uint32_t jc[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int j = c * G + l;
            okc[c] = j < nch;
            jc[c] = okc[c] ? uint32_t(j) : 0u;
        }
        u32x4 cw[C][R];
        float sc[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
#pragma unroll
            for (int r = 0; r < R; ++r) cw[c][r] = ld_stream16(codes[r] + 16u * jc[c]);
            sc[c] = TILE ? stile[jc[c] >> 3] : 1.f;
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (MT > 1 && t >= m) break;  // wave-uniform
                u32x4 xv[2];
                xv[0] = ld16(xp[t] + 16u * jc[c]);
                xv[1] = ld16(xp[t] + 16u * jc[c] + 8u);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float s = fp8_chunk_sum(cw[c][r], xv);
                    const float v = TILE ? fmaf(sc[c], s, acc[r][t]) : acc[r][t] + s;
                    acc[r][t] = okc[c] ? v : acc[r][t];
                }
            }
        }
    } else {
        for (int j = l; j < nch; j += G) {
            u32x4 cw[R];
#pragma unroll
            for (int r = 0; r < R; ++r) cw[r] = ld_stream16(codes[r] + 16u * j);
            const float scj = TILE ? stile[j >> 3] : 1.f;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t >= m) break;  // wave-uniform
                u32x4 xv[2];
                xv[0] = ld16(xp[t] + 16u * j);
                xv[1] = ld16(xp[t] + 16u * j + 8u);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float s = fp8_chunk_sum(cw[r], xv);
                    acc[r][t] = TILE ? fmaf(scj, s, acc[r][t]) : acc[r][t] + s;
                }
            }
        }
    }

    const float s_t = TILE ? 1.f : sp[0];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = TILE ? group_sum<G>(acc[r][t]) : group_sum<G>(acc[r][t]) * s_t;
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

struct Fp8Args {
    const uint8_t* w;
    int64_t soff;
    int n, k;
    const uint16_t* x;
    int m;
    float* y;
};

template <int G, int C, int MT, bool TILE>
hipError_t go(const Fp8Args& A, hipStream_t s) {
    constexpr int R = fp8_rows(C, MT);
    const int64_t units = (int64_t(A.n) + R - 1) / R;
    const int64_t per_block = (kBlock / kWave) * (kWave / G);
    const dim3 grid(unsigned((units + per_block - 1) / per_block));
    hipLaunchKernelGGL((k_gemv_fp8<R, MT, G, C, TILE>), grid, dim3(kBlock), 0, s, A.w, A.soff, A.n, A.k, A.x, A.m,
                       A.y);
    return hipGetLastError();
}

template <int G, int MT, bool TILE>
hipError_t by_chunks(const Fp8Args& A, hipStream_t s) {
    switch (fp8_chunks_per_lane(A.k / 16, G)) {
        case 1: return go<G, 1, MT, TILE>(A, s);
        case 2: return go<G, 2, MT, TILE>(A, s);
        case 3: return go<G, 3, MT, TILE>(A, s);
        case 4: return go<G, 4, MT, TILE>(A, s);
        case 6: return go<G, 6, MT, TILE>(A, s);
        case 8: return go<G, 8, MT, TILE>(A, s);
        case 12: return go<G, 12, MT, TILE>(A, s);
        case 16: return go<G, 16, MT, TILE>(A, s);
        default: return go<G, 0, MT, TILE>(A, s);
    }
}

template <bool TILE>
hipError_t dispatch(const Fp8Args& A, hipStream_t s) {
    const bool wide = A.k / 16 >= 64;
    const int tc = A.m <= 1 ? 1 : A.m <= 4 ? 4 : 16;
    if (tc == 1) return wide ? by_chunks<64, 1, TILE>(A, s) : by_chunks<16, 1, TILE>(A, s);
    if (tc == 4) return wide ? by_chunks<64, 4, TILE>(A, s) : by_chunks<16, 4, TILE>(A, s);
    return wide ? by_chunks<64, 16, TILE>(A, s) : by_chunks<16, 16, TILE>(A, s);
}

// Dequantizer for verification: one thread per 16-byte chunk.
__global__ __launch_bounds__(kBlock) void k_dequant_fp8(const uint8_t* __restrict__ w, int64_t soff, bool tile,
                                                        int64_t n, int k, float* __restrict__ out) {
    const int64_t idx = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    const int nch = k / 16;
    if (idx >= n * nch) return;
    const int64_t r = idx / nch;
    const int j = int(idx % nch);
    const u32x4 c = ld16(w + r * k + 16 * j);
    const float* sp = reinterpret_cast<const float*>(w + soff);
    const float sc = tile ? sp[(r / 128) * ((k + 127) / 128) + (j >> 3)] : sp[0];
    float* o = out + r * k + 16 * j;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bf16x2 a = e4m3x2_to_bf16x2<0>(c[q]), b = e4m3x2_to_bf16x2<1>(c[q]);
        o[4 * q + 0] = bf16x2_lo(a) * sc;
        o[4 * q + 1] = bf16x2_hi(a) * sc;
        o[4 * q + 2] = bf16x2_lo(b) * sc;
        o[4 * q + 3] = bf16x2_hi(b) * sc;
    }
}

}  // namespace

hipError_t launch_gemv_fp8(int fmt, const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, int m, float* y,
                           hipStream_t s) {
    const Fp8Args A{w, scale_plane_offset(fmt, n, k), int(n), int(k), x, m, y};
    return fmt == QG_FP8_B128 ? dispatch<true>(A, s) : dispatch<false>(A, s);
}

hipError_t launch_dequant_fp8(int fmt, const uint8_t* w, int64_t n, int64_t k, float* out, hipStream_t s) {
    const dim3 grid(unsigned((n * (k / 16) + kBlock - 1) / kBlock));
    hipLaunchKernelGGL(k_dequant_fp8, grid, dim3(kBlock), 0, s, w, scale_plane_offset(fmt, n, k),
                       fmt == QG_FP8_B128, n, int(k), out);
    return hipGetLastError();
}

}  // namespace qg
