// Row-dot cores shared by the dense and the MoE GEMV kernels.
//
// Work split (all formats): lanes form groups of G lanes; a group owns R
// rows; lane l of a group handles the 16-byte code chunks j = c*G + l of each
// row, c = 0..C-1.  When C > 0 is a compile-time count (C >= ceil(chunks/G);
// chunks past the end of the row are skipped), every code and scale load of
// the R*C chunks is issued before any arithmetic, so each wave keeps R*C*1 KB
// of weight reads in flight at once; C == 0 is the general fallback that loops
// over chunks with a runtime count.  Both accumulate each row in ascending
// chunk order, so every variant gives bitwise the same sums.
#pragma once

#include "qg_device.hpp"

namespace qg {

// ---------------------------------------------------------------- NVFP4

// Widen one 32-element chunk of E2M1 codes (4 dwords) to 16 bf16 pairs.
__device__ __forceinline__ void nvfp4_decode_chunk(const u32x4& c, bf16x2 (&d)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        d[4 * q + 0] = e2m1x2_to_bf16x2<0>(c[q]);
        d[4 * q + 1] = e2m1x2_to_bf16x2<1>(c[q]);
        d[4 * q + 2] = e2m1x2_to_bf16x2<2>(c[q]);
        d[4 * q + 3] = e2m1x2_to_bf16x2<3>(c[q]);
    }
}

// Add a decoded chunk's products with the bf16 activations xv into acc: each
// 16-element block is summed on its own, scaled by its block scale (s0, s1),
// and added in block order.
__device__ __forceinline__ float nvfp4_chunk_dot_decoded(const bf16x2 (&d)[16], float s0, float s1,
                                                         const u32x4 (&xv)[4], float acc) {
    float b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) b0 = dot2_bf16(d[p], xv[p / 4][p % 4], b0);
#pragma unroll
    for (int p = 8; p < 16; ++p) b1 = dot2_bf16(d[p], xv[p / 4][p % 4], b1);
    acc = fmaf(s0, b0, acc);
    return fmaf(s1, b1, acc);
}

// Decode one 32-element chunk (4 dwords of codes, 2 E4M3 scales in sc) and add
// its products with the bf16 activations xv into acc.
__device__ __forceinline__ float nvfp4_chunk_dot(const u32x4& c, uint32_t sc, const u32x4 (&xv)[4], float acc) {
    bf16x2 d[16];
    nvfp4_decode_chunk(c, d);
    return nvfp4_chunk_dot_decoded(d, e4m3_to_f32<0>(sc), e4m3_to_f32<1>(sc), xv, acc);
}

// Add this lane's share of R rows x up to MT tokens into acc.  Chunk j of a
// row is 32 elements: 16 code bytes at codes[r] + 16j and the two E4M3 block
// scales at scales[r] + 2j.  x[t] points at token t's bf16 activations.
template <int R, int MT, int G, int C>
__device__ __forceinline__ void nvfp4_partial(const uint8_t* const (&codes)[R],
                                              const uint8_t* const (&scales)[R],
                                              const uint16_t* const (&x)[MT], int m, int nchunks,
                                              int l, float (&acc)[R][MT]) {
    if constexpr (C > 0) {
        // Lanes whose chunk c lies past the end of the row load chunk 0 of the
        // row instead (a valid address) and drop the result.
        u32x4 cw[C][R];
        uint32_t sw[C][R];
        bool okc[C];
        uint32_t jc[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int j = c * G + l;
            okc[c] = j < nchunks;
            jc[c] = okc[c] ? uint32_t(j) : 0u;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                cw[c][r] = ld_stream16(codes[r] + 16u * jc[c]);
                sw[c][r] = ld<uint16_t>(scales[r] + 2u * jc[c]);
            }
        }
        if constexpr (MT == 1) {
            u32x4 xv[C][4];
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[c][i] = ld16(x[0] + 32u * jc[c] + 8u * i);
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float v = nvfp4_chunk_dot(cw[c][r], sw[c][r], xv[c], acc[r][0]);
                    acc[r][0] = okc[c] ? v : acc[r][0];
                }
        } else {
            // Several tokens, in blocks of up to four: per chunk, the block's
            // activations are loaded and each row's chunk is decoded once and
            // reused for the block's tokens (chunks stay in ascending order for
            // every token).  x[t] for t >= m points at a
            // valid token, so no load is conditional; those sums are dropped.
            constexpr int TB = MT < 4 ? MT : 4;
#pragma unroll
            for (int tb = 0; tb < MT; tb += TB) {
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    u32x4 xv[TB][4];
#pragma unroll
                    for (int t = 0; t < TB; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) xv[t][i] = ld16(x[tb + t] + 32u * jc[c] + 8u * i);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        bf16x2 d[16];
                        nvfp4_decode_chunk(cw[c][r], d);
                        const float s0 = e4m3_to_f32<0>(sw[c][r]), s1 = e4m3_to_f32<1>(sw[c][r]);
#pragma unroll
                        for (int t = 0; t < TB; ++t) {
                            const float v = nvfp4_chunk_dot_decoded(d, s0, s1, xv[t], acc[r][tb + t]);
                            acc[r][tb + t] = okc[c] ? v : acc[r][tb + t];
                        }
                    }
                    // Stage the activation loads per chunk and token block: hoisting
                    // them all above the arithmetic would not fit in registers.
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    } else {
        for (int j = l; j < nchunks; j += G) {
            u32x4 cw[R];
            uint32_t sw[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                cw[r] = ld_stream16(codes[r] + 16 * j);
                sw[r] = ld<uint16_t>(scales[r] + 2 * j);
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < m) {
                    u32x4 xv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) xv[i] = ld16(x[t] + 32 * j + 8 * i);
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[r][t] = nvfp4_chunk_dot(cw[r], sw[r], xv, acc[r][t]);
                }
            }
        }
    }
}

// As nvfp4_partial, but a call with a single token (m == 1, wave-uniform)
// runs the one-token form instead of computing MT token slots; both forms
// give bitwise the same per-token sums.
template <int R, int MT, int G, int C>
__device__ __forceinline__ void nvfp4_partial_m(const uint8_t* const (&codes)[R],
                                                const uint8_t* const (&scales)[R],
                                                const uint16_t* const (&x)[MT], int m, int nchunks,
                                                int l, float (&acc)[R][MT]) {
    if constexpr (MT > 1) {
        if (m == 1) {
            float a1[R][1];
#pragma unroll
            for (int r = 0; r < R; ++r) a1[r][0] = acc[r][0];
            const uint16_t* const x1[1] = {x[0]};
            nvfp4_partial<R, 1, G, C>(codes, scales, x1, 1, nchunks, l, a1);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][0] = a1[r][0];
            return;
        }
    }
    nvfp4_partial<R, MT, G, C>(codes, scales, x, m, nchunks, l, acc);
}

// ---------------------------------------------------------------- launch shape

// Compile-time chunks per lane for a row of nchunks chunks split over G
// lanes: the smallest of {1, 2, 3, 4, 6, 8} that covers the row, or 0 for the
// runtime-loop fallback (rows longer than 8*G chunks).
inline constexpr int chunks_per_lane(int64_t nchunks, int G) {
    const int64_t c = (nchunks + G - 1) / G;
    return c <= 4 ? int(c) : c <= 6 ? 6 : c <= 8 ? 8 : 0;
}

// Lanes per row: 64 when a row has at least 64 chunks, else 16.
inline constexpr int lanes_per_row(int64_t nchunks) { return nchunks >= 64 ? 64 : 16; }

// Token-count class: 1, 4 or 16 (m = 2..4 run the 4-token code, 5..16 the
// 16-token code; the extra slots are skipped at run time).
inline constexpr int token_class(int m) { return m <= 1 ? 1 : m <= 4 ? 4 : 16; }

// Rows per lane group: about 8 KB of weight loads in flight per wave (R*C
// chunks of 1 KB per wave-wide load); with several tokens at least 4 rows (2
// for rows of more than 4 chunks per lane) so that each activation load feeds
// several rows -- activations for 4 tokens are as many bytes per row as the
// weights -- and at most 2 rows at 16 tokens to bound the accumulators.
inline constexpr int rows_per_group(int C, int MT) {
    const int c = C == 0 ? 8 : C;
    int r = 8 / c;
    if (MT > 1 && r < 4 && C > 0 && C <= 4) r = 4;
    if (MT > 1 && r < 2) r = 2;
    if (MT >= 16 && r > 2) r = 2;
    return r >= 8 ? 8 : r >= 4 ? 4 : r >= 2 ? 2 : 1;
}

}  // namespace qg
