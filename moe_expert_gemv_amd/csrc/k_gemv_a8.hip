// W4A8 path for gfx950: the Q8_0 activation quantizer and the Q4_0 x Q8_0
// GEMV with exact int32 block dots (v_dot4_i32_i8), after the pages' dp4a /
// W4A8 integer decode path (bw24 README, NVFP4 (W4) decode path entry).
//
// Per 32-element block: isum = sum (q_w - 8) * q_x, computed as
// sum q_w * q_x - 8 * sum q_x so the 4-bit codes need no per-nibble offset
// (the activation block sums come from the quantizer), then one fp32 step
// y += (d_w * d_x) * isum.  Streaming shape as in the NVFP4 kernel.
#include <hip/hip_runtime.h>

#include "qg_device.hpp"
#include "qg_gemv_core.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"
#include "qg_mfma.hpp"
#include "qg_reduce.hpp"

namespace qg {

namespace {

constexpr int kBlock = 256;

// sum over the block of q_w * q_x (exact int32), codes c, activations x0|x1.
__device__ __forceinline__ int q4_block_dot(const u32x4& c, const u32x4& x0, const u32x4& x1) {
    int isum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t lo, hi;
        q4_unpack(c[q], lo, hi);
        isum = dot4_i8(lo, x0[q], isum);
        isum = dot4_i8(hi, x1[q], isum);
    }
    return isum;
}

struct XBlock {
    u32x4 x0, x1;
    float dx;
    int bsum8;  // 8 * sum of the block's q_x
};

// Block j of token t's activations (j must be a valid block).  The token's
// base addresses are wave-uniform; only the 32-bit block offset is per lane.
// Without XS the block sum is formed from the codes.
template <bool XS>
__device__ __forceinline__ XBlock load_xblock(const int8_t* xq, const uint16_t* xd, const int32_t* xs, int64_t t,
                                              int k, int nb, uint32_t j) {
    XBlock b;
    const int8_t* p = (xq + t * k) + 32u * j;
    b.x0 = ld16(p);
    b.x1 = ld16(p + 16);
    b.dx = f16_to_f32((xd + t * nb)[j]);
    int s;
    if constexpr (XS) {
        s = (xs + t * nb)[j];
    } else {
        s = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s = dot4_i8(0x01010101u, b.x0[q], s);
            s = dot4_i8(0x01010101u, b.x1[q], s);
        }
    }
    b.bsum8 = 8 * s;
    return b;
}

// Chunk j of a row = Q4_0 block j: 16 code bytes and one fp16 scale.  XS:
// the quantizer's int32 block sums are given (else formed from the codes).
template <int R, int MT, int G, int C, bool XS, bool LDSX = false>
__global__ __launch_bounds__(kBlock) void k_gemv_q4_0_a8(const uint8_t* __restrict__ w, int64_t soff,
                                                         int n, int k,
                                                         const int8_t* __restrict__ xq,
                                                         const uint16_t* __restrict__ xd,
                                                         const int32_t* __restrict__ xs, int m,
                                                         float* __restrict__ y) {
    constexpr int kGroups = kWave / G;
    const int lane = lane_id();
    const int grp = G == kWave ? 0 : lane / G;  // one group per wave: rows are wave-uniform
    const int l = G == kWave ? lane : lane % G;
    const int wave = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * (kBlock / kWave) + int(threadIdx.x) / kWave);
    const int unit = wave * kGroups + grp;
    const int64_t crow = k / 2, srow = (k / 32) * 2;
    const int nb = k / 32;

    const uint8_t* codes[R];
    const uint8_t* scales[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(unit * R + r, n - 1);
        codes[r] = w + row * crow;
        scales[r] = w + soff + row * srow;
    }
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = 0.f;

    // Token slots past m read token 0 (valid addresses); their sums are dropped.
    int64_t tok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) tok[t] = t < m ? t : 0;

    if constexpr (C > 0) {
        // Every code chunk and scale of the R*C blocks is loaded first, at a
        // clamped (always valid) block index; lanes whose block c lies past
        // the row end keep their sum unchanged.  With one token the lane's C
        // activation blocks are requested before the weights: loads complete
        // in order, so activations requested behind the weight stream would
        // wait for all of it, and then cost one more round trip per block.
        u32x4 cw[C][R];
        uint32_t sw[C][R];
        bool okc[C];
        uint32_t jc[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int j = c * G + l;
            okc[c] = j < nb;
            jc[c] = okc[c] ? uint32_t(j) : 0u;
        }
        XBlock x1[MT == 1 ? C : 1];
        if constexpr (MT == 1) {
#pragma unroll
            for (int c = 0; c < C; ++c) x1[c] = load_xblock<XS>(xq, xd, xs, 0, k, nb, jc[c]);
        }
        // LDSX (four token slots, k <= 6144): the slots' activation blocks
        // are staged in LDS once per workgroup -- every wave would otherwise
        // read about 2.5 times its weight bytes in activations through L1.
        // Codes: 16-byte unit h of block j at slot 2j + (h ^ (j/4 & 1)), so
        // the eight lanes of one 128-byte LDS cycle hit distinct banks.
        // Staging loads are clamped (a clamped thread re-stores the last unit)
        // and issued before the weights; the stores wait for them only.
        constexpr int kXU = LDSX ? C * 128 : 1;  // code units per slot (nb <= 64 * C)
        constexpr int kXB = LDSX ? C * 64 : 1;   // blocks per slot
        __shared__ u32x4 s_q[LDSX ? MT * kXU : 1];
        __shared__ uint16_t s_d[LDSX ? MT * kXB : 1];
        __shared__ int32_t s_s[LDSX && XS ? MT * kXB : 1];
        constexpr int kQPer = (kXU + kBlock - 1) / kBlock;
        u32x4 gq[LDSX ? MT : 1][LDSX ? kQPer : 1];
        uint16_t gd[LDSX ? MT : 1];
        int32_t gs[LDSX ? MT : 1];
        const int tid = int(threadIdx.x);
        const int nu = 2 * nb;
        if constexpr (LDSX) {
            static_assert(G == kWave && MT == 4, "four token slots, one lane group per wave");
#pragma unroll
            for (int t = 0; t < MT; ++t) {
#pragma unroll
                for (int q = 0; q < kQPer; ++q)
                    gq[t][q] = ld16(xq + tok[t] * k + 16 * min(tid + kBlock * q, nu - 1));
                gd[t] = (xd + tok[t] * nb)[min(tid, nb - 1)];
                if constexpr (XS) gs[t] = (xs + tok[t] * nb)[min(tid, nb - 1)];
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                cw[c][r] = ld_stream16(codes[r] + 16u * jc[c]);
                sw[c][r] = ld<uint16_t>(scales[r] + 2u * jc[c]);
            }
        }
        if constexpr (LDSX) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
#pragma unroll
                for (int q = 0; q < kQPer; ++q) {
                    const uint32_t u = uint32_t(min(tid + kBlock * q, nu - 1));
                    s_q[t * kXU + ((u & ~1u) | ((u & 1u) ^ ((u >> 3) & 1u)))] = gq[t][q];
                }
                const int jb = min(tid, nb - 1);
                s_d[t * kXB + jb] = gd[t];
                if constexpr (XS) s_s[t * kXB + jb] = gs[t];
            }
            lds_barrier();
        }
        // token slot t's block j from LDS, as load_xblock gives it
        auto lds_xblock = [&](int t, uint32_t j) {
            XBlock b;
            const uint32_t f = (j >> 2) & 1u;
            b.x0 = s_q[t * kXU + 2 * j + f];
            b.x1 = s_q[t * kXU + 2 * j + (1u ^ f)];
            b.dx = f16_to_f32(s_d[t * kXB + j]);
            int sum;
            if constexpr (XS) {
                sum = s_s[t * kXB + j];
            } else {
                sum = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    sum = dot4_i8(0x01010101u, b.x0[q], sum);
                    sum = dot4_i8(0x01010101u, b.x1[q], sum);
                }
            }
            b.bsum8 = 8 * sum;
            return b;
        };
        // Tokens in blocks of up to four: per block and chunk, the tokens'
        // activation blocks are loaded and each row's codes unpacked once.
        constexpr int TB = MT < 4 ? MT : 4;
#pragma unroll
        for (int tb = 0; tb < MT; tb += TB) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                XBlock b[TB];
#pragma unroll
                for (int t = 0; t < TB; ++t) {
                    if constexpr (LDSX)
                        b[t] = lds_xblock(tb + t, jc[c]);
                    else
                        b[t] = MT == 1 ? x1[c] : load_xblock<XS>(xq, xd, xs, tok[tb + t], k, nb, jc[c]);
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    uint32_t lo[4], hi[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) q4_unpack(cw[c][r][q], lo[q], hi[q]);
                    const float dwr = f16_to_f32(sw[c][r]);
#pragma unroll
                    for (int t = 0; t < TB; ++t) {
                        int isum = 0;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            isum = dot4_i8(lo[q], b[t].x0[q], isum);
                            isum = dot4_i8(hi[q], b[t].x1[q], isum);
                        }
                        const float v = fmaf(dwr * b[t].dx, float(isum - b[t].bsum8), acc[r][tb + t]);
                        acc[r][tb + t] = okc[c] ? v : acc[r][tb + t];
                    }
                }
                // Stage the activation loads per chunk and token block: hoisting
                // them all above the arithmetic would not fit in registers.
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        for (int j = l; j < nb; j += G) {
            u32x4 cw[R];
            float dw[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                cw[r] = ld_stream16(codes[r] + 16 * j);
                dw[r] = f16_to_f32(ld<uint16_t>(scales[r] + 2 * j));
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < m) {
                    const XBlock b = load_xblock<XS>(xq, xd, xs, t, k, nb, uint32_t(j));
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const int isum = q4_block_dot(cw[r], b.x0, b.x1) - b.bsum8;
                        acc[r][t] = fmaf(dw[r] * b.dx, float(isum), acc[r][t]);
                    }
                }
            }
        }
    }
    if constexpr (MT > 1 && G == kWave && ((R * MT) & (R * MT - 1)) == 0 && R * MT <= 64) {
        // several tokens: reduce-scatter, lane l ends with (row, token) index
        // bitrev(l % N), index = row * MT + token -- bitwise the butterfly sums
        constexpr int N = R * MT, L = log2i(N);
        float flat[N];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < MT; ++t) flat[r * MT + t] = acc[r][t];
        const float v = reduce_scatter64<N>(flat);
        const int idx = bitrev<L>(lane & (N - 1));
        const int r = idx / MT, t = idx % MT;
        const int row = unit * R + r;
        if (lane < N && t < m && row < n) y[int64_t(t) * n + row] = v;
        return;
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

// ------------------------------------------------------------------ quantizer

// One lane per element, one half-wave (32 lanes) per 32-element block: the
// block's amax and code sum are half-wave butterflies (exact in any order), so
// every element's division runs on its own lane instead of 32 in sequence on
// one thread.  Each lane's arithmetic is the oracle's reading step by step:
// d32 = amax / 127 and x / d32 as correctly rounded fp32 divisions (this
// library is built without fast-math), v_rndne_f32, clamp to +-127.
__global__ __launch_bounds__(kBlock) void k_quantize_q8_0(const float* __restrict__ x, int64_t nelem,
                                                          int8_t* __restrict__ xq,
                                                          uint16_t* __restrict__ xd,
                                                          int32_t* __restrict__ xs) {
    const int64_t e = int64_t(blockIdx.x) * kBlock + threadIdx.x;  // nelem % 32 == 0: whole half-waves
    if (e >= nelem) return;                                         // uniform per half-wave
    const float v = x[e];
    float amax = fabsf(v);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
    const float d32 = amax / 127.0f;
    const int q = d32 != 0.f ? int(fminf(fmaxf(rintf(v / d32), -127.f), 127.f)) : 0;
    int sum = q;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) sum += __shfl_xor(sum, o, 32);
    xq[e] = int8_t(q);
    if ((threadIdx.x & 31) == 0) {
        const int64_t b = e / 32;
        xd[b] = __builtin_bit_cast(uint16_t, _Float16(d32));
        if (xs) xs[b] = sum;
    }
}

struct Args {
    const uint8_t* w;
    int64_t soff;
    int n, k;
    const int8_t* xq;
    const uint16_t* xd;
    const int32_t* xs;
    int m;
    float* y;
};

template <int G, int C, int MT>
hipError_t go(const Args& A, hipStream_t s) {
    if constexpr (MT >= 16 && C > 4) {
        // 16 tokens over long rows: the all-loads-first form does not fit in
        // registers; use the block loop.
        return go<G, 0, MT>(A, s);
    } else {
        constexpr int R = rows_per_group(C, MT);
        const int64_t units = (int64_t(A.n) + R - 1) / R;
        const int64_t per_block = (kBlock / kWave) * (kWave / G);
        const dim3 grid(unsigned((units + per_block - 1) / per_block));
        // four token slots: activations staged in LDS when they fit (k <= 6144)
        constexpr bool L = G == kWave && MT == 4 && C > 0 && C <= 3;
        if (A.xs)
            hipLaunchKernelGGL((k_gemv_q4_0_a8<R, MT, G, C, true, L>), grid, dim3(kBlock), 0, s, A.w, A.soff, A.n,
                               A.k, A.xq, A.xd, A.xs, A.m, A.y);
        else
            hipLaunchKernelGGL((k_gemv_q4_0_a8<R, MT, G, C, false, L>), grid, dim3(kBlock), 0, s, A.w, A.soff,
                               A.n, A.k, A.xq, A.xd, A.xs, A.m, A.y);
        return hipGetLastError();
    }
}

template <int G, int MT>
hipError_t by_chunks(const Args& A, hipStream_t s) {
    const int C = chunks_per_lane(A.k / 32, G);
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

hipError_t launch_gemv_q4_0_a8(const uint8_t* w, int64_t n, int64_t k, const int8_t* xq,
                               const uint16_t* xd, const int32_t* xs, int m, float* y,
                               hipStream_t s) {
    const Args A{w, scale_plane_offset(QG_Q4_0, n, k), int(n), int(k), xq, xd, xs, m, y};
    const bool wide = lanes_per_row(k / 32) == 64;
    switch (token_class(m)) {
        case 1: return wide ? by_chunks<64, 1>(A, s) : by_chunks<16, 1>(A, s);
        case 4: return wide ? by_chunks<64, 4>(A, s) : by_chunks<16, 4>(A, s);
        default: return wide ? by_chunks<64, 16>(A, s) : by_chunks<16, 16>(A, s);
    }
}

hipError_t launch_quantize_q8_0(const float* x, int64_t m, int64_t k, int8_t* xq, uint16_t* xd,
                                int32_t* xs, hipStream_t s) {
    const int64_t nelem = m * k;
    hipLaunchKernelGGL(k_quantize_q8_0, dim3(unsigned((nelem + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, x,
                       nelem, xq, xd, xs);
    return hipGetLastError();
}

}  // namespace qg
