// Fused-dequant GEMV kernels for gfx950 (wave64): NVFP4 x bf16, Q8_0 x fp32,
// Q4_0 x Q8_0 (integer block dots), the Q8_0 activation quantizer and the
// verification dequantizer.
//
// The decode step streams every weight byte exactly once (the pages' decode
// sits at the DRAM bandwidth limit: memra README, known gaps on plain decode
// margins), so each kernel is shaped around HBM streaming:
//  * lanes are split into groups of G lanes (G = 64, or 16 for short rows);
//    lane l of a group handles the 16-byte code chunks l, l+G, l+2G, ... of
//    each of its R rows, so one wave-wide load reads G*16 contiguous bytes
//    of a row (fully coalesced, non-temporal);
//  * the R rows of a group share every activation load (x is read R times
//    less often than with one row per group);
//  * per-lane partial sums are combined with a fixed DPP/swizzle butterfly.
// The chunk-to-lane mapping and the reduction order depend only on k, so
// results are bitwise identical for any token count, grid or schedule.
#include <hip/hip_runtime.h>

#include "qg_device.hpp"
#include "qg_gemv_core.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"

namespace qg {

namespace {

constexpr int kBlock = 256;  // threads per workgroup (4 waves)

// ------------------------------------------------------------------ decoders
// (shared by the GEMVs and by the verification dequantizer)

// Unpack one dword of a Q4_0 block: lo = elements 4q..4q+3 (low nibbles),
// hi = elements 16+4q..16+4q+3 (high nibbles), one unsigned code per byte.
__device__ __forceinline__ void q4_unpack(uint32_t c, uint32_t& lo, uint32_t& hi) {
    lo = c & 0x0F0F0F0Fu;
    hi = (c >> 4) & 0x0F0F0F0Fu;
}

// Signed byte B of c as fp32.
template <int B>
__device__ __forceinline__ float i8_to_f32(uint32_t c) {
    return float(int32_t(c << (24 - 8 * B)) >> 24);
}

// Dense NVFP4 GEMV.  SWIGLU: the R rows of a group are RA = R/2 gate rows
// i0..i0+RA-1 and the matching up rows inter+i0..; the epilogue writes
// a = bf16(silu(g) * u) (and optionally g, u into h).
template <int R, int MT, int G, bool SWIGLU>
__global__ __launch_bounds__(kBlock) void k_gemv_nvfp4(const uint8_t* __restrict__ w, int64_t soff,
                                                       float s_t, int nout, int k,
                                                       const uint16_t* __restrict__ x, int m,
                                                       float* __restrict__ y,
                                                       uint16_t* __restrict__ a,
                                                       float* __restrict__ h) {
    constexpr int kGroups = kWave / G;
    const int lane = lane_id();
    const int grp = lane / G, l = lane % G;
    const int wave = int(blockIdx.x) * (kBlock / kWave) + int(threadIdx.x) / kWave;
    const int unit = wave * kGroups + grp;
    const int64_t crow = k / 2, srow = k / 16;

    int rows[R];
    if constexpr (!SWIGLU) {
#pragma unroll
        for (int r = 0; r < R; ++r) rows[r] = min(unit * R + r, nout - 1);
    } else {
        constexpr int RA = R / 2;
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            rows[r] = min(unit * RA + r, nout - 1);
            rows[RA + r] = nout + rows[r];
        }
    }
    const uint8_t* codes[R];
    const uint8_t* scales[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        codes[r] = w + rows[r] * crow;
        scales[r] = w + soff + rows[r] * srow;
    }
    const uint16_t* xp[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xp[t] = x + int64_t(t < m ? t : 0) * k;

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = 0.f;

    nvfp4_partial<R, MT, G>(codes, scales, xp, m, k / 32, l, acc);

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = group_sum<G>(acc[r][t]) * s_t;

    if (l != 0) return;
    if constexpr (!SWIGLU) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = unit * R + r;
            if (row >= nout) break;
#pragma unroll
            for (int t = 0; t < MT; ++t)
                if (t < m) y[int64_t(t) * nout + row] = acc[r][t];
        }
    } else {
        constexpr int RA = R / 2;
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            const int i = unit * RA + r;
            if (i >= nout) break;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < m) {
                    const float g = acc[r][t], u = acc[RA + r][t];
                    const float act = g / (1.0f + expf(-g)) * u;
                    a[int64_t(t) * nout + i] = uint16_t(f32_to_bf16_rne(act));
                    if (h) {
                        h[int64_t(t) * 2 * nout + i] = g;
                        h[int64_t(t) * 2 * nout + nout + i] = u;
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ Q8_0 x fp32

// Chunk j of a row is 16 int8 codes (half of block j/2).
template <int R, int MT, int G>
__global__ __launch_bounds__(kBlock) void k_gemv_q8_0(const uint8_t* __restrict__ w, int64_t soff,
                                                      int n, int k, const float* __restrict__ x,
                                                      int m, float* __restrict__ y) {
    constexpr int kGroups = kWave / G;
    const int lane = lane_id();
    const int grp = lane / G, l = lane % G;
    const int wave = int(blockIdx.x) * (kBlock / kWave) + int(threadIdx.x) / kWave;
    const int unit = wave * kGroups + grp;
    const int64_t srow = (k / 32) * 2;

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

    const int nchunks = k / 16;
    for (int j = l; j < nchunks; j += G) {
        u32x4 c[R];
        float d[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            c[r] = ld_stream16(codes[r] + 16 * j);
            d[r] = f16_to_f32(ld<uint16_t>(scales[r] + 2 * (j >> 1)));
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < m) {
                const float* xp = x + int64_t(t) * k + 16 * j;
                float4 xv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[i] = ld<float4>(xp + 4 * i);
                const float* xf = reinterpret_cast<const float*>(xv);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float s = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        s = fmaf(i8_to_f32<0>(c[r][q]), xf[4 * q + 0], s);
                        s = fmaf(i8_to_f32<1>(c[r][q]), xf[4 * q + 1], s);
                        s = fmaf(i8_to_f32<2>(c[r][q]), xf[4 * q + 2], s);
                        s = fmaf(i8_to_f32<3>(c[r][q]), xf[4 * q + 3], s);
                    }
                    acc[r][t] = fmaf(d[r], s, acc[r][t]);
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

// ------------------------------------------------------------------ W4A8

// Chunk j of a row is one Q4_0 block: 16 code bytes and one fp16 scale.
template <int R, int MT, int G>
__global__ __launch_bounds__(kBlock) void k_gemv_q4_0_a8(const uint8_t* __restrict__ w, int64_t soff,
                                                         int n, int k,
                                                         const int8_t* __restrict__ xq,
                                                         const uint16_t* __restrict__ xd,
                                                         const int32_t* __restrict__ xs, int m,
                                                         float* __restrict__ y) {
    constexpr int kGroups = kWave / G;
    const int lane = lane_id();
    const int grp = lane / G, l = lane % G;
    const int wave = int(blockIdx.x) * (kBlock / kWave) + int(threadIdx.x) / kWave;
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

    for (int j = l; j < nb; j += G) {
        uint32_t lo[R][4], hi[R][4];
        float dw[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32x4 c = ld_stream16(codes[r] + 16 * j);
            dw[r] = f16_to_f32(ld<uint16_t>(scales[r] + 2 * j));
#pragma unroll
            for (int q = 0; q < 4; ++q) q4_unpack(c[q], lo[r][q], hi[r][q]);
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < m) {
                const int8_t* xp = xq + int64_t(t) * k + 32 * j;
                const u32x4 x0 = ld16(xp), x1 = ld16(xp + 16);
                const float dx = f16_to_f32(xd[int64_t(t) * nb + j]);
                int bsum;
                if (xs) {
                    bsum = xs[int64_t(t) * nb + j];
                } else {
                    bsum = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        bsum = dot4_i8(0x01010101u, x0[q], bsum);
                        bsum = dot4_i8(0x01010101u, x1[q], bsum);
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    int isum = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        isum = dot4_i8(lo[r][q], x0[q], isum);
                        isum = dot4_i8(hi[r][q], x1[q], isum);
                    }
                    isum -= 8 * bsum;  // sum (q_w - 8) q_x = sum q_w q_x - 8 sum q_x
                    acc[r][t] = fmaf(dw[r] * dx, float(isum), acc[r][t]);
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

// ------------------------------------------------------------------ quantizer

// One thread per 32-element block.
__global__ __launch_bounds__(kBlock) void k_quantize_q8_0(const float* __restrict__ x,
                                                          int64_t nblocks,
                                                          int8_t* __restrict__ xq,
                                                          uint16_t* __restrict__ xd,
                                                          int32_t* __restrict__ xs) {
    const int64_t b = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    if (b >= nblocks) return;
    const float* p = x + 32 * b;
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 f = ld<float4>(p + 4 * i);
        v[4 * i] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float d32 = amax / 127.0f;  // correctly rounded (no fast-math in this library)
    const _Float16 d16 = _Float16(d32);
    uint32_t packed[8];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed[i] = 0;
    if (d32 != 0.f) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float r = fminf(fmaxf(rintf(v[i] / d32), -127.f), 127.f);
            const int q = int(r);
            sum += q;
            packed[i / 4] |= uint32_t(q & 0xff) << (8 * (i % 4));
        }
    }
    u32x4* o = reinterpret_cast<u32x4*>(xq + 32 * b);
    o[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
    o[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
    xd[b] = __builtin_bit_cast(uint16_t, d16);
    if (xs) xs[b] = sum;
}

// ------------------------------------------------------------------ dequant

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

// ------------------------------------------------------------------ dispatch

inline int pow2_tokens(int m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : m <= 8 ? 8 : 16; }

inline unsigned grid_for(int64_t units, int G) {
    const int64_t per_block = (kBlock / kWave) * (kWave / G);
    return unsigned((units + per_block - 1) / per_block);
}

template <int MT, int G, bool SWIGLU>
hipError_t nvfp4_go(const uint8_t* w, int64_t soff, float s_t, int nout, int k, const uint16_t* x,
                    int m, float* y, uint16_t* a, float* h, hipStream_t s) {
    constexpr int R = SWIGLU ? (MT <= 2 ? 4 : 2) : (MT <= 2 ? 4 : MT <= 8 ? 2 : 1);
    const int64_t units = SWIGLU ? (nout + R / 2 - 1) / (R / 2) : (nout + R - 1) / R;
    hipLaunchKernelGGL((k_gemv_nvfp4<R, MT, G, SWIGLU>), dim3(grid_for(units, G)), dim3(kBlock), 0, s,
                       w, soff, s_t, nout, k, x, m, y, a, h);
    return hipGetLastError();
}

template <int G, bool SWIGLU>
hipError_t nvfp4_mt(const uint8_t* w, int64_t soff, float s_t, int nout, int k, const uint16_t* x,
                    int m, float* y, uint16_t* a, float* h, hipStream_t s) {
    switch (pow2_tokens(m)) {
        case 1: return nvfp4_go<1, G, SWIGLU>(w, soff, s_t, nout, k, x, m, y, a, h, s);
        case 2: return nvfp4_go<2, G, SWIGLU>(w, soff, s_t, nout, k, x, m, y, a, h, s);
        case 4: return nvfp4_go<4, G, SWIGLU>(w, soff, s_t, nout, k, x, m, y, a, h, s);
        case 8: return nvfp4_go<8, G, SWIGLU>(w, soff, s_t, nout, k, x, m, y, a, h, s);
        default: return nvfp4_go<16, G, SWIGLU>(w, soff, s_t, nout, k, x, m, y, a, h, s);
    }
}

// Lanes per row: 64 when a row has at least 64 chunks of 32 elements, else 16.
inline bool wide_rows(int64_t nchunks) { return nchunks >= 64; }

template <int MT, int G>
hipError_t q8_go(const uint8_t* w, int64_t soff, int n, int k, const float* x, int m, float* y,
                 hipStream_t s) {
    constexpr int R = MT <= 2 ? 4 : MT <= 8 ? 2 : 1;
    hipLaunchKernelGGL((k_gemv_q8_0<R, MT, G>), dim3(grid_for((n + R - 1) / R, G)), dim3(kBlock), 0,
                       s, w, soff, n, k, x, m, y);
    return hipGetLastError();
}

template <int MT, int G>
hipError_t a8_go(const uint8_t* w, int64_t soff, int n, int k, const int8_t* xq, const uint16_t* xd,
                 const int32_t* xs, int m, float* y, hipStream_t s) {
    constexpr int R = MT <= 2 ? 4 : MT <= 8 ? 2 : 1;
    hipLaunchKernelGGL((k_gemv_q4_0_a8<R, MT, G>), dim3(grid_for((n + R - 1) / R, G)), dim3(kBlock), 0,
                       s, w, soff, n, k, xq, xd, xs, m, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_nvfp4(const uint8_t* w, float s_t, int64_t n, int64_t k, const uint16_t* x,
                             int m, float* y, hipStream_t s) {
    const int64_t soff = scale_plane_offset(QG_NVFP4, n, k);
    if (wide_rows(k / 32))
        return nvfp4_mt<64, false>(w, soff, s_t, int(n), int(k), x, m, y, nullptr, nullptr, s);
    return nvfp4_mt<16, false>(w, soff, s_t, int(n), int(k), x, m, y, nullptr, nullptr, s);
}

hipError_t launch_gemv_nvfp4_swiglu(const uint8_t* w, float s_t, int64_t inter, int64_t k,
                                    const uint16_t* x, int m, uint16_t* a, float* h, hipStream_t s) {
    const int64_t soff = scale_plane_offset(QG_NVFP4, 2 * inter, k);
    if (wide_rows(k / 32))
        return nvfp4_mt<64, true>(w, soff, s_t, int(inter), int(k), x, m, nullptr, a, h, s);
    return nvfp4_mt<16, true>(w, soff, s_t, int(inter), int(k), x, m, nullptr, a, h, s);
}

hipError_t launch_gemv_q8_0(const uint8_t* w, int64_t n, int64_t k, const float* x, int m, float* y,
                            hipStream_t s) {
    const int64_t soff = scale_plane_offset(QG_Q8_0, n, k);
    const bool wide = wide_rows(k / 16);
#define QG_Q8(MT)                                                                      \
    return wide ? q8_go<MT, 64>(w, soff, int(n), int(k), x, m, y, s)                   \
                : q8_go<MT, 16>(w, soff, int(n), int(k), x, m, y, s)
    switch (pow2_tokens(m)) {
        case 1: QG_Q8(1);
        case 2: QG_Q8(2);
        case 4: QG_Q8(4);
        case 8: QG_Q8(8);
        default: QG_Q8(16);
    }
#undef QG_Q8
}

hipError_t launch_gemv_q4_0_a8(const uint8_t* w, int64_t n, int64_t k, const int8_t* xq,
                               const uint16_t* xd, const int32_t* xs, int m, float* y,
                               hipStream_t s) {
    const int64_t soff = scale_plane_offset(QG_Q4_0, n, k);
    const bool wide = wide_rows(k / 32);
#define QG_A8(MT)                                                                      \
    return wide ? a8_go<MT, 64>(w, soff, int(n), int(k), xq, xd, xs, m, y, s)          \
                : a8_go<MT, 16>(w, soff, int(n), int(k), xq, xd, xs, m, y, s)
    switch (pow2_tokens(m)) {
        case 1: QG_A8(1);
        case 2: QG_A8(2);
        case 4: QG_A8(4);
        case 8: QG_A8(8);
        default: QG_A8(16);
    }
#undef QG_A8
}

hipError_t launch_quantize_q8_0(const float* x, int64_t m, int64_t k, int8_t* xq, uint16_t* xd,
                                int32_t* xs, hipStream_t s) {
    const int64_t nblocks = m * (k / 32);
    hipLaunchKernelGGL(k_quantize_q8_0, dim3(unsigned((nblocks + kBlock - 1) / kBlock)), dim3(kBlock),
                       0, s, x, nblocks, xq, xd, xs);
    return hipGetLastError();
}

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
