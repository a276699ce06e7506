// K-quant (Q4_K, Q5_K, Q6_K) and IQ4_XS weights x Q8_0 activations for
// gfx950 (wave64): the K-quant split-plane matvecs with integer dots of the
// memra README (feature list "Decode kernels"), which the pages run their
// GGUF models with (bw24 README, requirements; memra README, model table).
//
// Shape as the W4A8 kernel: a group of G lanes owns R rows; lane l takes the
// 32-element blocks j = c*G + l of each row, so every wave-wide code load
// reads 1 KB of a row contiguously (non-temporal), and every code, high-bit
// and scale load of the R*C blocks is issued before any arithmetic.  Per
// block the codes are rebuilt as int8 bytes -- the 4-bit plane, plus for
// Q5_K / Q6_K the high bits (stored one byte apart, so one shift and one mask
// place four of them), or for IQ4_XS two byte permutes into the codebook --
// and dotted with the int8 activations by v_dot4_i32_i8, exactly.  The fp32
// scale step per block and the fixed butterfly are the only roundings; blocks
// are added in ascending order, so results depend on k only.
#include <hip/hip_runtime.h>

#include "qg_device.hpp"
#include "qg_gemv_core.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"

namespace qg {

namespace {

constexpr int kBlock = 256;

// The IQ4_NL codebook as int8 bytes, four entries per dword (entry 4i + b in
// byte b of dword i).
constexpr uint32_t kIq4T0 = 0xBFAD9881u;  // -127, -104,  -83,  -65
constexpr uint32_t kIq4T1 = 0xF6EADDCFu;  //  -49,  -35,  -22,  -10
constexpr uint32_t kIq4T2 = 0x26190D01u;  //    1,   13,   25,   38
constexpr uint32_t kIq4T3 = 0x71594535u;  //   53,   69,   89,  113

// Four 4-bit indices, the low nibbles of the bytes of c -> their four
// codebook bytes.  Byte permutes take selectors 0..7 as byte indices, so
// one permute looks bits 0..2 of every index up in entries 0..7 and another
// in entries 8..15, and a third takes byte i from the first or the second by
// bit 3 of index i (selector i or i + 4).  The high nibbles: c >> 4.
__device__ __forceinline__ uint32_t iq4_lookup(uint32_t c) {
    const uint32_t sel = c & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(kIq4T1, kIq4T0, sel);  // entries 0..7
    const uint32_t hi = __builtin_amdgcn_perm(kIq4T3, kIq4T2, sel);  // entries 8..15
    // ((c >> 1) & 0x04040404) | 0x03020100 as one three-input bit operation
    // (truth table 0xEA: a & b | c)
    const uint32_t pick = __builtin_amdgcn_bitop3_b32(c >> 1, 0x04040404u, 0x03020100u, 0xEA);
    return __builtin_amdgcn_perm(hi, lo, pick);
}

// The raw data of one 32-element block of a row.
struct KqRaw {
    u32x4 c;       // the 4-bit plane (Q4_0 nibble order)
    uint32_t h0;   // Q5_K: high bits; Q6_K: high bits of elements 0..15
    uint32_t h1;   // Q6_K: high bits of elements 16..31
    uint32_t sup;  // the super-block part: d (| dmin << 16)
    uint32_t sub;  // the block part: sc | m << 8 (Q4_K / Q5_K), sc_lo | sc_hi << 8 (Q6_K), ls (IQ4_XS)
};

template <int FMT>
__device__ __forceinline__ KqRaw kq_load(const uint8_t* codes, const uint8_t* scales, int k, uint32_t j) {
    KqRaw o;
    o.c = ld_stream16(codes + 16u * j);
    o.h0 = o.h1 = 0;
    const uint8_t* hb = codes + uint32_t(k) / 2;
    if constexpr (FMT == QG_Q5_K) {
        o.h0 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(hb + 4u * j));
    } else if constexpr (FMT == QG_Q6_K) {
        o.h0 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(hb + 8u * j));
        o.h1 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(hb + 8u * j + 4u));
    }
    const uint32_t S = uint32_t(k) / 256u, s = j >> 3;
    if constexpr (FMT == QG_Q4_K || FMT == QG_Q5_K) {
        o.sup = ld<uint32_t>(scales + 4u * s);
        o.sub = ld<uint16_t>(scales + 4u * S + 2u * j);
    } else if constexpr (FMT == QG_Q6_K) {
        o.sup = ld<uint16_t>(scales + 2u * s);
        o.sub = ld<uint16_t>(scales + 2u * S + 2u * j);
    } else {
        o.sup = ld<uint16_t>(scales + 2u * s);
        o.sub = ld<uint8_t>(scales + 2u * S + j);
    }
    return o;
}

// Codes of the block as int8 bytes: lo[q] = elements 4q..4q+3, hi[q] =
// elements 16+4q..16+4q+3 (for IQ4_XS the codebook values).
template <int FMT>
__device__ __forceinline__ void kq_codes(const KqRaw& o, uint32_t (&lo)[4], uint32_t (&hi)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if constexpr (FMT == QG_IQ4_XS) {
            lo[q] = iq4_lookup(o.c[q]);
            hi[q] = iq4_lookup(o.c[q] >> 4);
            continue;
        }
        q4_unpack(o.c[q], lo[q], hi[q]);
        if constexpr (FMT == QG_Q5_K) {
            lo[q] |= ((o.h0 >> q) & 0x01010101u) << 4;
            hi[q] |= ((o.h0 >> (4 + q)) & 0x01010101u) << 4;
        } else if constexpr (FMT == QG_Q6_K) {
            lo[q] |= ((o.h0 >> (2 * q)) & 0x03030303u) << 4;
            hi[q] |= ((o.h1 >> (2 * q)) & 0x03030303u) << 4;
        }
    }
}

// Per-block scale factors, shared by every token.
struct KqScale {
    float a, b;  // Q4_K / Q5_K: d*sc and dmin*m (exact); Q6_K / IQ4_XS: d
    int s0, s1;  // Q6_K: the two int8 sub-scales; IQ4_XS: ls - 32
};

template <int FMT>
__device__ __forceinline__ KqScale kq_scale(const KqRaw& o) {
    KqScale s;
    if constexpr (FMT == QG_Q4_K || FMT == QG_Q5_K) {
        s.a = f16_to_f32(o.sup & 0xFFFFu) * float(o.sub & 0xFFu);
        s.b = f16_to_f32(o.sup >> 16) * float(o.sub >> 8);
        s.s0 = s.s1 = 0;
    } else {
        s.a = f16_to_f32(o.sup);
        s.b = 0.f;
        if constexpr (FMT == QG_Q6_K) {
            s.s0 = int(int8_t(o.sub & 0xFFu));
            s.s1 = int(int8_t(o.sub >> 8));
        } else {
            s.s0 = int(o.sub) - 32;
            s.s1 = 0;
        }
    }
    return s;
}

// Token t's Q8_0 block j: codes, scale, code sum and (Q6_K) the first half's sum.
struct KqX {
    u32x4 x0, x1;
    float dx;
    int sum, half;
};

template <int FMT>
__device__ __forceinline__ KqX kq_xblock(const int8_t* xq, const uint16_t* xd, const int32_t* xs, int64_t t,
                                         int k, int nb, uint32_t j) {
    KqX b;
    const int8_t* p = (xq + t * k) + 32u * j;
    b.x0 = ld16(p);
    b.x1 = ld16(p + 16);
    b.dx = f16_to_f32((xd + t * nb)[j]);
    b.sum = (xs + t * nb)[j];
    b.half = 0;
    if constexpr (FMT == QG_Q6_K) {
#pragma unroll
        for (int q = 0; q < 4; ++q) b.half = dot4_i8(0x01010101u, b.x0[q], b.half);
    }
    return b;
}

// acc + this block's contribution for one token.
template <int FMT>
__device__ __forceinline__ float kq_block(const uint32_t (&lo)[4], const uint32_t (&hi)[4], const KqScale& s,
                                          const KqX& x, float acc) {
    if constexpr (FMT == QG_Q6_K) {
        int ia = 0, ib = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ia = dot4_i8(lo[q], x.x0[q], ia);
            ib = dot4_i8(hi[q], x.x1[q], ib);
        }
        ia -= 32 * x.half;
        ib -= 32 * (x.sum - x.half);
        const int v = s.s0 * ia + s.s1 * ib;  // |v| < 2^24: exact in fp32
        return fmaf(s.a * x.dx, float(v), acc);
    } else {
        int isum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            isum = dot4_i8(lo[q], x.x0[q], isum);
            isum = dot4_i8(hi[q], x.x1[q], isum);
        }
        if constexpr (FMT == QG_IQ4_XS) {
            return fmaf(s.a * x.dx, float(s.s0 * isum), acc);
        } else {
            const float v = fmaf(s.a, float(isum), -(s.b * float(x.sum)));
            return fmaf(x.dx, v, acc);
        }
    }
}

template <int FMT, int R, int MT, int G, int C>
__global__ __launch_bounds__(kBlock) void k_gemv_kquant(const uint8_t* __restrict__ w, int64_t soff, int n, int k,
                                                        const int8_t* __restrict__ xq,
                                                        const uint16_t* __restrict__ xd,
                                                        const int32_t* __restrict__ xs, int m,
                                                        float* __restrict__ y) {
    constexpr int kGroups = kWave / G;
    const int lane = lane_id();
    const int grp = G == kWave ? 0 : lane / G;
    const int l = G == kWave ? lane : lane % G;
    const int wave = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * (kBlock / kWave) + int(threadIdx.x) / kWave);
    const int unit = wave * kGroups + grp;
    const int64_t crow = code_row_bytes(FMT, k), srow = scale_row_bytes(FMT, k);
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
        // All loads of the R*C blocks first, at a clamped (valid) block index;
        // lanes whose block lies past the row end keep their sums unchanged.
        KqRaw raw[C][R];
        bool okc[C];
        uint32_t jc[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int j = c * G + l;
            okc[c] = j < nb;
            jc[c] = okc[c] ? uint32_t(j) : 0u;
#pragma unroll
            for (int r = 0; r < R; ++r) raw[c][r] = kq_load<FMT>(codes[r], scales[r], k, jc[c]);
        }
        constexpr int TB = MT < 4 ? MT : 4;
#pragma unroll
        for (int tb = 0; tb < MT; tb += TB) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                KqX xb[TB];
#pragma unroll
                for (int t = 0; t < TB; ++t) xb[t] = kq_xblock<FMT>(xq, xd, xs, tok[tb + t], k, nb, jc[c]);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    uint32_t lo[4], hi[4];
                    kq_codes<FMT>(raw[c][r], lo, hi);
                    const KqScale s = kq_scale<FMT>(raw[c][r]);
#pragma unroll
                    for (int t = 0; t < TB; ++t) {
                        const float v = kq_block<FMT>(lo, hi, s, xb[t], acc[r][tb + t]);
                        acc[r][tb + t] = okc[c] ? v : acc[r][tb + t];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        for (int j = l; j < nb; j += G) {
            KqRaw raw[R];
#pragma unroll
            for (int r = 0; r < R; ++r) raw[r] = kq_load<FMT>(codes[r], scales[r], k, uint32_t(j));
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < m) {
                    const KqX xb = kq_xblock<FMT>(xq, xd, xs, t, k, nb, uint32_t(j));
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        uint32_t lo[4], hi[4];
                        kq_codes<FMT>(raw[r], lo, hi);
                        acc[r][t] = kq_block<FMT>(lo, hi, kq_scale<FMT>(raw[r]), xb, acc[r][t]);
                    }
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

// Verification dequantizer: one thread per 32-element block, the GEMV's own
// code rebuild, values rounded once to fp32.
template <int FMT>
__global__ __launch_bounds__(kBlock) void k_dequant_kquant(const uint8_t* __restrict__ w, int64_t soff, int n,
                                                           int k, float* __restrict__ out) {
    const int64_t nb = k / 32;
    const int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= int64_t(n) * nb) return;
    const int64_t row = i / nb;
    const uint32_t j = uint32_t(i % nb);
    const KqRaw raw = kq_load<FMT>(w + row * code_row_bytes(FMT, k), w + soff + row * scale_row_bytes(FMT, k), k, j);
    uint32_t lo[4], hi[4];
    kq_codes<FMT>(raw, lo, hi);
    const KqScale s = kq_scale<FMT>(raw);
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int e0 = 4 * q + b, e1 = 16 + 4 * q + b;
            if constexpr (FMT == QG_Q4_K || FMT == QG_Q5_K) {
                v[e0] = fmaf(s.a, float((lo[q] >> (8 * b)) & 0xFFu), -s.b);
                v[e1] = fmaf(s.a, float((hi[q] >> (8 * b)) & 0xFFu), -s.b);
            } else if constexpr (FMT == QG_Q6_K) {
                v[e0] = s.a * float(s.s0 * (int((lo[q] >> (8 * b)) & 0xFFu) - 32));
                v[e1] = s.a * float(s.s1 * (int((hi[q] >> (8 * b)) & 0xFFu) - 32));
            } else {
                v[e0] = s.a * float(s.s0 * int(int8_t(lo[q] >> (8 * b))));
                v[e1] = s.a * float(s.s0 * int(int8_t(hi[q] >> (8 * b))));
            }
        }
    float4* o = reinterpret_cast<float4*>(out + row * k + 32 * int64_t(j));
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = float4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
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

template <int FMT, int G, int C, int MT>
hipError_t go(const Args& A, hipStream_t s) {
    if constexpr (MT >= 16 && C > 4) {
        return go<FMT, G, 0, MT>(A, s);
    } else {
        constexpr int R = rows_per_group(C, MT);
        const int64_t units = (int64_t(A.n) + R - 1) / R;
        const int64_t per_block = (kBlock / kWave) * (kWave / G);
        const dim3 grid(unsigned((units + per_block - 1) / per_block));
        hipLaunchKernelGGL((k_gemv_kquant<FMT, R, MT, G, C>), grid, dim3(kBlock), 0, s, A.w, A.soff, A.n, A.k,
                           A.xq, A.xd, A.xs, A.m, A.y);
        return hipGetLastError();
    }
}

template <int FMT, int G, int MT>
hipError_t by_chunks(const Args& A, hipStream_t s) {
    const int C = chunks_per_lane(A.k / 32, G);
    if constexpr (G == 16) {
        switch (C) {
            case 1: return go<FMT, 16, 1, MT>(A, s);
            case 2: return go<FMT, 16, 2, MT>(A, s);
            case 3: return go<FMT, 16, 3, MT>(A, s);
            default: return go<FMT, 16, 4, MT>(A, s);
        }
    } else {
        switch (C) {
            case 1: return go<FMT, 64, 1, MT>(A, s);
            case 2: return go<FMT, 64, 2, MT>(A, s);
            case 3: return go<FMT, 64, 3, MT>(A, s);
            case 4: return go<FMT, 64, 4, MT>(A, s);
            case 6: return go<FMT, 64, 6, MT>(A, s);
            case 8: return go<FMT, 64, 8, MT>(A, s);
            default: return go<FMT, 64, 0, MT>(A, s);
        }
    }
}

template <int FMT>
hipError_t by_tokens(const Args& A, hipStream_t s) {
    const bool wide = lanes_per_row(A.k / 32) == 64;
    switch (token_class(A.m)) {
        case 1: return wide ? by_chunks<FMT, 64, 1>(A, s) : by_chunks<FMT, 16, 1>(A, s);
        case 4: return wide ? by_chunks<FMT, 64, 4>(A, s) : by_chunks<FMT, 16, 4>(A, s);
        default: return wide ? by_chunks<FMT, 64, 16>(A, s) : by_chunks<FMT, 16, 16>(A, s);
    }
}

template <int FMT>
hipError_t dequant(const uint8_t* w, int64_t n, int64_t k, float* out, hipStream_t s) {
    const int64_t blocks = n * (k / 32);
    hipLaunchKernelGGL(k_dequant_kquant<FMT>, dim3(unsigned((blocks + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
                       w, scale_plane_offset(FMT, n, k), int(n), int(k), out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_kquant_a8(int fmt, const uint8_t* w, int64_t n, int64_t k, const int8_t* xq,
                                 const uint16_t* xd, const int32_t* xs, int m, float* y, hipStream_t s) {
    const Args A{w, scale_plane_offset(fmt, n, k), int(n), int(k), xq, xd, xs, m, y};
    switch (fmt) {
        case QG_Q4_K: return by_tokens<QG_Q4_K>(A, s);
        case QG_Q5_K: return by_tokens<QG_Q5_K>(A, s);
        case QG_Q6_K: return by_tokens<QG_Q6_K>(A, s);
        default: return by_tokens<QG_IQ4_XS>(A, s);
    }
}

hipError_t launch_dequant_kquant(int fmt, const uint8_t* w, int64_t n, int64_t k, float* out, hipStream_t s) {
    switch (fmt) {
        case QG_Q4_K: return dequant<QG_Q4_K>(w, n, k, out, s);
        case QG_Q5_K: return dequant<QG_Q5_K>(w, n, k, out, s);
        case QG_Q6_K: return dequant<QG_Q6_K>(w, n, k, out, s);
        default: return dequant<QG_IQ4_XS>(w, n, k, out, s);
    }
}

}  // namespace qg
