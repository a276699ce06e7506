// Dense NVFP4 x bf16 GEMV for gfx950 (wave64), plain or with the SwiGLU
// epilogue of a fused gate+up projection.
//
// The decode step streams every weight byte once, so its speed limit is HBM
// bandwidth (memra README, known gaps), and the kernel is shaped around
// streaming:
//  * a group of G lanes (G = 64, or 16 for rows shorter than 2048 elements)
//    owns R rows; each lane loads 16-byte code chunks c*G + l, c < C, so one
//    wave-wide load reads 1 KB of a row contiguously (non-temporal);
//  * all R*C code and scale loads are issued before any arithmetic (about
//    8 KB of weights in flight per wave);
//  * E2M1 pairs are widened to bf16 by v_cvt_scalef32_pk_bf16_fp4 and
//    multiplied into fp32 by v_dot2_f32_bf16; each 16-element block's sum is
//    scaled once by its E4M3 scale, the row sum once by the tensor scale;
//  * per-lane sums are combined by a fixed DPP/swizzle butterfly.
// The chunk-to-lane mapping and the reduction order depend only on k, so
// results are bitwise identical for any token count, grid or schedule.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "qg_device.hpp"
#include "qg_gemv_core.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"
#include "qg_mfma.hpp"
#include "qg_reduce.hpp"

namespace qg {

namespace {

constexpr int kBlock = 256;  // threads per workgroup (4 waves)

// Streaming kernel shape, measured on MI355X over rows per unit R in
// {1, 2, 4, 8} and units per wave in {1, 2, 4, 8}: four rows per unit for
// short rows (8 KB of codes per wave at k = 4096), two for long rows (12 KB
// at k = 12288), one unit per wave.
template <int C>
constexpr int kStreamRows = C <= 2 ? 4 : 2;
// Activations staged in LDS once per workgroup (rather than loaded by every
// lane from L1/L2) for rows of three or more chunks per lane that fill every
// lane's chunk slots (k == 2048 * C; other rows keep the per-lane loads): measured on
// MI355X, the 4096 x 12288 down projection went from 7.35 to 6.9 us, while
// at two chunks per lane (4096-element rows) the staging's extra registers
// cost occupancy and time.
template <int G, int C>
constexpr bool kStreamLdsX = G == kWave && C >= 3;
// Two to four tokens: activations staged in LDS for full rows of one or an
// even number of chunks per lane, in passes of two chunks (32 KB of LDS at
// four tokens).
template <int G, int C, int MT>
constexpr bool kMultiLdsX = G == kWave && MT == 4 && (C == 1 || (C > 0 && C % 2 == 0));

// SWIGLU: the matrix is packed with gate/up rows interleaved (packed row 2i =
// gate i, 2i+1 = up i), so the R consecutive rows of a group are RA = R/2
// (gate, up) pairs; the epilogue writes a = bf16(silu(g) * u) (and optionally
// g, u into h).  nout is n (plain) or inter (SwiGLU).
template <int R, int MT, int G, int C, bool SWIGLU, bool LDSX = false, int NT = kBlock>
__global__ __launch_bounds__(NT) void k_gemv_nvfp4(const uint8_t* __restrict__ w, int64_t soff,
                                                       float s_t, int nout, int k,
                                                       const uint16_t* __restrict__ x, int m,
                                                       float* __restrict__ y,
                                                       uint16_t* __restrict__ a,
                                                       float* __restrict__ h) {
    constexpr int kGroups = kWave / G;
    const int lane = lane_id();
    const int grp = G == kWave ? 0 : lane / G;  // one group per wave: rows are wave-uniform
    const int l = G == kWave ? lane : lane % G;
    const int wave = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * (NT / kWave) + int(threadIdx.x) / kWave);
    const int unit = wave * kGroups + grp;
    const int64_t crow = k / 2, srow = k / 16;

    // SwiGLU matrices are packed with gate/up rows interleaved, so in both
    // modes a group's R rows are consecutive packed rows.
    const int nrows = SWIGLU ? 2 * nout : nout;
    int rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = min(unit * R + r, nrows - 1);
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

    if constexpr (LDSX) {
        // Two to four tokens over rows that fill every lane's chunk slots
        // (k == 32 * C * G): the MT token slots' activations are staged in
        // LDS once per workgroup instead of being read by every wave through
        // L1 (4 tokens bring 64 bytes per lane per chunk, more than the
        // weights).  Long rows go in passes of PC chunks (32 KB of LDS at
        // four tokens); the next pass's activations are loaded into
        // registers while the current pass is computed.  Same loads and
        // arithmetic per (row, token) as nvfp4_partial, so the sums are
        // bitwise the same.
        static_assert(G == kWave && MT <= 4 && C > 0, "one token block over full rows");
        constexpr int PC = C < 2 ? C : 2;  // chunks per pass
        constexpr int NP = C / PC;
        static_assert(NP * PC == C, "whole passes");
        constexpr int kU = PC * 256;  // 16-byte units of one token's activations per pass
        constexpr int PQ = kU / NT;   // of which each thread stages PQ
        static_assert(PQ * NT == kU, "whole staging loads per thread");
        __shared__ u32x4 xs[MT * kU];
        const int tid = int(threadIdx.x);
        u32x4 xg[MT][PQ];
        auto xload = [&](int pass) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int q = 0; q < PQ; ++q) xg[t][q] = ld16(xp[t] + 8u * (pass * kU + tid + NT * q));
        };
        // piece p of pass-chunk j of token t at slot t*kU + 4j + ((p + j/2) & 3):
        // conflict-free for the staging stores and the per-lane reads
        auto xstore = [&]() {
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int q = 0; q < PQ; ++q) {
                    const uint32_t u = uint32_t(tid + NT * q);
                    xs[t * kU + 4 * (u >> 2) + (((u & 3u) + (u >> 3)) & 3u)] = xg[t][q];
                }
        };
        xload(0);
        u32x4 cw[C][R];
        uint32_t sw[C][R];
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t j = uint32_t(c * G + l);
                cw[c][r] = ld_stream16(codes[r] + 16u * j);
                sw[c][r] = ld<uint16_t>(scales[r] + 2u * j);
            }
        __builtin_amdgcn_sched_barrier(0);
        xstore();
        lds_barrier();
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
            if (pass + 1 < NP) xload(pass + 1);
#pragma unroll
            for (int cc = 0; cc < PC; ++cc) {
                const int c = pass * PC + cc;
                const uint32_t jl = uint32_t(cc * G + l);  // chunk within the pass
                u32x4 xv[MT][4];
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xv[t][i] = xs[t * kU + 4 * jl + ((uint32_t(i) + (jl >> 1)) & 3u)];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    bf16x2 d[16];
                    nvfp4_decode_chunk(cw[c][r], d);
                    const float s0 = e4m3_to_f32<0>(sw[c][r]), s1 = e4m3_to_f32<1>(sw[c][r]);
#pragma unroll
                    for (int t = 0; t < MT; ++t) acc[r][t] = nvfp4_chunk_dot_decoded(d, s0, s1, xv[t], acc[r][t]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (pass + 1 < NP) {
                lds_barrier();  // every wave is done with this pass's activations
                xstore();
                lds_barrier();
            }
        }
    } else {
        nvfp4_partial<R, MT, G, C>(codes, scales, xp, m, k / 32, l, acc);
    }

    if constexpr (G == kWave && ((R * MT) & (R * MT - 1)) == 0 && R * MT <= 64) {
        // Reduce-scatter: lane l ends with (row, token) index bitrev(l % N),
        // index = row * MT + token.  For SwiGLU the up row of the same token
        // is MT indices further, i.e. the lane ^ bitrev(MT).
        constexpr int N = R * MT, L = log2i(N);
        float flat[N];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < MT; ++t) flat[r * MT + t] = acc[r][t];
        const float v = reduce_scatter64<N>(flat) * s_t;
        const int idx = bitrev<L>(lane & (N - 1));
        const int r = idx / MT, t = idx % MT;
        if constexpr (!SWIGLU) {
            const int row = unit * R + r;
            if (lane < N && t < m && row < nout) y[int64_t(t) * nout + row] = v;
        } else {
            constexpr int XU = 1 << (L - 1 - log2i(MT));  // bitrev(MT)
            const float other = xor_lane<XU>(v);
            const int i = unit * (R / 2) + r / 2;  // the a-row
            if (lane < N && (lane & XU) == 0 && t < m && i < nout) {
                const float g = v, u = other;
                a[int64_t(t) * nout + i] = uint16_t(f32_to_bf16_rne(g / (1.0f + expf(-g)) * u));
                if (h) {
                    h[int64_t(t) * 2 * nout + i] = g;
                    h[int64_t(t) * 2 * nout + nout + i] = u;
                }
            }
        }
        return;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = group_sum<G>(acc[r][t]) * s_t;

    if constexpr (!SWIGLU) {
        if (l != 0) return;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = unit * R + r;
            if (row >= nout) break;
#pragma unroll
            for (int t = 0; t < MT; ++t)
                if (t < m) y[int64_t(t) * nout + row] = acc[r][t];
        }
    } else {
        // Every lane of the group holds every sum: lane l evaluates the
        // SwiGLU of (a-row l / MT, token l % MT), so the RA * MT exponentials
        // run side by side instead of one after another on lane 0.
        constexpr int RA = R / 2;
        static_assert(RA * MT <= G, "one (a-row, token) per lane");
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int r = 0; r < RA; ++r)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                if (l == r * MT + t) {
                    g = acc[2 * r][t];
                    u = acc[2 * r + 1][t];
                }
        const int r = l / MT, t = l % MT;
        const int i = unit * RA + r;
        if (l < RA * MT && t < m && i < nout) {
            const float act = g / (1.0f + expf(-g)) * u;
            a[int64_t(t) * nout + i] = uint16_t(f32_to_bf16_rne(act));
            if (h) {
                h[int64_t(t) * 2 * nout + i] = g;
                h[int64_t(t) * 2 * nout + nout + i] = u;
            }
        }
    }
}

// One-token streaming variant: one unit (R rows per lane group) per wave,
// every code and scale load of the unit issued before any arithmetic, and the
// lane's activation chunks loaded once (a lane always covers the same k
// range).  Same per-row arithmetic and reduction order as k_gemv_nvfp4.
// (Two to eight units per wave in a straight-line register pipeline were
// measured on MI355X and were slower: 13.2-15.4 us against 11.6 us for the
// 24576 x 4096 gate+up.)
template <int R, int G, int C, bool SWIGLU, bool LDSX>
__global__ __launch_bounds__(kBlock) void k_gemv_nvfp4_stream(const uint8_t* __restrict__ w, int64_t soff,
                                                              float s_t, int nout, int k,
                                                              const uint16_t* __restrict__ x,
                                                              float* __restrict__ y,
                                                              uint16_t* __restrict__ a,
                                                              float* __restrict__ h, int n_wunits) {
    constexpr int kGroups = kWave / G;
    constexpr int kPer = SWIGLU ? R / 2 : R;  // output rows per group per unit
    const int lane = lane_id();
    const int grp = G == kWave ? 0 : lane / G;  // one group per wave: rows are wave-uniform
    const int l = G == kWave ? lane : lane % G;
    // wave-uniform, kept in a scalar register
    const int wave = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * (kBlock / kWave) + int(threadIdx.x) / kWave);
    const int64_t crow = k / 2, srow = k / 16;
    const int nchunks = k / 32;

    // Lanes whose chunk c lies past the end of a row load chunk 0 instead (a
    // valid address) and drop the result.  The LDSX instances are launched
    // only for rows that fill every chunk slot (k == 32 * C * G).
    bool okc[C];
    uint32_t jc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int j = c * G + l;
        okc[c] = LDSX || j < nchunks;
        jc[c] = okc[c] ? uint32_t(j) : 0u;
    }
    // Activations: per lane from global memory (its C chunks, 64 bytes
    // each), or with LDSX staged once per workgroup in LDS, which saves the
    // four waves' repeated L1 traffic on long rows.  Piece p of chunk j sits
    // at slot 4j + ((p + j/2) & 3): the eight lanes of one 128-byte LDS cycle
    // (consecutive j) then hit distinct banks, for the reads below and for
    // the staging stores.
    __shared__ u32x4 xs[LDSX ? C * 256 : 1];
    u32x4 xv[C][4];
    u32x4 xg[LDSX ? C : 1];
    if constexpr (LDSX) {
#pragma unroll
        for (int s = 0; s < C; ++s) xg[s] = ld16(x + 8u * (threadIdx.x + kBlock * s));
    } else {
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[c][i] = ld16(x + 32u * jc[c] + 8u * i);
    }

    const int nrows = SWIGLU ? 2 * nout : nout;  // packed rows (gate/up interleaved)
    const int wunit = min(wave, n_wunits - 1);    // a clamped wave stores nothing
    const int unit = wunit * kGroups + grp;
    u32x4 cw[C][R];
    uint32_t sw[C][R];
    {
        const uint8_t* cp[R];
        const uint8_t* sp[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = min(unit * R + r, nrows - 1);
            cp[r] = w + row * crow;
            sp[r] = w + soff + row * srow;
        }
        // row by row, or (LDSX) chunk by chunk across the rows
#pragma unroll
        for (int q = 0; q < R * C; ++q) {
            const int r = LDSX ? q % R : q / C, c = LDSX ? q / R : q % C;
            cw[c][r] = ld_stream16(cp[r] + 16u * jc[c]);
            sw[c][r] = ld<uint16_t>(sp[r] + 2u * jc[c]);
        }
    }
    if constexpr (LDSX) {
        // The x loads were issued before the weights, so the stores wait for
        // them only; the scheduling barrier keeps any decode of the weights
        // from being moved above the workgroup barrier (which would make that
        // barrier wait for every weight load).
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < C; ++s) {
            const uint32_t u = threadIdx.x + kBlock * s;
            xs[4 * (u >> 2) + (((u & 3u) + (u >> 3)) & 3u)] = xg[s];
        }
        lds_barrier();
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[c][i] = xs[4 * jc[c] + ((uint32_t(i) + (jc[c] >> 1)) & 3u)];
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool store = wave < n_wunits;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = nvfp4_chunk_dot(cw[c][r], sw[c][r], xv[c], acc[r]);
            acc[r] = okc[c] ? v : acc[r];
        }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = group_sum<G>(acc[r]) * s_t;
    if constexpr (!SWIGLU) {
        if (store && l == 0) {
#pragma unroll
            for (int r = 0; r < kPer; ++r) {
                const int i = unit * kPer + r;
                if (i < nout) y[i] = acc[r];
            }
        }
    } else {
        // lane l of the group evaluates the SwiGLU of its a-row l
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int r = 0; r < kPer; ++r)
            if (l == r) {
                g = acc[2 * r];
                u = acc[2 * r + 1];
            }
        const int i = unit * kPer + l;
        if (store && l < kPer && i < nout) {
            a[i] = uint16_t(f32_to_bf16_rne(g / (1.0f + expf(-g)) * u));
            if (h) {
                h[i] = g;
                h[nout + i] = u;
            }
        }
    }
}

struct Args {
    const uint8_t* w;
    int64_t soff;
    float s_t;
    int nout, k;
    const uint16_t* x;
    int m;
    float* y;
    uint16_t* a;
    float* h;
};

template <int G, int C, bool SW>
hipError_t go_stream(const Args& A, hipStream_t s) {
    constexpr int R0 = kStreamRows<C>;
    constexpr int R = SW ? (R0 < 2 ? 2 : R0) : R0;
    constexpr int per_unit = SW ? R / 2 : R;
    const int64_t units = (int64_t(A.nout) + per_unit - 1) / per_unit;
    const int64_t wunits = (units + (kWave / G) - 1) / (kWave / G);
    const dim3 grid(unsigned((wunits + kBlock / kWave - 1) / (kBlock / kWave)));
    if (kStreamLdsX<G, C> && A.k == 32 * C * G)
        hipLaunchKernelGGL((k_gemv_nvfp4_stream<R, G, C, SW, true>), grid, dim3(kBlock), 0, s, A.w, A.soff,
                           A.s_t, A.nout, A.k, A.x, A.y, A.a, A.h, int(wunits));
    else
        hipLaunchKernelGGL((k_gemv_nvfp4_stream<R, G, C, SW, false>), grid, dim3(kBlock), 0, s, A.w, A.soff,
                           A.s_t, A.nout, A.k, A.x, A.y, A.a, A.h, int(wunits));
    return hipGetLastError();
}

template <int G, int C, int MT, bool SW>
hipError_t go(const Args& A, hipStream_t s) {
    if constexpr (MT == 1 && C > 0 && C <= 6) {
        if (kernel_policy() != QG_KERNEL_GENERIC) return go_stream<G, C, SW>(A, s);
    }
    if constexpr (MT >= 16 && C > 4) {
        // 16 tokens over long rows: the all-loads-first form does not fit in
        // registers; use the chunk loop.
        return go<G, 0, MT, SW>(A, s);
    } else {
        constexpr int R0 = rows_per_group(C, MT);
        constexpr int R = SW ? (R0 < 2 ? 2 : R0) : R0;
        constexpr int per_unit = SW ? R / 2 : R;
        const int64_t units = (int64_t(A.nout) + per_unit - 1) / per_unit;
        if (kMultiLdsX<G, C, MT> && A.k == 32 * C * G) {
            // Rows of six or more chunks per lane: eight waves share one
            // staging of the activations (one 16-byte load per thread and
            // token per pass), which halves the L2 -> LDS activation reads;
            // these kernels hold two waves per SIMD either way.  Shorter
            // rows keep four-wave workgroups: there the wider workgroup
            // costs a resident wave per SIMD (batch-4 12288 x 4096 down
            // 13.2 -> 12.6 us; the 24576 x 4096 gate+up would go 15.7 -> 19 us).
            constexpr int NT = C % 2 == 0 && C >= 6 ? 2 * kBlock : kBlock;
            const int64_t per_block = (NT / kWave) * (kWave / G);
            const dim3 grid(unsigned((units + per_block - 1) / per_block));
            hipLaunchKernelGGL((k_gemv_nvfp4<R, MT, G, C, SW, kMultiLdsX<G, C, MT>, NT>), grid, dim3(NT), 0, s,
                               A.w, A.soff, A.s_t, A.nout, A.k, A.x, A.m, A.y, A.a, A.h);
        } else {
            const int64_t per_block = (kBlock / kWave) * (kWave / G);
            const dim3 grid(unsigned((units + per_block - 1) / per_block));
            hipLaunchKernelGGL((k_gemv_nvfp4<R, MT, G, C, SW>), grid, dim3(kBlock), 0, s, A.w, A.soff, A.s_t,
                               A.nout, A.k, A.x, A.m, A.y, A.a, A.h);
        }
        return hipGetLastError();
    }
}

template <int G, int MT, bool SW>
hipError_t by_chunks(const Args& A, hipStream_t s) {
    const int C = chunks_per_lane(A.k / 32, G);
    if constexpr (G == 16) {
        switch (C) {  // rows of fewer than 64 chunks: C <= 4
            case 1: return go<16, 1, MT, SW>(A, s);
            case 2: return go<16, 2, MT, SW>(A, s);
            case 3: return go<16, 3, MT, SW>(A, s);
            default: return go<16, 4, MT, SW>(A, s);
        }
    } else {
        switch (C) {
            case 1: return go<64, 1, MT, SW>(A, s);
            case 2: return go<64, 2, MT, SW>(A, s);
            case 3: return go<64, 3, MT, SW>(A, s);
            case 4: return go<64, 4, MT, SW>(A, s);
            case 6: return go<64, 6, MT, SW>(A, s);
            case 8: return go<64, 8, MT, SW>(A, s);
            default: return go<64, 0, MT, SW>(A, s);
        }
    }
}

template <bool SW>
hipError_t dispatch(const Args& A, hipStream_t s) {
    const bool wide = lanes_per_row(A.k / 32) == 64;
    switch (token_class(A.m)) {
        case 1: return wide ? by_chunks<64, 1, SW>(A, s) : by_chunks<16, 1, SW>(A, s);
        case 4: return wide ? by_chunks<64, 4, SW>(A, s) : by_chunks<16, 4, SW>(A, s);
        default: return wide ? by_chunks<64, 16, SW>(A, s) : by_chunks<16, 16, SW>(A, s);
    }
}

}  // namespace

hipError_t launch_gemv_nvfp4(const uint8_t* w, float s_t, int64_t n, int64_t k, const uint16_t* x,
                             int m, float* y, hipStream_t s) {
    const Args A{w, scale_plane_offset(QG_NVFP4, n, k), s_t, int(n), int(k), x, m, y, nullptr, nullptr};
    return dispatch<false>(A, s);
}

hipError_t launch_gemv_nvfp4_swiglu(const uint8_t* w, float s_t, int64_t inter, int64_t k,
                                    const uint16_t* x, int m, uint16_t* a, float* h, hipStream_t s) {
    const Args A{w, scale_plane_offset(QG_NVFP4, 2 * inter, k), s_t, int(inter), int(k), x, m, nullptr, a, h};
    return dispatch<true>(A, s);
}

}  // namespace qg
