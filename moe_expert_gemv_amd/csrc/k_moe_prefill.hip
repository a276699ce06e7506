// MoE over many tokens (prefill) on gfx950 matrix cores: route, group the
// (token, expert) pairs expert-major, grouped gate/up GEMM with the SwiGLU
// epilogue, grouped down GEMM, weighted combine.
//
// The LumenLLM README prefills its MoE models with a grouped NVFP4 MoE GEMM
// on tensor cores (feature list "Kernels"); the bw24 README groups routed
// pairs expert-major so each active expert's weights are read once for all
// its tokens (MoE feature entry).  Same layer and same results definition as
// the decode path (k_moe.hip), for any token count:
//   1. routing: k_route_topk, one wave per token;
//   2. grouping: k_mpf_place counts each expert's pairs and writes the
//      expert-major CSR (active experts ascending, then the shared expert;
//      inside an expert, pairs in (token, slot) order -- a stable placement,
//      so the CSR is exactly the decode path's) and the tile table of the
//      GEMMs (kPfPairs pairs per tile);
//   3. k_mpf_gemm<SWIGLU>: one workgroup per (tile, block of 256 weight
//      rows): the tile's activation rows are gathered into LDS (in passes of
//      512 k), the expert's NVFP4 rows decoded straight into MFMA fragments
//      (eight waves, each on 32 rows over the whole k range, one MFMA chain
//      per output); gate/up rows are interleaved, so SwiGLU pairs adjacent
//      columns;
//   4. k_mpf_combine: y = sum over slots of w * o, then + o_shared, in that
//      order (the decode path's order).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "qg_device.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"
#include "qg_mfma.hpp"

namespace qg {

namespace {

constexpr int kPfPairs = 32;    // pairs per GEMM tile (two 16-row MFMA blocks)
constexpr int kPfBlock = 512;   // GEMM workgroup: eight waves
constexpr int kPfNB = 2;        // 16-row weight blocks per wave
constexpr int kPfBN = 16 * kPfNB * (kPfBlock / 64);  // weight rows per GEMM workgroup: 256
// Workgroups are dealt to the XCDs round-robin by launch index, and each XCD
// has an L2 of its own; the GEMM grid is remapped so that neighbouring work
// items (the row blocks of one tile, which gather the same activation rows)
// run one after another on the same XCD.  Results do not depend on it.
constexpr int kXcds = 8;

constexpr int kGroupThreads = 256;  // placement workgroups
constexpr int kPfMaxExperts = 1024;  // routed experts of a prefill call, at most
constexpr int kIdsPerPass = 4 * kGroupThreads;  // ids a workgroup reads per pass (four per thread)
constexpr int kKeep = 4;  // passes of ids the placement keeps in registers

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Sum of v over the workgroup, returned to every thread.
__device__ __forceinline__ int block_sum_i(int v, int* s_tmp) {
    v = wave_sum_i(v);
    const int wave = int(threadIdx.x) / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[wave] = v;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int w = 0; w < kGroupThreads / kWave; ++w) r += s_tmp[w];
    return r;
}

// Exclusive prefix of v over the workgroup's threads (in thread order); the
// total goes to *total.
__device__ __forceinline__ int block_exclusive_i(int v, int* s_tmp, int* total) {
    const int lane = int(threadIdx.x) & (kWave - 1), wave = int(threadIdx.x) / kWave;
    int inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(inc, o);
        if (lane >= o) inc += u;
    }
    __syncthreads();
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kGroupThreads / kWave; ++w) {
        const int c = s_tmp[w];
        before += w < wave ? c : 0;
        all += c;
    }
    *total = all;
    return before + inc - v;
}

// Four ids starting at i (i % 4 == 0); entries at or past pr read as -1.
__device__ __forceinline__ int4 ids4(const int32_t* __restrict__ ids, int i, int pr) {
    if (i + 3 < pr) return *reinterpret_cast<const int4*>(ids + i);
    int4 v{-1, -1, -1, -1};
    if (i < pr) v.x = ids[i];
    if (i + 1 < pr) v.y = ids[i + 1];
    if (i + 2 < pr) v.z = ids[i + 2];
    return v;
}

// Every workgroup first counts the routed pairs of every expert (an LDS
// histogram of the t*k ids, four per thread per pass); workgroup e < E then
// writes counts[e], places expert e's pairs in pair-index order and
// describes its tiles; workgroup E places the shared expert's (if any) and
// writes the end entries and the tile count.  tile_info[0].x is the tile
// count, entry 1 + i (expert, first pair, pair count, 0) describes tile i,
// so that a GEMM workgroup finds its tile with two loads.
__global__ __launch_bounds__(kGroupThreads) void k_mpf_place(const int32_t* __restrict__ ids, int t, int k, int E,
                                                             int has_shared, int32_t* __restrict__ counts,
                                                             MoeWorkspace ws, int32_t* __restrict__ tile_off,
                                                             int32_t* __restrict__ pair_pos,
                                                             int4* __restrict__ tile_info) {
    __shared__ int s_tmp[kGroupThreads / kWave];
    __shared__ int s_hist[kPfMaxExperts];
    const int e = int(blockIdx.x), tid = int(threadIdx.x);
    const int pr = t * k;
    for (int j = tid; j < E; j += kGroupThreads) s_hist[j] = 0;
    // The ids of the first kKeep passes stay in registers for the placement
    // below (the same four ids per thread and pass), which then reads only
    // the passes beyond them again.
    int4 kept[kKeep];
#pragma unroll
    for (int j = 0; j < kKeep; ++j) kept[j] = ids4(ids, 4 * tid + j * kIdsPerPass, pr);
    __syncthreads();
    auto count = [&](const int4& v) {
        const int id4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (id4[q] >= 0 && id4[q] < E) atomicAdd(&s_hist[id4[q]], 1);  // padding and stray ids skipped
    };
#pragma unroll
    for (int j = 0; j < kKeep; ++j) count(kept[j]);
    for (int i = 4 * tid + kKeep * kIdsPerPass; i < pr; i += kIdsPerPass) count(ids4(ids, i, pr));
    __syncthreads();
    int off = 0, grp = 0, tiles = 0;  // over the experts before e
    for (int j = tid; j < e; j += kGroupThreads) {
        const int c = s_hist[j];
        off += c;
        grp += int(c > 0);
        tiles += (c + kPfPairs - 1) / kPfPairs;
    }
    off = block_sum_i(off, s_tmp);
    grp = block_sum_i(grp, s_tmp);
    tiles = block_sum_i(tiles, s_tmp);
    if (e < E) {
        const int c = s_hist[e];
        if (tid == 0) counts[e] = c;
        if (c == 0) return;  // uniform
        if (tid == 0) {
            ws.experts[grp] = e;
            ws.offsets[grp] = off;
            tile_off[grp] = tiles;
        }
        for (int j = tid; j * kPfPairs < c; j += kGroupThreads)
            tile_info[1 + tiles + j] = int4{e, off + j * kPfPairs, min(kPfPairs, c - j * kPfPairs), 0};
        int base = off;
        auto place = [&](const int4& v, int i) {  // one pass: ids i .. i + 3 of this thread
            const int hit[4] = {int(v.x == e), int(v.y == e), int(v.z == e), int(v.w == e)};
            int total;
            int pos = base + block_exclusive_i(hit[0] + hit[1] + hit[2] + hit[3], s_tmp, &total);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (hit[q]) {
                    const int tok = (i + q) / k, sl = (i + q) % k;
                    ws.pair_tok[pos] = tok;
                    ws.pair_slot[pos] = sl;
                    pair_pos[tok * (k + 1) + sl] = pos;
                    ++pos;
                }
            base += total;
        };
#pragma unroll
        for (int j = 0; j < kKeep; ++j)
            if (j * kIdsPerPass < pr) place(kept[j], 4 * tid + j * kIdsPerPass);  // uniform
        for (int i0 = kKeep * kIdsPerPass; i0 < pr; i0 += kIdsPerPass)  // uniform trip count
            place(ids4(ids, i0 + 4 * tid, pr), i0 + 4 * tid);
    } else {
        int g = grp;
        if (has_shared) {
            if (tid == 0) {
                ws.experts[g] = E;
                ws.offsets[g] = pr;
                tile_off[g] = tiles;
            }
            for (int j = tid; j * kPfPairs < t; j += kGroupThreads)
                tile_info[1 + tiles + j] = int4{E, pr + j * kPfPairs, min(kPfPairs, t - j * kPfPairs), 0};
            for (int tok = tid; tok < t; tok += kGroupThreads) {
                ws.pair_tok[pr + tok] = tok;
                ws.pair_slot[pr + tok] = k;
                pair_pos[tok * (k + 1) + k] = pr + tok;
            }
            ++g;
            tiles += (t + kPfPairs - 1) / kPfPairs;
        }
        if (tid == 0) {
            ws.offsets[g] = pr + (has_shared ? t : 0);
            tile_off[g] = tiles;
            *ws.n_groups = g;
            tile_info[0] = int4{tiles, 0, 0, 0};
        }
    }
}

struct GemmArgs {
    const uint8_t* w;        // expert e's matrix at w + e * stride
    int64_t stride, soff;    // bytes per expert; scale plane offset inside a matrix
    const float* scale;      // per-expert tensor scales
    int n;                   // weight rows (2I packed gate/up, or H)
    const uint16_t* src;     // activation rows: x (gathered by token) or a (by pair)
    uint16_t* a_out;         // SwiGLU output [P][n/2] bf16
    float* h_out;            // nullable [P][n] (g then u)
    float* o_out;            // plain output [P][n] fp32
};

// Instances that may run half row blocks: the gate/up GEMMs over K >= 1024.
// (The down GEMM's many short items leave no thin last round to shorten, and
// at K = 512 the second code path would cost the gate/up GEMM a third
// resident workgroup per CU.)
template <int KS, bool SWIGLU>
constexpr bool kPfHalf = SWIGLU && KS >= 4;

// One tile of up to kPfPairs pairs of one expert x kPfBN weight rows, over
// K = 256 * KS.  SWIGLU: activations gathered by token, output a (and h);
// else activations are the pairs' own rows of a, output o.
template <int KS, bool SWIGLU>
__global__ __launch_bounds__(kPfBlock, 4) void k_mpf_gemm(GemmArgs A, MoeWorkspace ws,
                                                          const int4* __restrict__ tile_info, int n_blocks,
                                                          int max_tiles, int xcd_slots) {
    constexpr int K = 2 * KW * KS;          // reduction length
    constexpr int NS = K / KW;              // 128-k weight slabs
    constexpr int MB = kPfPairs / 16;
    // The tile's activations are gathered in passes of 512 k through the same
    // 32 KB of LDS, so two workgroups share a CU and one's gathers overlap
    // the other's weight stream.
    constexpr int KP = K < 512 ? K : 512;   // k per pass
    constexpr int NP = K / KP;              // passes
    constexpr int SPP = KP / KW;            // slabs per pass
    constexpr int CPR = KP / 8;             // 16-byte chunks per LDS row
    constexpr int NCP = kPfPairs * CPR / kPfBlock;  // activation chunks per thread per pass
    // weight slabs in flight per wave: with several activation passes one
    // (each pass's activation loads return behind the weight requests
    // already out; at 512 tokens three slabs were 2.6 % slower for the whole
    // layer, two 0.5 %), with one pass four
    constexpr int WD = NP > 1 ? 1 : 4;
    static_assert(CPR >= 16 && (CPR & (CPR - 1)) == 0, "rows of a power-of-two count of 16 chunks");
    static_assert(K % KP == 0 && NCP * kPfBlock == kPfPairs * CPR && NS >= WD, "pass and slab shapes");
    __shared__ __attribute__((aligned(16))) uint16_t xs[kPfPairs * KP];
    // The item's weight scales: its rows are consecutive, so their scales are
    // one contiguous run of the scale plane, staged in LDS with the first
    // activation pass (rows padded by 16 bytes, so that the 16 rows of an MFMA
    // step spread over the banks) instead of one 2-byte load per slab.
    constexpr int SR = K / 16 + 16;                 // LDS bytes per row of scales
    constexpr int NSC = kPfBN * (K / 16) / 16 / kPfBlock;  // 16-byte pieces per thread
    static_assert(NSC >= 1 && NSC * 16 * kPfBlock == kPfBN * (K / 16), "scale run shape");
    __shared__ __attribute__((aligned(16))) uint8_t ss[kPfBN * SR];

    const int tid = int(threadIdx.x);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;

    // workgroup -> (tile ty, row block): workgroup b runs on XCD b % 8 as
    // that XCD's (b / 8)-th; tiles are dealt to the XCDs in turn, last tile
    // first (the shared expert's full tiles end the CSR, and the longest items
    // should start first), and an XCD takes every row block of a tile in a
    // row, so they share its L2.  Where an XCD's items would leave a last
    // round at most half as full as its xcd_slots resident workgroups (0: never),
    // its last tiles run as half row blocks (16 rows a wave), so that round
    // takes about half as long.  The tile's expert and pairs come from the
    // tile table.  The grid is sized for the worst case; the surplus
    // workgroups come last in launch order and exit.
    const int n_tiles = min(tile_info[0].x, max_tiles);
    const int xcd = int(blockIdx.x) % kXcds, xj = int(blockIdx.x) / kXcds;
    const int tx = n_tiles > xcd ? (n_tiles - xcd + kXcds - 1) / kXcds : 0;  // this XCD's tiles
    int qh = 0;                                                              // its tiles run as halves
    if (xcd_slots > 0 && tx * n_blocks > xcd_slots) {
        const int rem = tx * n_blocks % xcd_slots;
        if (rem > 0 && 2 * rem <= xcd_slots) qh = min(tx, (rem + n_blocks - 1) / n_blocks);
    }
    const int qf = tx - qh;
    const bool half = xj >= qf * n_blocks;
    const int q = half ? qf + (xj - qf * n_blocks) / (2 * n_blocks) : xj / n_blocks;
    const int blk = half ? (xj - qf * n_blocks) % (2 * n_blocks) : xj % n_blocks;
    if (q >= tx) return;
    const int ty = n_tiles - 1 - (xcd + kXcds * q);
    const int4 tinfo = tile_info[1 + ty];
    const int e = tinfo.x, p0 = tinfo.y, np = tinfo.z;  // np >= 1
    const uint8_t* w = A.w + int64_t(e) * A.stride;
    const float s_t = A.scale[e];

    // 1. activation rows into registers (rows past np repeat the last pair).
    // Each chunk's source (row and offset) is the same in every pass: found
    // once, so that a later pass's gather does not wait for the pair table.
    u32x4 xr[NCP];
    const uint16_t* xsrc[NCP];
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
        const int p = (wave + 8 * i) * kWave + lane;
        const int row = p / CPR, c = (p % CPR) ^ (row & 15);
        const int pos = p0 + min(row, np - 1);
        const int srow = SWIGLU ? ws.pair_tok[pos] : pos;
        xsrc[i] = A.src + int64_t(srow) * K + 8 * c;
    }
    auto x_load = [&](int pass) {
#pragma unroll
        for (int i = 0; i < NCP; ++i) xr[i] = ld16(xsrc[i] + pass * KP);
    };
    auto x_store = [&]() {
#pragma unroll
        for (int i = 0; i < NCP; ++i)
            *reinterpret_cast<u32x4*>(&xs[8 * ((wave + 8 * i) * kWave + lane)]) = xr[i];
    };
    x_load(0);
    const int item_rows = half ? kPfBN / 2 : kPfBN;
    const int row0 = blk * item_rows;  // the item's first weight row
    u32x4 sr[NSC];
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
        const int j = i * kPfBlock + tid;            // 16-byte piece of the run
        const int r = j / (K / 256), o = 16 * (j % (K / 256));
        const bool ok = r < item_rows && row0 + r < A.n;
        sr[i] = ok ? ld16(w + A.soff + int64_t(row0 + r) * (K / 16) + o) : u32x4{0u, 0u, 0u, 0u};
    }
    auto sc_store = [&]() {
#pragma unroll
        for (int i = 0; i < NSC; ++i) {
            const int j = i * kPfBlock + tid;
            const int r = j / (K / 256), o = 16 * (j % (K / 256));
            *reinterpret_cast<u32x4*>(&ss[r * SR + o]) = sr[i];
        }
    };
    __builtin_amdgcn_sched_barrier(0);

    // 2.-5. with NB 16-row blocks a wave: kPfNB, or 1 for half row blocks
    auto rows = [&](auto nb_c) {
        constexpr int NB = decltype(nb_c)::value;
        const int n0 = blk * (16 * NB * (kPfBlock / 64)) + wave * 16 * NB;  // this wave's first weight row
        // 2. weight slabs: slab s covers k = 128 s + [0, 128) of this wave's rows
        const uint8_t* wc[NB];
    #pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int64_t row = min(n0 + 16 * nb + lr, A.n - 1);
            wc[nb] = w + row * (K / 2);
        }
        auto w_load = [&](WStage<NB>& b, int sl) {  // codes only: the scales are in LDS
            const int kb = KW * sl + 32 * lg;
    #pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const u32x4 v = ld16(wc[nb] + kb / 2);  // fragment-shaped: ordinary loads (see k_prefill.hip)
    #pragma unroll
                for (int q = 0; q < 4; ++q) b.c[nb][q] = v[q];
            }
        };
        // one slab right behind the activation loads, the rest once the tile is
        // published (requested all up front, the weight stream delays the
        // activation data, which returns in order behind it)
        WStage<NB> wr[WD];
        w_load(wr[0], 0);
        __builtin_amdgcn_sched_barrier(0);

        // 3. publish the activation tile (the loads complete in order, ahead of
        // the weight loads; the LDS-only barrier leaves those in flight)
        x_store();
        sc_store();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
        for (int j = 1; j < WD; ++j) w_load(wr[j], j);
        __builtin_amdgcn_sched_barrier(0);

        // 4. one MFMA chain per output over the slabs in order
        floatx4 acc[MB][NB];
    #pragma unroll
        for (int i = 0; i < MB; ++i)
    #pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            if (NP > 1 && sl > 0 && sl % SPP == 0) {
                // next pass: every wave is done with the previous part of the
                // tile; gather the next part into the same space
                __builtin_amdgcn_sched_barrier(0);
                x_load(sl / SPP);
                lds_barrier();
                x_store();
                lds_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
            const WStage<NB> cur = wr[sl % WD];
            if (sl + WD < NS) w_load(wr[sl % WD], sl + WD);
            __builtin_amdgcn_sched_barrier(0);
            uint32_t scv[NB];  // this slab's two scale bytes of each row block
    #pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                scv[nb] = *reinterpret_cast<const uint16_t*>(
                    &ss[(wave * 16 * NB + 16 * nb + lr) * SR + (KW * sl + 32 * lg) / 16]);
    #pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4 bfr[NB];
    #pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const float sc = (q < 2) ? e4m3_to_f32<0>(scv[nb]) : e4m3_to_f32<1>(scv[nb]);
                    bfr[nb] = decode8_scaled(cur.c[nb][q], sc);
                }
                const int c = 16 * (sl % SPP) + 4 * lg + q;  // chunk within the pass
    #pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int row = 16 * mb + lr;
                    const u32x4 a = *reinterpret_cast<const u32x4*>(&xs[8 * (row * CPR + (c ^ (row & 15)))]);
    #pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_16x16x32_bf16(a, bfr[nb], acc[mb][nb]);
                }
            }
        }

        // 5. epilogue, per wave: tensor scale, then SwiGLU or the plain output
    #pragma unroll
        for (int mb = 0; mb < MB; ++mb)
    #pragma unroll
            for (int nb = 0; nb < NB; ++nb)
    #pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float sum = acc[mb][nb][v] * s_t;
                    const int row = 16 * mb + 4 * lg + v;  // pair of the tile
                    const int col = n0 + 16 * nb + lr;     // weight row
                    if constexpr (SWIGLU) {
                        // packed rows 2i (gate) and 2i+1 (up) sit in neighbouring lanes
                        const float other = __shfl_xor(sum, 1);
                        if ((lr & 1) == 0 && row < np && col < A.n) {
                            const int64_t pos = p0 + row;
                            const int I = A.n / 2, i = col / 2;
                            const float gv = sum, uv = other;
                            A.a_out[pos * I + i] = uint16_t(f32_to_bf16_rne(gv / (1.0f + expf(-gv)) * uv));
                            if (A.h_out) {
                                A.h_out[pos * 2 * I + i] = gv;
                                A.h_out[pos * 2 * I + I + i] = uv;
                            }
                        }
                    } else {
                        if (row < np && col < A.n) A.o_out[int64_t(p0 + row) * A.n + col] = sum;
                    }
                }
    };
    if constexpr (kPfHalf<KS, SWIGLU>) {
        if (half) {
            rows(std::integral_constant<int, 1>{});
            return;
        }
    }
    rows(std::integral_constant<int, kPfNB>{});
}

// y[t][h] = sum_s w[t][s] * o[pair (t, s)][h] (slots ascending), + o[pair
// (t, shared)][h].  Four outputs a thread (H is a multiple of 512), each
// pair row read with 16-byte loads, so a wave reads 1 KB runs; the sum of
// each output is the same chain as one output a thread.
constexpr int kCombineThreads = 256;
constexpr int kPfMaxTopK = 8;  // top_k of a MoE layer, at most
__global__ __launch_bounds__(kCombineThreads) void k_mpf_combine(const float* __restrict__ o,
                                                                 const float* __restrict__ wts,
                                                                 const int32_t* __restrict__ pair_pos, int k,
                                                                 int has_shared, int H, float* __restrict__ y) {
    const int tok = int(blockIdx.x);
    const int h = 4 * (int(blockIdx.y) * kCombineThreads + int(threadIdx.x));
    if (h >= H) return;
    // every row's load first (slots past k re-read slot k - 1; without a
    // shared expert its row is slot k - 1 too), then the sums in order
    const int32_t* pp = pair_pos + int64_t(tok) * (k + 1);
    floatx4 v[kPfMaxTopK + 1];
    float w[kPfMaxTopK];
#pragma unroll
    for (int s = 0; s < kPfMaxTopK; ++s) {
        const int sc = min(s, k - 1);
        v[s] = *reinterpret_cast<const floatx4*>(o + int64_t(pp[sc]) * H + h);
        w[s] = wts[int64_t(tok) * k + sc];
    }
    v[kPfMaxTopK] = *reinterpret_cast<const floatx4*>(o + int64_t(pp[has_shared ? k : k - 1]) * H + h);
    floatx4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kPfMaxTopK; ++s)
        if (s < k) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sum[j] = fmaf(w[s], v[s][j], sum[j]);
        }
    if (has_shared) {
#pragma unroll
        for (int j = 0; j < 4; ++j) sum[j] += v[kPfMaxTopK][j];
    }
    float* yo = y + int64_t(tok) * H + h;
#pragma unroll
    for (int j = 0; j < 4; ++j) yo[j] = sum[j];
}

template <int KS, bool SW>
hipError_t gemm(const GemmArgs& A, const MoeWorkspace& ws, const int4* tile_info, int max_tiles,
                hipStream_t s) {
    const int n_blocks = (A.n + kPfBN - 1) / kPfBN;
    // resident workgroups per XCD of this instance, for the half row blocks
    // (queried once per device)
    int xcd_slots = 0;
    if constexpr (kPfHalf<KS, SW>) {
        constexpr int kMaxDevices = 64;
        static std::atomic<int> cache[kMaxDevices];  // 0 = not yet queried
        int dev = 0;
        if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
        xcd_slots = dev >= 0 && dev < kMaxDevices ? cache[dev].load(std::memory_order_relaxed) : 0;
        if (xcd_slots == 0) {
            int cus = 0, per_cu = 0;
            if (hipError_t e = device_cu_count(&cus); e != hipSuccess) return e;
            if (hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_mpf_gemm<KS, SW>, kPfBlock, 0);
                e != hipSuccess)
                return e;
            xcd_slots = std::max(1, per_cu * cus / kXcds);
            if (dev >= 0 && dev < kMaxDevices) cache[dev].store(xcd_slots, std::memory_order_relaxed);
        }
    }
    // whole tiles per XCD, plus room for the half row blocks
    const int64_t per_xcd = int64_t(n_blocks) * ((max_tiles + kXcds - 1) / kXcds) +
                            int64_t(n_blocks) * ((xcd_slots / 2 + n_blocks - 1) / n_blocks);
    hipLaunchKernelGGL((k_mpf_gemm<KS, SW>), dim3(unsigned(per_xcd * kXcds)), dim3(kPfBlock), 0, s, A, ws, tile_info,
                       n_blocks, max_tiles, xcd_slots);
    return hipGetLastError();
}

template <bool SW>
hipError_t gemm_k(int64_t K, const GemmArgs& A, const MoeWorkspace& ws, const int4* tile_info, int max_tiles,
                  hipStream_t s) {
    switch (K) {
        case 512: return gemm<2, SW>(A, ws, tile_info, max_tiles, s);
        case 1024: return gemm<4, SW>(A, ws, tile_info, max_tiles, s);
        default: return gemm<8, SW>(A, ws, tile_info, max_tiles, s);
    }
}

}  // namespace

bool moe_prefill_shape_ok(int64_t hidden, int64_t inter) {
    auto ok = [](int64_t v) { return v == 512 || v == 1024 || v == 2048; };
    return ok(hidden) && ok(inter);
}

// GEMM tiles of a call, at most: full tiles of all routed pairs, one partial
// tile per active expert, and the shared expert's.
static int max_gemm_tiles(int64_t t, int k, int E, int has_shared) {
    const int64_t pr = t * k;
    return int((pr + kPfPairs - 1) / kPfPairs + std::min<int64_t>(E, pr) +
               (has_shared ? (t + kPfPairs - 1) / kPfPairs : 0));
}

size_t moe_prefill_layout(const qg_moe_desc* d, int64_t t, MoeWorkspace* ws, MoePrefillExtra* ex, void* base) {
    // the decode path's fields first (same layout), then the prefill's own
    size_t off = moe_workspace_layout(d, t, ws, base);
    const int64_t P = t * (d->top_k + (d->has_shared ? 1 : 0));
    auto take = [&](int64_t bytes) {
        const size_t at = off;
        off = size_t(align_up(int64_t(off) + bytes, kPlaneAlign));
        return at;
    };
    const size_t o_tiles = take(4 * (P + 2));
    const size_t o_cnt = take(4 * int64_t(d->n_experts));
    const size_t o_pos = take(4 * t * (d->top_k + 1));
    const size_t o_info = take(16 * (max_gemm_tiles(t, d->top_k, d->n_experts, d->has_shared) + 1));
    if (ex && base) {
        char* b = static_cast<char*>(base);
        ex->tile_off = reinterpret_cast<int32_t*>(b + o_tiles);
        ex->counts = reinterpret_cast<int32_t*>(b + o_cnt);
        ex->pair_pos = reinterpret_cast<int32_t*>(b + o_pos);
        ex->tile_info = reinterpret_cast<int4*>(b + o_info);
    }
    return off;
}

hipError_t launch_moe_prefill(const qg_moe_desc* d, const uint16_t* x, const float* logits, int t, float* y,
                              const MoeWorkspace& ws, const MoePrefillExtra& ex, hipStream_t s) {
    const int E = d->n_experts, k = d->top_k, hs = d->has_shared ? 1 : 0;
    const int H = int(d->hidden), I = int(d->inter);
    hipError_t err = launch_route_topk(logits, t, E, k, ws.ids, ws.wts, s);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_mpf_place, dim3(unsigned(E + 1)), dim3(kGroupThreads), 0, s, ws.ids, t, k, E, hs,
                       ex.counts, ws, ex.tile_off, ex.pair_pos, ex.tile_info);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int max_tiles = max_gemm_tiles(t, k, E, hs);
    GemmArgs gu{static_cast<const uint8_t*>(d->gate_up), d->gate_up_stride,
                scale_plane_offset(QG_NVFP4, 2 * int64_t(I), H), d->gate_up_scale, 2 * I, x, ws.a, ws.h, nullptr};
    if ((err = gemm_k<true>(H, gu, ws, ex.tile_info, max_tiles, s)) != hipSuccess) return err;
    GemmArgs dn{static_cast<const uint8_t*>(d->down), d->down_stride, scale_plane_offset(QG_NVFP4, int64_t(H), I),
                d->down_scale, H, ws.a, nullptr, nullptr, ws.o};
    if ((err = gemm_k<false>(I, dn, ws, ex.tile_info, max_tiles, s)) != hipSuccess) return err;
    hipLaunchKernelGGL(k_mpf_combine, dim3(unsigned(t), unsigned((H + 4 * kCombineThreads - 1) / (4 * kCombineThreads))),
                       dim3(kCombineThreads), 0, s, ws.o, ws.wts, ex.pair_pos, k, hs, H, y);
    return hipGetLastError();
}

}  // namespace qg
