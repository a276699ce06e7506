// W4A8 prefill on gfx950 matrix cores: Q4_0 weights x Q8_0 activations for
// any number of tokens, with the exact int32 block dots of the W4A8 GEMV.
//
// The bw24 README runs its prefill and its MoE expert GEMMs on int8 tensor
// cores over W4A8 operands (feature list: the NVFP4 (W4) decode path's int8
// W4A8 GEMM for prefill; MoE entry: the int8 tensor-core expert GEMM).  Here
// one v_mfma_i32_16x16x32_i8 covers exactly one 32-element Q4_0 block:
//  * lane group g of a fragment holds elements 8g..8g+7 of the block, which
//    in the Q4_0 layout are the low (g < 2) or high (g >= 2) nibbles of bytes
//    8(g%2)..8(g%2)+7 -- one 8-byte load per lane, one shift and mask, and a
//    byte-permute sign step turn them into the int8 values q - 8;
//  * activations are the quantizer's int8 codes, 8 bytes per lane;
//  * the block's int32 dots (exact) are scaled into fp32 per output as
//    acc = fma(d_w * d_x, isum, acc), blocks in ascending order, the same
//    scale step as the GEMV.  Every output depends only on its own token and
//    row, so results are bitwise reproducible and batch-invariant.
// Each 32-element block needs its own scale step per output (both operands
// have per-block fp16 scales), so the VALU work -- a convert, a multiply and
// an FMA per output per block -- bounds the kernel well before the matrix
// cores do.  Tiles: a wave computes 64 tokens x 16 NB rows (4 x NB MFMA
// tiles, so each decoded weight fragment serves four token tiles); a
// workgroup is four waves on 64 NB rows sharing the 64 tokens, whose fp32
// activation scales are staged in LDS block-major, so that one 16-byte LDS
// read gives the four tokens of a lane's outputs.  NB = 2, or 3 where the
// NB = 2 grid would not fit in one round of resident workgroups (three per CU
// either way): at 17408 x 5120 x 512 tokens, 1088 workgroups of 128 rows fill
// the 768 slots 1.42 times (233.8 us), 728 of 192 rows fit in one round
// (210.2 us).  The tile does not change any output's arithmetic.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "qg_device.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"
#include "qg_mfma.hpp"

namespace qg {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kMB = 4;                    // 16-token tiles per wave
constexpr int kTM = 16 * kMB;             // tokens per workgroup
constexpr int kS = 4;                     // 32-element blocks per stage
constexpr int kAL = kTM * 2 * kS / kThreads;  // 16-byte activation loads per thread per stage
constexpr int kXcds = 8;
constexpr int kSlotsPerCu = 3;            // resident workgroups per CU (LDS and VGPRs) for NB = 2 and 3
template <int NB>
constexpr int kTN = 16 * NB * kWaves;     // rows per workgroup
template <int NB>
constexpr int kBL = kTN<NB> * kS / kThreads;  // 16-byte weight loads per thread per stage
static_assert(kAL * kThreads == kTM * 2 * kS, "whole activation loads per thread");

// Four Q4_0 codes (bytes 0..15) -> the int8 values q - 8.
__device__ __forceinline__ uint32_t q4_to_s8(uint32_t q) {
    const uint32_t neg = __builtin_amdgcn_perm(0u, 0x000000F8u, (q >> 3) & 0x01010101u);  // 0xF8 where q < 8
    return (q & 0x07070707u) | neg;
}

// One stage of the workgroup's operands in LDS, block-major.
template <int TN>
struct Tile {
    uint8_t a[kS][kTM][32];   // activation codes: block, token, 32 bytes
    uint8_t b[kS][TN][16];    // weight codes: block, row, the block's 16 bytes
    float dx[kS][kTM];        // activation scales (fp32)
    uint16_t dw[kS][TN];      // weight scales (fp16 bits; 0 for blocks past k)
};

// The global loads of one stage, held in registers between the load and
// the LDS store (all 16-byte loads are whole-line reads of contiguous runs).
template <int BL>
struct Regs {
    u32x4 a[kAL];
    u32x4 b[BL];
    uint16_t dx[kS];
    uint32_t dw[2];
};

template <int NB>
__global__ __launch_bounds__(kThreads) void k_prefill_a8(const uint8_t* __restrict__ w, int64_t soff, int n,
                                                         int k, const int8_t* __restrict__ xq,
                                                         const uint16_t* __restrict__ xd, int m,
                                                         float* __restrict__ y, int m_blocks, int items) {
    constexpr int kNB = NB, kTN = qg::kTN<NB>, kBL = qg::kBL<NB>;
    static_assert(kBL * kThreads == kTN * kS, "whole weight loads per thread");
    static_assert(kS == 4 && kTN + kTM <= kThreads, "scale loads: one thread per row or token, two dwords of 2 blocks");
    using Tile = qg::Tile<kTN>;
    using Regs = qg::Regs<kBL>;
    __shared__ Tile tile[2];

    // work item -> (row block, token block): each XCD takes a contiguous run
    // of items, so the token blocks of one row block share its L2
    const int per_xcd = (items + kXcds - 1) / kXcds;
    const int item = int(blockIdx.x) % kXcds * per_xcd + int(blockIdx.x) / kXcds;
    if (item >= items) return;
    const int t0 = item % m_blocks * kTM;
    const int n0 = item / m_blocks * kTN;

    const int tid = int(threadIdx.x);
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lr = lane & 15, g = lane >> 4;
    const int nb = k / 32;
    const int nst = (nb + kS - 1) / kS;
    const int64_t crow = k / 2, srow = k / 16;

    // stage loads: activations (token, 16-byte part), weights (row, block),
    // the weight scales of 4 blocks of one row (one 8-byte run, read as two
    // dwords), the activation scales of one token (4 fp16)
    auto gload = [&](Regs& r, int st) {
        const int b0 = st * kS;
#pragma unroll
        for (int i = 0; i < kAL; ++i) {
            const int c = tid + kThreads * i;
            const int tok = c / (2 * kS), part = c % (2 * kS);
            const int blk = min(b0 + part / 2, nb - 1);
            r.a[i] = ld16(xq + int64_t(min(t0 + tok, m - 1)) * k + 32 * blk + 16 * (part % 2));
        }
#pragma unroll
        for (int i = 0; i < kBL; ++i) {
            const int c = tid + kThreads * i;
            const int row = c / kS, blk = min(b0 + c % kS, nb - 1);
            // 64 bytes of a row per stage, the line's other half next stage:
            // an ordinary load keeps the line in the cache
            r.b[i] = ld16(w + int64_t(min(n0 + row, n - 1)) * crow + 16 * blk);
        }
        if (tid < kTN) {
            const uint8_t* sp = w + soff + int64_t(min(n0 + tid, n - 1)) * srow;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ba = min(b0 + 2 * h, nb - 1), bb = min(b0 + 2 * h + 1, nb - 1);
                r.dw[h] = uint32_t(ld<uint16_t>(sp + 2 * ba)) | (uint32_t(ld<uint16_t>(sp + 2 * bb)) << 16);
            }
        } else if (tid < kTN + kTM) {
            const uint16_t* xp = xd + int64_t(min(t0 + tid - kTN, m - 1)) * nb;
#pragma unroll
            for (int j = 0; j < kS; ++j) r.dx[j] = xp[min(b0 + j, nb - 1)];
        }
    };
    auto lstore = [&](Tile& T, const Regs& r, int st) {
        const int b0 = st * kS;
#pragma unroll
        for (int i = 0; i < kAL; ++i) {
            const int c = tid + kThreads * i;
            const int tok = c / (2 * kS), part = c % (2 * kS);
            *reinterpret_cast<u32x4*>(&T.a[part / 2][tok][16 * (part % 2)]) = r.a[i];
        }
#pragma unroll
        for (int i = 0; i < kBL; ++i) {
            const int c = tid + kThreads * i;
            *reinterpret_cast<u32x4*>(&T.b[c % kS][c / kS][0]) = r.b[i];
        }
        if (tid < kTN) {
#pragma unroll
            for (int j = 0; j < kS; ++j)  // blocks past k scale by zero
                T.dw[j][tid] = b0 + j < nb ? uint16_t(r.dw[j / 2] >> (16 * (j % 2))) : uint16_t(0);
        } else if (tid < kTN + kTM) {
#pragma unroll
            for (int j = 0; j < kS; ++j) T.dx[j][tid - kTN] = f16_to_f32(r.dx[j]);
        }
    };

    floatx4 acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int rw = wave * 16 * kNB;  // this wave's first row in the tile
    const int shift = 4 * (g >> 1);
    // One stage: per block the eight tile products first (independent, so
    // the matrix core pipelines them), then the scale steps.
    auto compute = [&](const Tile& T) {
#pragma unroll 1
        for (int t = 0; t < kS; ++t) {
            uint64_t bf[kNB];
            float dwf[kNB];
#pragma unroll
            for (int j = 0; j < kNB; ++j) {
                const int row = rw + 16 * j + lr;
                const u32x2 v = *reinterpret_cast<const u32x2*>(&T.b[t][row][8 * (g & 1)]);
                const uint32_t lo = q4_to_s8((v[0] >> shift) & 0x0F0F0F0Fu);
                const uint32_t hi = q4_to_s8((v[1] >> shift) & 0x0F0F0F0Fu);
                bf[j] = uint64_t(lo) | (uint64_t(hi) << 32);
                dwf[j] = f16_to_f32(T.dw[t][row]);
            }
            i32x4 isum[kMB][kNB];
#pragma unroll
            for (int i = 0; i < kMB; ++i) {
                const uint64_t a = *reinterpret_cast<const uint64_t*>(&T.a[t][16 * i + lr][8 * g]);
#pragma unroll
                for (int j = 0; j < kNB; ++j)
                    isum[i][j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(long(a), long(bf[j]), i32x4{0, 0, 0, 0},
                                                                       0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < kMB; ++i) {
                const floatx4 dx = *reinterpret_cast<const floatx4*>(&T.dx[t][16 * i + 4 * g]);
#pragma unroll
                for (int j = 0; j < kNB; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[i][j][v] = fmaf(dwf[j] * dx[v], float(isum[i][j][v]), acc[i][j][v]);
            }
        }
    };

    // double-buffered stages: the next stage's global loads are in flight
    // while this one computes; one barrier per stage
    Regs r;
    gload(r, 0);
    lstore(tile[0], r, 0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int nx = min(st + 1, nst - 1);  // the last stage reloads itself into the idle buffer
        gload(r, nx);
        __builtin_amdgcn_sched_barrier(0);
        compute(tile[st & 1]);
        __builtin_amdgcn_sched_barrier(0);
        lstore(tile[(st + 1) & 1], r, nx);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const int row = n0 + rw + 16 * j + lr;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + 16 * i + 4 * g + v;
                if (t < m && row < n) y[int64_t(t) * n + row] = acc[i][j][v];
            }
        }
}

}  // namespace

bool prefill_a8_shape_ok(int64_t n, int64_t k, int64_t m) {
    if (m < 1 || m > (int64_t(1) << 24)) return false;
    const int64_t items = (m + kTM - 1) / kTM * ((n + kTN<2> - 1) / kTN<2>);  // the larger grid of the two tiles
    return items <= (int64_t(1) << 30) && m * k < (int64_t(1) << 40);
}

hipError_t launch_prefill_a8(const uint8_t* w, int64_t n, int64_t k, const int8_t* xq, const uint16_t* xd,
                             int64_t m, float* y, hipStream_t s) {
    const int m_blocks = int((m + kTM - 1) / kTM);
    int cus = 0;
    if (hipError_t e = device_cu_count(&cus); e != hipSuccess) return e;
    const int64_t soff = scale_plane_offset(QG_Q4_0, n, k);
    auto go = [&](auto nb_c) {
        constexpr int NB = decltype(nb_c)::value;
        const int items = m_blocks * int((n + kTN<NB> - 1) / kTN<NB>);
        const int per_xcd = (items + kXcds - 1) / kXcds;
        hipLaunchKernelGGL(k_prefill_a8<NB>, dim3(unsigned(per_xcd * kXcds)), dim3(kThreads), 0, s, w, soff, int(n),
                           int(k), xq, xd, int(m), y, m_blocks, items);
    };
    // 128-row tiles, or 192-row ones where the former need a second round
    if (int64_t(m_blocks) * ((n + kTN<2> - 1) / kTN<2>) > int64_t(kSlotsPerCu) * cus)
        go(std::integral_constant<int, 3>{});
    else
        go(std::integral_constant<int, 2>{});
    return hipGetLastError();
}

}  // namespace qg
