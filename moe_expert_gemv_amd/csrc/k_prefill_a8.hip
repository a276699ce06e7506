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
// cores do.  Tiles: a wave computes 64 tokens x 32 rows (4 x 2 MFMA tiles, so
// each decoded weight fragment serves four token tiles); a workgroup is four
// waves on 128 rows sharing the 64 tokens, whose fp32 activation scales are
// staged in LDS per chunk of 128 blocks, block-major, so that one 16-byte LDS
// read gives the four tokens of a lane's outputs.
#include <hip/hip_runtime.h>

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
constexpr int kNB = 2;                    // 16-row tiles per wave
constexpr int kTM = 16 * kMB;             // tokens per workgroup
constexpr int kTN = 16 * kNB * kWaves;    // rows per workgroup
constexpr int kChunk = 128;               // blocks whose activation scales sit in LDS at once
constexpr int kPitch = kTM + 4;           // LDS floats per block (padded, keeps 16-byte alignment)
constexpr int kXcds = 8;

// Four Q4_0 codes (bytes 0..15) -> the int8 values q - 8.
__device__ __forceinline__ uint32_t q4_to_s8(uint32_t q) {
    const uint32_t neg = __builtin_amdgcn_perm(0u, 0x000000F8u, (q >> 3) & 0x01010101u);  // 0xF8 where q < 8
    return (q & 0x07070707u) | neg;
}

// One block's operands of one wave.
struct Stage {
    uint64_t a[kMB];       // activation codes, 8 per lane per token tile
    uint32_t b[kNB][2];    // 8 raw code bytes per lane per row tile
    uint32_t dw[kNB];      // weight scale (fp16 bits)
};

__global__ __launch_bounds__(kThreads) void k_prefill_a8(const uint8_t* __restrict__ w, int64_t soff, int n,
                                                         int k, const int8_t* __restrict__ xq,
                                                         const uint16_t* __restrict__ xd, int m,
                                                         float* __restrict__ y, int m_blocks, int items) {
    __shared__ __attribute__((aligned(16))) float xd_s[kChunk * kPitch];

    // work item -> (row block, token block): each XCD takes a contiguous run
    // of items, so the token blocks of one row block share its L2
    const int per_xcd = (items + kXcds - 1) / kXcds;
    const int item = int(blockIdx.x) % kXcds * per_xcd + int(blockIdx.x) / kXcds;
    if (item >= items) return;
    const int t0 = item % m_blocks * kTM;
    const int rblk = item / m_blocks;

    const int tid = int(threadIdx.x);
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lr = lane & 15, g = lane >> 4;
    const int nb = k / 32;
    const int r0 = rblk * kTN + wave * 16 * kNB;

    const uint8_t* crow[kNB];
    const uint8_t* srow[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
        const int64_t row = min(r0 + 16 * j + lr, n - 1);
        crow[j] = w + row * (k / 2) + 8 * (g & 1);
        srow[j] = w + soff + row * (k / 16);
    }
    const int8_t* arow[kMB];
#pragma unroll
    for (int i = 0; i < kMB; ++i) arow[i] = xq + int64_t(min(t0 + 16 * i + lr, m - 1)) * k + 8 * g;
    const int shift = 4 * (g >> 1);

    auto load = [&](Stage& s, int blk) {
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(crow[j] + 16 * blk));
            s.b[j][0] = v[0];
            s.b[j][1] = v[1];
            s.dw[j] = ld<uint16_t>(srow[j] + 2 * blk);
        }
#pragma unroll
        for (int i = 0; i < kMB; ++i) s.a[i] = ld<uint64_t>(arow[i] + 32 * blk);
    };

    floatx4 acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Stage& s, int jj) {
        uint64_t bf[kNB];
        float dwf[kNB];
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const uint32_t lo = q4_to_s8((s.b[j][0] >> shift) & 0x0F0F0F0Fu);
            const uint32_t hi = q4_to_s8((s.b[j][1] >> shift) & 0x0F0F0F0Fu);
            bf[j] = uint64_t(lo) | (uint64_t(hi) << 32);
            dwf[j] = f16_to_f32(s.dw[j]);
        }
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
            const floatx4 dx = *reinterpret_cast<const floatx4*>(&xd_s[jj * kPitch + 16 * i + 4 * g]);
#pragma unroll
            for (int j = 0; j < kNB; ++j) {
                const i32x4 isum = __builtin_amdgcn_mfma_i32_16x16x32_i8(long(s.a[i]), long(bf[j]),
                                                                         i32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(dwf[j] * dx[v], float(isum[v]), acc[i][j][v]);
            }
        }
    };

    for (int c0 = 0; c0 < nb; c0 += kChunk) {
        const int len = min(kChunk, nb - c0);
        // activation scales of this chunk into LDS, block-major (tokens past
        // m repeat the last token; their outputs are not stored)
        if (c0 > 0) __syncthreads();
        for (int i = tid; i < kTM * len; i += kThreads) {
            const int tok = i / len, jj = i % len;
            const int t = min(t0 + tok, m - 1);
            xd_s[jj * kPitch + tok] = f16_to_f32(xd[int64_t(t) * nb + c0 + jj]);
        }
        __syncthreads();

        // four blocks of operands in flight; block indices past the chunk
        // load the chunk's last block again (valid) and are not computed
        Stage s0, s1, s2, s3;
        const int last = c0 + len - 1;
        load(s0, c0);
        load(s1, min(c0 + 1, last));
        load(s2, min(c0 + 2, last));
        load(s3, min(c0 + 3, last));
        for (int jj = 0; jj < len; jj += 4) {
            compute(s0, jj);
            load(s0, min(c0 + jj + 4, last));
            if (jj + 1 < len) compute(s1, jj + 1);
            load(s1, min(c0 + jj + 5, last));
            if (jj + 2 < len) compute(s2, jj + 2);
            load(s2, min(c0 + jj + 6, last));
            if (jj + 3 < len) compute(s3, jj + 3);
            load(s3, min(c0 + jj + 7, last));
        }
    }

#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const int row = r0 + 16 * j + lr;
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
    const int64_t items = (m + kTM - 1) / kTM * ((n + kTN - 1) / kTN);
    return items <= (int64_t(1) << 30) && m * k < (int64_t(1) << 40);
}

hipError_t launch_prefill_a8(const uint8_t* w, int64_t n, int64_t k, const int8_t* xq, const uint16_t* xd,
                             int64_t m, float* y, hipStream_t s) {
    const int m_blocks = int((m + kTM - 1) / kTM);
    const int items = m_blocks * int((n + kTN - 1) / kTN);
    const int per_xcd = (items + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(k_prefill_a8, dim3(unsigned(per_xcd * kXcds)), dim3(kThreads), 0, s, w,
                       scale_plane_offset(QG_Q4_0, n, k), int(n), int(k), xq, xd, int(m), y, m_blocks, items);
    return hipGetLastError();
}

}  // namespace qg
