// Small-M prefill GEMM over packed NVFP4 weights on gfx950 matrix cores.
//
// Y[t][r] = bf16_rne(s_t * sum_c D[r][c] * X[t][c]), D = e2m1 * e4m3 (exact in
// bf16).  This is the one place on the path that is a dense contraction, so it
// runs on MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  The pages keep
// prefill at bf16-activation numerics instead of W4A4 (memra README, known
// gaps), which is why the block-scaled FP4 MFMA of gfx950 is not used: its
// E8M0-per-32 scales and low-precision activations would change the result.
//
// Layout of the work:
//  * W is the streamed operand (0.5625 byte per weight, read once) and X the
//    reused one, so every wave owns distinct weight rows and decodes them
//    straight into MFMA B fragments in registers (no LDS round trip for W),
//    several stages ahead of use; X tiles go through LDS, double-buffered.
//  * Inside a 128-element slab, lane group g (lanes 16g..16g+15) covers 32
//    consecutive k, so one 16-byte code load per lane feeds 4 MFMA steps;
//    step s of the MFMA sums, for lane group g, the k range
//    slab + 32g + 8s .. +8 on both operands (A and B use the same permutation
//    of k, so the contraction is unchanged).
//  * Four shapes.  M <= 128 with k a multiple of 256, either entry point
//    (k_prefill_sm): one workgroup per 48 weight rows over all of k and
//    every token, X and the weights staged by LDS DMA, eight k chains added
//    in wave order.  M <= 128, other k, without a workspace (k_prefill_ks):
//    workgroups of 64 tokens x 48 weight rows; slab j of k goes to wave j
//    mod 4, each wave chains its slabs through the MFMAs in ascending order,
//    and the four partial sums are added in wave order through LDS.  M <= 128,
//    other k, with a workspace (k_prefill_sk + k_prefill_reduce): k is also
//    split over workgroups, 1024 per workgroup, whose fp32 partials are added
//    in range order by a second kernel.  M > 128: workgroups of 128 tokens x 192
//    weight rows; with k a multiple of 128 eight waves (k_prefill8, two
//    chains per output, added in a fixed order), otherwise four
//    (k_prefill, each wave 48 rows over all k in one ascending MFMA chain).
//    Within a shape the summation order of an output does not depend on M or
//    on the other rows, so a row's result does not depend on the batch it
//    came in (the shapes agree with each other to rounding).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "qg_device.hpp"
#include "qg_mfma.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"

namespace qg {

// Weight reads here are fragment-shaped (16 rows x 64 bytes per wave
// instruction), so each 128-byte line is read in two parts by different
// instructions: ordinary loads keep the line for the second part (the
// non-temporal form the GEMVs use measured about 10% slower here).

namespace {

constexpr int kBlock = 256;
// 4 x 4 transpose of dwords across the four 16-lane groups of a wave: on
// return, d[q] of lane group g holds what d[g] of lane group q held (same
// position inside the group).  v_permlane32_swap exchanges its first
// operand's lanes 32..63 with its second operand's lanes 0..31,
// v_permlane16_swap the first operand's odd 16-lane rows with the second's
// even rows.
__device__ __forceinline__ void transpose4_lane_groups(uint32_t (&d)[4]) {
    auto s32 = [](uint32_t& a, uint32_t& b) {
        const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
        a = r[0];
        b = r[1];
    };
    auto s16 = [](uint32_t& a, uint32_t& b) {
        const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
        a = r[0];
        b = r[1];
    };
    s32(d[0], d[2]);
    s32(d[1], d[3]);
    s16(d[0], d[1]);
    s16(d[2], d[3]);
}

// MB: 16-token blocks per wave; NB: 16-row blocks of W per wave; WN x WK = 4
// waves along W rows x along k; WD: stages of W loads in flight.

template <int MB, int NB, int WN, int WK, int WD>
struct PrefillShape {
    static constexpr int BM = 16 * MB;            // tokens per workgroup
    static constexpr int BN = 16 * NB * WN;       // weight rows per workgroup
    static constexpr int BK = KW * WK;            // k per stage
    static constexpr int SPS = KW / 32;           // MFMA steps per slab
    static constexpr int CPR = BK / 8;            // 16-byte X chunks per LDS row
    static constexpr int NCH = BM * CPR / kBlock; // X chunks staged per thread
    static_assert(WN * WK == 4 && (WK == 1 || WK == 4), "four waves, k split 1 or 4 ways");
    static_assert(CPR >= 16 && (CPR & (CPR - 1)) == 0, "X rows of a power-of-two count of 16 chunks");
    static_assert((BM * CPR) % kBlock == 0, "X tile split evenly over the threads");
};

template <int MB, int NB, int WN, int WK, int WD>
__global__ __launch_bounds__(kBlock) void k_prefill(const uint8_t* __restrict__ w, int64_t soff, float s_t,
                                                    int n, int k, const uint16_t* __restrict__ x, int m,
                                                    uint16_t* __restrict__ y) {
    using S = PrefillShape<MB, NB, WN, WK, WD>;
    constexpr int BM = S::BM, BN = S::BN, BK = S::BK, CPR = S::CPR, NCH = S::NCH, SPS = S::SPS;
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * BK];

    const int tid = int(threadIdx.x);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN, wk = wave / WN;
    const int lr = lane & 15, lg = lane >> 4;  // fragment row / column, lane group
    const int m0 = int(blockIdx.y) * BM;
    const int n0 = int(blockIdx.x) * BN + wn * 16 * NB;
    const int nst = (k + BK - 1) / BK;
    const int64_t crow = k / 2, srow = k / 16;

    // ---- X staging: thread t moves chunks p = t + 256 j of the BM x BK tile;
    // chunk (row, c) lands at row * CPR + (c ^ (row & 15)) (bank-conflict-free
    // fragment reads: 16 lanes reading one column of 16 rows hit 16 slots).
    // Chunks past k are zeroed when stored, not when loaded: a use right
    // after the prefetch would make the compiler wait for it (and, loads
    // completing in order, for every load issued before it).
    u32x4 xr[NCH];
    auto x_load = [&](int st) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int p = tid + kBlock * j;
            const int row = p / CPR, c = p % CPR;
            const int kk = st * BK + 8 * c;
            const int64_t gr = min(m0 + row, m - 1);
            xr[j] = ld16(x + gr * k + (kk < k ? kk : 0));
        }
    };
    auto x_store = [&](int buf, int st) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int p = tid + kBlock * j;
            const int row = p / CPR, c = p % CPR;
            const bool ok = st * BK + 8 * c < k;
            *reinterpret_cast<u32x4*>(&xs[buf][8 * (row * CPR + (c ^ (row & 15)))]) =
                ok ? xr[j] : u32x4{0u, 0u, 0u, 0u};
        }
    };

    // ---- W: this wave's rows n0 + 16 nb + lr, k range of lane group lg
    const uint8_t* wc[NB];
    const uint8_t* ws[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t row = min(n0 + 16 * nb + lr, n - 1);
        wc[nb] = w + row * crow;
        ws[nb] = w + soff + row * srow;
    }
    auto k_lane = [&](int st) { return st * BK + wk * KW + lg * (KW / 4); };
    auto w_load = [&](WStage<NB>& b, int st) {
        const int kl = k_lane(st);
        const int kc = kl < k ? kl : 0;  // lanes past the end read the row start
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const u32x4 v = ld16(wc[nb] + kc / 2);
#pragma unroll
            for (int q = 0; q < 4; ++q) b.c[nb][q] = v[q];
            b.s[nb] = ld<uint16_t>(ws[nb] + kc / 16);
        }
    };

    floatx4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // ---- prologue.  Every load in the loop is unconditional (stages past
    // the end read clamped addresses and contribute zeros), so the loop body
    // has no branches and the compiler's load counting stays exact: a branch
    // around a load would make it wait for every load in flight.
    WStage<NB> wr[WD];
#pragma unroll
    for (int d = 0; d < WD; ++d) w_load(wr[d], d);
    x_load(0);
    x_store(0, 0);
    x_load(1);
    lds_barrier();

    // ---- main loop, unrolled by WD so the W ring index is static; runs a
    // whole number of ring rounds (stages past nst multiply zeros)
    for (int st0 = 0; st0 < nst; st0 += WD) {
#pragma unroll
        for (int d = 0; d < WD; ++d) {
            const int st = st0 + d;
            const int buf = st & 1;
            // per MFMA step: decode this stage's W for the step into B
            // fragments, then the step's MFMAs with A from the swizzled X tile
            const bool okw = k_lane(st) < k;
            const uint16_t* xb = xs[buf];
            WStage<NB> cur = wr[d];
            // refill this ring slot with stage st + WD (its codes are in cur)
            w_load(wr[d], st + WD);
#pragma unroll
            for (int s = 0; s < SPS; ++s) {
                u32x4 bfr[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const float sc = (s < 2) ? e4m3_to_f32<0>(cur.s[nb]) : e4m3_to_f32<1>(cur.s[nb]);
                    const u32x4 v = decode8_scaled(cur.c[nb][s], sc);
                    bfr[nb] = okw ? v : u32x4{0u, 0u, 0u, 0u};
                }
                const int c = (wk * KW + lg * (KW / 4) + 8 * s) / 8;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int row = 16 * mb + lr;
                    const u32x4 a = *reinterpret_cast<const u32x4*>(&xb[8 * (row * CPR + (c ^ (row & 15)))]);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[mb][nb] = mfma_16x16x32_bf16(a, bfr[nb], acc[mb][nb]);
                }
            }
            // stage st + 1 into the other buffer (last read in stage st - 1,
            // before the barrier that closed it), then prefetch st + 2
            x_store(buf ^ 1, st + 1);
            x_load(st + 2);
            lds_barrier();  // the W ring stays in flight across it
        }
    }

    // ---- epilogue: D of a 16x16 tile: lane holds rows 4*(lane/16)+v, column lane%16
    if constexpr (WK == 1) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = m0 + 16 * mb + 4 * lg + v;
                    const int col = n0 + 16 * nb + lr;
                    if (row < m && col < n)
                        y[int64_t(row) * n + col] = uint16_t(f32_to_bf16_rne(acc[mb][nb][v] * s_t));
                }
    } else {
        // the four waves' partials through LDS, added in order; the X
        // buffers are free after the loop's last barrier
        static_assert(WN == 1, "k split across all four waves");
        float* red = reinterpret_cast<float*>(&xs[0][0]);
        static_assert(sizeof(float) * WK * BM * BN <= sizeof(xs), "reduction fits in the X buffers");
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[(wk * BM + 16 * mb + 4 * lg + v) * BN + 16 * nb + lr] = acc[mb][nb][v];
        __syncthreads();
        for (int idx = tid; idx < BM * BN; idx += kBlock) {
            const int r = idx / BN, c = idx % BN;
            float sum = red[r * BN + c];
#pragma unroll
            for (int q = 1; q < WK; ++q) sum += red[(q * BM + r) * BN + c];
            const int row = m0 + r, col = int(blockIdx.x) * BN + c;
            if (row < m && col < n) y[int64_t(row) * n + col] = uint16_t(f32_to_bf16_rne(sum * s_t));
        }
    }
}

// An LDS address, as the direct global -> LDS copies take it.
typedef __attribute__((address_space(3))) void* lds_ptr;

// M > 128, k a multiple of 128 (k_prefill8): 128 tokens x 192 weight rows
// per workgroup, eight waves (two per SIMD): waves w and w + 4 share 48 rows
// and take the two 64-k halves of every 128-k stage.  Everything a stage
// needs -- the X tile (128 x 128 bf16, 32 KB), the weight codes (192 rows x 64
// bytes) and their block scales (192 x 8 bytes) -- is copied global -> LDS by
// DMA (global_load_lds), into a ring of three stage slots, two stages ahead.
// With every load of the loop being such a copy, the wait for a stage is an
// exact vmcnt (the copies of the two later stages stay in flight), and one
// LDS barrier per stage both publishes the stage and frees the slot the next
// copy overwrites.  Fragments are then read from LDS: a lane group's 8 code
// bytes (16 k, one E4M3 block: both MFMA steps of the stage half), one scale
// byte, and the X chunks of the same 16 k (MFMA step s of lane group g takes
// k = stage + 64 half + 16 g + 8 s .. +8 on both operands).  Rows of codes
// sit 80 bytes apart in LDS (64 used), which puts the 16 rows of one
// fragment read on distinct banks.  Per output the two halves' chains (each
// over the stages in order) are added in a fixed order at the end.
constexpr int kP8Threads = 512;
constexpr int kP8BK = 128;                   // k per stage
constexpr int kP8Slots = 3;                  // stage slots in LDS
constexpr int kP8RowBytes = 80;              // LDS bytes per weight row of a stage (64 used)
constexpr int kP8WSlots = 1024;              // 16-byte LDS slots per stage for the codes (960 used)
constexpr int kP8Ops = 7;                    // copies per thread per stage: X 4, codes 2, scales 1

template <int MB, int NB>
__global__ __launch_bounds__(kP8Threads) void k_prefill8(const uint8_t* __restrict__ w, int64_t soff, float s_t,
                                                         int n, int k, const uint16_t* __restrict__ x, int m,
                                                         uint16_t* __restrict__ y) {
    constexpr int NT = kP8Threads, WN = 4, BK = kP8BK;
    constexpr int BM = 16 * MB, BN = 16 * NB * WN;
    constexpr int CPR = BK / 8;                 // 16-byte X chunks per token row
    constexpr int NCP = BM * CPR / NT;          // X copies per thread per stage
    constexpr int XW = BM * BK;                 // bf16 per X stage
    constexpr int WB = kP8WSlots * 16;          // code bytes per stage slot
    constexpr int SB = (NT / kWave) * kWave * 4;  // scale bytes per stage slot (512 dwords, 384 used)
    static_assert(NCP == 4 && BN == 192, "the copy counts below assume this tile");
    static_assert(BN * 5 <= kP8WSlots && BN * 2 <= NT, "code and scale slots");
    static_assert(sizeof(float) * 2 * NB * 4 * kWave * WN <= XW * 2, "two token blocks' second-half sums fit in an X slot");
    // The kP8Slots = 3 slots are separate objects, and the stage loop below is
    // unrolled by three so that every read and every copy names its slot at
    // compile time: the compiler then sees that the copies in flight into one
    // slot cannot alias the reads of another and leaves them outstanding (with
    // one array indexed by a run-time slot it waits for every copy before any
    // LDS read).
    static_assert(kP8Slots == 3, "the slot objects below and the loop's unroll");
    __shared__ __attribute__((aligned(16))) uint16_t x0[XW], x1[XW], x2[XW];
    __shared__ __attribute__((aligned(16))) uint8_t w0[WB], w1[WB], w2[WB];
    __shared__ __attribute__((aligned(16))) uint8_t s0[SB], s1[SB], s2[SB];

    const int tid = int(threadIdx.x);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN, wk = wave / WN;
    const int lr = lane & 15, lg = lane >> 4;
    const int m0 = int(blockIdx.y) * BM;
    const int nw = int(blockIdx.x) * BN;  // the workgroup's first weight row
    const int nst = k / BK;
    const int64_t crow = k / 2, srow = k / 16;

    // Copies of stage st (clamped to the last: the two issued past the end
    // reload it into slots not read any more) into one slot.  Every thread
    // issues kP8Ops copies per stage, so a wave's wait count is exact.  Each
    // source is a workgroup-uniform base for the stage plus a 32-bit offset
    // fixed for the whole loop (computed once here, so the loop spends no
    // arithmetic on addresses):
    //  * X: slot p of the tile holds X[row][st BK + 8c], row = p / CPR, c =
    //    (p % CPR) ^ (row & 15); copy i of this wave fills slots (wave + 8 i) *
    //    64 ..; rows past m repeat row m - 1.  Offsets in elements from X[m0]:
    //    row < 128 and k <= 2^24 keep them below 2^31.
    //  * codes: 16-byte slot q = 5 r + part holds bytes 16 part .. of weight
    //    row r's 64 code bytes of the stage (part 4 and slots past 5 BN:
    //    padding, filled from the workgroup's first row).
    //  * scales: dword slot q = 2 r + h holds bytes 4 h .. 4 h + 3 of row r's 8
    //    scale bytes of the stage (slots past 2 BN: padding, as above).
    const uint16_t* xt = x + int64_t(m0) * k;
    const uint8_t* wt = w + int64_t(nw) * crow;
    const uint8_t* stt = w + soff + int64_t(nw) * srow;
    uint32_t xo[NCP], wo[2], so;
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
        const int p = (wave + (NT / kWave) * i) * kWave + lane;
        const int row = p / CPR, c = (p % CPR) ^ (row & 15);
        xo[i] = uint32_t(min(row, m - 1 - m0)) * uint32_t(k) + uint32_t(8 * c);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = (wave + (NT / kWave) * i) * kWave + lane;
        const int r = q / 5, part = q % 5;
        wo[i] = (r < BN && part < 4) ? uint32_t(min(r, n - 1 - nw)) * uint32_t(crow) + uint32_t(16 * part) : 0u;
    }
    {
        const int q = wave * kWave + lane;
        const int r = q / 2, h = q % 2;
        so = r < BN ? uint32_t(min(r, n - 1 - nw)) * uint32_t(srow) + uint32_t(4 * h) : 0u;
    }
    // (the sources are passed as const void *: without the cast the host pass
    // of this file silently drops the kernel's launch stub)
    auto issue = [&](int st, uint16_t* xd, uint8_t* wd, uint8_t* sd) {
        const int sc = min(st, nst - 1);
        const uint16_t* xs_ = xt + sc * BK;
        const uint8_t* ws_ = wt + sc * (BK / 2);
        const uint8_t* ss_ = stt + sc * (BK / 16);
#pragma unroll
        for (int i = 0; i < NCP; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(xs_ + xo[i]), (lds_ptr)(xd + 8 * (wave + (NT / kWave) * i) * kWave), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(ws_ + wo[i]), (lds_ptr)(wd + 16 * (wave + (NT / kWave) * i) * kWave), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(ss_ + so), (lds_ptr)(sd + 4 * wave * kWave), 4, 0, 0);
    };

    floatx4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // stage st from slot (xb, wb, sb), after its copies have landed; the
    // copies of stage st + 2 go to slot (xn, wnx, sn), freed by the barrier
    auto stage = [&](int st, const uint16_t* xb, const uint8_t* wb, const uint8_t* sb, uint16_t* xn, uint8_t* wnx,
                     uint8_t* sn) {
        // vmcnt(kP8Ops): this wave's copies of stage st have landed, the next
        // stage's stay in flight; lgkmcnt(0): its reads of the slot of stage
        // st - 1 are done.  Then a bare barrier: every wave's copies of stage
        // st have landed and no wave still reads the slot the copies below
        // overwrite.  No release fence: the loop writes LDS only by copies,
        // which such a fence would wait for in full; the acquire keeps the
        // reads below the barrier.
        static_assert(kP8Ops < 16, "vmcnt in the low field");
        __builtin_amdgcn_s_waitcnt(0x0070 | kP8Ops);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        issue(st + 2, xn, wnx, sn);
        __builtin_amdgcn_sched_barrier(0);
        uint32_t sv[NB];
        u32x2 cv[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int r = wn * 16 * NB + 16 * nb + lr;
            cv[nb] = *reinterpret_cast<const u32x2*>(&wb[r * kP8RowBytes + wk * 32 + 8 * lg]);
            sv[nb] = sb[r * 8 + wk * 4 + lg];
        }
        u32x4 aa[2][MB];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int c = wk * 8 + 2 * lg + s2;  // k = stage + 64 wk + 16 lg + 8 s2
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = 16 * mb + lr;
                aa[s2][mb] = *reinterpret_cast<const u32x4*>(&xb[8 * (row * CPR + (c ^ (row & 15)))]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const u32x4* a = aa[s2];
            u32x4 bfr[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) bfr[nb] = decode8_scaled(cv[nb][s2], e4m3_to_f32<0>(sv[nb]));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_16x16x32_bf16(a[mb], bfr[nb], acc[mb][nb]);
        }
    };

    issue(0, x0, w0, s0);
    issue(1, x1, w1, s1);
    // slot of stage st: st % 3.  Whole triples in the loop, the one or two
    // stages left after it: with no conditional stage inside the loop every
    // path into a stage has the same copies outstanding, which the compiler
    // needs in order to keep the exact wait.
    int st = 0;
    for (; st + 3 <= nst; st += 3) {
        stage(st, x0, w0, s0, x2, w2, s2);
        stage(st + 1, x1, w1, s1, x0, w0, s0);
        stage(st + 2, x2, w2, s2, x1, w1, s1);
    }
    if (st < nst) stage(st, x0, w0, s0, x2, w2, s2);
    if (st + 1 < nst) stage(st + 1, x1, w1, s1, x0, w0, s0);

    // second half's sums through LDS, two 16-token blocks at a time in X slot
    // 0 (every copy has landed and every wave is done with the slots), added
    // to the first half's in that order
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the trailing copies past the end
    __syncthreads();
    float* red = reinterpret_cast<float*>(x0) + wn * (2 * NB * 4 * kWave);
    const int n0 = nw + wn * 16 * NB;
#pragma unroll
    for (int mp = 0; mp < MB; mp += 2) {
        if (wk == 1) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) red[((h * NB + nb) * 4 + v) * kWave + lane] = acc[mp + h][nb][v];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float sum = acc[mp + h][nb][v] + red[((h * NB + nb) * 4 + v) * kWave + lane];
                        const int row = m0 + 16 * (mp + h) + 4 * lg + v;
                        const int col = n0 + 16 * nb + lr;
                        if (row < m && col < n) y[int64_t(row) * n + col] = uint16_t(f32_to_bf16_rne(sum * s_t));
                    }
        }
        __syncthreads();
    }
}

// M <= 128: the k range is split over the four waves (slab j of 128 k to
// wave j mod 4), so a wave's X operand is its own: A fragments are loaded
// from global memory (L2) straight into registers, two slabs ahead, and W
// four slabs ahead; the main loop has no LDS traffic and no barrier.  The
// four partial sums meet in LDS at the end and are added in wave order.
// Inside a slab, MFMA step q of lane group g takes k = 32q + 8g .. +8, so an
// A load reads 64 contiguous bytes of each of 16 rows; W is loaded as 16
// contiguous bytes per lane (k = 32g .. 32g+31) and redistributed across the
// lane groups by a 4 x 4 transpose.  Workgroup: 16*MB tokens x 16*NB rows.
template <int MB, int NB>
__global__ __launch_bounds__(kBlock) void k_prefill_ks(const uint8_t* __restrict__ w, int64_t soff, float s_t,
                                                       int n, int k, const uint16_t* __restrict__ x, int m,
                                                       uint16_t* __restrict__ y) {
    constexpr int BM = 16 * MB, BN = 16 * NB;
    constexpr int AD = 2, WD = 4, U = 4;  // ring depths (slabs) and the unroll that makes them static
    __shared__ float red[4 * BM * BN];

    const int tid = int(threadIdx.x);
    const int lane = tid & 63;
    const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int m0 = int(blockIdx.y) * BM, n0 = int(blockIdx.x) * BN;
    const int nslab = (k + KW - 1) / KW;
    const int nw = (nslab - wk + 3) / 4;            // slabs wk, wk + 4, ... of this wave
    const int ilast = nw > 0 ? nw - 1 : 0;

    const uint16_t* xrow[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) xrow[mb] = x + int64_t(min(m0 + 16 * mb + lr, m - 1)) * k;
    const uint8_t* wc[NB];
    const uint8_t* ws[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t row = min(n0 + 16 * nb + lr, n - 1);
        wc[nb] = w + row * (k / 2);
        ws[nb] = w + soff + row * (k / 16);
    }
    // first k of the wave's i-th slab (clamped to a valid slab)
    auto slab_k = [&](int i) { return KW * (wk + 4 * min(i, ilast)); };

    u32x4 ar[AD][MB][4];
    WStage<NB> wr[WD];
    auto a_load = [&](u32x4 (&a)[MB][4], int i) {
        const int k0 = slab_k(i);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kq = k0 + 32 * q;            // step q is valid for all lanes or none
            const int kc = (kq < k ? kq : 0) + 8 * lg;  // past the end: a valid address, zeroed at use
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) a[mb][q] = ld16(xrow[mb] + kc);
        }
    };
    auto w_load = [&](WStage<NB>& b, int i) {
        const int kb = slab_k(i) + 32 * lg;
        const int kc = kb < k ? kb : 0;  // past the end: the row's own first block
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const u32x4 v = ld16(wc[nb] + kc / 2);
#pragma unroll
            for (int q = 0; q < 4; ++q) b.c[nb][q] = v[q];
            b.s[nb] = ld<uint16_t>(ws[nb] + kc / 16);  // blocks of k = kc .. kc+31
        }
    };

    floatx4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int d = 0; d < WD; ++d) w_load(wr[d], d);
#pragma unroll
    for (int d = 0; d < AD; ++d) a_load(ar[d], d);

    for (int i0 = 0; i0 < nw; i0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u;
            if (i < nw) {  // wave-uniform: compute slab i (no load inside)
                const int k0 = KW * (wk + 4 * i);
                if (k0 + KW > k) {  // the last slab runs past k: zero its X there
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            ar[u % AD][mb][q] = k0 + 32 * q < k ? ar[u % AD][mb][q] : u32x4{0u, 0u, 0u, 0u};
                }
                // W to step-major order: codes, and the scale byte of each step
                // (lane group g, step q: block 2q + g/2 of the slab)
                uint32_t cq[NB][4], sq[NB][4];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) cq[nb][q] = wr[u % WD].c[nb][q];
                    transpose4_lane_groups(cq[nb]);
                    const uint32_t s2 = wr[u % WD].s[nb];  // this lane group's blocks 2g, 2g+1
                    sq[nb][0] = sq[nb][1] = s2 & 0xffu;
                    sq[nb][2] = sq[nb][3] = s2 >> 8;
                    transpose4_lane_groups(sq[nb]);  // sq[q] = block 2q + g/2 (from lane group q)
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u32x4 bfr[NB];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) bfr[nb] = decode8_scaled(cq[nb][q], e4m3_to_f32<0>(sq[nb][q]));
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[mb][nb] = mfma_16x16x32_bf16(ar[u % AD][mb][q], bfr[nb], acc[mb][nb]);
                }
            }
            // refill both ring slots (unconditional: clamped slab index)
            a_load(ar[u % AD], i + AD);
            w_load(wr[u % WD], i + WD);
        }
    }

    // partial sums through LDS, added in wave order
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[(wk * BM + 16 * mb + 4 * lg + v) * BN + 16 * nb + lr] = acc[mb][nb][v];
    __syncthreads();
    for (int idx = tid; idx < BM * BN; idx += kBlock) {
        const int r = idx / BN, c = idx % BN;
        float sum = red[r * BN + c];
#pragma unroll
        for (int q = 1; q < 4; ++q) sum += red[(q * BM + r) * BN + c];
        const int row = m0 + r, col = n0 + c;
        if (row < m && col < n) y[int64_t(row) * n + col] = uint16_t(f32_to_bf16_rne(sum * s_t));
    }
}

// M <= 128 in one pass (k_prefill_sm): a workgroup owns 48 weight rows over
// all of k and every token (TB blocks of 64), so each weight byte is read
// once, nothing leaves the workgroup but its outputs, and the grid (n / 48
// workgroups) fills the machine.  X, the codes and the scales come through
// an LDS DMA ring of 256-k stages as in k_prefill8 (four slots for one token
// block -- 160 KB, three stages in flight -- two for two); wave s (of eight)
// takes k = stage + 32 s .. +32, one MFMA step per stage, so each wave runs
// one chain per output over the stages in order, and the eight chains are
// added in wave order at the end.  The per-token arithmetic is the same for
// TB = 1 and 2, so a token's result does not depend on m within m <= 128.
constexpr int kSmThreads = 512;
constexpr int kSmBK = 256;         // k per stage
constexpr int kSmRows = 48;        // weight rows per workgroup
constexpr int kSmRowBytes = 144;   // LDS bytes per weight row of a stage (128 used; 144 keeps 16 rows on distinct banks)
constexpr int kSmScaleOff = kSmRows * kSmRowBytes;  // the stage's 16 scale bytes a row follow the codes: 6912
constexpr int kSmTileStride = 36;  // floats a column in the epilogue's [column][32 tokens] tiles

template <int TB>
__global__ __launch_bounds__(kSmThreads) void k_prefill_sm(const uint8_t* __restrict__ w, int64_t soff, float s_t,
                                                           int n, int k, const uint16_t* __restrict__ x, int m,
                                                           uint16_t* __restrict__ y) {
    constexpr int NT = kSmThreads, BK = kSmBK, NB = kSmRows / 16, MB = 4 * TB;
    constexpr int BM = 16 * MB;                 // tokens
    constexpr int CPR = BK / 8;                 // 16-byte X chunks per token row: 32
    constexpr int NCP = BM * CPR / NT;          // X copies per thread per stage: 4 or 8
    constexpr int XW = BM * BK;                 // bf16 per X slot
    constexpr int WB = NT * 16;                 // code and scale bytes per slot (one 16-byte copy per thread)
    constexpr int OPS = NCP + 1;                // copies per thread per stage
    constexpr int SLOTS = TB == 1 ? 4 : 2;
    constexpr int TILE = kSmRows * kSmTileStride;  // epilogue floats a wave
    static_assert(kSmRows * 9 + kSmRows <= NT && kSmScaleOff + 16 * kSmRows <= WB, "code and scale copies");
    static_assert(4 * TILE * 4 <= XW * 2, "four waves' epilogue tiles fit one X slot");
    // separate slot objects, the loop unrolled by the slot count (see k_prefill8)
    __shared__ __attribute__((aligned(16))) uint16_t xa[XW], xb_[XW], xc[SLOTS > 2 ? XW : 8], xd_[SLOTS > 3 ? XW : 8];
    __shared__ __attribute__((aligned(16))) uint8_t wa[WB], wb_[WB], wc[SLOTS > 2 ? WB : 16], wd[SLOTS > 3 ? WB : 16];

    const int tid = int(threadIdx.x);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // the 32-k slice of every stage
    const int lr = lane & 15, lg = lane >> 4;
    const int nw = int(blockIdx.x) * kSmRows;
    const int nst = k / BK;
    const int64_t crow = k / 2, srow = k / 16;

    // Copy sources: a workgroup-uniform base per stage plus a 32-bit offset
    // fixed for the loop.
    //  * X: slot p holds X[tok][st BK + 8c], tok = p / CPR, c = (p % CPR) ^
    //    (tok & 15); copy i of this wave fills slots (wave + 8 i) * 64 ..;
    //    tokens past m repeat token m - 1.
    //  * codes and scales, one 16-byte copy a thread: thread q < 432 = 9 r +
    //    part, part < 8, copies bytes 16 part .. of row r's 128 code bytes of
    //    the stage to r * 144 + 16 part (part 8: padding, from the workgroup's
    //    first row); thread 432 + r copies row r's 16 scale bytes of the stage
    //    to 6912 + 16 r; the rest copy row 0's scales into the padding after.
    uint32_t xo[NCP];
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
        const int p = (wave + (NT / kWave) * i) * kWave + lane;
        const int tok = p / CPR, c = (p % CPR) ^ (tok & 15);
        xo[i] = uint32_t(min(tok, m - 1)) * uint32_t(k) + uint32_t(8 * c);
    }
    uint32_t wo;
    bool wsc;  // this thread copies scales
    {
        const int q = tid, r = q / 9, part = q % 9;
        if (q < 9 * kSmRows) {
            wsc = false;
            wo = part < 8 ? uint32_t(min(r, n - 1 - nw)) * uint32_t(crow) + uint32_t(16 * part) : 0u;
        } else {
            wsc = true;
            const int rs = q - 9 * kSmRows;
            wo = rs < kSmRows ? uint32_t(min(rs, n - 1 - nw)) * uint32_t(srow) : 0u;
        }
    }
    const uint8_t* wt = w + int64_t(nw) * crow;
    const uint8_t* stt = w + soff + int64_t(nw) * srow;
    // (sources passed as const void *: see k_prefill8)
    auto issue = [&](int st, uint16_t* xd, uint8_t* wd) {
        const int sc = min(st, nst - 1);
        const uint16_t* xs_ = x + sc * BK;
#pragma unroll
        for (int i = 0; i < NCP; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(xs_ + xo[i]),
                                             (lds_ptr)(xd + 8 * (wave + (NT / kWave) * i) * kWave), 16, 0, 0);
        const uint8_t* src = wsc ? stt + sc * (BK / 16) + wo : wt + sc * (BK / 2) + wo;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(wd + 16 * wave * kWave), 16, 0, 0);
    };

    floatx4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // step weights of this wave's 32 k of a stage, decoded from slot ws_
    auto decode_w = [&](const uint8_t* ws_, u32x4* bfr) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int r = 16 * nb + lr;
            const uint32_t cw = *reinterpret_cast<const uint32_t*>(&ws_[r * kSmRowBytes + 16 * wave + 4 * lg]);
            const uint32_t sv = ws_[kSmScaleOff + r * 16 + 2 * wave + (lg >> 1)];  // block (32 wave + 8 lg) / 16
            bfr[nb] = decode8_scaled(cw, e4m3_to_f32<0>(sv));
        }
    };
    auto mfma_x = [&](const uint16_t* xs_, const u32x4* bfr) {
        const int c = 4 * wave + lg;  // k = stage + 32 wave + 8 lg
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int tok = 16 * mb + lr;
            const u32x4 a = *reinterpret_cast<const u32x4*>(&xs_[8 * (tok * CPR + (c ^ (tok & 15)))]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_16x16x32_bf16(a, bfr[nb], acc[mb][nb]);
        }
    };
    // this wave's copies of stage st have landed (the later ones stay in
    // flight) and its LDS reads are done (a slot read in the previous stage
    // is the next copy's target), then a bare barrier and an acquire (see
    // k_prefill8)
    auto sync = [&](auto ahead) {
        constexpr int vm = OPS * (SLOTS - 2 - decltype(ahead)::value);
        static_assert(vm < 16, "vmcnt in the low field");
        __builtin_amdgcn_s_waitcnt(0x0070 | vm);  // lgkmcnt(0) vmcnt(vm)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    using ahead0 = std::integral_constant<int, 0>;

    auto stage = [&](int st, const uint16_t* xs_, const uint8_t* ws_, uint16_t* xn, uint8_t* wn_) {
        sync(ahead0{});
        issue(st + SLOTS - 1, xn, wn_);
        __builtin_amdgcn_sched_barrier(0);
        u32x4 bfr[NB];
        decode_w(ws_, bfr);
        mfma_x(xs_, bfr);
    };
    if constexpr (SLOTS == 4) {
        issue(0, xa, wa);
        issue(1, xb_, wb_);
        issue(2, xc, wc);
        int st = 0;
        for (; st + 4 <= nst; st += 4) {
            stage(st, xa, wa, xd_, wd);
            stage(st + 1, xb_, wb_, xa, wa);
            stage(st + 2, xc, wc, xb_, wb_);
            stage(st + 3, xd_, wd, xc, wc);
        }
        if (st < nst) stage(st, xa, wa, xd_, wd);
        if (st + 1 < nst) stage(st + 1, xb_, wb_, xa, wa);
        if (st + 2 < nst) stage(st + 2, xc, wc, xb_, wb_);
    } else {
        issue(0, xa, wa);
        int st = 0;
        for (; st + 2 <= nst; st += 2) {
            stage(st, xa, wa, xb_, wb_);
            stage(st + 1, xb_, wb_, xa, wa);
        }
        if (st < nst) stage(st, xa, wa, xb_, wb_);
    }

    // the eight chains of each output through LDS, 32 tokens at a time,
    // added in wave order: wave v's [column][token] tile sits in xa (v < 4)
    // or xb_
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the trailing copies
    __syncthreads();
    float* const tile = reinterpret_cast<float*>(wave < 4 ? xa : xb_) + (wave & 3) * TILE;
#pragma unroll
    for (int h = 0; h < 2 * TB; ++h) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                *reinterpret_cast<floatx4*>(&tile[(16 * nb + lr) * kSmTileStride + 16 * mb + 4 * lg]) =
                    acc[2 * h + mb][nb];
        __syncthreads();
        if (tid < kSmRows * 8) {  // column tid % 48, tokens 4 (tid / 48) .. + 4
            const int col = tid % kSmRows, t4 = tid / kSmRows;
            const int off = col * kSmTileStride + 4 * t4;
            floatx4 sum = *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(xa) + off);
#pragma unroll
            for (int v = 1; v < 8; ++v)
                sum += *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(v < 4 ? xa : xb_) +
                                                         (v & 3) * TILE + off);
            const int gc = nw + col;
            if (gc < n) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tok = 32 * h + 4 * t4 + e;
                    if (tok < m) y[int64_t(tok) * n + gc] = uint16_t(f32_to_bf16_rne(sum[e] * s_t));
                }
            }
        }
        __syncthreads();
    }
}

// M <= 128 with a workspace: the k range is split over several workgroups
// (kSkRange each), so a workgroup reads only its slice of X -- 64 tokens x
// 1024 k, 128 KB, staged into LDS -- instead of all of X.  A workgroup owns
// 192 weight rows of one k range for every token block (one for m <= 64, two
// for m <= 128: the weights stay in registers and the second X block replaces
// the first in LDS), so the grid is one round of workgroups and each weight
// byte is read once.  Eight waves, two per SIMD: waves w and w + 4 take the
// same 48 weight rows, w the even 128-k slabs of the range and w + 4 the odd
// ones, so one wave's weight decode (VALU) runs while the other's MFMAs do.
//
// Memory order.  Every wave first requests its part of the X block and of the
// block scales of the workgroup's rows (16-byte loads, contiguous across the
// wave); the weight slabs are requested once that X block is in LDS.  Issued
// together with the X loads, the whole grid's 28 MB of weight requests share
// the memory queues with X and the first MFMA waits for X for several
// microseconds more (measured: X staged 3 us after a workgroup starts with
// the weights behind it, 12 us with them beside it).  The scales go through
// LDS because a lane needs only two of a row's bytes per slab: 2-byte loads
// scattered over 16 rows per instruction cost more than the codes
// themselves.  The two halves' sums and the result tile go through LDS too,
// so each token's fp32 partials leave as one contiguous 768-byte row
// segment; k_prefill_reduce adds the ranges' partials in range order.
constexpr int kSkRange = 1024;                       // k per workgroup
constexpr int kSkBlock = 512;                        // threads per workgroup
constexpr int kSkHalves = 2;                         // waves sharing a row set
constexpr int kSkSlabs = kSkRange / KW / kSkHalves;  // slabs per wave: 4
constexpr int kSkRows = 64;                          // tokens per block
constexpr int kSkNB = 3;                             // 16-row blocks per wave
constexpr int kSkCols = 16 * kSkNB * (kSkBlock / kWave / kSkHalves);  // weight rows per workgroup: 192
constexpr int kSkScaleStride = 80;  // LDS bytes per weight row of scales (64 used; 80 keeps 16 rows on distinct banks)
constexpr int kSkTileStride = kSkCols + 4;  // floats per token of the LDS result tile (padding: no bank conflicts)

template <bool TAIL, int TB>
__global__ __launch_bounds__(kSkBlock) void k_prefill_sk(const uint8_t* __restrict__ w, int64_t soff, int n, int k,
                                                         const uint16_t* __restrict__ x, int m,
                                                         float* __restrict__ part) {
    constexpr int NB = kSkNB;
    constexpr int MB = kSkRows / 16;
    constexpr int RW = kSkBlock / kWave / kSkHalves;  // row sets per workgroup: 4
    constexpr int CPR = kSkRange / 8;                  // 16-byte chunks per X row
    constexpr int kCopies = kSkRows * CPR / kSkBlock;  // X chunks per lane: 16
    constexpr int SPR = kSkRange / 32;                 // scale pairs (2 bytes, 32 k) per row of the range
    constexpr int kScale16 = kSkCols * (SPR * 2 / 16);  // 16-byte scale chunks per workgroup: 768
    constexpr int kScale16PerLane = (kScale16 + kSkBlock - 1) / kSkBlock;
    constexpr int kScale2PerLane = kSkCols * SPR / kSkBlock;  // 2-byte scale pairs per lane: 12
    static_assert(kSkCols * SPR % kSkBlock == 0, "scale pairs split evenly");
    static_assert(2 * kSkRows * kSkTileStride * 4 <= kSkRows * kSkRange * 2, "result tile fits in the X buffer");
    __shared__ __attribute__((aligned(16))) uint16_t xs[kSkRows * kSkRange];
    __shared__ __attribute__((aligned(16))) uint8_t ss[kSkCols * kSkScaleStride];

    const int tid = int(threadIdx.x);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rs = wave % RW, half = wave / RW;
    const int lr = lane & 15, lg = lane >> 4;
    const int nw = int(blockIdx.x) * kSkCols;  // the workgroup's first weight row
    const int n0 = nw + rs * 16 * NB;          // this wave's
    const int kz = int(blockIdx.z) * kSkRange;

    // X block loads: chunk slot p of the LDS tile holds X[row][kz + 8c],
    // row = p / CPR, c = (p % CPR) ^ (row & 15) (fragment reads then hit 16
    // distinct slots per 16 lanes); lane i of copy step cp fills slot
    // cp * 64 + i.  Tokens past m repeat token m-1 (their results are not
    // stored); chunks past k are zero.
    auto x_load = [&](u32x4(&xr)[kCopies], int m0) {
#pragma unroll
        for (int i = 0; i < kCopies; ++i) {
            const int p = (wave + (kSkBlock / kWave) * i) * kWave + lane;
            const int row = p / CPR, c = (p % CPR) ^ (row & 15);
            const int kk = kz + 8 * c;
            xr[i] = ld16(x + int64_t(min(m0 + row, m - 1)) * k + (kk < k ? kk : 0));
        }
    };
    // (the chunks past k are zeroed here, not at the load: a select there
    // would wait for the data before the weight loads are issued)
    auto x_store = [&](const u32x4(&xr)[kCopies]) {
#pragma unroll
        for (int i = 0; i < kCopies; ++i) {
            const int p = (wave + (kSkBlock / kWave) * i) * kWave + lane;
            const int row = p / CPR, c = (p % CPR) ^ (row & 15);
            *reinterpret_cast<u32x4*>(&xs[8 * p]) = TAIL ? zero_unless(kz + 8 * c < k, xr[i]) : xr[i];
        }
    };

    // 1. X block 0 and the scales of rows nw.. (rows past n repeat row n-1).
    // Scale pair e of a row covers k = kz + 32 e .. +32; pairs past k take
    // the row's first pair, as the codes past k take the row's first codes
    // (they meet zero X).  Without a k tail every row's range of scales is 64
    // aligned bytes: four 16-byte loads; with one, 2-byte loads.
    u32x4 xr[kCopies];
    x_load(xr, 0);
    u32x4 sr16[kScale16PerLane];
    uint32_t sr2[kScale2PerLane];
    if constexpr (!TAIL) {
#pragma unroll
        for (int i = 0; i < kScale16PerLane; ++i) {
            const int c = min(tid + kSkBlock * i, kScale16 - 1);
            const int64_t row = min(nw + c / 4, n - 1);
            sr16[i] = ld16(w + soff + row * (k / 16) + kz / 16 + 16 * (c % 4));
        }
    } else {
#pragma unroll
        for (int i = 0; i < kScale2PerLane; ++i) {
            const int e = tid + kSkBlock * i;
            const int64_t row = min(nw + e / SPR, n - 1);
            const int kk = kz + 32 * (e % SPR);
            sr2[i] = ld<uint16_t>(w + soff + row * (k / 16) + (kk < k ? kk / 16 : 0));
        }
    }

    // 2. this wave's weight slabs, all of them (issued after step 3); slab j
    // covers k = kz + 128 (2 j + half) + [0, 128), lane group lg its 32 k from
    // kz + 128 (2 j + half) + 32 lg (past k: the row's first 32)
    WStage<NB> wr[kSkSlabs];
    auto w_load = [&]() {
#pragma unroll
        for (int j = 0; j < kSkSlabs; ++j) {
            const int kb = kz + KW * (kSkHalves * j + half) + 32 * lg;
            const int kc = kb < k ? kb : 0;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int64_t row = min(n0 + 16 * nb + lr, n - 1);
                const u32x4 v = ld16(w + row * (k / 2) + kc / 2);
#pragma unroll
                for (int q = 0; q < 4; ++q) wr[j].c[nb][q] = v[q];
            }
        }
    };

    // 3. publish X block 0 and the scales, then request the weights
    x_store(xr);
    if constexpr (!TAIL) {
        // lanes past the last chunk store the last chunk again (the same
        // bytes): no branch, which would let the compiler sink the load
        // behind the weight loads and wait for all of them
#pragma unroll
        for (int i = 0; i < kScale16PerLane; ++i) {
            const int c = min(tid + kSkBlock * i, kScale16 - 1);
            *reinterpret_cast<u32x4*>(&ss[(c / 4) * kSkScaleStride + 16 * (c % 4)]) = sr16[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < kScale2PerLane; ++i) {
            const int e = tid + kSkBlock * i;
            *reinterpret_cast<uint16_t*>(&ss[(e / SPR) * kSkScaleStride + 2 * (e % SPR)]) = uint16_t(sr2[i]);
        }
    }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);  // no decode is hoisted above the barrier
    w_load();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (TB > 1) x_load(xr, kSkRows);  // block 1, queued behind the weights

    // this wave's scale pairs: slab j, row block nb
    uint32_t sc2[kSkSlabs][NB];
#pragma unroll
    for (int j = 0; j < kSkSlabs; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            sc2[j][nb] = *reinterpret_cast<const uint16_t*>(
                &ss[(rs * 16 * NB + 16 * nb + lr) * kSkScaleStride + 2 * (4 * (kSkHalves * j + half) + lg)]);

    float* tile = reinterpret_cast<float*>(xs);  // [half][token][column], after the MFMAs
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        if (tb > 0) {
            // a later block decodes the weights again: kept decoded they would
            // take 192 registers, so the registers are marked as rewritten here
            // (an empty asm), which stops the compiler from reusing block 0's
            // decode.  Every weight load has completed by now.
#pragma unroll
            for (int j = 0; j < kSkSlabs; ++j)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(wr[j].c[nb][q]));
                    asm volatile("" : "+v"(sc2[j][nb]));
                }
        }
        // 4. MFMAs, slab by slab, without a runtime branch (slabs past k meet
        // zero X and add nothing)
        floatx4 acc[MB][NB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kSkSlabs; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4 bfr[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const float sc = (q < 2) ? e4m3_to_f32<0>(sc2[j][nb]) : e4m3_to_f32<1>(sc2[j][nb]);
                    bfr[nb] = decode8_scaled(wr[j].c[nb][q], sc);
                }
                const int c = 16 * (kSkHalves * j + half) + 4 * lg + q;  // k = 128 slab + 32 lg + 8 q
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int row = 16 * mb + lr;
                    const u32x4 a = *reinterpret_cast<const u32x4*>(&xs[8 * (row * CPR + (c ^ (row & 15)))]);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_16x16x32_bf16(a, bfr[nb], acc[mb][nb]);
                }
            }
        }

        // 5. both halves' sums into the tile (the X block is no longer read),
        // then even half + odd half per output, stored as contiguous row
        // segments of part[z][token][column]
        lds_barrier();
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    tile[(half * kSkRows + 16 * mb + 4 * lg + v) * kSkTileStride + rs * 16 * NB + 16 * nb + lr] =
                        acc[mb][nb][v];
        lds_barrier();
        float* pz = part + int64_t(blockIdx.z) * m * n;
        constexpr int C4 = kSkCols / 4;
#pragma unroll
        for (int i = 0; i < kSkRows * C4 / kSkBlock; ++i) {
            const int c = tid + kSkBlock * i;
            const int r = c / C4, col = 4 * (c % C4);
            const floatx4 a = *reinterpret_cast<const floatx4*>(&tile[r * kSkTileStride + col]);
            const floatx4 b = *reinterpret_cast<const floatx4*>(&tile[(kSkRows + r) * kSkTileStride + col]);
            const floatx4 sum = {a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]};
            const int tok = tb * kSkRows + r, gc = nw + col;
            if (tok < m && gc < n) {
                float* dst = pz + int64_t(tok) * n + gc;
                if (n % 4 == 0) {
                    *reinterpret_cast<floatx4*>(dst) = sum;
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (gc + v < n) dst[v] = sum[v];
                }
            }
        }
        if constexpr (TB > 1) {
            if (tb + 1 < TB) {
                lds_barrier();  // the tile is read
                x_store(xr);
                lds_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// y = bf16_rne(s_t * sum over the nz ranges of part[z]), ranges in order
// (the first range's value is the start, so a lone -0 stays -0).  Four
// outputs per thread when count % 4 == 0 (every slice then starts 16-byte
// aligned), else one; the ranges' loads are issued four at a time.
__global__ __launch_bounds__(kBlock) void k_prefill_reduce(const float* __restrict__ part, int nz, int64_t count,
                                                           float s_t, uint16_t* __restrict__ y) {
    const int64_t n4 = count % 4 == 0 ? count / 4 : 0;
    for (int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x; i < n4; i += int64_t(gridDim.x) * kBlock) {
        floatx4 sum = *reinterpret_cast<const floatx4*>(part + 4 * i);
        for (int z0 = 1; z0 < nz; z0 += 4) {
            floatx4 v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (z0 + j < nz) v[j] = *reinterpret_cast<const floatx4*>(part + (z0 + j) * count + 4 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (z0 + j < nz) {
                    sum[0] += v[j][0];
                    sum[1] += v[j][1];
                    sum[2] += v[j][2];
                    sum[3] += v[j][3];
                }
        }
        const uint32_t lo = f32_to_bf16_rne(sum[0] * s_t) | (f32_to_bf16_rne(sum[1] * s_t) << 16);
        const uint32_t hi = f32_to_bf16_rne(sum[2] * s_t) | (f32_to_bf16_rne(sum[3] * s_t) << 16);
        *reinterpret_cast<u32x2*>(y + 4 * i) = u32x2{lo, hi};
    }
    for (int64_t i = 4 * n4 + int64_t(blockIdx.x) * kBlock + threadIdx.x; i < count;
         i += int64_t(gridDim.x) * kBlock) {
        float sum = part[i];
        for (int z = 1; z < nz; ++z) sum += part[z * count + i];
        y[i] = uint16_t(f32_to_bf16_rne(sum * s_t));
    }
}

template <int MB, int NB, int WN, int WK, int WD>
hipError_t go(const uint8_t* w, int64_t soff, float s_t, int64_t n, int64_t k, const uint16_t* x, int64_t m,
              uint16_t* y, hipStream_t s) {
    using S = PrefillShape<MB, NB, WN, WK, WD>;
    const dim3 grid(unsigned((n + S::BN - 1) / S::BN), unsigned((m + S::BM - 1) / S::BM));
    hipLaunchKernelGGL((k_prefill<MB, NB, WN, WK, WD>), grid, dim3(kBlock), 0, s, w, soff, s_t, int(n),
                       int(k), x, int(m), y);
    return hipGetLastError();
}

}  // namespace

// The k-split kernel only where the one-pass kernel (k_prefill_sm) does not
// run: m <= 128 with k not a multiple of 256.
static bool prefill_splits_k(int64_t k, int64_t m) { return m <= 2 * kSkRows && k % kSmBK != 0; }

size_t prefill_workspace_bytes(int64_t n, int64_t k, int64_t m) {
    if (!prefill_splits_k(k, m)) return 0;
    const int64_t nz = (k + kSkRange - 1) / kSkRange;
    return size_t(nz * m * n * 4);
}

hipError_t launch_prefill_ws(const uint8_t* w, float s_t, int64_t n, int64_t k, const uint16_t* x, int64_t m,
                             uint16_t* y, float* ws, hipStream_t s) {
    if (!prefill_splits_k(k, m) || kernel_policy() == QG_KERNEL_GENERIC) return launch_prefill(w, s_t, n, k, x, m, y, s);
    const int64_t soff = scale_plane_offset(QG_NVFP4, n, k);
    const int nz = int((k + kSkRange - 1) / kSkRange);
    const dim3 grid(unsigned((n + kSkCols - 1) / kSkCols), 1u, unsigned(nz));
    const bool tail = k % kSkRange != 0;
    auto kern = m > kSkRows ? (tail ? k_prefill_sk<true, 2> : k_prefill_sk<false, 2>)
                            : (tail ? k_prefill_sk<true, 1> : k_prefill_sk<false, 1>);
    hipLaunchKernelGGL(kern, grid, dim3(kSkBlock), 0, s, w, soff, int(n), int(k), x, int(m), ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t count = m * n;
    const unsigned blocks = unsigned(std::max<int64_t>(1, std::min<int64_t>((count / 4 + kBlock - 1) / kBlock, 4096)));
    hipLaunchKernelGGL(k_prefill_reduce, dim3(blocks), dim3(kBlock), 0, s, ws, nz, count, s_t, y);
    return hipGetLastError();
}

hipError_t launch_prefill(const uint8_t* w, float s_t, int64_t n, int64_t k, const uint16_t* x,
                          int64_t m, uint16_t* y, hipStream_t s) {
    const int64_t soff = scale_plane_offset(QG_NVFP4, n, k);
    if (m <= 128 && k % kSmBK == 0) {
        const dim3 grid(unsigned((n + kSmRows - 1) / kSmRows));
        if (m > 64)
            hipLaunchKernelGGL(k_prefill_sm<2>, grid, dim3(kSmThreads), 0, s, w, soff, s_t, int(n), int(k), x, int(m), y);
        else
            hipLaunchKernelGGL(k_prefill_sm<1>, grid, dim3(kSmThreads), 0, s, w, soff, s_t, int(n), int(k), x, int(m), y);
        return hipGetLastError();
    }
    if (m <= 128) {
        constexpr int MB = 4, NB = 3;
        const dim3 grid(unsigned((n + 16 * NB - 1) / (16 * NB)), unsigned((m + 16 * MB - 1) / (16 * MB)));
        hipLaunchKernelGGL((k_prefill_ks<MB, NB>), grid, dim3(kBlock), 0, s, w, soff, s_t, int(n), int(k), x,
                           int(m), y);
        return hipGetLastError();
    }
    if (k % kP8BK == 0) {
        constexpr int MB = 8, NB = 3, BN = 16 * NB * 4, BM = 16 * MB;
        const dim3 grid(unsigned((n + BN - 1) / BN), unsigned((m + BM - 1) / BM));
        hipLaunchKernelGGL((k_prefill8<MB, NB>), grid, dim3(512), 0, s, w, soff, s_t, int(n), int(k), x, int(m), y);
        return hipGetLastError();
    }
    return go<8, 3, 4, 1, 4>(w, soff, s_t, n, k, x, m, y, s);
}

}  // namespace qg
