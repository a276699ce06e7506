// MoE decode on gfx950: softmax top-k router, expert-major grouping, grouped
// gate/up GEMV with SwiGLU, grouped down GEMV and the weighted combine.
//
// The pages batch routed (token, expert) pairs expert-major so that every
// active expert's weights are streamed once for all its tokens (bw24 README,
// MoE feature entry: expert-major CSR batching), and keep routing on the device
// (bw24 README, CUDA-graph decode: a few bytes of host traffic per token).
// Here a layer is three launches on one stream:
//   1. k_route_topk       logits -> ids, weights (one wave per token)
//   2. k_moe_gate_up      every workgroup rebuilds the CSR from ids in LDS (a
//                         few hundred integer ops), then one (expert group x
//                         row tile) of the grouped gate/up GEMV + SwiGLU;
//                         workgroup (0,0) also publishes the CSR in the
//                         workspace
//   3. k_moe_down         one row tile of the grouped down GEMV, one wave per
//                         expert group, then the weighted sum of the routed
//                         outputs in slot order plus the shared expert, done
//                         inside the workgroup through LDS
// Grids are sized for the worst case (t * top_k + 1 groups); workgroups whose
// group does not exist return at once.
#include <hip/hip_runtime.h>

#include "qg_device.hpp"
#include "qg_gemv_core.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"

namespace qg {

namespace {

constexpr int kBlock = 256;
constexpr int kMaxTokens = QG_MAX_M;
constexpr int kMaxTopK = 8;
constexpr int kMaxPairs = kMaxTokens * (kMaxTopK + 1);

// ------------------------------------------------------------------ router

// (value, index) pair order of the router: larger logit first, ties to the
// lower expert index; index kNoExpert marks an empty slot (always last).
constexpr int kNoExpert = 0x7fffffff;

__device__ __forceinline__ bool route_better(float v, int i, float bv, int bi) {
    return i != kNoExpert && (bi == kNoExpert || v > bv || (v == bv && i < bi));
}

template <int CTRL>
__device__ __forceinline__ void route_step_dpp(float& bv, int& bi) {
    const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xf, 0xf, false));
    const int oi = __builtin_amdgcn_update_dpp(kNoExpert, bi, CTRL, 0xf, 0xf, false);
    if (route_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
    }
}

// Wave-wide best (value, index): the same fixed butterfly as group_sum
// (DPP within rows of 16, a swizzle across rows, then the two 32-lane halves);
// every lane returns the winner.
__device__ __forceinline__ void route_wave_best(float& bv, int& bi) {
    route_step_dpp<0xB1>(bv, bi);   // lane ^ 1
    route_step_dpp<0x4E>(bv, bi);   // lane ^ 2
    route_step_dpp<0x141>(bv, bi);  // half-row mirror
    route_step_dpp<0x140>(bv, bi);  // row mirror
    {
        const float ov = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(bv), 0x401F));
        const int oi = __builtin_amdgcn_ds_swizzle(bi, 0x401F);
        if (route_better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
    const int i0 = __builtin_amdgcn_readlane(bi, 0);
    const float v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 32));
    const int i1 = __builtin_amdgcn_readlane(bi, 32);
    const bool second = route_better(v1, i1, v0, i0);
    bv = second ? v1 : v0;
    bi = second ? i1 : i0;
}

// Top-k of one token's e logits by the calling wave (e <= 64 * PER).  Lane s
// (s < top_k) returns selection s: its logit in sel_v, its expert in sel_i and
// its renormalised softmax weight in sel_w.  All lanes must call it.
template <int PER>
__device__ __forceinline__ void route_one_token(const float* __restrict__ logits, int e, int top_k,
                                                float& sel_v, int& sel_i, float& sel_w) {
    const int lane = lane_id();
    float v[PER];
    bool taken[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int ex = i * kWave + lane;
        const int exs = ex < e ? ex : 0;
        v[i] = logits[exs];
        taken[i] = ex >= e;
    }
    sel_v = 0.f;
    sel_i = kNoExpert;
    for (int s = 0; s < top_k; ++s) {
        float bv = 0.f;
        int bi = kNoExpert;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (!taken[i] && route_better(v[i], i * kWave + lane, bv, bi)) {
                bv = v[i];
                bi = i * kWave + lane;
            }
        route_wave_best(bv, bi);
        if (lane == s) {
            sel_v = bv;
            sel_i = bi;
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) taken[i] = taken[i] || (i * kWave + lane == bi);
    }
    // weights: exp(l - l_max) / sum over the selection, summed in slot order
    const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_v), 0));
    const float ex = lane < top_k ? expf(sel_v - vmax) : 0.f;
    float sum = 0.f;
    for (int s = 0; s < top_k; ++s) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), s));
    sel_w = ex / sum;
}

// One wave per token.
template <int PER>
__global__ __launch_bounds__(kBlock) void k_route_topk(const float* __restrict__ logits, int t, int e,
                                                       int top_k, int32_t* __restrict__ ids,
                                                       float* __restrict__ wts) {
    const int tok = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * (kBlock / kWave) + int(threadIdx.x) / kWave);
    if (tok >= t) return;  // uniform per wave
    float sv, sw;
    int si;
    route_one_token<PER>(logits + int64_t(tok) * e, e, top_k, sv, si, sw);
    const int lane = lane_id();
    if (lane < top_k) {
        ids[int64_t(tok) * top_k + lane] = si;
        wts[int64_t(tok) * top_k + lane] = sw;
    }
}

// ------------------------------------------------------------------ grouping

struct Csr {
    int n_groups;
    int experts[kMaxPairs];
    int offsets[kMaxPairs + 1];
    int tok[kMaxPairs];
    int slot[kMaxPairs];
};

// Expert-major CSR of the t*k routed pairs (pair p = token p/k, slot p%k):
// active experts ascending, pairs inside an expert in ascending (token, slot)
// order, then the shared expert with every token.  Ids are clamped into
// [0, E) so that bad ids can never index outside the expert arrays.
__device__ void build_csr(const int32_t* __restrict__ ids, int t, int k, int E, int has_shared,
                          Csr& c, int* s_e, int* s_first) {
    const int P = t * k;
    const int tid = int(threadIdx.x);
    for (int p = tid; p < P; p += kBlock) s_e[p] = min(max(ids[p], 0), E - 1);
    __syncthreads();
    for (int p = tid; p < P; p += kBlock) {
        const int e = s_e[p];
        int less = 0, before = 0;
        for (int q = 0; q < P; ++q) {
            const int eq = s_e[q];
            less += eq < e;
            before += (q < p) & (eq == e);
        }
        const int rank = less + before;
        c.tok[rank] = p / k;
        c.slot[rank] = p % k;
        s_first[p] = (before == 0) ? less + 1 : 0;  // 1 + offset of the group, or 0
    }
    __syncthreads();
    for (int p = tid; p < P; p += kBlock) {
        if (s_first[p]) {
            const int e = s_e[p];
            int g = 0;
            for (int q = 0; q < P; ++q) g += (s_first[q] != 0) & (s_e[q] < e);
            c.experts[g] = e;
            c.offsets[g] = s_first[p] - 1;
        }
    }
    if (tid == 0) {
        int U = 0;
        for (int q = 0; q < P; ++q) U += s_first[q] != 0;
        c.offsets[U] = P;
        if (has_shared) {
            c.experts[U] = E;
            c.offsets[U + 1] = P + t;
        }
        c.n_groups = U + (has_shared ? 1 : 0);
    }
    if (has_shared)
        for (int i = tid; i < t; i += kBlock) {
            c.tok[P + i] = i;
            c.slot[P + i] = k;
        }
    __syncthreads();
}

struct MoeArgs {
    int E, k, has_shared, flags;
    int H, I;
    const uint8_t* gate_up;
    int64_t gu_stride;
    const uint8_t* down;
    int64_t dn_stride;
    const float* gu_scale;
    const float* dn_scale;
};

// ------------------------------------------------------------------ gate/up + SwiGLU

// blockIdx.y = expert group, blockIdx.x = tile of a-rows.  Each group of G
// lanes owns RA a-rows (RA gate rows and the RA matching up rows).
// ROUTE: the workgroup first routes every token itself from the logits
// (route_one_token, one wave per token) into LDS; workgroup (0,0) publishes
// the ids and weights in the workspace for the down kernel.
template <int MT, int G, int C, int RA, bool ROUTE, int PER>
__global__ __launch_bounds__(kBlock) void k_moe_gate_up(MoeArgs A, const uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ ids_in,
                                                        const float* __restrict__ logits, int t,
                                                        MoeWorkspace ws) {
    __shared__ Csr c;
    __shared__ int s_e[kMaxPairs], s_first[kMaxPairs];
    __shared__ int s_ids[kMaxTokens * kMaxTopK];
    const int tid = int(threadIdx.x);
    const int32_t* ids = ids_in;
    if constexpr (ROUTE) {
        const int lane = lane_id();
        for (int tok = tid / kWave; tok < t; tok += kBlock / kWave) {  // uniform per wave
            float sv, sw;
            int si;
            route_one_token<PER>(logits + int64_t(tok) * A.E, A.E, A.k, sv, si, sw);
            if (lane < A.k) {
                s_ids[tok * A.k + lane] = si;
                if (blockIdx.x == 0 && blockIdx.y == 0) {
                    ws.ids[tok * A.k + lane] = si;
                    ws.wts[tok * A.k + lane] = sw;
                }
            }
        }
        __syncthreads();
        ids = s_ids;
    }
    build_csr(ids, t, A.k, A.E, A.has_shared, c, s_e, s_first);
    if (blockIdx.x == 0 && blockIdx.y == 0) {
        const int P = t * (A.k + A.has_shared);
        if (tid == 0) *ws.n_groups = c.n_groups;
        for (int i = tid; i < P; i += kBlock) {
            ws.pair_tok[i] = c.tok[i];
            ws.pair_slot[i] = c.slot[i];
        }
        for (int i = tid; i < c.n_groups; i += kBlock) ws.experts[i] = c.experts[i];
        for (int i = tid; i <= c.n_groups; i += kBlock) ws.offsets[i] = c.offsets[i];
    }
    const int g = int(blockIdx.y);
    if (g >= c.n_groups) return;
    const int e = c.experts[g];
    const int p0 = c.offsets[g];
    const int mg = c.offsets[g + 1] - p0;

    constexpr int R = 2 * RA;
    constexpr int kGroups = kWave / G;
    const int lane = lane_id();
    const int grp = lane / G, l = lane % G;
    const int wave = int(blockIdx.x) * (kBlock / kWave) + tid / kWave;
    const int unit = wave * kGroups + grp;
    const int I = A.I, H = A.H;

    const uint8_t* w = A.gate_up + int64_t(e) * A.gu_stride;
    const int64_t soff = scale_plane_offset(QG_NVFP4, 2 * int64_t(I), H);
    const float s_t = A.gu_scale[e];
    // gate/up rows are interleaved in the packed matrix: R consecutive rows
    int rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = min(unit * R + r, 2 * I - 1);
    const uint8_t* codes[R];
    const uint8_t* scales[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        codes[r] = w + int64_t(rows[r]) * (H / 2);
        scales[r] = w + soff + int64_t(rows[r]) * (H / 16);
    }
    const uint16_t* xp[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) xp[i] = x + int64_t(c.tok[p0 + (i < mg ? i : 0)]) * H;

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[r][i] = 0.f;
    nvfp4_partial<R, MT, G, C>(codes, scales, xp, mg, H / 32, l, acc);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[r][i] = group_sum<G>(acc[r][i]) * s_t;
    if (l != 0) return;
#pragma unroll
    for (int r = 0; r < RA; ++r) {
        const int row = unit * RA + r;
        if (row >= I) break;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (i < mg) {
                const int p = p0 + i;
                const float gv = acc[2 * r][i], uv = acc[2 * r + 1][i];
                const float act = gv / (1.0f + expf(-gv)) * uv;
                ws.a[int64_t(p) * I + row] = uint16_t(f32_to_bf16_rne(act));
                if (ws.h) {
                    ws.h[int64_t(p) * 2 * I + row] = gv;
                    ws.h[int64_t(p) * 2 * I + I + row] = uv;
                }
            }
        }
    }
}

// ------------------------------------------------------------------ down + combine

// blockIdx.x = tile of output rows; the workgroup has one wave per expert
// group (up to 16; wave w takes groups w, w+16, ...).  Every wave computes
// its groups' down outputs for the tile into LDS, then the workgroup sums them
// per token in slot order plus the shared expert: a fixed order, and no
// synchronisation between workgroups.
template <int MT, int G, int C, int R>
__global__ __launch_bounds__(1024) void k_moe_down(MoeArgs A, const float* __restrict__ wts, int t,
                                                   float* __restrict__ y, MoeWorkspace ws) {
    constexpr int kGroups = kWave / G;
    constexpr int kRows = kGroups * R;  // rows per tile
    __shared__ int s_off[kMaxPairs + 1];
    __shared__ int s_exp[kMaxPairs];
    __shared__ int s_pair[kMaxTokens][kMaxTopK + 1];
    __shared__ float s_o[kMaxPairs][kRows];
    const int tid = int(threadIdx.x);
    const int nthreads = int(blockDim.x);
    const int nw = nthreads / kWave;
    const int ng = *ws.n_groups;
    const int P = t * (A.k + A.has_shared);
    for (int i = tid; i <= ng; i += nthreads) s_off[i] = ws.offsets[i];
    for (int i = tid; i < ng; i += nthreads) s_exp[i] = ws.experts[i];
    for (int i = tid; i < P; i += nthreads) s_pair[ws.pair_tok[i]][ws.pair_slot[i]] = i;
    __syncthreads();

    const int lane = lane_id();
    const int grp = lane / G, l = lane % G;
    const int I = A.I, H = A.H;
    const int tile0 = int(blockIdx.x) * kRows;
    const int64_t soff = scale_plane_offset(QG_NVFP4, H, I);
    for (int g = tid / kWave; g < ng; g += nw) {  // uniform per wave
        const int e = s_exp[g];
        const int p0 = s_off[g];
        const int mg = s_off[g + 1] - p0;
        const uint8_t* w = A.down + int64_t(e) * A.dn_stride;
        const float s_t = A.dn_scale[e];
        const uint8_t* codes[R];
        const uint8_t* scales[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(tile0 + grp * R + r, H - 1);
            codes[r] = w + int64_t(row) * (I / 2);
            scales[r] = w + soff + int64_t(row) * (I / 16);
        }
        const uint16_t* xp[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) xp[i] = ws.a + int64_t(p0 + (i < mg ? i : 0)) * I;
        float acc[R][MT];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[r][i] = 0.f;
        nvfp4_partial<R, MT, G, C>(codes, scales, xp, mg, I / 32, l, acc);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[r][i] = group_sum<G>(acc[r][i]) * s_t;
        if (l == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = tile0 + grp * R + r;
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    if (i < mg) {
                        s_o[p0 + i][grp * R + r] = acc[r][i];
                        if (row < H) ws.o[int64_t(p0 + i) * H + row] = acc[r][i];
                    }
                }
            }
        }
    }
    __syncthreads();
    for (int idx = tid; idx < t * kRows; idx += nthreads) {
        const int tt = idx / kRows, rr = idx % kRows;
        const int row = tile0 + rr;
        if (row >= H) continue;
        float sum = 0.f;
        for (int s = 0; s < A.k; ++s) sum = fmaf(wts[int64_t(tt) * A.k + s], s_o[s_pair[tt][s]][rr], sum);
        if (A.has_shared) sum += s_o[s_pair[tt][A.k]][rr];
        y[int64_t(tt) * H + row] = sum;
    }
}

// C = 1 when a row fits in one chunk per lane, else the runtime chunk loop.
template <int MT, int GU, int CU, int GD, int CD>
hipError_t moe_go(const MoeArgs& A, const uint16_t* x, const int32_t* ids, const float* w, const float* logits,
                  int t, float* y, const MoeWorkspace& ws, hipStream_t s) {
    constexpr int RA = 2;
    const int max_groups = t * A.k + (A.has_shared ? 1 : 0);
    const int a_rows_per_block = (kBlock / kWave) * (kWave / GU) * RA;
    const dim3 g1((A.I + a_rows_per_block - 1) / a_rows_per_block, max_groups);
    if (logits) {
        const int per = (A.E + kWave - 1) / kWave;
        if (per <= 4)
            hipLaunchKernelGGL((k_moe_gate_up<MT, GU, CU, RA, true, 4>), g1, dim3(kBlock), 0, s, A, x, nullptr,
                               logits, t, ws);
        else
            hipLaunchKernelGGL((k_moe_gate_up<MT, GU, CU, RA, true, 16>), g1, dim3(kBlock), 0, s, A, x, nullptr,
                               logits, t, ws);
        w = ws.wts;
    } else {
        hipLaunchKernelGGL((k_moe_gate_up<MT, GU, CU, RA, false, 1>), g1, dim3(kBlock), 0, s, A, x, ids, nullptr,
                           t, ws);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    constexpr int kRowsDown = kWave / GD;  // one row per lane group
    const int waves = max_groups < 16 ? max_groups : 16;
    const dim3 g2((A.H + kRowsDown - 1) / kRowsDown);
    hipLaunchKernelGGL((k_moe_down<MT, GD, CD, 1>), g2, dim3(kWave * waves), 0, s, A, w, t, y, ws);
    return hipGetLastError();
}

template <int MT, int GU, int CU>
hipError_t moe_down_shape(const MoeArgs& A, const uint16_t* x, const int32_t* ids, const float* w,
                          const float* logits, int t, float* y, const MoeWorkspace& ws, hipStream_t s) {
    const int jd = A.I / 32;
    if (lanes_per_row(jd) == 64)
        return jd <= 64 ? moe_go<MT, GU, CU, 64, 1>(A, x, ids, w, logits, t, y, ws, s)
                        : moe_go<MT, GU, CU, 64, 0>(A, x, ids, w, logits, t, y, ws, s);
    return jd <= 16 ? moe_go<MT, GU, CU, 16, 1>(A, x, ids, w, logits, t, y, ws, s)
                    : moe_go<MT, GU, CU, 16, 0>(A, x, ids, w, logits, t, y, ws, s);
}

template <int MT>
hipError_t moe_mt(const MoeArgs& A, const uint16_t* x, const int32_t* ids, const float* w, const float* logits,
                  int t, float* y, const MoeWorkspace& ws, hipStream_t s) {
    const int ju = A.H / 32;
    if (lanes_per_row(ju) == 64)
        return ju <= 64 ? moe_down_shape<MT, 64, 1>(A, x, ids, w, logits, t, y, ws, s)
                        : moe_down_shape<MT, 64, 0>(A, x, ids, w, logits, t, y, ws, s);
    return ju <= 16 ? moe_down_shape<MT, 16, 1>(A, x, ids, w, logits, t, y, ws, s)
                    : moe_down_shape<MT, 16, 0>(A, x, ids, w, logits, t, y, ws, s);
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int64_t t, int e, int top_k, int32_t* ids, float* w,
                             hipStream_t s) {
    const dim3 grid(unsigned((t + 3) / 4));
    const int per = (e + kWave - 1) / kWave;
    if (per <= 1)
        hipLaunchKernelGGL(k_route_topk<1>, grid, dim3(kBlock), 0, s, logits, int(t), e, top_k, ids, w);
    else if (per <= 4)
        hipLaunchKernelGGL(k_route_topk<4>, grid, dim3(kBlock), 0, s, logits, int(t), e, top_k, ids, w);
    else
        hipLaunchKernelGGL(k_route_topk<16>, grid, dim3(kBlock), 0, s, logits, int(t), e, top_k, ids, w);
    return hipGetLastError();
}

// Workspace regions, each 256-byte aligned, in the documented order.  With
// base == nullptr only the size is computed.
size_t moe_workspace_layout(const qg_moe_desc* d, int64_t t, MoeWorkspace* ws, void* base) {
    const int64_t P = t * (d->top_k + (d->has_shared ? 1 : 0));
    const int64_t H = d->hidden, I = d->inter;
    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        const int64_t at = off;
        off = align_up(off + bytes, kPlaneAlign);
        return at;
    };
    const int64_t o_ng = take(4);
    const int64_t o_ex = take(4 * P);
    const int64_t o_off = take(4 * (P + 1));
    const int64_t o_tok = take(4 * P);
    const int64_t o_slot = take(4 * P);
    const int64_t o_a = take(2 * P * I);
    const int64_t o_h = (d->flags & QG_MOE_KEEP_H) ? take(4 * P * 2 * I) : -1;
    const int64_t o_o = take(4 * P * H);
    const int64_t o_ids = take(4 * t * d->top_k);
    const int64_t o_wts = take(4 * t * d->top_k);
    if (ws && base) {
        char* b = static_cast<char*>(base);
        ws->n_groups = reinterpret_cast<int32_t*>(b + o_ng);
        ws->experts = reinterpret_cast<int32_t*>(b + o_ex);
        ws->offsets = reinterpret_cast<int32_t*>(b + o_off);
        ws->pair_tok = reinterpret_cast<int32_t*>(b + o_tok);
        ws->pair_slot = reinterpret_cast<int32_t*>(b + o_slot);
        ws->a = reinterpret_cast<uint16_t*>(b + o_a);
        ws->h = o_h >= 0 ? reinterpret_cast<float*>(b + o_h) : nullptr;
        ws->o = reinterpret_cast<float*>(b + o_o);
        ws->ids = reinterpret_cast<int32_t*>(b + o_ids);
        ws->wts = reinterpret_cast<float*>(b + o_wts);
    }
    return size_t(off);
}

hipError_t launch_moe(const qg_moe_desc* d, const uint16_t* x, const int32_t* ids, const float* w,
                      const float* logits, int t, float* y, const MoeWorkspace& ws, hipStream_t s) {
    MoeArgs A;
    A.E = d->n_experts;
    A.k = d->top_k;
    A.has_shared = d->has_shared ? 1 : 0;
    A.flags = d->flags;
    A.H = int(d->hidden);
    A.I = int(d->inter);
    A.gate_up = static_cast<const uint8_t*>(d->gate_up);
    A.gu_stride = d->gate_up_stride;
    A.down = static_cast<const uint8_t*>(d->down);
    A.dn_stride = d->down_stride;
    A.gu_scale = d->gate_up_scale;
    A.dn_scale = d->down_scale;
    switch (token_class(t)) {
        case 1: return moe_mt<1>(A, x, ids, w, logits, t, y, ws, s);
        case 4: return moe_mt<4>(A, x, ids, w, logits, t, y, ws, s);
        default: return moe_mt<16>(A, x, ids, w, logits, t, y, ws, s);
    }
}

}  // namespace qg
