// MoE decode on gfx950: softmax top-k router, expert-major grouping, grouped
// gate/up GEMV with SwiGLU, grouped down GEMV and the weighted combine.
//
// The pages batch routed (token, expert) pairs expert-major so that every
// active expert's weights are streamed once for all its tokens (bw24 README,
// MoE feature entry: expert-major CSR batching), and keep routing on the device
// (bw24 README, CUDA-graph decode: a few bytes of host traffic per token).
// A layer is two launches on one stream:
//   1. gate/up: the routing (moe_forward: one wave per token, from the logits;
//      moe_gemv_grouped: ids given) and the expert-major grouping are done
//      inside every workgroup (a CSR in LDS, or for two to four tokens
//      ballots over the routed ids), then the grouped gate/up GEMV + SwiGLU;
//      the first workgroup publishes routing and CSR in the workspace;
//   2. down: the grouped down GEMV, then the weighted sum of the routed
//      outputs in slot order plus the shared expert, inside the workgroup
//      through LDS (no synchronisation between workgroups).
// One token: a workgroup per (expert group, row tile), grids sized for the
// worst case (t * top_k + 1 groups), absent groups return at once.  Two to
// four tokens: the tile path below, one workgroup per row tile holding every
// group.  moe_route_topk is the routing alone.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "qg_device.hpp"
#include "qg_gemv_core.hpp"
#include "qg_internal.hpp"
#include "qg_layout.hpp"
#include "qg_mfma.hpp"

namespace qg {

namespace {

constexpr int kBlock = 256;
constexpr int kMaxTokens = QG_MAX_M;
constexpr int kMaxTopK = 8;
constexpr int kMaxPairs = kMaxTokens * (kMaxTopK + 1);
// Per-expert tensor scales are staged in LDS at kernel start (their load then
// overlaps the routing instead of trailing the GEMV) for up to this many
// experts including the shared one; larger rosters read them from memory.
constexpr int kMaxScaleLds = 1025;
static_assert(kMaxTokens * kMaxTopK <= kBlock, "build_csr gives each routed pair its own thread");
static_assert(kMaxPairs % 4 == 0 && kMaxPairs >= kMaxTokens * kMaxTopK, "CSR scratch is read four entries at a time");

// ------------------------------------------------------------------ router

// Router keys.  A logit v of expert i becomes the 64-bit key
// (order(v) << 32) | ~i, where order() maps the fp32 bit pattern to an
// unsigned integer with the same order as the values (-0 counts as +0, NaN
// below every number); a larger key is a larger logit, ties going to the
// lower expert index.  Key 0 marks an empty slot and loses to every logit.
__device__ __forceinline__ uint64_t route_key(float v, int i) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;  // -0 == +0
    uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    if (v != v) ord = 1u;          // NaN: below every number
    return (uint64_t(ord) << 32) | uint64_t(~uint32_t(i));
}

__device__ __forceinline__ float route_key_value(uint64_t key) {
    const uint32_t ord = uint32_t(key >> 32);
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

__device__ __forceinline__ int route_key_index(uint64_t key) { return int(~uint32_t(key)); }

// One DPP exchange of a wave-wide unsigned maximum.  Lanes of rows outside
// ROW_MASK (and lanes without a source) see 0, the identity of the maximum,
// so the exchange folds into one v_max_u32 with a DPP operand.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t route_max_step(uint32_t v) {
    const uint32_t o = __builtin_amdgcn_update_dpp(0u, v, CTRL, ROW_MASK, 0xf, false);
    return o > v ? o : v;
}

// Largest value of the wave, returned to every lane: butterflies inside rows
// of 16 lanes, then row broadcasts that leave the total in lane 63.
__device__ __forceinline__ uint32_t route_wave_max(uint32_t v) {
    v = route_max_step<0xB1>(v);        // quad_perm [1,0,3,2]
    v = route_max_step<0x4E>(v);        // quad_perm [2,3,0,1]
    v = route_max_step<0x141>(v);       // row_half_mirror
    v = route_max_step<0x140>(v);       // row_mirror: every lane holds its row's maximum
    v = route_max_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = route_max_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __builtin_amdgcn_readlane(v, 63);
}

// Loads of one token's e logits for route_select (e <= 64 * PER): lane l
// gets logits l, l + 64, ...  All loads are unconditional, at clamped (valid)
// addresses, so they are in flight together.
template <int PER>
__device__ __forceinline__ void route_load(const float* __restrict__ logits, int e, float (&v)[PER]) {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = logits[min(i * kWave + lane, e - 1)];
}

// Top-k of one token's logits (loaded by route_load) by the calling wave.
// Lane s (s < top_k) returns selection s: its logit in sel_v, its expert in
// sel_i and its renormalised softmax weight in sel_w.  All lanes must call
// it.  Each lane sorts its PER keys once; a round takes the wave maximum of
// the lanes' leading keys and the winning lane moves to its next key.
template <int PER>
__device__ __forceinline__ void route_select(const float (&v)[PER], int e, int top_k, float& sel_v, int& sel_i,
                                             float& sel_w) {
    const int lane = lane_id();
    uint64_t key[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int ex = i * kWave + lane;
        const uint64_t keep = ex < e ? ~0ull : 0ull;  // slots past e: key 0
        key[i] = route_key(v[i], ex) & keep;
    }
    // descending insertion sort of the lane's keys (a fixed network)
#pragma unroll
    for (int i = 1; i < PER; ++i)
#pragma unroll
        for (int j = i; j > 0; --j) {
            const uint64_t a = key[j - 1], b = key[j];
            key[j - 1] = a > b ? a : b;
            key[j] = a > b ? b : a;
        }
    // A round's maximum is taken over the keys' high words (the logit order)
    // alone; the low word (~expert) decides only among lanes whose leading
    // logits are equal, in a second reduction that is skipped when one lane
    // holds the maximum (the usual case).  The result is the 64-bit key
    // maximum either way.
    uint64_t mine = 0;
    for (int s = 0; s < top_k; ++s) {
        const uint32_t hi = uint32_t(key[0] >> 32);
        const uint32_t m = route_wave_max(hi);
        const uint64_t tie = __ballot(hi == m);
        const uint32_t lo = __popcll(tie) == 1
                                ? __builtin_amdgcn_readlane(uint32_t(key[0]), __builtin_ctzll(tie))
                                : route_wave_max(hi == m ? uint32_t(key[0]) : 0u);
        const uint64_t best = (uint64_t(m) << 32) | lo;
        if (lane == s) mine = best;
        if (key[0] == best) {  // the winner (keys are distinct) moves to its next key
#pragma unroll
            for (int i = 0; i + 1 < PER; ++i) key[i] = key[i + 1];
            key[PER - 1] = 0;
        }
    }
    sel_v = route_key_value(mine);
    sel_i = route_key_index(mine);
    // weights: exp(l - l_max) / sum over the selection, summed in slot order
    const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_v), 0));
    const float ex = lane < top_k ? expf(sel_v - vmax) : 0.f;
    float sum = 0.f;
    for (int s = 0; s < top_k; ++s) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), s));
    sel_w = ex / sum;
}

template <int PER>
__device__ __forceinline__ void route_one_token(const float* __restrict__ logits, int e, int top_k,
                                                float& sel_v, int& sel_i, float& sel_w) {
    float v[PER];
    route_load<PER>(logits, e, v);
    route_select<PER>(v, e, top_k, sel_v, sel_i, sel_w);
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
// [0, E) so that bad ids can never index outside the expert arrays.  Thread p
// handles pair p (t*k <= kBlock); s_e and s_first hold at least t*k rounded up
// to 4 entries, 16-byte aligned, and are read four at a time.
__device__ void build_csr(const int32_t* __restrict__ ids, int t, int k, int E, int has_shared,
                          Csr& c, int* s_e, int* s_first) {
    const int P = t * k;
    const int P4 = (P + 3) & ~3;
    const int p = int(threadIdx.x);
    const int e = p < P ? min(max(ids[p], 0), E - 1) : 0x7fffffff;  // padding sorts after every expert
    if (p < P4) s_e[p] = e;
    lds_barrier();
    int less = 0, before = 0;  // pairs of a smaller expert; earlier pairs of the same expert
    if (p < P) {
#pragma unroll 4
        for (int q = 0; q < P4; q += 4) {
            const int4 v = *reinterpret_cast<const int4*>(s_e + q);
            less += int(v.x < e) + int(v.y < e) + int(v.z < e) + int(v.w < e);
            before += int(v.x == e && q < p) + int(v.y == e && q + 1 < p) + int(v.z == e && q + 2 < p) +
                      int(v.w == e && q + 3 < p);
        }
        const int rank = less + before;
        c.tok[rank] = p / k;
        c.slot[rank] = p % k;
    }
    const bool first = p < P && before == 0;  // the expert's first pair
    if (p < P4) s_first[p] = first ? 1 : 0;
    lds_barrier();
    if (first) {
        int g = 0;  // active experts below e
#pragma unroll 4
        for (int q = 0; q < P4; q += 4) {
            const int4 v = *reinterpret_cast<const int4*>(s_e + q);
            const int4 f = *reinterpret_cast<const int4*>(s_first + q);
            g += (f.x & int(v.x < e)) + (f.y & int(v.y < e)) + (f.z & int(v.z < e)) + (f.w & int(v.w < e));
        }
        c.experts[g] = e;
        c.offsets[g] = less;
    }
    if (p == 0) {
        int U = 0;  // active experts
#pragma unroll 4
        for (int q = 0; q < P4; q += 4) {
            const int4 f = *reinterpret_cast<const int4*>(s_first + q);
            U += f.x + f.y + f.z + f.w;
        }
        c.offsets[U] = P;
        if (has_shared) {
            c.experts[U] = E;
            c.offsets[U + 1] = P + t;
        }
        c.n_groups = U + (has_shared ? 1 : 0);
    }
    if (has_shared && p < t) {
        c.tok[P + p] = p;
        c.slot[P + p] = k;
    }
    lds_barrier();
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
    __shared__ __align__(16) int s_e[kMaxPairs];
    __shared__ __align__(16) int s_first[kMaxPairs];
    __shared__ int s_ids[kMaxTokens * kMaxTopK];
    __shared__ float s_scale[kMaxScaleLds];
    const int tid = int(threadIdx.x);
    const int32_t* ids = ids_in;
    const int n_scales = A.E + A.has_shared;
    // One routed token: its k experts are distinct, so group k is the shared
    // expert, with pair k.  Its workgroups need neither the routing nor the
    // CSR and request their rows at once.
    const bool shared_only = ROUTE && t == 1 && A.has_shared && int(blockIdx.y) == A.k;
    const bool scales_in_lds = n_scales <= kMaxScaleLds && !shared_only;
    // The scales go to LDS (visible after the CSR barrier) through the waves
    // that do not route when there are such, so that a routing wave's first
    // request is its logits.
    const int w0 = ROUTE && t < kBlock / kWave ? t : 0;  // first staging wave
    if (scales_in_lds && tid >= w0 * kWave)
        for (int i = tid - w0 * kWave; i < n_scales; i += kBlock - w0 * kWave) s_scale[i] = A.gu_scale[i];
    bool csr_done = shared_only;
    if constexpr (ROUTE) {
        if (!shared_only) {
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
                if (t == 1) {
                    // One token: its k experts are distinct, so the CSR is their
                    // ascending order, one pair each (what build_csr produces),
                    // written by this wave -- one barrier instead of four.
                    int rank = 0;
                    for (int j = 0; j < A.k; ++j) rank += int(__builtin_amdgcn_readlane(si, j) < si);
                    if (lane < A.k) {
                        c.experts[rank] = si;
                        c.offsets[rank] = rank;
                        c.tok[rank] = 0;
                        c.slot[rank] = lane;
                    }
                    if (lane == 0) {
                        c.offsets[A.k] = A.k;
                        if (A.has_shared) {
                            c.experts[A.k] = A.E;
                            c.offsets[A.k + 1] = A.k + 1;
                            c.tok[A.k] = 0;
                            c.slot[A.k] = A.k;
                        }
                        c.n_groups = A.k + A.has_shared;
                    }
                }
            }
            __syncthreads();
            ids = s_ids;
            csr_done = t == 1;
        }
    }
    if (!csr_done) build_csr(ids, t, A.k, A.E, A.has_shared, c, s_e, s_first);
    if (blockIdx.x == 0 && blockIdx.y == 0) {  // never a shared_only workgroup (k >= 1)
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
    if (!shared_only && g >= c.n_groups) return;
    const int e = shared_only ? A.E : c.experts[g];
    const int p0 = shared_only ? A.k : c.offsets[g];
    const int mg = shared_only ? 1 : c.offsets[g + 1] - p0;

    constexpr int R = 2 * RA;
    constexpr int kGroups = kWave / G;
    const int lane = lane_id();
    const int grp = lane / G, l = lane % G;
    const int wave = int(blockIdx.x) * (kBlock / kWave) + tid / kWave;
    const int unit = wave * kGroups + grp;
    const int I = A.I, H = A.H;

    const uint8_t* w = A.gate_up + int64_t(e) * A.gu_stride;
    const int64_t soff = scale_plane_offset(QG_NVFP4, 2 * int64_t(I), H);
    const float s_t = scales_in_lds ? s_scale[e] : A.gu_scale[e];
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
    for (int i = 0; i < MT; ++i) xp[i] = x + int64_t(shared_only ? 0 : c.tok[p0 + (i < mg ? i : 0)]) * H;

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[r][i] = 0.f;
    nvfp4_partial_m<R, MT, G, C>(codes, scales, xp, mg, H / 32, l, acc);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[r][i] = group_sum<G>(acc[r][i]) * s_t;
    // every lane of the group holds every sum: lane l evaluates the SwiGLU
    // of (a-row q / MT, token q % MT) for q = l, l + G, ..., side by side
    // rather than all on lane 0
#pragma unroll
    for (int q0 = 0; q0 < RA * MT; q0 += G) {
        const int q = q0 + l;
        float gv = 0.f, uv = 0.f;
#pragma unroll
        for (int r = 0; r < RA; ++r)
#pragma unroll
            for (int i = 0; i < MT; ++i)
                if (q == r * MT + i) {
                    gv = acc[2 * r][i];
                    uv = acc[2 * r + 1][i];
                }
        const int ra = q / MT, ti = q % MT;
        const int row = unit * RA + ra;
        if (q < RA * MT && ti < mg && row < I) {
            const int p = p0 + ti;
            const float act = gv / (1.0f + expf(-gv)) * uv;
            ws.a[int64_t(p) * I + row] = uint16_t(f32_to_bf16_rne(act));
            if (ws.h) {
                ws.h[int64_t(p) * 2 * I + row] = gv;
                ws.h[int64_t(p) * 2 * I + I + row] = uv;
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
    __shared__ float s_scale[kMaxScaleLds];
    const int tid = int(threadIdx.x);
    const int nthreads = int(blockDim.x);
    const int nw = nthreads / kWave;
    const int n_scales = A.E + A.has_shared;
    const bool scales_in_lds = n_scales <= kMaxScaleLds;
    if (scales_in_lds)
        for (int i = tid; i < n_scales; i += nthreads) s_scale[i] = A.dn_scale[i];  // visible after the barrier below
    // The CSR header is read up to the worst-case group count (the workspace
    // holds that many entries), so these loads do not wait for n_groups.
    const int ng = *ws.n_groups;
    const int P = t * (A.k + A.has_shared);
    const int gmax = t * A.k + A.has_shared;
    for (int i = tid; i <= gmax; i += nthreads) s_off[i] = ws.offsets[i];
    for (int i = tid; i < gmax; i += nthreads) s_exp[i] = ws.experts[i];
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
        const float s_t = scales_in_lds ? s_scale[e] : A.dn_scale[e];
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
        nvfp4_partial_m<R, MT, G, C>(codes, scales, xp, mg, I / 32, l, acc);
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

// ------------------------------------------------------------------ tile path (t <= 4)

// For two to four tokens the layer runs as two launches of kTileBlock-thread
// workgroups, one row tile per workgroup and every expert group in it: wave w
// takes groups w, w + 8, w + 16, ... and issues the weight loads of all of
// them before any arithmetic, while activations and per-expert scales sit in
// LDS (loaded at kernel start, alongside the routing).  The routing and the
// CSR are thus built once per workgroup rather than once per (group, tile),
// and with one workgroup per CU the grid is resident at once.  Eight waves
// per workgroup leave each wave up to 256 registers for the weights in
// flight; the down kernel with one chunk per lane fits in 128 and runs
// sixteen waves, so that each takes at most two routed groups (t = 4:
// 20.75 -> 20.45 us per layer; the gate/up kernel spills at sixteen waves
// and was 3.5 us slower).
constexpr int kTileBlock = 512;
constexpr int kTileWaves = kTileBlock / kWave;
constexpr int kTileMaxPairs = 4 * (kMaxTopK + 1);  // pairs of a tile-path call (t <= 4)
#ifndef QG_TILE_DEPTH
#define QG_TILE_DEPTH 1
#endif
#ifndef QG_TILE_DEPTH_DN
#define QG_TILE_DEPTH_DN 1
#endif
// Expert groups whose loads a wave keeps in flight ahead of the group it
// computes (gate/up, down).  Measured at four tokens on MI355X: one ahead
// 26.4 us, two 27.7 us, three 27.9 us, all groups at once 28.4 us; with the
// groups taken from ballots, one ahead 22.3 us against gate/up two ahead
// 23.2 us, down two ahead 22.5 us and four ahead 22.8 us.
constexpr int kTileDepth = QG_TILE_DEPTH;
constexpr int kTileDepthDn = QG_TILE_DEPTH_DN;
constexpr int kStageBytes = 64 * 1024;  // LDS activation staging per workgroup
static_assert(kMaxTokens * kMaxTopK <= kTileBlock, "build_csr gives each routed pair its own thread");

// One expert group's weights for one wave: R rows x C chunks per lane.
template <int C, int R>
struct GroupW {
    u32x4 cw[C][R];
    uint32_t sw[C][R];
};

template <int C, int R>
__device__ __forceinline__ void load_group_w(GroupW<C, R>& b, const uint8_t* const (&codes)[R],
                                             const uint8_t* const (&scales)[R], const uint32_t (&jc)[C]) {
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            b.cw[c][r] = ld_stream16(codes[r] + 16u * jc[c]);
            b.sw[c][r] = ld<uint16_t>(scales[r] + 2u * jc[c]);
        }
}

// Calls f(std::integral_constant<int, n>) for the runtime count n in
// [N, NMAX], so that f's body is straight-line code for that count.
template <int NMAX, int N = 1, typename F>
__device__ __forceinline__ void dispatch_count(int n, F&& f) {
    if constexpr (N <= NMAX) {
        if (n == N)
            f(std::integral_constant<int, N>{});
        else
            dispatch_count<NMAX, N + 1>(n, f);
    }
}

// Row sums of one token from a group's preloaded weights; the token's bf16
// activations at xl (LDS).  Same arithmetic and order per row as
// nvfp4_partial: chunks ascending, each 16-element block summed, scaled and
// added in order.  Tokens of a group are taken one at a time (the few groups
// with several tokens decode their chunks once per token).
template <int R, int C>
__device__ __forceinline__ void nvfp4_token_dot(const GroupW<C, R>& b, const bool (&okc)[C], const uint32_t (&jc)[C],
                                                const uint16_t* xl, float (&acc)[R]) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
        u32x4 xv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[q] = ld16(xl + 32u * jc[c] + 8u * q);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = nvfp4_chunk_dot(b.cw[c][r], b.sw[c][r], xv, acc[r]);
            acc[r] = okc[c] ? v : acc[r];
        }
    }
}

// Routing and CSR of a tile-path call for the down kernel (workspace header),
// by one wave: lane q < P = t*k (P <= 32) holds pair q's expert in idv, and
// s_ids[0, P) the same ids unclamped (padding is ignored).  The same CSR as
// build_csr: active experts ascending, pairs of an expert in (token, slot)
// order, then the shared expert with every token.  Per lane, bit q of lt / eq
// marks pairs of a smaller / the same expert.
__device__ __forceinline__ void publish_csr(int idv, const int* s_ids, int P, int t, int k, int E, int has_shared,
                                            const MoeWorkspace& ws) {
    const int lane = lane_id();
    uint32_t lt = 0, eq = 0;
#pragma unroll
    for (int q = 0; q < 32; q += 4) {
        const int4 v = *reinterpret_cast<const int4*>(s_ids + q);
        const int e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = min(max(e4[i], 0), E - 1);
            const bool ok = q + i < P;
            lt |= (ok && e < idv) ? 1u << (q + i) : 0u;
            eq |= (ok && e == idv) ? 1u << (q + i) : 0u;
        }
    }
    const uint32_t earlier = eq & (lane < 32 ? (1u << lane) - 1u : ~0u);  // lanes >= 32 hold no pair
    const bool first = lane < P && earlier == 0;       // the expert's first pair
    const uint32_t fmask = uint32_t(__ballot(first));
    const int less = __popc(lt), rank = less + __popc(earlier), g = __popc(lt & fmask);
    if (lane < P) {
        ws.pair_tok[rank] = lane / k;
        ws.pair_slot[rank] = lane % k;
        if (first) {
            ws.experts[g] = idv;
            ws.offsets[g] = less;
        }
    }
    const int U = __popc(fmask);
    if (lane == 0) {
        ws.offsets[U] = P;
        if (has_shared) {
            ws.experts[U] = E;
            ws.offsets[U + 1] = P + t;
        }
        *ws.n_groups = U + has_shared;
    }
    if (has_shared && lane < t) {
        ws.pair_tok[P + lane] = lane;
        ws.pair_slot[P + lane] = k;
    }
}

// Gate/up + SwiGLU, tile path.  blockIdx.x = tile of R consecutive packed
// rows (R/2 a-rows; gate/up rows interleaved), every group; a row of H/32
// chunks spread over the whole wave (G = 64).  ROUTE as in k_moe_gate_up.
// No CSR is built here: every wave holds the t*k routed experts one per lane
// and takes the pairs q = wave, wave + 8, ... that are their expert's first
// pair (so each active expert has one owner), finding the expert's other
// pairs and its place in the expert-major order with ballots.  The shared
// expert needs no routing: its token i goes to wave 7 - i, which requests the
// shared rows before anything else and computes them while its first routed
// group is in flight (the barrier before publishes LDS only, so those loads
// stay outstanding).  GW bounds the routed groups of one wave.
template <int C, int R, bool ROUTE, int PER, int GW>
__global__ __launch_bounds__(kTileBlock) void k_moe_gate_up_tile(MoeArgs A, const uint16_t* __restrict__ x,
                                                                 const int32_t* __restrict__ ids_in,
                                                                 const float* __restrict__ logits, int t,
                                                                 MoeWorkspace ws) {
    static_assert(R % 2 == 0, "gate and up rows come in pairs");
    __shared__ __align__(16) int s_ids[kMaxTokens * kMaxTopK];
    __shared__ float s_scale[kMaxScaleLds];
    __shared__ __align__(16) uint16_t s_x[kStageBytes / 2];
    __shared__ uint16_t s_act[kTileMaxPairs][R / 2];
    __shared__ float s_h[kTileMaxPairs][R];
    const int tid = int(threadIdx.x);
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int H = A.H, I = A.I, E = A.E;
    const int P = t * A.k;  // routed pairs (<= 32 on this path)
    const int nchunks = H / 32;
    bool okc[C];
    uint32_t jc[C];
#pragma unroll
    for (int cc = 0; cc < C; ++cc) {
        const int j = cc * kWave + lane;
        okc[cc] = j < nchunks;
        jc[cc] = okc[cc] ? uint32_t(j) : 0u;
    }
    const int row0 = int(blockIdx.x) * R;
    const int64_t soff = scale_plane_offset(QG_NVFP4, 2 * int64_t(I), H);
    auto load_rows = [&](GroupW<C, R>& b, int e) {  // this tile's rows of expert e
        const uint8_t* w = A.gate_up + int64_t(e) * A.gu_stride;
        const uint8_t* codes[R];
        const uint8_t* scales[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = min(row0 + r, 2 * I - 1);
            codes[r] = w + row * (H / 2);
            scales[r] = w + soff + row * (H / 16);
        }
        load_group_w<C, R>(b, codes, scales, jc);
    };
    // A group's row sums, reduction and SwiGLU, one pair at a time: the
    // pairs are the set bits of m (bit n: token n / div), at CSR positions
    // p0, p0 + 1, ...  Results to LDS, stored after the last group (stores
    // count on the same counter as loads).
    auto compute = [&](const GroupW<C, R>& b, int e, int p0, uint64_t m, int div) {
        const float s_t = s_scale[e];
        for (int p = p0; m; ++p, m &= m - 1) {
            const int tok = int(__builtin_ctzll(m)) / div;
            float acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.f;
            nvfp4_token_dot<R, C>(b, okc, jc, s_x + tok * H, acc);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = group_sum<kWave>(acc[r]) * s_t;
            // lane r evaluates the SwiGLU of a-row r
            float gv = 0.f, uv = 0.f;
#pragma unroll
            for (int r = 0; r < R / 2; ++r)
                if (lane == r) {
                    gv = acc[2 * r];
                    uv = acc[2 * r + 1];
                }
            if (lane < R / 2) {
                s_act[p][lane] = uint16_t(f32_to_bf16_rne(gv / (1.0f + expf(-gv)) * uv));
                s_h[p][2 * lane] = gv;
                s_h[p][2 * lane + 1] = uv;
            }
        }
    };
    auto store = [&](int p0, int mg) {  // a group's pairs (its run of the CSR) to the workspace
        for (int idx = lane; idx < mg * (R / 2); idx += kWave) {
            const int p = p0 + idx / (R / 2), r = idx % (R / 2);
            const int row = row0 / 2 + r;
            if (row < I) {
                ws.a[int64_t(p) * I + row] = s_act[p][r];
                if (ws.h) {
                    ws.h[int64_t(p) * 2 * I + row] = s_h[p][2 * r];
                    ws.h[int64_t(p) * 2 * I + I + row] = s_h[p][2 * r + 1];
                }
            }
        }
    };

    // 0. the shared expert's rows (the waves of its tokens); with two chunks
    // per lane they are requested after the routing instead, as holding them
    // through it runs out of registers
    const int sh_tok = kTileWaves - 1 - wave;
    const bool own_shared = A.has_shared && sh_tok < t;
    constexpr bool kEarly = C == 1;
    GroupW<C, R> gs;
    if (kEarly && own_shared) load_rows(gs, E);
    // 1. loads: the routing waves (one per token) their token's logits; the
    // other waves the scales and x into LDS, so that the routing waits for
    // its logits only
    float lv[PER];
    if constexpr (ROUTE) {
        if (wave < t) route_load<PER>(logits + int64_t(wave) * E, E, lv);
    }
    const int w0 = ROUTE ? t : 0;  // first staging wave
    if (wave >= w0) {
        const int st = tid - w0 * kWave, nst = kTileBlock - w0 * kWave;
        const int ns = E + A.has_shared, n16 = t * H / 8;  // x [t][H] in 16-byte units
        for (int i = st; i < ns; i += nst) s_scale[i] = A.gu_scale[i];
        for (int b = 0; b < n16; b += 4 * nst) {
            u32x4 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = ld16(x + 8 * int64_t(min(b + st + q * nst, n16 - 1)));
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (b + st + q * nst < n16) reinterpret_cast<u32x4*>(s_x)[b + st + q * nst] = v[q];
        }
    }
    // 2. routing (one wave per token)
    if constexpr (ROUTE) {
        if (wave < t) {
            float sv, sw;
            int si;
            route_select<PER>(lv, E, A.k, sv, si, sw);
            if (lane < A.k) {
                s_ids[wave * A.k + lane] = si;
                if (blockIdx.x == 0) {
                    ws.ids[wave * A.k + lane] = si;
                    ws.wts[wave * A.k + lane] = sw;
                }
            }
        }
    } else {
        if (tid < P) s_ids[tid] = ids_in[tid];
    }
    lds_barrier();  // x, scales and the routed ids
    // 3. every wave: pair q's expert in lane q; this wave's groups
    int idv = -1;
    if (lane < P) idv = min(max(s_ids[lane], 0), E - 1);
    uint32_t own = 0;  // bit j: pair wave + 8j is its expert's first pair
#pragma unroll
    for (int j = 0; j < GW; ++j) {
        const int q = wave + kTileWaves * j;
        if (q < P) {
            const int e = __builtin_amdgcn_readlane(idv, q);
            if (__builtin_ctzll(__ballot(idv == e)) == q) own |= 1u << j;
        }
    }
    if (blockIdx.x == 0 && wave == 0) publish_csr(idv, s_ids, P, t, A.k, E, A.has_shared, ws);

    // 4. weight loads and, per group, row sums, reduction and SwiGLU.  The
    // group count is turned into straight-line code (dispatch_count), and a
    // wave keeps kTileDepth groups' loads ahead of the group it computes, so
    // the data of its groups arrives one after another and the decode of
    // each overlaps the stream of the next.
    const int nv = __popc(own);
    auto run = [&](auto nv_c) {
        constexpr int NV = decltype(nv_c)::value;
        constexpr int NA = NV > 0 ? NV : 1;
        GroupW<C, R> gw[NA];
        int ge[NA];
        uint32_t rem = own;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            ge[j] = __builtin_amdgcn_readlane(idv, wave + kTileWaves * int(__builtin_ctz(rem)));
            rem &= rem - 1;
        }
#pragma unroll
        for (int j = 0; j < NV && j < kTileDepth; ++j) load_rows(gw[j], ge[j]);
        if (!kEarly && own_shared) load_rows(gs, E);
        if (own_shared) compute(gs, E, P + sh_tok, 1ull << sh_tok, 1);
        int gp[NA], gm[NA];  // each group's first CSR position and pair count
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if (j + kTileDepth < NV) load_rows(gw[j + kTileDepth], ge[j + kTileDepth]);
            __builtin_amdgcn_sched_barrier(0);
            const uint64_t m = __ballot(idv == ge[j]);
            gp[j] = __popcll(__ballot(lane < P && idv < ge[j]));
            gm[j] = __popcll(m);
            compute(gw[j], ge[j], gp[j], m, A.k);
        }
        if (own_shared) store(P + sh_tok, 1);
#pragma unroll
        for (int j = 0; j < NV; ++j) store(gp[j], gm[j]);
    };
    dispatch_count<GW, 0>(nv, run);
}

// Down + combine, tile path.  blockIdx.x = tile of (64 / G) * R output rows,
// every group; the SwiGLU outputs of all pairs are staged in LDS.  NW waves:
// routed group g goes to wave g % NW, the shared expert's pair of token i to
// wave NW - 1 - i, which requests the shared rows before the header is read.
// The combine is the same fixed-order sum as in k_moe_down.
template <int G, int C, int R, int GW, int NW = kTileWaves>
__global__ __launch_bounds__(NW * kWave) void k_moe_down_tile(MoeArgs A, const float* __restrict__ wts, int t,
                                                              float* __restrict__ y, MoeWorkspace ws) {
    constexpr int kGroups = kWave / G;
    constexpr int kRows = kGroups * R;  // rows per tile
    constexpr int kNT = NW * kWave;     // threads
    constexpr int kStPT = kStageBytes / 16 / kNT;
    constexpr int kScPT = (kMaxScaleLds + kNT - 1) / kNT;
    __shared__ int s_off[kMaxPairs + 1];
    __shared__ int s_exp[kMaxPairs];
    __shared__ int s_pair[kMaxTokens][kMaxTopK + 1];
    __shared__ float s_o[kMaxPairs][kRows];
    __shared__ float s_scale[kMaxScaleLds];
    __shared__ __align__(16) uint16_t s_a[kStageBytes / 2];
    const int tid = int(threadIdx.x);
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int I = A.I, H = A.H;
    const int grp = lane / G, l = lane % G;
    const int tile0 = int(blockIdx.x) * kRows;
    const int nchunks = I / 32;
    bool okc[C];
    uint32_t jc[C];
#pragma unroll
    for (int cc = 0; cc < C; ++cc) {
        const int j = cc * G + l;
        okc[cc] = j < nchunks;
        jc[cc] = okc[cc] ? uint32_t(j) : 0u;
    }
    const int64_t soff = scale_plane_offset(QG_NVFP4, H, I);
    auto load_rows = [&](GroupW<C, R>& b, int e) {  // this lane group's rows of expert e
        const uint8_t* w = A.down + int64_t(e) * A.dn_stride;
        const uint8_t* codes[R];
        const uint8_t* scales[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = min(tile0 + grp * R + r, H - 1);
            codes[r] = w + row * (I / 2);
            scales[r] = w + soff + row * (I / 16);
        }
        load_group_w<C, R>(b, codes, scales, jc);
    };
    auto compute = [&](const GroupW<C, R>& b, int e, int p0, int mg) {  // the group's pairs, one at a time
        const float s_t = s_scale[e];
        for (int i = 0; i < mg; ++i) {
            const int p = p0 + i;
            float acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.f;
            nvfp4_token_dot<R, C>(b, okc, jc, s_a + p * I, acc);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = group_sum<G>(acc[r]) * s_t;
            if (l == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) s_o[p][grp * R + r] = acc[r];
            }
        }
    };

    const int sh_tok = NW - 1 - wave;
    const bool own_shared = A.has_shared && sh_tok < t;
    GroupW<C, R> gs;
    if (own_shared) load_rows(gs, A.E);
    // header up to the worst-case group count, scales and a: one round of
    // loads.  The header goes to LDS first, so that the waves request their
    // first groups' rows before the staged scales and a are stored (those
    // loads were issued earlier and complete before the weights).
    const int ng = *ws.n_groups;
    const int P = t * (A.k + A.has_shared);
    const int gmax = t * A.k + A.has_shared;
    const int n_sc = A.E + A.has_shared, n16 = P * I / 8;  // scales; a [P][I] in 16-byte units
    float scv[kScPT];
    u32x4 av[kStPT];
    {  // gmax < P < kNT: one entry per thread, loads first
        const int oo = ws.offsets[min(tid, gmax)];
        const int ee = ws.experts[min(tid, gmax - 1)];
        const int pt = ws.pair_tok[min(tid, P - 1)], ps = ws.pair_slot[min(tid, P - 1)];
#pragma unroll
        for (int q = 0; q < kScPT; ++q) scv[q] = A.dn_scale[min(tid + q * kNT, n_sc - 1)];
#pragma unroll
        for (int q = 0; q < kStPT; ++q) av[q] = ld16(ws.a + 8 * int64_t(min(tid + q * kNT, n16 - 1)));
        if (tid <= gmax) s_off[tid] = oo;
        if (tid < gmax) s_exp[tid] = ee;
        if (tid < P) s_pair[pt][ps] = tid;
    }
    lds_barrier();
    auto store_staged = [&]() {
#pragma unroll
        for (int q = 0; q < kScPT; ++q)
            if (tid + q * kNT < n_sc) s_scale[tid + q * kNT] = scv[q];
#pragma unroll
        for (int q = 0; q < kStPT; ++q)
            if (tid + q * kNT < n16) reinterpret_cast<u32x4*>(s_a)[tid + q * kNT] = av[q];
        lds_barrier();
    };

    const int nr = ng - A.has_shared;                                   // routed groups
    const int nv = min(GW, (nr - wave + NW - 1) / NW);  // of this wave (uniform, >= 0)
    // As in the gate/up tile kernel: straight-line code per group count,
    // kTileDepthDn groups' loads in flight ahead of the computed one, and no
    // global store until every weight load has been consumed.
    auto run = [&](auto nv_c) {
        constexpr int NV = decltype(nv_c)::value;
        GroupW<C, R> gw[NV > 0 ? NV : 1];
#pragma unroll
        for (int j = 0; j < NV && j < kTileDepthDn; ++j) load_rows(gw[j], s_exp[wave + NW * j]);
        __builtin_amdgcn_sched_barrier(0);
        store_staged();
        if (own_shared) compute(gs, A.E, s_off[nr] + sh_tok, 1);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if (j + kTileDepthDn < NV)
                load_rows(gw[j + kTileDepthDn], s_exp[wave + NW * (j + kTileDepthDn)]);
            __builtin_amdgcn_sched_barrier(0);
            const int g = wave + NW * j;
            compute(gw[j], s_exp[g], s_off[g], s_off[g + 1] - s_off[g]);
        }
    };
    dispatch_count<GW, 0>(nv, run);
    __syncthreads();
    // per-pair down outputs to the workspace, then the combine
    for (int idx = tid; idx < P * kRows; idx += kNT) {
        const int pp = idx / kRows, rr = idx % kRows;
        const int row = tile0 + rr;
        if (row < H) ws.o[int64_t(pp) * H + row] = s_o[pp][rr];
    }
    for (int idx = tid; idx < t * kRows; idx += kNT) {
        const int tt = idx / kRows, rr = idx % kRows;
        const int row = tile0 + rr;
        if (row >= H) continue;
        float sum = 0.f;
        for (int s = 0; s < A.k; ++s) sum = fmaf(wts[int64_t(tt) * A.k + s], s_o[s_pair[tt][s]][rr], sum);
        if (A.has_shared) sum += s_o[s_pair[tt][A.k]][rr];
        y[int64_t(tt) * H + row] = sum;
    }
}

// Launch of the tile path; false when the shapes are outside it.
bool moe_tile_go(const MoeArgs& A, const uint16_t* x, const int32_t* ids, const float* w, const float* logits,
                 int t, float* y, const MoeWorkspace& ws, hipStream_t s, hipError_t& err) {
    constexpr int RU = 4;  // packed gate/up rows per tile
    constexpr int RD = 2;  // down rows per lane group
    const int ju = A.H / 32, jd = A.I / 32;
    const int nrmax = t * A.k;  // routed groups at most
    const int P = t * (A.k + A.has_shared);
    const int cu = chunks_per_lane(ju, 64);
    const bool down16 = lanes_per_row(jd) == 16;
    const int cd = chunks_per_lane(jd, down16 ? 16 : 64);
    // one token: the per-(group, tile) kernels are as fast and need no staging
    if (t < 2 || t > 4 || nrmax > 4 * kTileWaves) return false;
    if (lanes_per_row(ju) != 64 || (cu != 1 && cu != 2) || (cd != 1 && cd != 2)) return false;
    if (int64_t(t) * A.H * 2 > kStageBytes || int64_t(P) * A.I * 2 > kStageBytes) return false;
    if (A.E + A.has_shared > kMaxScaleLds) return false;
    const bool gw1 = nrmax <= 2 * kTileWaves;  // else up to 4 routed groups per wave
    if (cu == 2 && !gw1) return false;          // too many registers: the general path
    const dim3 g1((2 * A.I + RU - 1) / RU);
    auto up = [&](auto cu_c, auto gw_c) {
        constexpr int CU = decltype(cu_c)::value, GWc = decltype(gw_c)::value;
        if (logits) {
            if ((A.E + kWave - 1) / kWave <= 4)
                hipLaunchKernelGGL((k_moe_gate_up_tile<CU, RU, true, 4, GWc>), g1, dim3(kTileBlock), 0, s, A, x,
                                   nullptr, logits, t, ws);
            else
                hipLaunchKernelGGL((k_moe_gate_up_tile<CU, RU, true, 16, GWc>), g1, dim3(kTileBlock), 0, s, A,
                                   x, nullptr, logits, t, ws);
        } else {
            hipLaunchKernelGGL((k_moe_gate_up_tile<CU, RU, false, 1, GWc>), g1, dim3(kTileBlock), 0, s, A, x,
                               ids, nullptr, t, ws);
        }
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    if (cu == 1) gw1 ? up(I1{}, I2{}) : up(I1{}, I4{});
    else up(I2{}, I2{});
    err = hipGetLastError();
    if (err != hipSuccess) return true;
    if (logits) w = ws.wts;
    auto down = [&](auto g_c, auto cd_c, auto gw_c) {
        constexpr int GD = decltype(g_c)::value, CD = decltype(cd_c)::value, GWc = decltype(gw_c)::value;
        constexpr int kRowsDown = (kWave / GD) * RD;
        const dim3 g2((A.H + kRowsDown - 1) / kRowsDown);
        if constexpr (CD == 1)  // sixteen waves: at most two routed groups each
            hipLaunchKernelGGL((k_moe_down_tile<GD, CD, RD, 2, 2 * kTileWaves>), g2, dim3(2 * kTileBlock), 0, s, A, w,
                               t, y, ws);
        else
            hipLaunchKernelGGL((k_moe_down_tile<GD, CD, RD, GWc>), g2, dim3(kTileBlock), 0, s, A, w, t, y, ws);
    };
    using I16 = std::integral_constant<int, 16>;
    using I64 = std::integral_constant<int, 64>;
    if (down16) {
        if (cd == 1) gw1 ? down(I16{}, I1{}, I2{}) : down(I16{}, I1{}, I4{});
        else gw1 ? down(I16{}, I2{}, I2{}) : down(I16{}, I2{}, I4{});
    } else {
        if (cd == 1) gw1 ? down(I64{}, I1{}, I2{}) : down(I64{}, I1{}, I4{});
        else gw1 ? down(I64{}, I2{}, I2{}) : down(I64{}, I2{}, I4{});
    }
    err = hipGetLastError();
    return true;
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
    // One token with a row in one chunk per 16-lane group: the tile down
    // kernel reads the same CSR header, and its shared-expert preload and
    // split barrier take the layer from 12.53 to 11.96 us (E = 256, k = 8,
    // H = 2048, I = 512); P * I * 2 <= 9 * 512 * 2 bytes fits its staging.
    if constexpr (MT == 1 && GD == 16 && CD == 1) {
        if (t == 1 && A.k <= kMaxTopK && A.E + A.has_shared <= kMaxScaleLds) {
            constexpr int kRowsTile = (kWave / 16) * 2;
            const dim3 gt((A.H + kRowsTile - 1) / kRowsTile);
            hipLaunchKernelGGL((k_moe_down_tile<16, 1, 2, 2, 2 * kTileWaves>), gt, dim3(2 * kTileBlock), 0, s, A, w, t,
                               y, ws);
            return hipGetLastError();
        }
    }
    // two rows per lane group: each wave's weight request is twice as large
    // (measured at one token: 12.96 us with one row, 12.65 with two, 13.4
    // with four)
    constexpr int RDn = 2;
    constexpr int kRowsDown = kWave / GD * RDn;
    const int waves = max_groups < 16 ? max_groups : 16;
    const dim3 g2((A.H + kRowsDown - 1) / kRowsDown);
    hipLaunchKernelGGL((k_moe_down<MT, GD, CD, RDn>), g2, dim3(kWave * waves), 0, s, A, w, t, y, ws);
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
    hipError_t err = hipSuccess;
    switch (token_class(t)) {
        case 1:
            if (moe_tile_go(A, x, ids, w, logits, t, y, ws, s, err)) return err;
            return moe_mt<1>(A, x, ids, w, logits, t, y, ws, s);
        case 4:
            if (kernel_policy() != QG_KERNEL_GENERIC && moe_tile_go(A, x, ids, w, logits, t, y, ws, s, err))
                return err;
            return moe_mt<4>(A, x, ids, w, logits, t, y, ws, s);
        default: return moe_mt<16>(A, x, ids, w, logits, t, y, ws, s);
    }
}

}  // namespace qg
