// Internal launch interface between the C entry points (qg_api.cpp) and the
// kernel translation units.  Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "qgemv.h"

namespace qg {

void record_hip_error(hipError_t e);

// Compute units of the current device (cached per device after the first call).
hipError_t device_cu_count(int* cus);
// The kernel policy (QG_KERNEL_TUNED or QG_KERNEL_GENERIC) in force for a new call.
int kernel_policy();

// Returns hipSuccess or the launch error.
hipError_t launch_dequant(int fmt, const uint8_t* w, float s_t, int64_t n, int64_t k, float* out,
                          hipStream_t s);
hipError_t launch_gemv_q8_0(const uint8_t* w, int64_t n, int64_t k, const float* x, int m, float* y,
                            hipStream_t s);
hipError_t launch_gemv_nvfp4(const uint8_t* w, float s_t, int64_t n, int64_t k, const uint16_t* x,
                             int m, float* y, hipStream_t s);
hipError_t launch_gemv_fp8(int fmt, const uint8_t* w, int64_t n, int64_t k, const uint16_t* x, int m, float* y,
                           hipStream_t s);
hipError_t launch_dequant_fp8(int fmt, const uint8_t* w, int64_t n, int64_t k, float* out, hipStream_t s);
hipError_t launch_gemv_kquant_a8(int fmt, const uint8_t* w, int64_t n, int64_t k, const int8_t* xq,
                                 const uint16_t* xd, const int32_t* xs, int m, float* y, hipStream_t s);
hipError_t launch_dequant_kquant(int fmt, const uint8_t* w, int64_t n, int64_t k, float* out, hipStream_t s);
bool prefill_a8_shape_ok(int64_t n, int64_t k, int64_t m);
hipError_t launch_prefill_a8(const uint8_t* w, int64_t n, int64_t k, const int8_t* xq, const uint16_t* xd,
                             int64_t m, float* y, hipStream_t s);
hipError_t launch_gemv_nvfp4_swiglu(const uint8_t* w, float s_t, int64_t inter, int64_t k,
                                    const uint16_t* x, int m, uint16_t* a, float* h, hipStream_t s);
hipError_t launch_quantize_q8_0(const float* x, int64_t m, int64_t k, int8_t* xq, uint16_t* xd,
                                int32_t* xs, hipStream_t s);
hipError_t launch_gemv_q4_0_a8(const uint8_t* w, int64_t n, int64_t k, const int8_t* xq,
                               const uint16_t* xd, const int32_t* xs, int m, float* y,
                               hipStream_t s);
hipError_t launch_route_topk(const float* logits, int64_t t, int e, int top_k, int32_t* ids,
                             float* w, hipStream_t s);

struct MoeWorkspace {
    int32_t* n_groups;
    int32_t* experts;
    int32_t* offsets;
    int32_t* pair_tok;
    int32_t* pair_slot;
    uint16_t* a;
    float* h;       // nullable
    float* o;
    int32_t* ids;   // routing written by the fused path (moe_forward)
    float* wts;
};
size_t moe_workspace_layout(const qg_moe_desc* d, int64_t t, MoeWorkspace* ws, void* base);
// ids/w given: grouped GEMVs only.  logits given (ids, w null): routing is
// done inside the gate/up kernel and written to ws.ids / ws.wts.
hipError_t launch_moe(const qg_moe_desc* d, const uint16_t* x, const int32_t* ids, const float* w,
                      const float* logits, int t, float* y, const MoeWorkspace& ws, hipStream_t s);

// MoE over many tokens: the decode workspace fields, then these.
struct MoePrefillExtra {
    int32_t* tile_off;  // [P + 2] first GEMM tile of each group
    int32_t* counts;    // [n_experts] routed pairs per expert
    int32_t* pair_pos;  // [t * (top_k + 1)] CSR position of pair (token, slot)
    int4* tile_info;    // [1 + max tiles]: the tile count, then (expert, first pair, pairs, 0) per GEMM tile
};
bool moe_prefill_shape_ok(int64_t hidden, int64_t inter);
size_t moe_prefill_layout(const qg_moe_desc* d, int64_t t, MoeWorkspace* ws, MoePrefillExtra* ex, void* base);
hipError_t launch_moe_prefill(const qg_moe_desc* d, const uint16_t* x, const float* logits, int t, float* y,
                              const MoeWorkspace& ws, const MoePrefillExtra& ex, hipStream_t s);

hipError_t launch_prefill(const uint8_t* w, float s_t, int64_t n, int64_t k, const uint16_t* x,
                          int64_t m, uint16_t* y, hipStream_t s);
// Workspace bytes of launch_prefill_ws (0: the single-pass kernel, no workspace).
size_t prefill_workspace_bytes(int64_t n, int64_t k, int64_t m);
hipError_t launch_prefill_ws(const uint8_t* w, float s_t, int64_t n, int64_t k, const uint16_t* x, int64_t m,
                             uint16_t* y, float* ws, hipStream_t s);

// Achievable-peak probes (k_probe.hip).
hipError_t launch_probe_read(const void* buf, int64_t bytes, uint32_t* sink, int wg_per_cu, hipStream_t s);
hipError_t launch_probe_mfma(int64_t iters, float* sink, hipStream_t s, int64_t* flops);

}  // namespace qg
