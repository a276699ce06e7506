// The C entry points: argument validation on the host, then one launch (or a
// short fixed sequence of launches) on the caller's stream.  Nothing here
// allocates, synchronises or keeps per-call state; the only process-wide
// setting is the kernel policy (the rollback seam).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "qg_internal.hpp"
#include "qg_layout.hpp"
#include "qgemv.h"

namespace qg {

extern std::atomic<int> g_last_hip_error;

void record_hip_error(hipError_t e) { g_last_hip_error.store(int(e)); }

hipError_t device_cu_count(int* cus) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];  // 0 = not yet queried
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) {
        if (const int v = cache[dev].load(std::memory_order_relaxed)) {
            *cus = v;
            return hipSuccess;
        }
    }
    int v = 0;
    if (hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev); e != hipSuccess)
        return e;
    if (v < 1) v = 1;
    if (dev >= 0 && dev < kMaxDevices) cache[dev].store(v, std::memory_order_relaxed);
    *cus = v;
    return hipSuccess;
}

namespace {

std::atomic<int> g_policy{QG_KERNEL_TUNED};
std::once_flag g_policy_env;

// QG_FORCE_KERNEL, read once: "generic" selects the generic kernels.
void read_policy_env() {
    const char* v = std::getenv("QG_FORCE_KERNEL");
    if (v && std::strcmp(v, "generic") == 0) g_policy.store(QG_KERNEL_GENERIC);
}

}  // namespace

int kernel_policy() {
    std::call_once(g_policy_env, read_policy_env);
    return g_policy.load(std::memory_order_relaxed);
}

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

inline int finish(hipError_t e) {
    if (e == hipSuccess) return QG_OK;
    record_hip_error(e);
    return QG_EHIP;
}

// Largest token count of moe_prefill (grid and index ranges stay well inside int).
constexpr int64_t kMoePrefillMaxT = 65536;

// Checks shared by the GEMV entry points.
inline int check_gemv(const void* w, int64_t n, int64_t k, const void* x, int64_t m, const void* y) {
    if (!w || !x || !y) return QG_EINVAL;
    if (!aligned(w, 256) || !aligned(x, 16) || !aligned(y, 16)) return QG_EINVAL;
    if (!valid_shape(n, k) || m < 1) return QG_EINVAL;
    if (m > QG_MAX_M) return QG_EUNSUPPORTED;
    return QG_OK;
}

}  // namespace
}  // namespace qg

using namespace qg;

extern "C" {

int qg_set_kernel_policy(int policy) {
    if (policy != QG_KERNEL_TUNED && policy != QG_KERNEL_GENERIC) return QG_EINVAL;
    std::call_once(g_policy_env, read_policy_env);
    g_policy.store(policy);
    return QG_OK;
}

int qg_kernel_policy(void) { return kernel_policy(); }

int qg_dequant(int fmt, const void* w, float tensor_scale, int64_t n, int64_t k, float* out,
               void* stream) {
    if (!valid_fmt(fmt) || !w || !out || !aligned(w, 256) || !aligned(out, 16)) return QG_EINVAL;
    if (!valid_fmt_shape(fmt, n, k)) return QG_EINVAL;
    if (is_kquant(fmt))
        return finish(launch_dequant_kquant(fmt, static_cast<const uint8_t*>(w), n, k, out, as_stream(stream)));
    if (is_fp8(fmt))
        return finish(launch_dequant_fp8(fmt, static_cast<const uint8_t*>(w), n, k, out, as_stream(stream)));
    return finish(launch_dequant(fmt, static_cast<const uint8_t*>(w), tensor_scale, n, k, out,
                                 as_stream(stream)));
}

int qgemv_fp8(int fmt, const void* w, int64_t n, int64_t k, const uint16_t* x, int64_t m, float* y,
              void* stream) {
    if (!is_fp8(fmt)) return QG_EINVAL;
    if (int st = check_gemv(w, n, k, x, m, y)) return st;
    return finish(launch_gemv_fp8(fmt, static_cast<const uint8_t*>(w), n, k, x, int(m), y, as_stream(stream)));
}

int qgemv_q8_0(const void* w, int64_t n, int64_t k, const float* x, int64_t m, float* y,
               void* stream) {
    if (int st = check_gemv(w, n, k, x, m, y)) return st;
    return finish(launch_gemv_q8_0(static_cast<const uint8_t*>(w), n, k, x, int(m), y,
                                   as_stream(stream)));
}

int qgemv_nvfp4(const void* w, float tensor_scale, int64_t n, int64_t k, const uint16_t* x,
                int64_t m, float* y, void* stream) {
    if (int st = check_gemv(w, n, k, x, m, y)) return st;
    return finish(launch_gemv_nvfp4(static_cast<const uint8_t*>(w), tensor_scale, n, k, x, int(m), y,
                                    as_stream(stream)));
}

int qgemv_nvfp4_swiglu(const void* w_gu, float tensor_scale, int64_t inter, int64_t k,
                       const uint16_t* x, int64_t m, uint16_t* a, float* h, void* stream) {
    if (inter < 1 || inter > (int64_t(1) << 30)) return QG_EINVAL;
    if (int st = check_gemv(w_gu, 2 * inter, k, x, m, a)) return st;
    if (h && !aligned(h, 16)) return QG_EINVAL;
    return finish(launch_gemv_nvfp4_swiglu(static_cast<const uint8_t*>(w_gu), tensor_scale, inter, k,
                                           x, int(m), a, h, as_stream(stream)));
}

int qg_quantize_q8_0_act(const float* x, int64_t m, int64_t k, int8_t* xq, uint16_t* xd,
                         int32_t* xs, void* stream) {
    if (!x || !xq || !xd) return QG_EINVAL;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xd, 2) || (xs && !aligned(xs, 4)))
        return QG_EINVAL;
    if (m < 1 || !valid_shape(1, k) || m > (int64_t(1) << 31) / (k / 32)) return QG_EINVAL;
    return finish(launch_quantize_q8_0(x, m, k, xq, xd, xs, as_stream(stream)));
}

int qgemv_q4_0_a8(const void* w, int64_t n, int64_t k, const int8_t* xq, const uint16_t* xd,
                  const int32_t* xs, int64_t m, float* y, void* stream) {
    if (int st = check_gemv(w, n, k, xq, m, y)) return st;
    if (!xd || !aligned(xd, 2) || (xs && !aligned(xs, 4))) return QG_EINVAL;
    return finish(launch_gemv_q4_0_a8(static_cast<const uint8_t*>(w), n, k, xq, xd, xs, int(m), y,
                                      as_stream(stream)));
}

int qgemm_prefill_a8(const void* w, int64_t n, int64_t k, const int8_t* xq, const uint16_t* xd, int64_t m,
                     float* y, void* stream) {
    if (!w || !xq || !xd || !y) return QG_EINVAL;
    if (!aligned(w, 256) || !aligned(xq, 16) || !aligned(xd, 2) || !aligned(y, 16)) return QG_EINVAL;
    if (!valid_shape(n, k) || m < 1) return QG_EINVAL;
    if (!prefill_a8_shape_ok(n, k, m)) return QG_EUNSUPPORTED;
    return finish(launch_prefill_a8(static_cast<const uint8_t*>(w), n, k, xq, xd, m, y, as_stream(stream)));
}

int qgemv_kquant_a8(int fmt, const void* w, int64_t n, int64_t k, const int8_t* xq, const uint16_t* xd,
                    const int32_t* xs, int64_t m, float* y, void* stream) {
    if (!is_kquant(fmt)) return QG_EINVAL;
    if (int st = check_gemv(w, n, k, xq, m, y)) return st;
    if (k % kKqSuper != 0) return QG_EINVAL;
    if (!xd || !xs || !aligned(xd, 2) || !aligned(xs, 4)) return QG_EINVAL;
    return finish(launch_gemv_kquant_a8(fmt, static_cast<const uint8_t*>(w), n, k, xq, xd, xs, int(m), y,
                                        as_stream(stream)));
}

int moe_route_topk(const float* logits, int64_t t, int64_t n_experts, int64_t top_k, int32_t* ids,
                   float* weights, void* stream) {
    if (!logits || !ids || !weights) return QG_EINVAL;
    if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(weights, 4)) return QG_EINVAL;
    if (t < 1 || t > (int64_t(1) << 24) || top_k < 1 || n_experts < top_k) return QG_EINVAL;
    if (top_k > 16 || n_experts > 1024) return QG_EUNSUPPORTED;
    return finish(launch_route_topk(logits, t, int(n_experts), int(top_k), ids, weights,
                                    as_stream(stream)));
}

static int check_moe_desc(const qg_moe_desc* d) {
    if (!d) return QG_EINVAL;
    if (d->layout_version != QG_LAYOUT_VERSION) return QG_EVERSION;
    if (!d->gate_up || !d->down || !d->gate_up_scale || !d->down_scale || d->reserved != 0) return QG_EINVAL;
    if (d->n_experts < 1 || d->top_k < 1 || d->top_k > d->n_experts) return QG_EINVAL;
    if (d->has_shared != 0 && d->has_shared != 1) return QG_EINVAL;
    if (d->flags & ~QG_MOE_KEEP_H) return QG_EINVAL;
    if (!valid_shape(2 * d->inter, d->hidden) || !valid_shape(d->hidden, d->inter)) return QG_EINVAL;
    if (d->top_k > 8) return QG_EUNSUPPORTED;
    if (!aligned(d->gate_up, 256) || !aligned(d->down, 256)) return QG_EINVAL;
    if (d->gate_up_stride % 256 || d->down_stride % 256) return QG_EINVAL;
    if (d->gate_up_stride < int64_t(packed_bytes(QG_NVFP4, 2 * d->inter, d->hidden))) return QG_EINVAL;
    if (d->down_stride < int64_t(packed_bytes(QG_NVFP4, d->hidden, d->inter))) return QG_EINVAL;
    if (d->hidden > (int64_t(1) << 20) || d->inter > (int64_t(1) << 20)) return QG_EUNSUPPORTED;
    return QG_OK;
}

size_t moe_workspace_bytes(const qg_moe_desc* d, int64_t t) {
    if (check_moe_desc(d) != QG_OK || t < 1 || t > QG_MAX_M) return 0;
    return moe_workspace_layout(d, t, nullptr, nullptr);
}

int moe_gemv_grouped(const qg_moe_desc* d, const uint16_t* x, const int32_t* ids,
                     const float* weights, int64_t t, float* y, void* ws, size_t ws_bytes,
                     void* stream) {
    if (int st = check_moe_desc(d)) return st;
    if (!x || !ids || !weights || !y || !ws) return QG_EINVAL;
    if (!aligned(x, 16) || !aligned(ids, 4) || !aligned(weights, 4) || !aligned(y, 16) ||
        !aligned(ws, 256))
        return QG_EINVAL;
    if (t < 1) return QG_EINVAL;
    if (t > QG_MAX_M) return QG_EUNSUPPORTED;
    MoeWorkspace lay;
    const size_t need = moe_workspace_layout(d, t, &lay, ws);
    if (ws_bytes < need) return QG_ENOSPC;
    return finish(launch_moe(d, x, ids, weights, nullptr, int(t), y, lay, as_stream(stream)));
}

}  // extern "C"

// Workspace of moe_forward_noalloc: a library-owned device array, one copy per
// GPU (each device holds its own instance at its own address), kept until the
// process ends.  In host code the name `scratch` is only a host-side stand-in
// for the symbol: every use goes through the device address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch).
static __device__ __align__(256) unsigned char scratch[QG_MOE_NOALLOC_SCRATCH_BYTES];

namespace qg {
namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device: looked up once per
// device (with that device current) and cached.
hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    if (void* p = g_scratch_ptr[dev].load(std::memory_order_acquire)) {
        *out = p;
        return hipSuccess;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace
}  // namespace qg

extern "C" {

int moe_forward_noalloc(const qg_moe_desc* d, const uint16_t* x, const float* logits, int64_t t, float* y,
                        void* stream) {
    if (int st = check_moe_desc(d)) return st;
    if (!x || !logits || !y) return QG_EINVAL;
    if (!aligned(x, 16) || !aligned(logits, 4) || !aligned(y, 16)) return QG_EINVAL;
    if (t < 1) return QG_EINVAL;
    if (t > QG_MAX_M || d->n_experts > 1024) return QG_EUNSUPPORTED;
    const size_t need = moe_workspace_layout(d, t, nullptr, nullptr);
    if (need > size_t(QG_MOE_NOALLOC_SCRATCH_BYTES)) return QG_ENOSPC;
    void* base = nullptr;
    if (hipError_t e = noalloc_scratch(&base); e != hipSuccess) return finish(e);
    MoeWorkspace lay;
    moe_workspace_layout(d, t, &lay, base);
    // Every workspace region is written before it is read within the call,
    // so nothing left over from an earlier call needs clearing.
    return finish(launch_moe(d, x, nullptr, nullptr, logits, int(t), y, lay, as_stream(stream)));
}

int moe_forward(const qg_moe_desc* d, const uint16_t* x, const float* logits, int64_t t, float* y, void* ws,
                size_t ws_bytes, void* stream) {
    if (int st = check_moe_desc(d)) return st;
    if (!x || !logits || !y || !ws) return QG_EINVAL;
    if (!aligned(x, 16) || !aligned(logits, 4) || !aligned(y, 16) || !aligned(ws, 256)) return QG_EINVAL;
    if (t < 1) return QG_EINVAL;
    if (t > QG_MAX_M || d->n_experts > 1024) return QG_EUNSUPPORTED;
    MoeWorkspace lay;
    const size_t need = moe_workspace_layout(d, t, &lay, ws);
    if (ws_bytes < need) return QG_ENOSPC;
    return finish(launch_moe(d, x, nullptr, nullptr, logits, int(t), y, lay, as_stream(stream)));
}

size_t moe_prefill_workspace_bytes(const qg_moe_desc* d, int64_t t) {
    if (check_moe_desc(d) || t < 1 || t > kMoePrefillMaxT) return 0;
    if (!moe_prefill_shape_ok(d->hidden, d->inter) || d->n_experts > 1024) return 0;
    return moe_prefill_layout(d, t, nullptr, nullptr, nullptr);
}

int moe_prefill(const qg_moe_desc* d, const uint16_t* x, const float* logits, int64_t t, float* y, void* ws,
                size_t ws_bytes, void* stream) {
    if (int st = check_moe_desc(d)) return st;
    if (!x || !logits || !y || !ws) return QG_EINVAL;
    if (!aligned(x, 16) || !aligned(logits, 4) || !aligned(y, 16) || !aligned(ws, 256)) return QG_EINVAL;
    if (t < 1) return QG_EINVAL;
    if (t > kMoePrefillMaxT || d->n_experts > 1024 || !moe_prefill_shape_ok(d->hidden, d->inter))
        return QG_EUNSUPPORTED;
    MoeWorkspace lay;
    MoePrefillExtra ex;
    const size_t need = moe_prefill_layout(d, t, &lay, &ex, ws);
    if (ws_bytes < need) return QG_ENOSPC;
    return finish(launch_moe_prefill(d, x, logits, int(t), y, lay, ex, as_stream(stream)));
}

int qgemm_prefill(const void* w, float tensor_scale, int64_t n, int64_t k, const uint16_t* x,
                  int64_t m, uint16_t* y, void* stream) {
    if (!w || !x || !y || !aligned(w, 256) || !aligned(x, 16) || !aligned(y, 16)) return QG_EINVAL;
    if (!valid_shape(n, k) || m < 1 || m > (int64_t(65535) * 64)) return QG_EINVAL;
    return finish(launch_prefill(static_cast<const uint8_t*>(w), tensor_scale, n, k, x, m, y,
                                 as_stream(stream)));
}

size_t qgemm_prefill_workspace_bytes(int64_t n, int64_t k, int64_t m) {
    if (!valid_shape(n, k) || m < 1 || m > (int64_t(65535) * 64)) return 0;
    return prefill_workspace_bytes(n, k, m);
}

int qgemm_prefill_ws(const void* w, float tensor_scale, int64_t n, int64_t k, const uint16_t* x,
                     int64_t m, uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
    if (!w || !x || !y || !aligned(w, 256) || !aligned(x, 16) || !aligned(y, 16)) return QG_EINVAL;
    if (!valid_shape(n, k) || m < 1 || m > (int64_t(65535) * 64)) return QG_EINVAL;
    const size_t need = prefill_workspace_bytes(n, k, m);
    if (need > 0) {
        if (!ws || !aligned(ws, 256)) return QG_EINVAL;
        if (ws_bytes < need) return QG_ENOSPC;
    }
    return finish(launch_prefill_ws(static_cast<const uint8_t*>(w), tensor_scale, n, k, x, m, y,
                                    static_cast<float*>(ws), as_stream(stream)));
}

int qg_probe_read(const void* buf, size_t bytes, int wg_per_cu, uint32_t* sink, void* stream) {
    if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4)) return QG_EINVAL;
    if (bytes < 16 || bytes % 16 || bytes > (size_t(1) << 40) || wg_per_cu < 1 || wg_per_cu > 8) return QG_EINVAL;
    return finish(launch_probe_read(buf, int64_t(bytes), sink, wg_per_cu, as_stream(stream)));
}

int qg_probe_mfma_bf16(int64_t iters, float* sink, int64_t* flops, void* stream) {
    if (!sink || !flops || !aligned(sink, 4) || iters < 1 || iters > (int64_t(1) << 32)) return QG_EINVAL;
    return finish(launch_probe_mfma(iters, sink, as_stream(stream), flops));
}

}  // extern "C"
