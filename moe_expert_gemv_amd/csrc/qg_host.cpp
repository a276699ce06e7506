// Host side of the library: versions, status text and the packers.
//
// The packers implement the split-plane repack of the pages (bw24 README and
// memra README, feature lists: split-plane matvecs over repacked weights).
// They are exact bit moves: codes and scale bit patterns are copied into the
// device layout described in qgemv.h and can be recovered unchanged.
#include <atomic>
#include <cstring>

#include "qg_layout.hpp"
#include "qgemv.h"

namespace qg {
std::atomic<int> g_last_hip_error{0};
}

extern "C" {

int qg_abi_version(void) { return QG_ABI_VERSION; }
int qg_layout_version(void) { return QG_LAYOUT_VERSION; }
int qg_last_hip_error(void) { return qg::g_last_hip_error.load(); }

const char* qg_status_string(int status) {
    switch (status) {
        case QG_OK: return "ok";
        case QG_EINVAL: return "invalid argument (null pointer, bad shape, misalignment or bad code)";
        case QG_EUNSUPPORTED: return "shape outside what the kernels implement";
        case QG_ENOSPC: return "destination or workspace buffer too small";
        case QG_EHIP: return "HIP runtime or launch error";
        default: return "unknown status";
    }
}

size_t qg_packed_bytes(int fmt, int64_t n, int64_t k) {
    if (!qg::valid_fmt(fmt) || !qg::valid_shape(n, k)) return 0;
    return size_t(qg::packed_bytes(fmt, n, k));
}

size_t qg_scale_plane_offset(int fmt, int64_t n, int64_t k) {
    if (!qg::valid_fmt(fmt) || !qg::valid_shape(n, k)) return 0;
    return size_t(qg::scale_plane_offset(fmt, n, k));
}

// ---------------------------------------------------------------- packers

static int check_pack_args(int fmt, const void* a, const void* b, int64_t n, int64_t k,
                           const void* buf, size_t bytes) {
    if (!a || !b || !buf) return QG_EINVAL;
    if (!qg::valid_shape(n, k)) return QG_EINVAL;
    if (bytes < size_t(qg::packed_bytes(fmt, n, k))) return QG_ENOSPC;
    return QG_OK;
}

int qg_pack_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, void* dst,
                  size_t dst_bytes) {
    int st = check_pack_args(QG_NVFP4, codes, scales, n, k, dst, dst_bytes);
    if (st) return st;
    for (int64_t i = 0; i < n * k; ++i)
        if (codes[i] > 15) return QG_EINVAL;
    uint8_t* out = static_cast<uint8_t*>(dst);
    std::memset(out, 0, size_t(qg::packed_bytes(QG_NVFP4, n, k)));
    const int64_t crow = k / 2;
    for (int64_t r = 0; r < n; ++r) {
        const uint8_t* c = codes + r * k;
        uint8_t* o = out + r * crow;
        for (int64_t j = 0; j < crow; ++j) o[j] = uint8_t(c[2 * j] | (c[2 * j + 1] << 4));
    }
    std::memcpy(out + qg::scale_plane_offset(QG_NVFP4, n, k), scales, size_t(n * (k / 16)));
    return QG_OK;
}

int qg_pack_q4_0(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, void* dst,
                 size_t dst_bytes) {
    int st = check_pack_args(QG_Q4_0, codes, scales, n, k, dst, dst_bytes);
    if (st) return st;
    for (int64_t i = 0; i < n * k; ++i)
        if (codes[i] > 15) return QG_EINVAL;
    uint8_t* out = static_cast<uint8_t*>(dst);
    std::memset(out, 0, size_t(qg::packed_bytes(QG_Q4_0, n, k)));
    const int64_t crow = k / 2;
    for (int64_t r = 0; r < n; ++r) {
        const uint8_t* c = codes + r * k;
        uint8_t* o = out + r * crow;
        for (int64_t b = 0; b < k / 32; ++b)
            for (int i = 0; i < 16; ++i)
                o[16 * b + i] = uint8_t(c[32 * b + i] | (c[32 * b + 16 + i] << 4));
    }
    std::memcpy(out + qg::scale_plane_offset(QG_Q4_0, n, k), scales, size_t(n * (k / 32)) * 2);
    return QG_OK;
}

int qg_pack_q8_0(const int8_t* codes, const uint16_t* scales, int64_t n, int64_t k, void* dst,
                 size_t dst_bytes) {
    int st = check_pack_args(QG_Q8_0, codes, scales, n, k, dst, dst_bytes);
    if (st) return st;
    uint8_t* out = static_cast<uint8_t*>(dst);
    std::memset(out, 0, size_t(qg::packed_bytes(QG_Q8_0, n, k)));
    std::memcpy(out, codes, size_t(n * k));
    std::memcpy(out + qg::scale_plane_offset(QG_Q8_0, n, k), scales, size_t(n * (k / 32)) * 2);
    return QG_OK;
}

// Fused gate/up matrix: logical rows [0, inter) gate, [inter, 2*inter) up;
// packed row 2i = gate row i, packed row 2i+1 = up row i.
int qg_pack_nvfp4_gate_up(const uint8_t* codes, const uint8_t* scales, int64_t inter, int64_t k, void* dst,
                          size_t dst_bytes) {
    const int64_t n = 2 * inter;
    int st = check_pack_args(QG_NVFP4, codes, scales, n, k, dst, dst_bytes);
    if (st) return st;
    for (int64_t i = 0; i < n * k; ++i)
        if (codes[i] > 15) return QG_EINVAL;
    uint8_t* out = static_cast<uint8_t*>(dst);
    std::memset(out, 0, size_t(qg::packed_bytes(QG_NVFP4, n, k)));
    const int64_t crow = k / 2, srow = k / 16;
    uint8_t* splane = out + qg::scale_plane_offset(QG_NVFP4, n, k);
    for (int64_t r = 0; r < n; ++r) {
        const int64_t pr = r < inter ? 2 * r : 2 * (r - inter) + 1;  // packed row
        const uint8_t* c = codes + r * k;
        uint8_t* o = out + pr * crow;
        for (int64_t j = 0; j < crow; ++j) o[j] = uint8_t(c[2 * j] | (c[2 * j + 1] << 4));
        std::memcpy(splane + pr * srow, scales + r * srow, size_t(srow));
    }
    return QG_OK;
}

// ---------------------------------------------------------------- unpackers

int qg_unpack_nvfp4(const void* src, size_t src_bytes, int64_t n, int64_t k, uint8_t* codes,
                    uint8_t* scales) {
    int st = check_pack_args(QG_NVFP4, codes, scales, n, k, src, src_bytes);
    if (st) return st;
    const uint8_t* in = static_cast<const uint8_t*>(src);
    const int64_t crow = k / 2;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < crow; ++j) {
            uint8_t v = in[r * crow + j];
            codes[r * k + 2 * j] = v & 15;
            codes[r * k + 2 * j + 1] = v >> 4;
        }
    std::memcpy(scales, in + qg::scale_plane_offset(QG_NVFP4, n, k), size_t(n * (k / 16)));
    return QG_OK;
}

int qg_unpack_nvfp4_gate_up(const void* src, size_t src_bytes, int64_t inter, int64_t k, uint8_t* codes,
                            uint8_t* scales) {
    const int64_t n = 2 * inter;
    int st = check_pack_args(QG_NVFP4, codes, scales, n, k, src, src_bytes);
    if (st) return st;
    const uint8_t* in = static_cast<const uint8_t*>(src);
    const int64_t crow = k / 2, srow = k / 16;
    const uint8_t* splane = in + qg::scale_plane_offset(QG_NVFP4, n, k);
    for (int64_t r = 0; r < n; ++r) {
        const int64_t pr = r < inter ? 2 * r : 2 * (r - inter) + 1;
        for (int64_t j = 0; j < crow; ++j) {
            const uint8_t v = in[pr * crow + j];
            codes[r * k + 2 * j] = v & 15;
            codes[r * k + 2 * j + 1] = v >> 4;
        }
        std::memcpy(scales + r * srow, splane + pr * srow, size_t(srow));
    }
    return QG_OK;
}

int qg_unpack_q4_0(const void* src, size_t src_bytes, int64_t n, int64_t k, uint8_t* codes,
                   uint16_t* scales) {
    int st = check_pack_args(QG_Q4_0, codes, scales, n, k, src, src_bytes);
    if (st) return st;
    const uint8_t* in = static_cast<const uint8_t*>(src);
    const int64_t crow = k / 2;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < k / 32; ++b)
            for (int i = 0; i < 16; ++i) {
                uint8_t v = in[r * crow + 16 * b + i];
                codes[r * k + 32 * b + i] = v & 15;
                codes[r * k + 32 * b + 16 + i] = v >> 4;
            }
    std::memcpy(scales, in + qg::scale_plane_offset(QG_Q4_0, n, k), size_t(n * (k / 32)) * 2);
    return QG_OK;
}

int qg_unpack_q8_0(const void* src, size_t src_bytes, int64_t n, int64_t k, int8_t* codes,
                   uint16_t* scales) {
    int st = check_pack_args(QG_Q8_0, codes, scales, n, k, src, src_bytes);
    if (st) return st;
    const uint8_t* in = static_cast<const uint8_t*>(src);
    std::memcpy(codes, in, size_t(n * k));
    std::memcpy(scales, in + qg::scale_plane_offset(QG_Q8_0, n, k), size_t(n * (k / 32)) * 2);
    return QG_OK;
}

int qg_pack_fp8(int fmt, const uint8_t* codes, const float* scales, int64_t n, int64_t k, void* dst,
                size_t dst_bytes) {
    if (!qg::is_fp8(fmt)) return QG_EINVAL;
    int st = check_pack_args(fmt, codes, scales, n, k, dst, dst_bytes);
    if (st) return st;
    uint8_t* out = static_cast<uint8_t*>(dst);
    std::memset(out, 0, size_t(qg::packed_bytes(fmt, n, k)));
    std::memcpy(out, codes, size_t(n * k));
    std::memcpy(out + qg::scale_plane_offset(fmt, n, k), scales, size_t(qg::scale_plane_bytes(fmt, n, k)));
    return QG_OK;
}

int qg_unpack_fp8(int fmt, const void* src, size_t src_bytes, int64_t n, int64_t k, uint8_t* codes,
                  float* scales) {
    if (!qg::is_fp8(fmt)) return QG_EINVAL;
    int st = check_pack_args(fmt, codes, scales, n, k, src, src_bytes);
    if (st) return st;
    const uint8_t* in = static_cast<const uint8_t*>(src);
    std::memcpy(codes, in, size_t(n * k));
    std::memcpy(scales, in + qg::scale_plane_offset(fmt, n, k), size_t(qg::scale_plane_bytes(fmt, n, k)));
    return QG_OK;
}

}  // extern "C"
