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
        case QG_EVERSION: return "packed buffer or descriptor of another layout version";
        case QG_ENOSPC: return "destination or workspace buffer too small";
        case QG_EHIP: return "HIP runtime or launch error";
        default: return "unknown status";
    }
}

size_t qg_packed_bytes(int fmt, int64_t n, int64_t k) {
    if (!qg::valid_fmt(fmt) || !qg::valid_fmt_shape(fmt, n, k)) return 0;
    return size_t(qg::packed_bytes(fmt, n, k));
}

size_t qg_scale_plane_offset(int fmt, int64_t n, int64_t k) {
    if (!qg::valid_fmt(fmt) || !qg::valid_fmt_shape(fmt, n, k)) return 0;
    return size_t(qg::scale_plane_offset(fmt, n, k));
}

// ---------------------------------------------------------------- layout stamp

namespace {

void write_stamp(void* buf, int fmt, uint32_t kind, int64_t n, int64_t k) {
    qg::Stamp st{qg::kStampMagic, uint32_t(QG_LAYOUT_VERSION), uint32_t(fmt), kind, n, k};
    std::memcpy(static_cast<uint8_t*>(buf) + qg::stamp_offset(fmt, n, k), &st, sizeof st);
}

// The stamp of a packed host buffer of at least packed_bytes(fmt, n, k).
int check_stamp(const void* buf, int fmt, uint32_t kind, int64_t n, int64_t k) {
    qg::Stamp st;
    std::memcpy(&st, static_cast<const uint8_t*>(buf) + qg::stamp_offset(fmt, n, k), sizeof st);
    if (st.magic != qg::kStampMagic) return QG_EINVAL;
    if (st.version != uint32_t(QG_LAYOUT_VERSION)) return QG_EVERSION;
    if (st.fmt != uint32_t(fmt) || st.kind != kind || st.n != n || st.k != k) return QG_EINVAL;
    return QG_OK;
}

}  // namespace

int qg_packed_check(int fmt, const void* buf, size_t bytes, int64_t n, int64_t k) {
    const uint32_t kind = fmt == QG_NVFP4_GATE_UP ? qg::kKindGateUp : qg::kKindPlain;
    if (fmt == QG_NVFP4_GATE_UP) {
        fmt = QG_NVFP4;
        if (n % 2) return QG_EINVAL;
    }
    if (!buf || !qg::valid_fmt(fmt) || !qg::valid_fmt_shape(fmt, n, k)) return QG_EINVAL;
    if (bytes < size_t(qg::packed_bytes(fmt, n, k))) return QG_ENOSPC;
    return check_stamp(buf, fmt, kind, n, k);
}

// ---------------------------------------------------------------- packers

static int check_pack_args(int fmt, const void* a, const void* b, int64_t n, int64_t k,
                           const void* buf, size_t bytes) {
    if (!a || !b || !buf) return QG_EINVAL;
    if (!qg::valid_fmt_shape(fmt, n, k)) return QG_EINVAL;
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
    write_stamp(out, QG_NVFP4, qg::kKindPlain, n, k);
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
    write_stamp(out, QG_Q4_0, qg::kKindPlain, n, k);
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
    write_stamp(out, QG_Q8_0, qg::kKindPlain, n, k);
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
    write_stamp(out, QG_NVFP4, qg::kKindGateUp, n, k);
    return QG_OK;
}

// ---------------------------------------------------------------- unpackers

int qg_unpack_nvfp4(const void* src, size_t src_bytes, int64_t n, int64_t k, uint8_t* codes,
                    uint8_t* scales) {
    int st = check_pack_args(QG_NVFP4, codes, scales, n, k, src, src_bytes);
    if (st) return st;
    if ((st = check_stamp(src, QG_NVFP4, qg::kKindPlain, n, k))) return st;
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
    if ((st = check_stamp(src, QG_NVFP4, qg::kKindGateUp, n, k))) return st;
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
    if ((st = check_stamp(src, QG_Q4_0, qg::kKindPlain, n, k))) return st;
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
    if ((st = check_stamp(src, QG_Q8_0, qg::kKindPlain, n, k))) return st;
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
    write_stamp(out, fmt, qg::kKindPlain, n, k);
    return QG_OK;
}

int qg_unpack_fp8(int fmt, const void* src, size_t src_bytes, int64_t n, int64_t k, uint8_t* codes,
                  float* scales) {
    if (!qg::is_fp8(fmt)) return QG_EINVAL;
    int st = check_pack_args(fmt, codes, scales, n, k, src, src_bytes);
    if (st) return st;
    if ((st = check_stamp(src, fmt, qg::kKindPlain, n, k))) return st;
    const uint8_t* in = static_cast<const uint8_t*>(src);
    std::memcpy(codes, in, size_t(n * k));
    std::memcpy(scales, in + qg::scale_plane_offset(fmt, n, k), size_t(qg::scale_plane_bytes(fmt, n, k)));
    return QG_OK;
}

// ---------------------------------------------------------------- K-quants

static int kq_code_limit(int fmt) { return fmt == QG_Q5_K ? 32 : fmt == QG_Q6_K ? 64 : 16; }
static bool kq_has_min(int fmt) { return fmt == QG_Q4_K || fmt == QG_Q5_K; }
// Bit position of the high code bits of element e (0..31) of a block in its
// dword: Q5_K one bit, Q6_K two bits (e < 16 in the first dword, else the
// second).  Four consecutive elements land one byte apart.
static int kq5_bit(int e) { return 8 * (e % 4) + e / 4; }
static int kq6_bit(int e) { return 8 * (e % 16 % 4) + 2 * (e % 16 / 4); }

static int check_kquant_args(int fmt, const void* codes, const void* d, const void* dmin, const void* sub,
                             const void* mins, int64_t n, int64_t k, const void* buf, size_t bytes) {
    if (!qg::is_kquant(fmt) || !codes || !d || !sub || !buf) return QG_EINVAL;
    if (kq_has_min(fmt) && (!dmin || !mins)) return QG_EINVAL;
    if (!qg::valid_fmt_shape(fmt, n, k)) return QG_EINVAL;
    if (bytes < size_t(qg::packed_bytes(fmt, n, k))) return QG_ENOSPC;
    return QG_OK;
}

int qg_pack_kquant(int fmt, const uint8_t* codes, const uint16_t* d, const uint16_t* dmin, const uint8_t* sub,
                   const uint8_t* mins, int64_t n, int64_t k, void* dst, size_t dst_bytes) {
    int st = check_kquant_args(fmt, codes, d, dmin, sub, mins, n, k, dst, dst_bytes);
    if (st) return st;
    const int lim = kq_code_limit(fmt);
    for (int64_t i = 0; i < n * k; ++i)
        if (codes[i] >= lim) return QG_EINVAL;
    if (fmt != QG_Q6_K)
        for (int64_t i = 0; i < n * (k / 32); ++i)
            if (sub[i] > 63 || (kq_has_min(fmt) && mins[i] > 63)) return QG_EINVAL;
    uint8_t* out = static_cast<uint8_t*>(dst);
    std::memset(out, 0, size_t(qg::packed_bytes(fmt, n, k)));
    const int64_t crow = qg::code_row_bytes(fmt, k), srow = qg::scale_row_bytes(fmt, k);
    const int64_t S = k / qg::kKqSuper, B = k / 32, sup = qg::kq_super_bytes(fmt, k);
    uint8_t* splane = out + qg::scale_plane_offset(fmt, n, k);
    for (int64_t r = 0; r < n; ++r) {
        const uint8_t* c = codes + r * k;
        uint8_t* o = out + r * crow;
        uint8_t* hb = o + k / 2;
        for (int64_t b = 0; b < B; ++b) {
            for (int i = 0; i < 16; ++i)
                o[16 * b + i] = uint8_t((c[32 * b + i] & 15) | ((c[32 * b + 16 + i] & 15) << 4));
            if (fmt == QG_Q5_K) {
                uint32_t h = 0;
                for (int e = 0; e < 32; ++e) h |= uint32_t(c[32 * b + e] >> 4) << kq5_bit(e);
                std::memcpy(hb + 4 * b, &h, 4);
            } else if (fmt == QG_Q6_K) {
                uint32_t h[2] = {0, 0};
                for (int e = 0; e < 32; ++e) h[e / 16] |= uint32_t(c[32 * b + e] >> 4) << kq6_bit(e);
                std::memcpy(hb + 8 * b, h, 8);
            }
        }
        uint8_t* so = splane + r * srow;
        for (int64_t s = 0; s < S; ++s) {
            if (kq_has_min(fmt)) {
                const uint32_t v = uint32_t(d[r * S + s]) | (uint32_t(dmin[r * S + s]) << 16);
                std::memcpy(so + 4 * s, &v, 4);
            } else {
                std::memcpy(so + 2 * s, &d[r * S + s], 2);
            }
        }
        if (kq_has_min(fmt)) {
            for (int64_t b = 0; b < B; ++b) {
                so[sup + 2 * b] = sub[r * B + b];
                so[sup + 2 * b + 1] = mins[r * B + b];
            }
        } else {
            std::memcpy(so + sup, sub + r * qg::kq_sub_bytes(fmt, k), size_t(qg::kq_sub_bytes(fmt, k)));
        }
    }
    write_stamp(out, fmt, qg::kKindPlain, n, k);
    return QG_OK;
}

int qg_unpack_kquant(int fmt, const void* src, size_t src_bytes, int64_t n, int64_t k, uint8_t* codes,
                     uint16_t* d, uint16_t* dmin, uint8_t* sub, uint8_t* mins) {
    int st = check_kquant_args(fmt, codes, d, dmin, sub, mins, n, k, src, src_bytes);
    if (st) return st;
    if ((st = check_stamp(src, fmt, qg::kKindPlain, n, k))) return st;
    const uint8_t* in = static_cast<const uint8_t*>(src);
    const int64_t crow = qg::code_row_bytes(fmt, k), srow = qg::scale_row_bytes(fmt, k);
    const int64_t S = k / qg::kKqSuper, B = k / 32, sup = qg::kq_super_bytes(fmt, k);
    const uint8_t* splane = in + qg::scale_plane_offset(fmt, n, k);
    for (int64_t r = 0; r < n; ++r) {
        const uint8_t* o = in + r * crow;
        const uint8_t* hb = o + k / 2;
        uint8_t* c = codes + r * k;
        for (int64_t b = 0; b < B; ++b) {
            for (int i = 0; i < 16; ++i) {
                c[32 * b + i] = o[16 * b + i] & 15;
                c[32 * b + 16 + i] = o[16 * b + i] >> 4;
            }
            if (fmt == QG_Q5_K) {
                uint32_t h;
                std::memcpy(&h, hb + 4 * b, 4);
                for (int e = 0; e < 32; ++e) c[32 * b + e] |= uint8_t(((h >> kq5_bit(e)) & 1) << 4);
            } else if (fmt == QG_Q6_K) {
                uint32_t h[2];
                std::memcpy(h, hb + 8 * b, 8);
                for (int e = 0; e < 32; ++e) c[32 * b + e] |= uint8_t(((h[e / 16] >> kq6_bit(e)) & 3) << 4);
            }
        }
        const uint8_t* so = splane + r * srow;
        for (int64_t s = 0; s < S; ++s) {
            if (kq_has_min(fmt)) {
                uint32_t v;
                std::memcpy(&v, so + 4 * s, 4);
                d[r * S + s] = uint16_t(v & 0xFFFF);
                dmin[r * S + s] = uint16_t(v >> 16);
            } else {
                std::memcpy(&d[r * S + s], so + 2 * s, 2);
            }
        }
        if (kq_has_min(fmt)) {
            for (int64_t b = 0; b < B; ++b) {
                sub[r * B + b] = so[sup + 2 * b];
                mins[r * B + b] = so[sup + 2 * b + 1];
            }
        } else {
            std::memcpy(sub + r * qg::kq_sub_bytes(fmt, k), so + sup, size_t(qg::kq_sub_bytes(fmt, k)));
        }
    }
    return QG_OK;
}

}  // extern "C"
