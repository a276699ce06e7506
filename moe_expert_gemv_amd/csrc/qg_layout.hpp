// Packed layout (version QG_LAYOUT_VERSION): plane sizes and offsets (host and
// device code).
//
// A packed matrix is [codes plane][pad][scale plane][pad][stamp], every plane
// 256-byte aligned.  Rows of both planes are stored back to back; with
// k % 32 == 0 every row starts on a 16-byte boundary.
#pragma once

#include <cstddef>
#include <cstdint>

#include "qgemv.h"

namespace qg {

constexpr int64_t kPlaneAlign = 256;

inline constexpr int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

inline constexpr bool is_fp8(int fmt) { return fmt == QG_FP8_TENSOR || fmt == QG_FP8_B128; }
inline constexpr bool is_kquant(int fmt) { return fmt >= QG_Q4_K && fmt <= QG_IQ4_XS; }

// K-quants and IQ4_XS: super-blocks of 256 elements.  Codes row: the 4-bit
// plane (Q4_0 nibble order per 32 elements), then the high code bits (Q5_K
// one, Q6_K two per element).  Scale row: the per-super-block part (fp16 d,
// plus fp16 dmin for Q4_K / Q5_K), then the per-32-element part.
constexpr int64_t kKqSuper = 256;
inline constexpr int64_t kq_high_bytes(int fmt, int64_t k) {
    return fmt == QG_Q5_K ? k / 8 : fmt == QG_Q6_K ? k / 4 : 0;
}
inline constexpr int64_t kq_super_bytes(int fmt, int64_t k) {
    return (fmt == QG_Q4_K || fmt == QG_Q5_K ? 4 : 2) * (k / kKqSuper);
}
inline constexpr int64_t kq_sub_bytes(int fmt, int64_t k) { return (fmt == QG_IQ4_XS ? 1 : 2) * (k / 32); }

// Elements per scale block (row-blocked formats).
inline constexpr int64_t block_len(int fmt) { return fmt == QG_NVFP4 ? 16 : 32; }
// Bytes per scale (row-blocked formats).
inline constexpr int64_t scale_bytes(int fmt) { return fmt == QG_NVFP4 ? 1 : 2; }
// Bytes of codes per row.
inline constexpr int64_t code_row_bytes(int fmt, int64_t k) {
    return fmt == QG_Q8_0 || is_fp8(fmt) ? k : k / 2 + kq_high_bytes(fmt, k);
}
// Bytes of scales per row (row-blocked formats and K-quants).
inline constexpr int64_t scale_row_bytes(int fmt, int64_t k) {
    return is_kquant(fmt) ? kq_super_bytes(fmt, k) + kq_sub_bytes(fmt, k) : k / block_len(fmt) * scale_bytes(fmt);
}

// FP8 block-128: scale tiles of 128 x 128 weights.
constexpr int64_t kFp8Tile = 128;
// Number of fp32 scales of an FP8 matrix.
inline constexpr int64_t fp8_scale_count(int fmt, int64_t n, int64_t k) {
    return fmt == QG_FP8_TENSOR ? 1 : ((n + kFp8Tile - 1) / kFp8Tile) * ((k + kFp8Tile - 1) / kFp8Tile);
}

inline constexpr bool valid_fmt(int fmt) {
    return fmt == QG_NVFP4 || fmt == QG_Q8_0 || fmt == QG_Q4_0 || is_fp8(fmt) || is_kquant(fmt);
}

// Shape rule shared by every entry point: n >= 1, k a positive multiple of 32,
// and sizes small enough that all byte offsets fit comfortably in int64.
inline constexpr bool valid_shape(int64_t n, int64_t k) {
    return n >= 1 && k >= 32 && k % 32 == 0 && n < (int64_t(1) << 31) && k <= (int64_t(1) << 24);
}

// The shape rule plus the format's own: K-quant rows are whole super-blocks.
inline constexpr bool valid_fmt_shape(int fmt, int64_t n, int64_t k) {
    return valid_shape(n, k) && (!is_kquant(fmt) || k % kKqSuper == 0);
}

inline constexpr int64_t scale_plane_offset(int fmt, int64_t n, int64_t k) {
    return align_up(n * code_row_bytes(fmt, k), kPlaneAlign);
}

inline constexpr int64_t scale_plane_bytes(int fmt, int64_t n, int64_t k) {
    return is_fp8(fmt) ? 4 * fp8_scale_count(fmt, n, k) : n * scale_row_bytes(fmt, k);
}

// Layout stamp: the last kStampBytes of every packed matrix name its layout
// version, format, row order and shape, so that a buffer written by another
// layout version is rejected rather than misread.  The kernels never read it.
constexpr int64_t kStampBytes = 256;
constexpr uint32_t kStampMagic = 0x4B504751u;  // the bytes "QGPK"
constexpr uint32_t kKindPlain = 0;             // rows in logical order
constexpr uint32_t kKindGateUp = 1;            // fused gate/up, rows interleaved
struct Stamp {
    uint32_t magic;
    uint32_t version;
    uint32_t fmt;
    uint32_t kind;
    int64_t n;
    int64_t k;
};

inline constexpr int64_t stamp_offset(int fmt, int64_t n, int64_t k) {
    return scale_plane_offset(fmt, n, k) + align_up(scale_plane_bytes(fmt, n, k), kPlaneAlign);
}

inline constexpr int64_t packed_bytes(int fmt, int64_t n, int64_t k) { return stamp_offset(fmt, n, k) + kStampBytes; }

}  // namespace qg
