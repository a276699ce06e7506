// Packed layout V1: plane sizes and offsets (host and device code).
//
// A packed matrix is [codes plane][pad][scale plane][pad], every plane
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

// Elements per scale block (row-blocked formats).
inline constexpr int64_t block_len(int fmt) { return fmt == QG_NVFP4 ? 16 : 32; }
// Bytes per scale (row-blocked formats).
inline constexpr int64_t scale_bytes(int fmt) { return fmt == QG_NVFP4 ? 1 : 2; }
// Bytes of codes per row.
inline constexpr int64_t code_row_bytes(int fmt, int64_t k) {
    return fmt == QG_Q8_0 || is_fp8(fmt) ? k : k / 2;
}
// Bytes of scales per row (row-blocked formats).
inline constexpr int64_t scale_row_bytes(int fmt, int64_t k) { return k / block_len(fmt) * scale_bytes(fmt); }

// FP8 block-128: scale tiles of 128 x 128 weights.
constexpr int64_t kFp8Tile = 128;
// Number of fp32 scales of an FP8 matrix.
inline constexpr int64_t fp8_scale_count(int fmt, int64_t n, int64_t k) {
    return fmt == QG_FP8_TENSOR ? 1 : ((n + kFp8Tile - 1) / kFp8Tile) * ((k + kFp8Tile - 1) / kFp8Tile);
}

inline constexpr bool valid_fmt(int fmt) {
    return fmt == QG_NVFP4 || fmt == QG_Q8_0 || fmt == QG_Q4_0 || is_fp8(fmt);
}

// Shape rule shared by every entry point: n >= 1, k a positive multiple of 32,
// and sizes small enough that all byte offsets fit comfortably in int64.
inline constexpr bool valid_shape(int64_t n, int64_t k) {
    return n >= 1 && k >= 32 && k % 32 == 0 && n < (int64_t(1) << 31) && k <= (int64_t(1) << 24);
}

inline constexpr int64_t scale_plane_offset(int fmt, int64_t n, int64_t k) {
    return align_up(n * code_row_bytes(fmt, k), kPlaneAlign);
}

inline constexpr int64_t scale_plane_bytes(int fmt, int64_t n, int64_t k) {
    return is_fp8(fmt) ? 4 * fp8_scale_count(fmt, n, k) : n * scale_row_bytes(fmt, k);
}

inline constexpr int64_t packed_bytes(int fmt, int64_t n, int64_t k) {
    return scale_plane_offset(fmt, n, k) + align_up(scale_plane_bytes(fmt, n, k), kPlaneAlign);
}

}  // namespace qg
