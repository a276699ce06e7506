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

// Elements per scale block.
inline constexpr int64_t block_len(int fmt) { return fmt == QG_NVFP4 ? 16 : 32; }
// Bytes per scale.
inline constexpr int64_t scale_bytes(int fmt) { return fmt == QG_NVFP4 ? 1 : 2; }
// Bytes of codes per row.
inline constexpr int64_t code_row_bytes(int fmt, int64_t k) { return fmt == QG_Q8_0 ? k : k / 2; }
// Bytes of scales per row.
inline constexpr int64_t scale_row_bytes(int fmt, int64_t k) { return k / block_len(fmt) * scale_bytes(fmt); }

inline constexpr bool valid_fmt(int fmt) { return fmt == QG_NVFP4 || fmt == QG_Q8_0 || fmt == QG_Q4_0; }

// Shape rule shared by every entry point: n >= 1, k a positive multiple of 32,
// and sizes small enough that all byte offsets fit comfortably in int64.
inline constexpr bool valid_shape(int64_t n, int64_t k) {
    return n >= 1 && k >= 32 && k % 32 == 0 && n <= (int64_t(1) << 31) && k <= (int64_t(1) << 24);
}

inline constexpr int64_t scale_plane_offset(int fmt, int64_t n, int64_t k) {
    return align_up(n * code_row_bytes(fmt, k), kPlaneAlign);
}

inline constexpr int64_t packed_bytes(int fmt, int64_t n, int64_t k) {
    return scale_plane_offset(fmt, n, k) + align_up(n * scale_row_bytes(fmt, k), kPlaneAlign);
}

}  // namespace qg
