// Cross-lane reduce-scatter for wave64 kernels that end with several row sums
// per lane (several rows x several tokens): the sums leave the wave one per
// lane instead of through one full butterfly per sum.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "qg_device.hpp"

namespace qg {

// Exchange with lane ^ X inside aligned 32-lane halves (X < 32), or across
// the halves (X == 32).
template <int X>
__device__ __forceinline__ float xor_lane(float v) {
    if constexpr (X == 1) return dpp_mov<0xB1>(v);  // quad_perm [1,0,3,2]
    if constexpr (X == 2) return dpp_mov<0x4E>(v);  // quad_perm [2,3,0,1]
    if constexpr (X >= 4 && X <= 16)
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (X << 10)));
    if constexpr (X == 32)
        return __int_as_float(__builtin_amdgcn_ds_bpermute((lane_id() ^ 32) << 2, __float_as_int(v)));
    return v;
}

constexpr int log2i(int n) { return n <= 1 ? 0 : 1 + log2i(n / 2); }

// Reduce-scatter of N = 2^L values over the 64 lanes of a wave: the result
// for value index bitrev_L(lane % N) ends in that lane (and in every lane
// congruent to it mod N).  Level j pairs lane l with l ^ 2^j, exactly as
// group_sum<64> does (its row mirrors pair the same quads and halves), and
// adds the two partial sums of the same lane sets, so every value is
// bitwise the group_sum<64> result -- with about 3 instructions per value
// pair per level instead of one butterfly per value.
template <int N>
__device__ __forceinline__ float reduce_scatter64(float (&v)[N]) {
    static_assert((N & (N - 1)) == 0 && N >= 1 && N <= 64, "power of two up to 64");
    const int lane = lane_id();
    float w[N];
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = v[i];
    auto level = [&](auto x_c, auto h_c) {
        constexpr int X = decltype(x_c)::value, H = decltype(h_c)::value;
        const bool hi = (lane & X) != 0;
#pragma unroll
        for (int i = 0; i < H; ++i) {
            const float keep = hi ? w[i + H] : w[i];
            const float send = hi ? w[i] : w[i + H];
            w[i] = keep + xor_lane<X>(send);
        }
    };
    using std::integral_constant;
    if constexpr (N >= 2) level(integral_constant<int, 1>{}, integral_constant<int, N / 2>{});
    if constexpr (N >= 4) level(integral_constant<int, 2>{}, integral_constant<int, N / 4>{});
    if constexpr (N >= 8) level(integral_constant<int, 4>{}, integral_constant<int, N / 8>{});
    if constexpr (N >= 16) level(integral_constant<int, 8>{}, integral_constant<int, N / 16>{});
    if constexpr (N >= 32) level(integral_constant<int, 16>{}, integral_constant<int, N / 32>{});
    if constexpr (N >= 64) level(integral_constant<int, 32>{}, integral_constant<int, 1>{});
    float r = w[0];
    if constexpr (N < 2) r += xor_lane<1>(r);
    if constexpr (N < 4) r += xor_lane<2>(r);
    if constexpr (N < 8) r += xor_lane<4>(r);
    if constexpr (N < 16) r += xor_lane<8>(r);
    if constexpr (N < 32) r += xor_lane<16>(r);
    if constexpr (N < 64) r += xor_lane<32>(r);
    return r;
}

// bit-reversal of the low L bits
template <int L>
__device__ __forceinline__ int bitrev(int x) {
    int r = 0;
#pragma unroll
    for (int b = 0; b < L; ++b) r |= ((x >> b) & 1) << (L - 1 - b);
    return r;
}

}  // namespace qg
