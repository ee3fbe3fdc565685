// Cross-lane exchanges within a 64-lane wavefront (gfx950).
//
// lane_xor<M>(v) returns v from lane (lane ^ M).  xor 1 and 2 use DPP quad
// permutes (plain VALU moves), xor 4, 8 and 16 use ds_swizzle in bit mode
// (no address computation), xor 32 uses ds_bpermute.  All of them move the
// exact bits, so reductions built on them give the same values as any other
// exchange.
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {

template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    const int x = __builtin_bit_cast(int, v);
    if constexpr (M == 1) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
    } else if constexpr (M == 2) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
    } else if constexpr (M == 4 || M == 8 || M == 16) {
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(x, (M << 10) | 0x1F));
    } else {
        return __shfl_xor(v, M, 64);
    }
}

// lane_xor_row<M>(v, lane) for M in {1, 2, 4, 8}: the value of lane (lane ^ M),
// from DPP moves alone (no LDS-pipe swizzle).  Within a 16-lane row, row_ror:n
// hands lane i the value of lane (i - n) mod 16; the partner at distance 4 is
// lane i + 4 (rotation by 12) when bit 2 of i is clear and i - 4 (rotation by 4)
// otherwise, and the one at distance 8 is lane (i + 8) mod 16 either way.
template <int M>
__device__ __forceinline__ float lane_xor_row(float v, int lane) {
    const int x = __builtin_bit_cast(int, v);
    if constexpr (M == 1 || M == 2) {
        return lane_xor<M>(v);
    } else if constexpr (M == 4) {
        const int down = __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, true);  // row_ror:4  -> lane i - 4
        const int up = __builtin_amdgcn_mov_dpp(x, 0x12C, 0xF, 0xF, true);    // row_ror:12 -> lane i + 4
        return __builtin_bit_cast(float, (lane & 4) ? down : up);
    } else {
        static_assert(M == 8, "distance within a 16-lane row");
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true));  // row_ror:8
    }
}

}  // namespace pkv
