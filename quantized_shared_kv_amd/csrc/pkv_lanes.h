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

}  // namespace pkv
