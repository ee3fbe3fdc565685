// Matrix-core pool decode kernel: host launcher and the fused-finish form (the templates and the
// kernel's description are in pkv_decode_mfma.h).
#include "pkv_decode_mfma.h"

namespace pkv {

int launch_pool_mfma(const DecodeLaunch& a, int total_wg, hipStream_t s) {
    // rows per workgroup: the largest row block of the launch's pools (the plan keeps blocks at
    // most 64 rows, 48 with fp32 queries, whose hi + lo operands take twice the registers)
    // fp32 queries, and queries carrying a per-channel pool's K scales, take fp16 hi + lo operands
    int rows = 1;
    bool split = a.q_dtype == PKV_F32;
    for (int p = 0; p < a.n_pools; ++p)
        if (a.pools[p].seg_begin < 0) {
            rows = rows > a.pools[p].rb_rows ? rows : a.pools[p].rb_rows;
            split = split || a.pools[p].kmode == PKV_KSCALE_CHANNEL;
        }
    if (rows > (split ? 48 : kMaxRows)) return PKV_EUNSUPPORTED;
    const int rt = (rows + 15) / 16;
    return a.fused ? launch_pool_mfma_form<true>(a, total_wg, s, rt, split)
                   : launch_pool_mfma_split(a, total_wg, s, rt, split);
}

}  // namespace pkv
