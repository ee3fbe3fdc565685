// Matrix-core pool decode kernel: the split-record form (partial records for k_merge).
#include "pkv_decode_mfma.h"

namespace pkv {

int launch_pool_mfma_split(const DecodeLaunch& a, int total_wg, hipStream_t s, int rt, bool split_q) {
    return launch_pool_mfma_form<false>(a, total_wg, s, rt, split_q);
}

}  // namespace pkv
