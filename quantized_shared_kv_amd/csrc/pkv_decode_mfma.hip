// Matrix-core (MFMA) pool decode kernel for gfx950.  Not yet enabled.
#include "pkv_decode.h"

namespace pkv {

bool mfma_supported(const DecodeLaunch&) { return false; }

int launch_pool_mfma(const DecodeLaunch&, int, hipStream_t) { return PKV_EUNSUPPORTED; }

}  // namespace pkv
