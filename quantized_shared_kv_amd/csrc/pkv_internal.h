// Internal declarations shared by the translation units of libpolykv.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "polykv.h"

namespace pkv {

// fp32 Lloyd-Max N(0,1) tables for 2, 3 and 4 bits, index [bits - 2].
// Thresholds beyond 2^bits - 1 and centroids beyond 2^bits are padding.
struct CodebookTables {
    float thr[3][15];
    float cent[3][16];
    // fp16 operand scale of each table: fp16(fp32(s * c)) / s is within the smallest relative
    // distance of c, over s = 1 + j / 2^16 (j < 2^16), that any s reaches for every centroid
    // at once.  The matrix-core decode takes its centroids as fp16 (s * c) and divides s back
    // out of the weights; fp16 (c) itself is off by up to 4.9e-4 (4 bits).
    float fp16_scale[3];
    float fp16_err[3];  // that largest relative distance, per table
};

// Computed once on the host from the Lloyd-Max conditions (see pkv_host.cpp).
const CodebookTables& codebook_tables();

constexpr int kGroupTokens = 8;   // tokens per packed V code group
constexpr int kTokenRound = 32;   // capacity rounding (one decode step of tokens)
constexpr uint64_t kAlign = 256;

inline uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool config_valid(const pkv_pool_config* cfg, int* err);

// Offset of layer l's code region relative to off_vc[0]: Hkv * tc * d / 8 * (sum of earlier bits).
inline uint64_t vc_layer_offset(int hkv, int tc, int d, const uint8_t* bits, int l) {
    uint64_t acc = 0;
    for (int i = 0; i < l; ++i) acc += bits[i];
    return (uint64_t)hkv * tc * (d / 8) * acc;
}

int launch_status();  // PKV_OK or PKV_EHIP from hipGetLastError

}  // namespace pkv
