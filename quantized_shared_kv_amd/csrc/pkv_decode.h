// Internal decode-attention plan shared by the decode translation units.
#pragma once

#include "pkv_internal.h"

namespace pkv {

constexpr int kMaxPoolsPerLaunch = 16;
constexpr int kMaxAgentsPerLaunch = 128;

// One pool of a decode launch.  The launch's agents are ordered by pool; pool
// rows are (agent of the pool, head of the kv head's group): row r of kv head g
// -> launch agent agent0 + r / G, q head g*G + r % G.
struct PoolEntry {
    const uint8_t* base;
    uint64_t off_kq, off_vn, off_ks, off_vmax, off_vc0;
    uint64_t part_off;     // float offset of this pool's partial records in the workspace
    uint32_t ge3[4];       // bit l set: layer l uses >= 3 bits
    uint32_t eq4[4];       // bit l set: layer l uses 4 bits
    int32_t T;             // tokens in the pool's layers of the call
    int32_t tc;            // token capacity rounded to 32
    int32_t rows;          // agents of this pool * G
    int32_t agent0;        // first launch agent of this pool
    int32_t splits;        // token splits per (layer, kv head)
    int32_t chunk;         // tokens per split (multiple of 32)
    int32_t rblocks;       // row blocks per (layer, kv head, split)
    int32_t rb_rows;       // rows per row block (the last block may hold fewer)
    int32_t wg_begin;      // first workgroup of this pool in the launch
    int32_t seg_begin;     // >= 0: a private segment decoded by k_seg (no pool-kernel workgroups),
                           // its first unit there; -1: decoded by the pool kernel
    int32_t agent_base;    // >= 0: the pool's launch agents agent0 + i are call agents
                           // agent_base + i (no table lookup needed); -1 otherwise
    uint32_t vsign[4];     // V rotation sign mask: output dimension i negated after the inverse FWHT
    int32_t kmode;         // K-scale granularity (PKV_KSCALE_*): where the K scale of a token lives
};

// K scales of pool layer l, kv head g: per tensor [tc] (shared by the heads), per token [tc],
// per channel [d]
__host__ __device__ inline uint64_t ks_offset(const PoolEntry& p, int l, int g, int hkv, int d) {
    if (p.kmode == PKV_KSCALE_TOKEN) return ((uint64_t)l * hkv + g) * p.tc;
    if (p.kmode == PKV_KSCALE_CHANNEL) return ((uint64_t)l * hkv + g) * d;
    return (uint64_t)l * p.tc;
}

struct DecodeLaunch {
    PoolEntry pools[kMaxPoolsPerLaunch];
    int16_t agent_id[kMaxAgentsPerLaunch];    // call-level agent index of each launch agent
    int16_t agent_pool[kMaxAgentsPerLaunch];  // pool entry of each launch agent
    int16_t agent_pos[kMaxAgentsPerLaunch];   // index of the agent among its pool's agents
    int16_t agent_pool2[kMaxAgentsPerLaunch]; // private pool entry of each launch agent, -1 for none
    int16_t agent_pos2[kMaxAgentsPerLaunch];  // index of the agent among its private pool's agents
    int32_t sfx_len[kMaxAgentsPerLaunch];
    const void* q;
    const void* sfx_k;
    const void* sfx_v;
    float* out;
    float* part;            // workspace base (floats)
    uint64_t sfx_part_off;  // float offset of suffix partial records
    int32_t n_pools, n_agents;
    int32_t q_dtype, sfx_dtype;
    int32_t hq, hkv, G, d;
    int32_t l0, lc;         // first pool layer of the call, layers in the call
    int32_t sfx_cap;
    int32_t has_sfx;
    int32_t fused;          // the pool kernel finishes the outputs itself (one split everywhere)
    int32_t has_private;    // some agent also attends a private pool (outputs merged by k_merge)
    int32_t seg_units;      // k_seg units: (agent, layer, kv head) of the small private pools
    int32_t sfx_wg_begin;   // >= 0: the pool kernel's workgroups from this one on do the native-window
                            // work (4 units each) instead of a separate kernel; -1: none
    float sm_log2;          // softmax scale * log2(e)
};

// V bits and prefix-sum of bits of pool layer l (bits of earlier layers).
__host__ __device__ inline int layer_bits(const PoolEntry& p, int l) {
    return 2 + ((p.ge3[l >> 5] >> (l & 31)) & 1u) + ((p.eq4[l >> 5] >> (l & 31)) & 1u);
}

__device__ inline int layer_bits_prefix(const PoolEntry& p, int l) {
    int acc = 2 * l;
    const int w = l >> 5, bit = l & 31;
    for (int i = 0; i < w; ++i) acc += __popc(p.ge3[i]) + __popc(p.eq4[i]);
    const uint32_t m = bit ? ((1u << bit) - 1u) : 0u;
    acc += __popc(p.ge3[w] & m) + __popc(p.eq4[w] & m);
    return acc;
}

// Matrix-core kernel: the pool-local workgroup index w -> (item, row block), item = (layer,
// kv head, split) in split-fastest order.  The row blocks of one item sit 8 workgroups apart, so
// with workgroups dealt to the 8 XCDs in turn they share an XCD (and its L2) when the pool's
// start is a multiple of 8; with one row block this is the identity.
__host__ __device__ inline int pool_item_of_wg(int w, int items, int rblocks, int* rb) {
    if (rblocks == 1) {
        *rb = 0;
        return w;
    }
    const int grp = w / (8 * rblocks), within = w % (8 * rblocks);
    const int cnt = items - grp * 8 < 8 ? items - grp * 8 : 8;
    *rb = within / cnt;
    return grp * 8 + within % cnt;
}

// Records of partial softmax state: [m (log2 units), l, acc[d]].
inline int record_floats(int d) { return 2 + d; }

// Launches implemented in pkv_decode_mfma.hip.
int launch_pool_mfma(const DecodeLaunch& a, int total_wg, hipStream_t s);

}  // namespace pkv
