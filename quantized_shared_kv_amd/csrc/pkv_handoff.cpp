// Handing a pool over: a POD header that, with the image bytes, recreates the
// pool elsewhere (another buffer, process or device), and kv-head shards.
//
// PolyKV explainer, section 2.A: the shared context is computed once,
// compressed and stored as one object that every agent reads.  The image is
// position-independent (every region is an offset from the buffer's start), so
// handing it over is copying its bytes plus the header below.  A kv-head shard
// is the pool restricted to a contiguous range of kv heads: every region of the
// image is [layer][kv head]-major, so per layer each region of the range is one
// contiguous span, and the K scales ([layer][token], shared by the heads) are
// copied whole.  Decoding a shard with the matching query-head groups gives the
// same outputs as decoding the whole pool, because every (layer, kv head) is
// decoded independently; this is how the pool would be split over GPUs.
#include <hip/hip_runtime.h>

#include <cstring>

#include "pkv_internal.h"

namespace {

constexpr uint32_t kMagic = 0x31564B50u;  // "PKV1" in little-endian byte order

bool ranges_overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool pool_ok(const pkv_pool* p) {
    int err;
    if (!p || !p->base || !pkv::config_valid(&p->cfg, &err)) return false;
    for (int l = 0; l < p->cfg.n_layers; ++l)
        if (p->n_tokens[l] < 0 || p->n_tokens[l] > p->cfg.capacity_tokens) return false;
    return p->bytes == pool_bytes(&p->cfg);
}

}  // namespace

extern "C" {

int pool_export_header(const pkv_pool* pool, pkv_pool_header* out) {
    if (!out || !pool_ok(pool)) return PKV_EINVAL;
    pkv_pool_header h;
    std::memset(&h, 0, sizeof(h));
    h.magic = kMagic;
    h.abi_version = pkv_version();
    h.cfg = pool->cfg;
    for (int l = 0; l < pool->cfg.n_layers; ++l) h.n_tokens[l] = pool->n_tokens[l];
    h.image_bytes = pool->bytes;
    *out = h;
    return PKV_OK;
}

int pool_import(const pkv_pool_header* hdr, void* dev_buf, size_t dev_bytes, pkv_pool* out) {
    if (!hdr || !out) return PKV_EINVAL;
    if (hdr->magic != kMagic || hdr->abi_version / 100 != pkv_version() / 100) return PKV_EINVAL;
    int err;
    if (!pkv::config_valid(&hdr->cfg, &err)) return err;
    if (hdr->image_bytes != pool_bytes(&hdr->cfg)) return PKV_EINVAL;
    for (int l = 0; l < hdr->cfg.n_layers; ++l)
        if (hdr->n_tokens[l] < 0 || hdr->n_tokens[l] > hdr->cfg.capacity_tokens) return PKV_EINVAL;
    pkv_pool p;
    const int st = pool_build(&hdr->cfg, dev_buf, dev_bytes, &p);
    if (st != PKV_OK) return st;
    for (int l = 0; l < hdr->cfg.n_layers; ++l) p.n_tokens[l] = hdr->n_tokens[l];
    *out = p;
    return PKV_OK;
}

int pool_shard(const pkv_pool* src, int32_t head_begin, int32_t head_count, void* dev_buf, size_t dev_bytes,
               pkv_pool* out, void* stream) {
    if (!out || !pool_ok(src)) return PKV_EINVAL;
    const int H = src->cfg.n_kv_heads;
    if (head_begin < 0 || head_count < 1 || head_begin + head_count > H) return PKV_EINVAL;
    pkv_pool_config cfg = src->cfg;
    cfg.n_kv_heads = head_count;
    pkv_pool p;
    const int st = pool_build(&cfg, dev_buf, dev_bytes, &p);
    if (st != PKV_OK) return st;
    if (ranges_overlap(src->base, src->bytes, dev_buf, p.bytes)) return PKV_EINVAL;
    for (int l = 0; l < cfg.n_layers; ++l) p.n_tokens[l] = src->n_tokens[l];

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t* sb = static_cast<const uint8_t*>(src->base);
    uint8_t* db = static_cast<uint8_t*>(dev_buf);
    const uint64_t L = cfg.n_layers, tc = src->tc, d = cfg.head_dim, h0 = head_begin, hc = head_count;
    auto copy = [&](uint64_t dst_off, uint64_t src_off, uint64_t n) {
        return hipMemcpyAsync(db + dst_off, sb + src_off, n, hipMemcpyDeviceToDevice, s) == hipSuccess;
    };
    // K scales: per tensor one per token, shared by every head (copied whole); per token
    // [L][H][tc] and per channel [L][H][d] (the range's heads, layer by layer)
    const uint64_t kper = cfg.k_scale == PKV_KSCALE_TOKEN ? tc : cfg.k_scale == PKV_KSCALE_CHANNEL ? d : 0;
    bool ok = kper ? true : copy(p.off_ks, src->off_ks, L * tc * 4);
    for (uint64_t l = 0; ok && l < L; ++l) {
        const uint64_t bits = cfg.v_bits[l];
        ok = (!kper || copy(p.off_ks + l * hc * kper * 4, src->off_ks + (l * H + h0) * kper * 4, hc * kper * 4)) &&
             copy(p.off_kq + l * hc * tc * d, src->off_kq + (l * H + h0) * tc * d, hc * tc * d) &&
             copy(p.off_vn + l * hc * tc * 4, src->off_vn + (l * H + h0) * tc * 4, hc * tc * 4) &&
             copy(p.off_vmax + l * hc * 4, src->off_vmax + (l * H + h0) * 4, hc * 4) &&
             copy(p.off_vc[l], src->off_vc[l] + h0 * (tc / 8) * d * bits, hc * (tc / 8) * d * bits);
    }
    if (!ok) return PKV_EHIP;
    *out = p;
    return PKV_OK;
}

}  // extern "C"
