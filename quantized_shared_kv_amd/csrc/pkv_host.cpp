// Host-side parts of libpolykv: Lloyd-Max tables, pool layout, error strings.
//
// PolyKV explainer, section 2.B: rotated V coordinates are mapped to
// Lloyd-Max centroids for N(0, 1).  The pages print no table, so it is
// computed here from the two optimality conditions (thresholds are midpoints
// of neighbouring centroids; each centroid is the mean of N(0, 1) restricted
// to its cell) by Lloyd iteration in double on the positive half-line, then
// mirrored and rounded to fp32.
#include <cmath>
#include <cstring>
#include <mutex>

#include "pkv_internal.h"

namespace pkv {
namespace {

double normal_pdf(double x) {
    if (std::isinf(x)) return 0.0;
    return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
}

// P(a < X <= b) for 0 <= a < b <= inf, from upper-tail probabilities.
double upper_mass(double a, double b) {
    const double r = 1.0 / std::sqrt(2.0);
    const double ta = 0.5 * std::erfc(a * r);
    const double tb = std::isinf(b) ? 0.0 : 0.5 * std::erfc(b * r);
    return ta - tb;
}

// Positive-half centroids of the 2^bits-level quantiser.
void lloyd_positive(int bits, double* c) {
    const int half = (1 << bits) / 2;
    for (int j = 0; j < half; ++j) c[j] = (j + 0.5) * 3.0 / half;  // any increasing start converges
    double lo[8], hi[8], nc[8];
    for (int it = 0; it < 200000; ++it) {
        lo[0] = 0.0;
        for (int j = 1; j < half; ++j) lo[j] = 0.5 * (c[j - 1] + c[j]);
        for (int j = 0; j + 1 < half; ++j) hi[j] = lo[j + 1];
        hi[half - 1] = INFINITY;
        double delta = 0.0;
        for (int j = 0; j < half; ++j) {
            nc[j] = (normal_pdf(lo[j]) - normal_pdf(hi[j])) / upper_mass(lo[j], hi[j]);
            delta = std::fmax(delta, std::fabs(nc[j] - c[j]));
        }
        for (int j = 0; j < half; ++j) c[j] = nc[j];
        if (delta <= 1e-14) break;
    }
}

// x rounded to the nearest fp16 value, ties to even (x a normal fp16 magnitude: 2^-14 <= |x| < 65504)
double round_fp16(float x) {
    int e = 0;
    std::frexp(x, &e);  // |x| in [2^(e-1), 2^e): 11 significant bits in fp16
    return std::ldexp(std::nearbyint(std::ldexp((double)x, 11 - e)), e - 11);
}

// The scale s of one table (see CodebookTables::fp16_scale): the positive centroids are
// enough (the table is symmetric).
void fp16_operand_scale(const float* cpos, int half, float* scale, float* err) {
    double best = INFINITY;
    float best_s = 1.0f;
    for (int j = 0; j < (1 << 16); ++j) {
        const float sc = 1.0f + (float)j / 65536.0f;  // exact in fp32
        double worst = 0.0;
        for (int k = 0; k < half && worst < best; ++k) {
            const float v = sc * cpos[k];  // the fp32 value the device rounds to fp16
            worst = std::fmax(worst, std::fabs(round_fp16(v) / sc - (double)cpos[k]) / (double)cpos[k]);
        }
        if (worst < best) {
            best = worst;
            best_s = sc;
        }
    }
    *scale = best_s;
    *err = (float)best;
}

CodebookTables build_tables() {
    CodebookTables t;
    std::memset(&t, 0, sizeof(t));
    for (int bits = 2; bits <= 4; ++bits) {
        const int levels = 1 << bits, half = levels / 2;
        double cpos[8];
        lloyd_positive(bits, cpos);
        float* cent = t.cent[bits - 2];
        float* thr = t.thr[bits - 2];
        for (int j = 0; j < half; ++j) {
            cent[half + j] = (float)cpos[j];
            cent[half - 1 - j] = (float)(-cpos[j]);
        }
        thr[half - 1] = 0.0f;
        for (int j = 1; j < half; ++j) {
            const double m = 0.5 * (cpos[j - 1] + cpos[j]);
            thr[half - 1 + j] = (float)m;
            thr[half - 1 - j] = (float)(-m);
        }
        fp16_operand_scale(cent + half, half, &t.fp16_scale[bits - 2], &t.fp16_err[bits - 2]);
    }
    return t;
}

}  // namespace

const CodebookTables& codebook_tables() {
    static const CodebookTables t = build_tables();
    return t;
}

bool config_valid(const pkv_pool_config* cfg, int* err) {
    *err = PKV_EINVAL;
    if (!cfg) return false;
    if (cfg->n_layers < 1 || cfg->n_layers > PKV_MAX_LAYERS) return false;
    if (cfg->n_kv_heads < 1 || cfg->capacity_tokens < 1) return false;
    *err = PKV_EUNSUPPORTED;
    if (cfg->head_dim != 64 && cfg->head_dim != 128) return false;
    for (int l = 0; l < cfg->n_layers; ++l)
        if (cfg->v_bits[l] < 2 || cfg->v_bits[l] > 4) return false;
    if (cfg->k_scale > PKV_KSCALE_CHANNEL || cfg->v_norm > PKV_VNORM_CORRECTED) return false;
    *err = PKV_EINVAL;
    for (int i = cfg->head_dim / 8; i < 16; ++i)
        if (cfg->v_signs[i]) return false;  // sign bits past head_dim
    if (cfg->reserved[0] || cfg->reserved[1]) return false;
    // keep every region offset inside 64-bit arithmetic with a wide margin
    const double est = (double)cfg->n_layers * cfg->n_kv_heads * ((double)cfg->capacity_tokens + 32) *
                       (cfg->head_dim * 1.5 + 8.0);
    *err = PKV_EINVAL;
    if (est > 1e15) return false;
    *err = PKV_OK;
    return true;
}

int launch_status() { return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP; }

namespace {

void fill_layout(const pkv_pool_config* cfg, pkv_pool* p) {
    const uint64_t L = cfg->n_layers, H = cfg->n_kv_heads, d = cfg->head_dim;
    const uint64_t tc = ((uint64_t)cfg->capacity_tokens + kTokenRound - 1) / kTokenRound * kTokenRound;
    p->tc = (int32_t)tc;
    p->off_kq = 0;
    p->off_vn = align_up(p->off_kq + L * H * tc * d);
    p->off_ks = align_up(p->off_vn + L * H * tc * 4);
    const uint64_t ks_bytes = cfg->k_scale == PKV_KSCALE_TOKEN     ? L * H * tc * 4
                              : cfg->k_scale == PKV_KSCALE_CHANNEL ? L * H * d * 4
                                                                   : L * tc * 4;
    p->off_vmax = align_up(p->off_ks + ks_bytes);
    p->off_vc[0] = align_up(p->off_vmax + L * H * 4);
    for (uint64_t l = 0; l < L; ++l) p->off_vc[l + 1] = p->off_vc[l] + H * tc * d * cfg->v_bits[l] / 8;
    p->off_amax = align_up(p->off_vc[L]);
    p->bytes = align_up(p->off_amax + (cfg->k_scale == PKV_KSCALE_CHANNEL ? L * H * d * 4 : L * 4));
}

}  // namespace
}  // namespace pkv

extern "C" {

size_t pool_bytes(const pkv_pool_config* cfg) {
    int err;
    if (!pkv::config_valid(cfg, &err)) return 0;
    pkv_pool p;
    std::memset(&p, 0, sizeof(p));
    pkv::fill_layout(cfg, &p);
    return (size_t)p.bytes;
}

int pool_build(const pkv_pool_config* cfg, void* dev_buf, size_t dev_bytes, pkv_pool* out) {
    int err;
    if (!out) return PKV_EINVAL;
    if (!pkv::config_valid(cfg, &err)) return err;
    if (!dev_buf || ((uintptr_t)dev_buf % pkv::kAlign) != 0) return PKV_EINVAL;
    pkv_pool p;
    std::memset(&p, 0, sizeof(p));
    p.cfg = *cfg;
    for (int l = cfg->n_layers; l < PKV_MAX_LAYERS; ++l) p.cfg.v_bits[l] = 0;
    pkv::fill_layout(cfg, &p);
    if (dev_bytes < p.bytes) return PKV_ENOSPACE;
    p.base = dev_buf;
    *out = p;
    return PKV_OK;
}

const char* pkv_strerror(int code) {
    switch (code) {
        case PKV_OK: return "ok";
        case PKV_EINVAL: return "invalid argument";
        case PKV_EUNSUPPORTED: return "unsupported head_dim, bit width or dtype";
        case PKV_ECAPACITY: return "append exceeds pool capacity";
        case PKV_ENOSPACE: return "buffer or workspace too small";
        case PKV_EHIP: return "HIP kernel launch failed";
        default: return "unknown error";
    }
}

int pkv_version(void) { return 106; }

size_t pkv_abi_sizeof(int32_t which) {
    switch (which) {
        case 0: return sizeof(pkv_pool_config);
        case 1: return sizeof(pkv_pool);
        case 2: return sizeof(pkv_decode_args);
        case 3: return sizeof(pkv_comix_args);
        case 4: return sizeof(pkv_pool_header);
        default: return 0;
    }
}

int pkv_lloyd_max_table(int32_t bits, float* centroids, float* thresholds) {
    if (bits < 2 || bits > 4) return PKV_EUNSUPPORTED;
    const pkv::CodebookTables& t = pkv::codebook_tables();
    if (centroids) std::memcpy(centroids, t.cent[bits - 2], sizeof(float) * (1u << bits));
    if (thresholds) std::memcpy(thresholds, t.thr[bits - 2], sizeof(float) * ((1u << bits) - 1));
    return PKV_OK;
}

}  // extern "C"
