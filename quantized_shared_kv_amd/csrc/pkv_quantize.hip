// Pool write path: per-tensor int8 K and FWHT/Lloyd-Max V codes for gfx950.
//
// PolyKV explainer, section 2.B (asymmetric compression scheme):
//  - K: one linear int8 scale per tensor (here: per layer and per append).
//  - V: FWHT rotation, normalisation to N(0, 1)-like coordinates, Lloyd-Max
//    code per coordinate, and a per-vector norm.
// CoMixKV news article ("incremental quantization strategy"): appended tokens
// are encoded once and earlier tokens are never rewritten; V bits per layer.
//
// Three launches per append, all on the caller's stream:
//   1. k_reset      clear the per-layer amax scratch (and Vmax on a fresh layer)
//   2. k_amax       max |k| per layer, reduced with an atomic max on fp32 bits
//   3. k_encode     one wavefront per 8-token code group of one (layer, kv head):
//                   int8 K rows, then per token an in-register FWHT across the
//                   wave (head_dim 64: one element per lane; 128: two), the
//                   norm by a fixed halving tree, and the code search; the
//                   wave collects the group's code fields and stores them.
// Every floating-point step uses one IEEE rounding (no FMA contraction, correctly
// rounded division and square root), so codes are reproducible bit for bit.
#include <cstring>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kMaxLayersArg = PKV_MAX_LAYERS;

struct EncodeArgs {
    const void* k;
    const void* v;
    uint8_t* base;
    uint64_t off_kq, off_vn, off_ks, off_vmax, off_amax;
    uint64_t off_vc[kMaxLayersArg];  // absolute code-region offset of each call layer
    int32_t dtype;                   // pkv_dtype
    int32_t n;                       // tokens appended
    int32_t t0;                      // first token index of the append
    int32_t hkv, d, tc;
    int32_t l0, nl;
    uint8_t bits[kMaxLayersArg];     // bits of each call layer
    float thr[3][15];
};

__device__ __forceinline__ float load_elem(const void* p, int dtype, uint64_t i) {
    if (dtype == PKV_BF16) {
        const uint16_t b = static_cast<const uint16_t*>(p)[i];
        return __uint_as_float(static_cast<uint32_t>(b) << 16);
    }
    return static_cast<const float*>(p)[i];
}

__global__ void k_reset(EncodeArgs a) {
    const int j = blockIdx.x;
    if (j >= a.nl) return;
    const int l = a.l0 + j;
    if (threadIdx.x == 0) reinterpret_cast<uint32_t*>(a.base + a.off_amax)[l] = 0u;
    if (a.t0 == 0) {
        float* vmax = reinterpret_cast<float*>(a.base + a.off_vmax);
        for (int g = threadIdx.x; g < a.hkv; g += blockDim.x) vmax[(uint64_t)l * a.hkv + g] = 0.0f;
    }
}

// grid (blocks per layer, nl), 256 threads
__global__ void __launch_bounds__(256) k_amax(EncodeArgs a) {
    const int j = blockIdx.y;
    const uint64_t per_layer = (uint64_t)a.hkv * a.n * a.d;
    const uint64_t base = (uint64_t)j * per_layer;
    float m = 0.0f;
    if (a.dtype == PKV_BF16) {
        // 8 bf16 per 16-byte load; per_layer and base are multiples of 64 elements
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + base);
        const uint64_t nv = per_layer / 8;
        for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nv;
             i += (uint64_t)gridDim.x * blockDim.x) {
            const uint4 w = p[i];
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                m = fmaxf(m, fabsf(__uint_as_float(u[e] << 16)));
                m = fmaxf(m, fabsf(__uint_as_float(u[e] & 0xffff0000u)));
            }
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.k) + base);
        const uint64_t nv = per_layer / 4;
        for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nv;
             i += (uint64_t)gridDim.x * blockDim.x) {
            const float4 w = p[i];
            m = fmaxf(fmaxf(m, fabsf(w.x)), fmaxf(fabsf(w.y), fmaxf(fabsf(w.z), fabsf(w.w))));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float wmax[4];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) wmax[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        // non-negative floats order like their bit patterns
        atomicMax(reinterpret_cast<uint32_t*>(a.base + a.off_amax) + (a.l0 + j), __float_as_uint(r));
    }
}

// One wavefront per (group, kv head, layer); EPL = head_dim / 64 elements per lane.
// Lane lam holds dimensions EPL*lam .. EPL*lam + EPL-1.
template <int EPL>
__device__ void encode_group(const EncodeArgs& a, int grp, int g, int j) {
#pragma clang fp contract(off)
    constexpr int D = 64 * EPL;
    const int lane = threadIdx.x & 63;
    const int l = a.l0 + j;
    const int b = a.bits[j];
    const int nthr = (1 << b) - 1;
    const float* thr = a.thr[b - 2];

    const float amax = __uint_as_float(reinterpret_cast<const uint32_t*>(a.base + a.off_amax)[l]);
    const float s = amax > 0.0f ? amax / 127.0f : 0.0f;

    const int gt0 = grp * kGroupTokens;
    const int tb = max(a.t0, gt0);
    const int te = min(a.t0 + a.n, gt0 + kGroupTokens);

    uint8_t* vc = a.base + a.off_vc[j] + ((uint64_t)g * (a.tc / kGroupTokens) + grp) * (uint64_t)(D * b);
    uint32_t field[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        field[e] = 0u;
        if (gt0 < a.t0) {  // first group of an append that starts mid-group: keep earlier tokens
            const int dim = EPL * lane + e;
            uint32_t old = 0u;
            for (int k = 0; k < b; ++k) old |= static_cast<uint32_t>(vc[dim * b + k]) << (8 * k);
            field[e] = old & ((1u << (b * (a.t0 - gt0))) - 1u);
        }
    }

    int8_t* kq = reinterpret_cast<int8_t*>(a.base + a.off_kq) + ((uint64_t)l * a.hkv + g) * a.tc * D;
    float* vn = reinterpret_cast<float*>(a.base + a.off_vn) + ((uint64_t)l * a.hkv + g) * a.tc;
    float* ks = reinterpret_cast<float*>(a.base + a.off_ks) + (uint64_t)l * a.tc;
    float nmax = 0.0f;

    for (int t = tb; t < te; ++t) {
        const uint64_t src = (((uint64_t)j * a.hkv + g) * a.n + (t - a.t0)) * D + EPL * lane;
        // ---- K row: q = clamp(rint(k / s), -127, 127)
        int8_t qv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float x = load_elem(a.k, a.dtype, src + e);
            float q = 0.0f;
            if (s > 0.0f) q = fminf(fmaxf(rintf(x / s), -127.0f), 127.0f);
            qv[e] = static_cast<int8_t>(static_cast<int>(q));
        }
        if (EPL == 2) {
            const uint16_t pair = static_cast<uint16_t>(static_cast<uint8_t>(qv[0])) |
                                  static_cast<uint16_t>(static_cast<uint16_t>(static_cast<uint8_t>(qv[EPL - 1])) << 8);
            reinterpret_cast<uint16_t*>(kq + (uint64_t)t * D)[lane] = pair;
        } else {
            kq[(uint64_t)t * D + lane] = qv[0];
        }
        // ---- V vector
        float x[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = load_elem(a.v, a.dtype, src + e);
        // sum of squares: halving tree, element i pairs with i + h for h = D/2 .. 1
        float sq[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) sq[e] = x[e] * x[e];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sq[e] = sq[e] + __shfl_xor(sq[e], off, 64);
        }
        float ss = sq[0];
        if (EPL == 2) ss = sq[0] + sq[EPL - 1];
        const float nrm = sqrtf(ss);
        // FWHT, ascending half-width h: in-lane stage first when EPL == 2
        float z[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) z[e] = x[e];
        if (EPL == 2) {
            const float u = z[0], w = z[EPL - 1];
            z[0] = u + w;
            z[EPL - 1] = u - w;
        }
#pragma unroll
        for (int off = 1; off <= 32; off <<= 1) {
            const bool upper = (lane & off) != 0;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float p = __shfl_xor(z[e], off, 64);
                z[e] = upper ? (p - z[e]) : (z[e] + p);
            }
        }
        // codes: number of thresholds strictly below y = z * (1/n)
        if (nrm > 0.0f) {
            const float r = 1.0f / nrm;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float y = z[e] * r;
                uint32_t c = 0;
                for (int k = 0; k < nthr; ++k) c += (y > thr[k]) ? 1u : 0u;
                field[e] |= c << (b * (t - gt0));
            }
        }
        if (lane == 0) {
            vn[t] = nrm;
            if (g == 0) ks[t] = s;
        }
        nmax = fmaxf(nmax, nrm);
    }
    // store this lane's code fields: dimension dim -> bytes [dim*b, dim*b + b)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int dim = EPL * lane + e;
        for (int k = 0; k < b; ++k) vc[dim * b + k] = static_cast<uint8_t>(field[e] >> (8 * k));
    }
    if (lane == 0 && te > tb) {
        float* vmax = reinterpret_cast<float*>(a.base + a.off_vmax);
        atomicMax(reinterpret_cast<uint32_t*>(vmax + (uint64_t)l * a.hkv + g), __float_as_uint(nmax));
    }
}

// grid (ceil(groups / 4), hkv, nl), 256 threads = 4 wavefronts, one group each
__global__ void __launch_bounds__(256) k_encode(EncodeArgs a, int grp_first, int n_grp) {
    const int wave = threadIdx.x >> 6;
    const int gi = blockIdx.x * 4 + wave;
    if (gi >= n_grp) return;
    if (a.d == 128)
        encode_group<2>(a, grp_first + gi, blockIdx.y, blockIdx.z);
    else
        encode_group<1>(a, grp_first + gi, blockIdx.y, blockIdx.z);
}

}  // namespace
}  // namespace pkv

extern "C" int pool_quantize_append(pkv_pool* pool, int32_t layer_begin, int32_t layer_count,
                                    const void* k, const void* v, pkv_dtype dtype, int32_t n_tokens,
                                    void* stream) {
    using namespace pkv;
    if (!pool || !pool->base) return PKV_EINVAL;
    int err;
    if (!config_valid(&pool->cfg, &err)) return err;
    if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_EUNSUPPORTED;
    const pkv_pool_config& c = pool->cfg;
    if (layer_count < 0 || n_tokens < 0 || layer_begin < 0 || layer_begin + layer_count > c.n_layers)
        return PKV_EINVAL;
    if (layer_count == 0 || n_tokens == 0) return PKV_OK;
    if (!k || !v) return PKV_EINVAL;
    if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) % 16) return PKV_EINVAL;
    const int t0 = pool->n_tokens[layer_begin];
    for (int l = layer_begin; l < layer_begin + layer_count; ++l)
        if (pool->n_tokens[l] != t0) return PKV_EINVAL;
    if ((int64_t)t0 + n_tokens > c.capacity_tokens) return PKV_ECAPACITY;

    EncodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.k = k;
    a.v = v;
    a.base = static_cast<uint8_t*>(pool->base);
    a.off_kq = pool->off_kq;
    a.off_vn = pool->off_vn;
    a.off_ks = pool->off_ks;
    a.off_vmax = pool->off_vmax;
    a.off_amax = pool->off_amax;
    for (int j = 0; j < layer_count; ++j) {
        a.off_vc[j] = pool->off_vc[layer_begin + j];
        a.bits[j] = c.v_bits[layer_begin + j];
    }
    a.dtype = dtype;
    a.n = n_tokens;
    a.t0 = t0;
    a.hkv = c.n_kv_heads;
    a.d = c.head_dim;
    a.tc = pool->tc;
    a.l0 = layer_begin;
    a.nl = layer_count;
    std::memcpy(a.thr, codebook_tables().thr, sizeof(a.thr));

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(k_reset, dim3(layer_count), dim3(64), 0, s, a);
    const uint64_t per_layer = (uint64_t)c.n_kv_heads * n_tokens * c.head_dim;
    const uint64_t vecs = per_layer / 8;
    unsigned blocks = (unsigned)std::min<uint64_t>(1024, (vecs + 255) / 256);
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(k_amax, dim3(blocks, layer_count), dim3(256), 0, s, a);
    const int grp_first = t0 / kGroupTokens;
    const int grp_last = (t0 + n_tokens - 1) / kGroupTokens;
    const int n_grp = grp_last - grp_first + 1;
    hipLaunchKernelGGL(k_encode, dim3((n_grp + 3) / 4, c.n_kv_heads, layer_count), dim3(256), 0, s, a,
                       grp_first, n_grp);
    const int st = launch_status();
    if (st != PKV_OK) return st;
    for (int l = layer_begin; l < layer_begin + layer_count; ++l) pool->n_tokens[l] = t0 + n_tokens;
    return PKV_OK;
}
