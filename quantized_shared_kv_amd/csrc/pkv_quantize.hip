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
//                   (k_amax_channel per (layer, kv head, channel) on a per-channel pool's
//                   first append; none for per-token scales, found inside k_encode)
//   3. k_encode     a wavefront encodes one 8-token code group of one (layer,
//                   kv head) at a time: int8 K rows, then for the 8 tokens
//                   together an in-register FWHT across the wave (head_dim 64:
//                   one element per lane; 128: two), the norm by a fixed
//                   halving tree, and the code search; the group's code fields
//                   are staged in LDS and stored as dwords.
// Every floating-point step uses one IEEE rounding (no FMA contraction, correctly
// rounded division and square root), so codes are reproducible bit for bit.
#include <cmath>
#include <cstring>
#include <type_traits>

#include "pkv_internal.h"
#include "pkv_lanes.h"

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
    float cent[3][16];               // Lloyd-Max centroids (the corrected norm's ||c_hat||)
    uint32_t vsign[4];               // V rotation sign mask: bit i set = coordinate i negated
    int32_t kmode;                   // PKV_KSCALE_*
    int32_t vcorr;                   // corrected V norm
    float sd;                        // fl(sqrt(head_dim))
};

// k_encode reads its EncodeArgs in place at the start of the kernel-argument segment, where the
// first explicit argument of a kernel sits (HSA code-object ABI): a plain, standard-layout block.
static_assert(std::is_standard_layout<EncodeArgs>::value && std::is_trivially_copyable<EncodeArgs>::value,
              "EncodeArgs is read as raw kernel-argument memory");

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
    if (a.kmode == PKV_KSCALE_CHANNEL) {  // per (kv head, channel) maxima of the first append
        uint32_t* am = reinterpret_cast<uint32_t*>(a.base + a.off_amax) + (uint64_t)l * a.hkv * a.d;
        for (int i = threadIdx.x; i < a.hkv * a.d; i += blockDim.x) am[i] = 0u;
    } else if (threadIdx.x == 0) {
        reinterpret_cast<uint32_t*>(a.base + a.off_amax)[l] = 0u;
    }
    if (a.t0 == 0) {
        float* vmax = reinterpret_cast<float*>(a.base + a.off_vmax);
        for (int g = threadIdx.x; g < a.hkv; g += blockDim.x) vmax[(uint64_t)l * a.hkv + g] = 0.0f;
    }
}

// grid (kAmaxBlocks, nl), 256 threads.  Few blocks per layer keep the number of
// same-address atomics small (the per-layer maxima share one cache line).
constexpr int kAmaxBlocks = 16;

__global__ void __launch_bounds__(256) k_amax(EncodeArgs a) {
    const int j = blockIdx.y;
    const uint64_t per_layer = (uint64_t)a.hkv * a.n * a.d;
    const uint64_t base = (uint64_t)j * per_layer;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    float m0 = 0.0f, m1 = 0.0f;
    if (a.dtype == PKV_BF16) {
        // 8 bf16 per 16-byte load; per_layer and base are multiples of 64 elements
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + base);
        const uint64_t nv = per_layer / 8;
        uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
        for (; i + 3 * stride < nv; i += 4 * stride) {
            uint4 w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = p[i + r * stride];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t u[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    m0 = fmaxf(m0, fabsf(__uint_as_float(u[e] << 16)));
                    m1 = fmaxf(m1, fabsf(__uint_as_float(u[e] & 0xffff0000u)));
                }
            }
        }
        for (; i < nv; i += stride) {
            const uint4 w = p[i];
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                m0 = fmaxf(m0, fabsf(__uint_as_float(u[e] << 16)));
                m1 = fmaxf(m1, fabsf(__uint_as_float(u[e] & 0xffff0000u)));
            }
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.k) + base);
        const uint64_t nv = per_layer / 4;
        uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
        for (; i + 3 * stride < nv; i += 4 * stride) {
            float4 w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = p[i + r * stride];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                m0 = fmaxf(fmaxf(m0, fabsf(w[r].x)), fmaxf(fabsf(w[r].y), fmaxf(fabsf(w[r].z), fabsf(w[r].w))));
        }
        for (; i < nv; i += stride) {
            const float4 w = p[i];
            m1 = fmaxf(fmaxf(m1, fabsf(w.x)), fmaxf(fabsf(w.y), fmaxf(fabsf(w.z), fabsf(w.w))));
        }
    }
    float m = fmaxf(m0, m1);
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

// grid (kAmaxBlocks, hkv, nl), 256 threads: max |k| per (layer, kv head, channel) over the
// append's tokens (a per-channel pool's first append).  Thread t reads channel t % d of every
// (256 / d)-th token of its block's share, so a wavefront reads whole token rows.
__global__ void __launch_bounds__(256) k_amax_channel(EncodeArgs a) {
    const int j = blockIdx.z, g = blockIdx.y;
    const int c = threadIdx.x % a.d, tl = threadIdx.x / a.d, tper = 256 / a.d;
    const uint64_t row0 = ((uint64_t)j * a.hkv + g) * a.n;
    float m = 0.0f;
    for (int t = blockIdx.x * tper + tl; t < a.n; t += gridDim.x * tper)
        m = fmaxf(m, fabsf(load_elem(a.k, a.dtype, (row0 + t) * a.d + c)));
    // non-negative floats order like their bit patterns
    uint32_t* am = reinterpret_cast<uint32_t*>(a.base + a.off_amax) + ((uint64_t)(a.l0 + j) * a.hkv + g) * a.d;
    atomicMax(am + c, __float_as_uint(m));
}

constexpr int kEncWaves = 4;
constexpr int kGroupsPerWg = 64;  // 512 tokens per workgroup: one Vmax atomic per workgroup

// One level of the halving-tree sum of squares across lanes: s <- s + s[lane ^ M].
template <int M, int EPL>
__device__ __forceinline__ void tree_level(float (&sq)[kGroupTokens][EPL]) {
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i)
#pragma unroll
        for (int e = 0; e < EPL; ++e) sq[i][e] = sq[i][e] + lane_xor<M>(sq[i][e]);
}

// One FWHT stage across lanes: the lane with bit M clear keeps z + p, the one with
// it set gets p - z (p = partner's z); fma(+-1, z, p) is exactly that sum.
template <int M, int EPL>
__device__ __forceinline__ void butterfly(float (&z)[kGroupTokens][EPL], int lane) {
    const float sgn = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i)
#pragma unroll
        for (int e = 0; e < EPL; ++e) z[i][e] = __builtin_fmaf(sgn, z[i][e], lane_xor<M>(z[i][e]));
}

// Raw K and V of one 8-token group for this lane: its EPL elements of each token, as
// stored (bf16 bit patterns, or fp32 bits), 0 for tokens outside the append.
template <int EPL, bool BF16>
struct EncRaw {
    static constexpr int W = BF16 ? (EPL + 1) / 2 : EPL;  // 32-bit words per token per tensor
    uint32_t k[kGroupTokens][W], v[kGroupTokens][W];
};

template <int EPL, bool BF16>
__device__ __forceinline__ void enc_load(const EncodeArgs& a, int grp, int g, int j, EncRaw<EPL, BF16>& r) {
    constexpr int D = 64 * EPL;
    const int lane = threadIdx.x & 63;
    const int gt0 = grp * kGroupTokens;
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i) {
        const bool valid = gt0 + i >= a.t0 && gt0 + i < a.t0 + a.n;
        const uint64_t src = (((uint64_t)j * a.hkv + g) * a.n + (valid ? gt0 + i - a.t0 : 0)) * D + EPL * lane;
        if constexpr (BF16 && EPL == 2) {  // one dword: the lane's two bf16 values
            r.k[i][0] = valid ? static_cast<const uint32_t*>(a.k)[src / 2] : 0u;
            r.v[i][0] = valid ? static_cast<const uint32_t*>(a.v)[src / 2] : 0u;
        } else if constexpr (BF16) {
            r.k[i][0] = valid ? static_cast<const uint16_t*>(a.k)[src] : 0u;
            r.v[i][0] = valid ? static_cast<const uint16_t*>(a.v)[src] : 0u;
        } else if constexpr (EPL == 2) {
            const uint2 kk = valid ? static_cast<const uint2*>(a.k)[src / 2] : make_uint2(0u, 0u);
            const uint2 vv = valid ? static_cast<const uint2*>(a.v)[src / 2] : make_uint2(0u, 0u);
            r.k[i][0] = kk.x;
            r.k[i][EPL - 1] = kk.y;
            r.v[i][0] = vv.x;
            r.v[i][EPL - 1] = vv.y;
        } else {
            r.k[i][0] = valid ? static_cast<const uint32_t*>(a.k)[src] : 0u;
            r.v[i][0] = valid ? static_cast<const uint32_t*>(a.v)[src] : 0u;
        }
    }
}

template <int EPL, bool BF16>
__device__ __forceinline__ float enc_elem(const uint32_t (&w)[EncRaw<EPL, BF16>::W], int e) {
    if constexpr (BF16 && EPL == 2) return __uint_as_float(e == 0 ? w[0] << 16 : w[0] & 0xffff0000u);
    else if constexpr (BF16) return __uint_as_float(w[0] << 16);
    else return __uint_as_float(w[e]);
}

// c ? x : y on register values: the empty asm hands the select values rather than the
// table's elements, so the compiler does not turn it into an indexed load of the table
__device__ __forceinline__ float sel(bool c, float x, float y) {
    asm("" : "+v"(x), "+v"(y));
    return c ? x : y;
}

// Lloyd-Max code of y: the number of thresholds t[0] < ... < t[2^BITS - 2] strictly below
// y, found by a binary search over the sorted table (each level one comparison; the
// threshold of the next level picked by the bits found so far).
template <int BITS>
__device__ __forceinline__ uint32_t lm_code(float y, const float* t) {
    if constexpr (BITS == 2) {
        const bool b1 = y > t[1];
        const bool b0 = y > sel(b1, t[2], t[0]);
        return (b1 ? 2u : 0u) + (b0 ? 1u : 0u);
    } else if constexpr (BITS == 3) {
        const bool b2 = y > t[3];
        const bool b1 = y > sel(b2, t[5], t[1]);
        const float u0 = sel(b1, t[2], t[0]), u1 = sel(b1, t[6], t[4]);
        const bool b0 = y > sel(b2, u1, u0);
        return (b2 ? 4u : 0u) + (b1 ? 2u : 0u) + (b0 ? 1u : 0u);
    } else {
        const bool b3 = y > t[7];
        const bool b2 = y > sel(b3, t[11], t[3]);
        const bool b1 = y > sel(b3, sel(b2, t[13], t[9]), sel(b2, t[5], t[1]));
        const float u0 = sel(b1, t[2], t[0]), u1 = sel(b1, t[6], t[4]), u2 = sel(b1, t[10], t[8]),
                    u3 = sel(b1, t[14], t[12]);
        const bool b0 = y > sel(b3, sel(b2, u3, u2), sel(b2, u1, u0));
        return (b3 ? 8u : 0u) + (b2 ? 4u : 0u) + (b1 ? 2u : 0u) + (b0 ? 1u : 0u);
    }
}

// One wavefront encodes one 8-token code group of one (layer, kv head); the 8
// tokens are processed together so their cross-lane reductions and butterflies
// are independent and overlap.  Lane lam holds dimensions EPL*lam .. EPL*lam + EPL-1.
template <int EPL, int BITS, bool BF16>
__device__ __forceinline__ void encode_group(const EncodeArgs& a, int grp, int g, int j, const EncRaw<EPL, BF16>& raw,
                             uint8_t* stage, float& nmax, const float* cent, const float (&sch)[EPL],
                             const float (&rch)[EPL], uint64_t off_vc) {
#pragma clang fp contract(off)
    constexpr int D = 64 * EPL;
    const int lane = threadIdx.x & 63;
    const int l = a.l0 + j;
    float thr[(1 << BITS) - 1];
#pragma unroll
    for (int k = 0; k < (1 << BITS) - 1; ++k) thr[k] = a.thr[BITS - 2][k];


    const int gt0 = grp * kGroupTokens;
    bool valid[kGroupTokens];
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i) valid[i] = gt0 + i >= a.t0 && gt0 + i < a.t0 + a.n;

    float kx[kGroupTokens][EPL], vx[kGroupTokens][EPL];
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i)
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            kx[i][e] = enc_elem<EPL, BF16>(raw.k[i], e);
            vx[i][e] = enc_elem<EPL, BF16>(raw.v[i], e);
        }
    // ---- K scales: per tensor, one per layer and append (from k_amax); per token, each token's
    // max |k| over the wavefront; per channel, this lane's channels' (sch)
    float sk[kGroupTokens], rk[kGroupTokens];  // scale and its reciprocal per token
    if (a.kmode == PKV_KSCALE_TENSOR) {
        const float amax = __uint_as_float(reinterpret_cast<const uint32_t*>(a.base + a.off_amax)[l]);
        const float s = amax > 0.0f ? amax / 127.0f : 0.0f;
        const float rs = s > 0.0f ? 1.0f / s : 0.0f;
#pragma unroll
        for (int i = 0; i < kGroupTokens; ++i) {
            sk[i] = s;
            rk[i] = rs;
        }
    } else if (a.kmode == PKV_KSCALE_TOKEN) {
#pragma unroll
        for (int i = 0; i < kGroupTokens; ++i) {
            float m = fabsf(kx[i][0]);
            if (EPL == 2) m = fmaxf(m, fabsf(kx[i][EPL - 1]));
            m = fmaxf(m, lane_xor<32>(m));
            m = fmaxf(m, lane_xor<16>(m));
            m = fmaxf(m, lane_xor<8>(m));
            m = fmaxf(m, lane_xor<4>(m));
            m = fmaxf(m, lane_xor<2>(m));
            m = fmaxf(m, lane_xor<1>(m));
            sk[i] = m > 0.0f ? m / 127.0f : 0.0f;
            rk[i] = sk[i] > 0.0f ? 1.0f / sk[i] : 0.0f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kGroupTokens; ++i) sk[i] = rk[i] = 0.0f;
    }
    // ---- K rows: q = clamp(rint(k / s), -127, 127).  k * (1/s) is within 1.5e-5 of the
    // correctly rounded quotient (|k / s| <= 127), so it rounds the same way unless it lies
    // within 3e-5 of a half-integer; only then is the quotient itself computed (past 127.5 the
    // code clamps either way).
    int8_t* kq = reinterpret_cast<int8_t*>(a.base + a.off_kq) + ((uint64_t)l * a.hkv + g) * a.tc * D;
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i) {
        if (!valid[i]) continue;
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const bool ch = a.kmode == PKV_KSCALE_CHANNEL;
            const float s = ch ? sch[e] : sk[i];
            float q = 0.0f;
            if (s > 0.0f) {
                const float t = kx[i][e] * (ch ? rch[e] : rk[i]);
                const float fr = t - floorf(t);
                q = rintf(t);
                if (fabsf(fr - 0.5f) < 3.0e-5f) q = rintf(kx[i][e] / s);
                q = fminf(fmaxf(q, -127.0f), 127.0f);
            }
            packed |= static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(static_cast<int>(q)))) << (8 * e);
        }
        if (EPL == 2)
            reinterpret_cast<uint16_t*>(kq + (uint64_t)(gt0 + i) * D)[lane] = static_cast<uint16_t>(packed);
        else
            kq[(uint64_t)(gt0 + i) * D + lane] = static_cast<int8_t>(packed);
    }
    // ---- V: sum of squares by the halving tree (element i pairs with i + h, h = D/2 .. 1)
    float sq[kGroupTokens][EPL];
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i)
#pragma unroll
        for (int e = 0; e < EPL; ++e) sq[i][e] = vx[i][e] * vx[i][e];
    tree_level<32>(sq);
    tree_level<16>(sq);
    tree_level<8>(sq);
    tree_level<4>(sq);
    tree_level<2>(sq);
    tree_level<1>(sq);
    // every lane now holds the 8 sums; lane i < 8 takes the square root and reciprocal of
    // token i's, and the wave reads them back from those lanes
    float mine = 0.0f;
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i) {
        float ss = sq[i][0];
        if (EPL == 2) ss = sq[i][0] + sq[i][EPL - 1];
        mine = lane == i ? ss : mine;
    }
    const float n_l = sqrtf(mine);
    const float r_l = n_l > 0.0f ? 1.0f / n_l : 0.0f;
    float nrm[kGroupTokens], rcp[kGroupTokens];
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i) {
        nrm[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(n_l), i));
        rcp[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r_l), i));
    }
    // ---- the rotation's signs (coordinate EPL * lane + e negated where its mask bit is set;
    // the norm above does not see them), then the FWHT, ascending half-width (the in-lane
    // stage first when EPL == 2)
    {
        const int d0 = EPL * lane;
        const int wsel = d0 >> 5;  // a select over the four words, not an index into the argument block
        const uint32_t word = wsel == 0 ? a.vsign[0] : wsel == 1 ? a.vsign[1] : wsel == 2 ? a.vsign[2] : a.vsign[3];
        const uint32_t sb = (word >> (d0 & 31)) & ((1u << EPL) - 1u);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const uint32_t flip = ((sb >> e) & 1u) << 31;
#pragma unroll
            for (int i = 0; i < kGroupTokens; ++i) vx[i][e] = __uint_as_float(__float_as_uint(vx[i][e]) ^ flip);
        }
    }
    if (EPL == 2) {
#pragma unroll
        for (int i = 0; i < kGroupTokens; ++i) {
            const float u = vx[i][0], w = vx[i][EPL - 1];
            vx[i][0] = u + w;
            vx[i][EPL - 1] = u - w;
        }
    }
    butterfly<1>(vx, lane);
    butterfly<2>(vx, lane);
    butterfly<4>(vx, lane);
    butterfly<8>(vx, lane);
    butterfly<16>(vx, lane);
    butterfly<32>(vx, lane);
    // ---- codes of y = z * (1/n); 8 tokens per field
    uint32_t field[EPL];
    uint32_t code[kGroupTokens][EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) field[e] = 0u;
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i) {
        const bool coded = valid[i] && nrm[i] > 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            code[i][e] = coded ? lm_code<BITS>(vx[i][e] * rcp[i], thr) : 0u;
            field[e] |= code[i][e] << (BITS * i);
        }
    }
    // ---- the stored norm: ||v||, or the corrected n' = fl(fl(n * sqrt(d)) / ||c_hat||) with the
    // centroids' squares summed by the same halving tree (lane i < 8 holds token i's)
    float n_store = n_l;
    if (a.vcorr) {
        float cq[kGroupTokens][EPL];
#pragma unroll
        for (int i = 0; i < kGroupTokens; ++i)
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float c = cent[code[i][e]];
                cq[i][e] = c * c;
            }
        tree_level<32>(cq);
        tree_level<16>(cq);
        tree_level<8>(cq);
        tree_level<4>(cq);
        tree_level<2>(cq);
        tree_level<1>(cq);
        float cs = 0.0f;
#pragma unroll
        for (int i = 0; i < kGroupTokens; ++i) {
            float ss = cq[i][0];
            if (EPL == 2) ss = cq[i][0] + cq[i][EPL - 1];
            cs = lane == i ? ss : cs;
        }
        const float cn = sqrtf(cs);
        n_store = n_l > 0.0f ? (n_l * a.sd) / cn : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i) {
        const float ni = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(n_store), i));
        if (valid[i] && nrm[i] > 0.0f) nmax = fmaxf(nmax, ni);
    }
    uint8_t* vc = a.base + off_vc + ((uint64_t)g * (a.tc / kGroupTokens) + grp) * (uint64_t)(D * BITS);
    if (gt0 < a.t0) {  // the append starts inside this group: keep the earlier tokens' bits
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int dim = EPL * lane + e;
            uint32_t old = 0u;
#pragma unroll
            for (int k = 0; k < BITS; ++k) old |= static_cast<uint32_t>(vc[dim * BITS + k]) << (8 * k);
            field[e] |= old & ((1u << (BITS * (a.t0 - gt0))) - 1u);
        }
    }
    // ---- norms and per-tensor / per-token scales of the valid tokens: lane i < 8 stores token i
    float* vn = reinterpret_cast<float*>(a.base + a.off_vn) + ((uint64_t)l * a.hkv + g) * a.tc;
    bool mine_ok = false;
    float s_mine = 0.0f;
#pragma unroll
    for (int i = 0; i < kGroupTokens; ++i) {
        mine_ok = lane == i ? valid[i] : mine_ok;
        s_mine = lane == i ? sk[i] : s_mine;
    }
    if (lane < kGroupTokens && mine_ok) {
        vn[gt0 + lane] = n_store;
        if (a.kmode == PKV_KSCALE_TENSOR && g == 0)
            reinterpret_cast<float*>(a.base + a.off_ks)[(uint64_t)l * a.tc + gt0 + lane] = s_mine;
        else if (a.kmode == PKV_KSCALE_TOKEN)
            reinterpret_cast<float*>(a.base + a.off_ks)[((uint64_t)l * a.hkv + g) * a.tc + gt0 + lane] = s_mine;
    }
    // ---- code fields: dimension dim -> bytes [dim*BITS, dim*BITS + BITS), staged in LDS
#pragma unroll
    for (int e = 0; e < EPL; ++e)
#pragma unroll
        for (int k = 0; k < BITS; ++k) stage[(EPL * lane + e) * BITS + k] = static_cast<uint8_t>(field[e] >> (8 * k));
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    constexpr int NW = D * BITS / 4;  // dwords of the group
    for (int w = lane; w < NW; w += 64)
        reinterpret_cast<uint32_t*>(vc)[w] = reinterpret_cast<const uint32_t*>(stage)[w];
    __builtin_amdgcn_wave_barrier();
}

// grid (ceil(groups / kGroupsPerWg), hkv, nl), 256 threads; each wavefront loads its next
// group while it encodes the current one
template <int EPL, int BITS, bool BF16>
__device__ __forceinline__ void encode_wg(const EncodeArgs& a, int grp_first, int n_grp, uint64_t off_vc) {
    __shared__ __align__(16) uint8_t stage[kEncWaves][128 * 4];
    __shared__ float wmax[kEncWaves];
    __shared__ float cent[16];
    const int wave = threadIdx.x >> 6;
    const int g = blockIdx.y, j = blockIdx.z;
    const int lane = threadIdx.x & 63;
    if (threadIdx.x == 0) {  // compile-time indices: a thread-dependent index into the kernel
                             // argument would copy the whole argument block to scratch
#pragma unroll
        for (int k = 0; k < 16; ++k) cent[k] = a.cent[BITS - 2][k];
    }
    // per-channel scales of this lane's channels: from the first append's maxima (and stored
    // by the first workgroup of each (layer, kv head)), or as stored by it for later appends
    float sch[EPL], rch[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) sch[e] = rch[e] = 0.0f;
    if (a.kmode == PKV_KSCALE_CHANNEL) {
        const uint64_t cb = ((uint64_t)(a.l0 + j) * a.hkv + g) * a.d + EPL * lane;
        float* ks = reinterpret_cast<float*>(a.base + a.off_ks);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            if (a.t0 == 0) {
                const float amax = __uint_as_float(reinterpret_cast<const uint32_t*>(a.base + a.off_amax)[cb + e]);
                sch[e] = amax > 0.0f ? amax / 127.0f : 0.0f;
                if (blockIdx.x == 0 && wave == 0) ks[cb + e] = sch[e];
            } else {
                sch[e] = ks[cb + e];
            }
            rch[e] = sch[e] > 0.0f ? 1.0f / sch[e] : 0.0f;
        }
    }
    __syncthreads();
    float nmax = 0.0f;
    const int gb = blockIdx.x * kGroupsPerWg;
    const int ge = min(n_grp, gb + kGroupsPerWg);
    if (gb + wave < ge) {
        EncRaw<EPL, BF16> cur;
        enc_load<EPL, BF16>(a, grp_first + gb + wave, g, j, cur);
        for (int gi = gb + wave; gi < ge; gi += kEncWaves) {
            // the last group loads itself again rather than branching around the load
            EncRaw<EPL, BF16> nxt;
            enc_load<EPL, BF16>(a, grp_first + min(gi + kEncWaves, ge - 1), g, j, nxt);
            encode_group<EPL, BITS, BF16>(a, grp_first + gi, g, j, cur, stage[wave], nmax, cent, sch, rch, off_vc);
            cur = nxt;
        }
    }
    if ((threadIdx.x & 63) == 0) wmax[wave] = nmax;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float r = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        float* vmax = reinterpret_cast<float*>(a.base + a.off_vmax);
        atomicMax(reinterpret_cast<uint32_t*>(vmax + (uint64_t)(a.l0 + j) * a.hkv + g), __float_as_uint(r));
    }
}

template <bool BF16>
__device__ __forceinline__ void encode_dispatch(const EncodeArgs& a, int grp_first, int n_grp, int b, uint64_t off_vc) {
    if (a.d == 128) {
        if (b == 2) encode_wg<2, 2, BF16>(a, grp_first, n_grp, off_vc);
        else if (b == 3) encode_wg<2, 3, BF16>(a, grp_first, n_grp, off_vc);
        else encode_wg<2, 4, BF16>(a, grp_first, n_grp, off_vc);
    } else {
        if (b == 2) encode_wg<1, 2, BF16>(a, grp_first, n_grp, off_vc);
        else if (b == 3) encode_wg<1, 3, BF16>(a, grp_first, n_grp, off_vc);
        else encode_wg<1, 4, BF16>(a, grp_first, n_grp, off_vc);
    }
}

// The argument block is read in place, through the kernel-argument segment (it is the first
// argument, at offset 0): handing the by-value parameter to the large inlined body made the
// compiler copy all of it to per-lane scratch first.
__global__ void __launch_bounds__(256) k_encode(EncodeArgs args, int grp_first, int n_grp) {
    (void)args;
    const EncodeArgs& a = *static_cast<const EncodeArgs*>((const void*)__builtin_amdgcn_kernarg_segment_ptr());
    const int b = a.bits[blockIdx.z];
    const uint64_t off_vc = a.off_vc[blockIdx.z];
    if (a.dtype == PKV_BF16) encode_dispatch<true>(a, grp_first, n_grp, b, off_vc);
    else encode_dispatch<false>(a, grp_first, n_grp, b, off_vc);
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
    std::memcpy(a.cent, codebook_tables().cent, sizeof(a.cent));
    std::memcpy(a.vsign, c.v_signs, sizeof(a.vsign));
    a.kmode = c.k_scale;
    a.vcorr = c.v_norm == PKV_VNORM_CORRECTED;
    a.sd = (float)std::sqrt((double)c.head_dim);

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(k_reset, dim3(layer_count), dim3(64), 0, s, a);
    if (c.k_scale == PKV_KSCALE_TENSOR)
        hipLaunchKernelGGL(k_amax, dim3(kAmaxBlocks, layer_count), dim3(256), 0, s, a);
    else if (c.k_scale == PKV_KSCALE_CHANNEL && t0 == 0)
        hipLaunchKernelGGL(k_amax_channel, dim3(kAmaxBlocks, c.n_kv_heads, layer_count), dim3(256), 0, s, a);
    const int grp_first = t0 / kGroupTokens;
    const int grp_last = (t0 + n_tokens - 1) / kGroupTokens;
    const int n_grp = grp_last - grp_first + 1;
    hipLaunchKernelGGL(k_encode, dim3((n_grp + kGroupsPerWg - 1) / kGroupsPerWg, c.n_kv_heads, layer_count),
                       dim3(256), 0, s, a, grp_first, n_grp);
    const int st = launch_status();
    if (st != PKV_OK) return st;
    for (int l = layer_begin; l < layer_begin + layer_count; ++l) pool->n_tokens[l] = t0 + n_tokens;
    return PKV_OK;
}
