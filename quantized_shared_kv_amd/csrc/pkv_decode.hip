// Decode attention of many agents over shared compressed pools (gfx950).
//
// PolyKV explainer, section 2.A: agents hold a reference to one shared pool
// and attend over it; section 2.B: V is dequantised by centroid lookup and an
// inverse FWHT.  CoMixKV news article: the most recent tokens of each agent
// stay at native precision.  Here the pool is never dequantised into memory:
// the kernels read the compressed bytes, form scores from int8 K times the
// per-token scale, and accumulate p * norm * centroid in the rotated domain;
// the merge kernel applies one inverse FWHT per output row.
//
// Launch sequence of one call (all on the caller's stream):
//   1. native window per (agent, layer, kv head): partial softmax state over the
//      agent's bf16 suffix tokens (k_sfx_fast; k_sfx for fp32 operands); in a
//      split-record matrix-core launch that leaves compute units free, extra
//      workgroups of the pool kernel do this work beside the pool workgroups
//   2. k_seg per (agent, layer, kv head) of a small private pool, if any
//   3. pool kernel per (pool, layer, kv head, token split): partial state of
//      all rows that read the pool (every agent of the pool times every q head
//      of the kv head's group), rotated domain; the matrix-core kernel of
//      pkv_decode_mfma.hip (k_pool_valu when asked for).  With one split per
//      (layer, kv head) it finishes the rows itself (inverse FWHT, suffix
//      record, normalise); otherwise
//   4. k_merge per output row: combine splits, inverse FWHT, add the suffix
// Softmax state is kept in log2 units: scores are scaled by sigma * log2(e).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "pkv_decode.h"
#include "pkv_lanes.h"
#include "pkv_sfx.h"

namespace pkv {
namespace {

constexpr int kValuRows = 32;  // rows per VALU workgroup
constexpr int kTile = 32;      // tokens per tile
constexpr int kThreads = 256;

struct Centroids {
    float c[3][16];
};

__device__ __forceinline__ float ld_elem(const void* p, int dtype, uint64_t i) {
    if (dtype == PKV_BF16) {
        const uint16_t b = static_cast<const uint16_t*>(p)[i];
        return __uint_as_float(static_cast<uint32_t>(b) << 16);
    }
    return static_cast<const float*>(p)[i];
}

template <int D>
struct ValuSmem {
    float q[kValuRows][D];
    float k[kTile][D + 1];
    float v[kTile][D + 1];
    float sc[kValuRows][kTile + 1];
    float f[kTile];
    float nn[kTile];
    float m[kValuRows], l[kValuRows], al[kValuRows];
    int valid[kTile];
};

// Online softmax over tokens [t_begin, t_end) for nr rows whose queries are in sm.q.
// acc[k] holds element idx = tid + 256 k of the row-major [nr][D] accumulator.
template <int D, class Src>
__device__ void valu_attend(ValuSmem<D>& sm, int nr, int t_begin, int t_end, const Src& src,
                            float* acc) {
    constexpr int ACC = kValuRows * D / kThreads;
    const int tid = threadIdx.x;
    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
        src.load_tile(sm, t0, t_end);
        __syncthreads();
        for (int pair = tid; pair < nr * kTile; pair += kThreads) {
            const int r = pair / kTile, t = pair % kTile;
            float dot = 0.0f;
#pragma unroll 8
            for (int i = 0; i < D; ++i) dot += sm.q[r][i] * sm.k[t][i];
            sm.sc[r][t] = sm.valid[t] ? dot * sm.f[t] : -INFINITY;
        }
        __syncthreads();
        if (tid < nr) {
            const float mold = sm.m[tid];
            float mx = mold;
            for (int t = 0; t < kTile; ++t) mx = fmaxf(mx, sm.sc[tid][t]);
            const float alpha = (mold == -INFINITY) ? 0.0f : exp2f(mold - mx);
            float sum = 0.0f;
            for (int t = 0; t < kTile; ++t) {
                const float s = sm.sc[tid][t];
                const float p = (s == -INFINITY) ? 0.0f : exp2f(s - mx);
                sum += p;
                sm.sc[tid][t] = p * sm.nn[t];
            }
            sm.l[tid] = sm.l[tid] * alpha + sum;
            sm.m[tid] = mx;
            sm.al[tid] = alpha;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < ACC; ++k) {
            const int idx = tid + kThreads * k;
            const int r = idx / D, i = idx % D;
            if (r < nr) {
                float v = acc[k] * sm.al[r];
                for (int t = 0; t < kTile; ++t) v += sm.sc[r][t] * sm.v[t][i];
                acc[k] = v;
            }
        }
        __syncthreads();
    }
}

// Token source reading a compressed pool: int8 K * scale, V centroids * norm.
template <int D>
struct PoolSrc {
    const int8_t* kq;
    const float* vn;
    const float* ks;
    const uint8_t* vc;
    const float* cent;
    const float* kch;  // per-channel K scales, or nullptr (per tensor / per token: ks)
    int bits;
    float sm_log2;
    __device__ void load_tile(ValuSmem<D>& sm, int t0, int t_end) const {
        const int tid = threadIdx.x;
        for (int idx = tid; idx < kTile * D; idx += kThreads) {
            const int t = idx / D, i = idx % D;
            const int tok = t0 + t;
            const float k = tok < t_end ? static_cast<float>(kq[(uint64_t)tok * D + i]) : 0.0f;
            sm.k[t][i] = kch ? k * kch[i] : k;
        }
        const uint32_t mask = (1u << bits) - 1u;
        for (int idx = tid; idx < 4 * D; idx += kThreads) {
            const int gi = idx / D, dim = idx % D;
            const uint8_t* fp = vc + ((uint64_t)(t0 / kGroupTokens + gi) * D + dim) * bits;
            uint32_t field = 0;
            for (int b = 0; b < bits; ++b) field |= static_cast<uint32_t>(fp[b]) << (8 * b);
            for (int i = 0; i < kGroupTokens; ++i) sm.v[gi * kGroupTokens + i][dim] = cent[(field >> (bits * i)) & mask];
        }
        if (tid < kTile) {
            const int tok = t0 + tid;
            const bool ok = tok < t_end;
            sm.valid[tid] = ok;
            sm.f[tid] = ok ? (kch ? sm_log2 : ks[tok] * sm_log2) : 0.0f;
            sm.nn[tid] = ok ? vn[tok] : 0.0f;
        }
    }
};

// Token source reading an agent's native suffix K/V rows.
template <int D>
struct SfxSrc {
    const void* k;
    const void* v;
    int dtype;
    uint64_t base;  // element offset of token 0
    float sm_log2;
    __device__ void load_tile(ValuSmem<D>& sm, int t0, int t_end) const {
        const int tid = threadIdx.x;
        for (int idx = tid; idx < kTile * D; idx += kThreads) {
            const int t = idx / D, i = idx % D;
            const int tok = t0 + t;
            const bool ok = tok < t_end;
            sm.k[t][i] = ok ? ld_elem(k, dtype, base + (uint64_t)tok * D + i) : 0.0f;
            sm.v[t][i] = ok ? ld_elem(v, dtype, base + (uint64_t)tok * D + i) : 0.0f;
        }
        if (tid < kTile) {
            const bool ok = t0 + tid < t_end;
            sm.valid[tid] = ok;
            sm.f[tid] = sm_log2;
            sm.nn[tid] = ok ? 1.0f : 0.0f;
        }
    }
};

template <int D>
__device__ void load_rows_and_init(ValuSmem<D>& sm, const DecodeLaunch& a, int nr, int lj,
                                   const int* agents, const int* heads, float* acc) {
    const int tid = threadIdx.x;
    for (int idx = tid; idx < kValuRows * D; idx += kThreads) {
        const int r = idx / D, i = idx % D;
        float x = 0.0f;
        if (r < nr) x = ld_elem(a.q, a.q_dtype, (((uint64_t)agents[r] * a.lc + lj) * a.hq + heads[r]) * D + i);
        sm.q[r][i] = x;
    }
    if (tid < kValuRows) {
        sm.m[tid] = -INFINITY;
        sm.l[tid] = 0.0f;
    }
    constexpr int ACC = kValuRows * D / kThreads;
#pragma unroll
    for (int k = 0; k < ACC; ++k) acc[k] = 0.0f;
    __syncthreads();
}

template <int D>
__device__ void store_records(const ValuSmem<D>& sm, int nr, float* const* recs, const float* acc) {
    constexpr int ACC = kValuRows * D / kThreads;
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < ACC; ++k) {
        const int idx = tid + kThreads * k;
        const int r = idx / D, i = idx % D;
        if (r < nr) recs[r][2 + i] = acc[k];
    }
    if (tid < nr) {
        recs[tid][0] = sm.m[tid];
        recs[tid][1] = sm.l[tid];
    }
}

__device__ __forceinline__ int find_pool(const DecodeLaunch& a, int wg) {
    int p = 0;
    while (p + 1 < a.n_pools && wg >= a.pools[p + 1].wg_begin) ++p;
    return p;
}

// grid: one workgroup per (pool, layer, kv head, split, row block of 32 rows)
template <int D>
__global__ void __launch_bounds__(kThreads) k_pool_valu(DecodeLaunch a, Centroids cents) {
    __shared__ ValuSmem<D> sm;
    __shared__ int agents[kValuRows], heads[kValuRows];
    __shared__ float* recs[kValuRows];
    const int p = find_pool(a, blockIdx.x);
    const PoolEntry& P = a.pools[p];
    int local = blockIdx.x - P.wg_begin;
    const int rb = local % P.rblocks;
    local /= P.rblocks;
    const int s = local % P.splits;
    local /= P.splits;
    const int g = local % a.hkv;
    const int lj = local / a.hkv;
    const int l = a.l0 + lj;
    const int r0 = rb * kValuRows;
    const int nr = min(kValuRows, P.rows - r0);
    if (threadIdx.x < kValuRows) {
        const int rho = min(r0 + (int)threadIdx.x, P.rows - 1);
        agents[threadIdx.x] = a.agent_id[P.agent0 + rho / a.G];
        heads[threadIdx.x] = g * a.G + rho % a.G;
        recs[threadIdx.x] = a.part + P.part_off +
                            ((((uint64_t)lj * a.hkv + g) * P.splits + s) * P.rows + rho) * (2 + D);
    }
    __syncthreads();
    float acc[kValuRows * D / kThreads];
    load_rows_and_init(sm, a, nr, lj, agents, heads, acc);

    const int bits = layer_bits(P, l);
    PoolSrc<D> src;
    src.kq = reinterpret_cast<const int8_t*>(P.base + P.off_kq) + ((uint64_t)l * a.hkv + g) * P.tc * D;
    src.vn = reinterpret_cast<const float*>(P.base + P.off_vn) + ((uint64_t)l * a.hkv + g) * P.tc;
    src.ks = reinterpret_cast<const float*>(P.base + P.off_ks) + ks_offset(P, l, g, a.hkv, D);
    src.kch = P.kmode == PKV_KSCALE_CHANNEL ? src.ks : nullptr;
    src.vc = P.base + P.off_vc0 + (uint64_t)a.hkv * P.tc * (D / 8) * layer_bits_prefix(P, l) +
             (uint64_t)g * (P.tc / kGroupTokens) * D * bits;
    src.cent = cents.c[bits - 2];
    src.bits = bits;
    src.sm_log2 = a.sm_log2;
    const int tb = s * P.chunk;
    const int te = min(P.T, tb + P.chunk);
    valu_attend<D>(sm, nr, tb, te, src, acc);
    store_records<D>(sm, nr, recs, acc);
}

// grid (lc * hkv, n_agents): one workgroup per (agent, layer, kv head); rows = the G heads
template <int D>
__global__ void __launch_bounds__(kThreads) k_sfx_valu(DecodeLaunch a) {
    __shared__ ValuSmem<D> sm;
    __shared__ int agents[kValuRows], heads[kValuRows];
    __shared__ float* recs[kValuRows];
    const int k = blockIdx.y;
    const int lj = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
    const int agent = a.agent_id[k];
    const int S = a.sfx_len[k];
    for (int r0 = 0; r0 < a.G; r0 += kValuRows) {
        const int nr = min(kValuRows, a.G - r0);
        if (threadIdx.x < kValuRows) {
            const int h = g * a.G + min(r0 + (int)threadIdx.x, a.G - 1);
            agents[threadIdx.x] = agent;
            heads[threadIdx.x] = h;
            recs[threadIdx.x] = a.part + a.sfx_part_off + (((uint64_t)k * a.lc + lj) * a.hq + h) * (2 + D);
        }
        __syncthreads();
        float acc[kValuRows * D / kThreads];
        load_rows_and_init(sm, a, nr, lj, agents, heads, acc);
        SfxSrc<D> src;
        src.k = a.sfx_k;
        src.v = a.sfx_v;
        src.dtype = a.sfx_dtype;
        src.base = (((uint64_t)agent * a.lc + lj) * a.hkv + g) * (uint64_t)a.sfx_cap * D;
        src.sm_log2 = a.sm_log2;
        valu_attend<D>(sm, nr, 0, S, src, acc);
        store_records<D>(sm, nr, recs, acc);
        __syncthreads();
    }
}

// Native suffix attention, one wavefront per (launch agent, layer, kv head):
// lanes own tokens for the scores (bf16 K rows times bf16 queries with
// v_dot2c_f32_bf16, exact products, fp32 accumulation; any fp32 operand takes a
// plain fp32 FMA path), the softmax state is kept per row across the wave, and for the value
// sum each lane owns D/64 dimensions while the probabilities of a 64-token
// chunk are broadcast from LDS.  Rows are the kv head's q heads (G <= 8 per
// pass; larger groups take several passes).
constexpr int kSfxRows = 8;

template <int D, bool BF16>  // BF16: bf16 queries and bf16 suffix (dot2 path)
__device__ void sfx_wave(const DecodeLaunch& a, int unit, float* pbuf, uint32_t* qbuf) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int g = unit % a.hkv;
    const int lj = (unit / a.hkv) % a.lc;
    const int k = unit / (a.hkv * a.lc);
    const int agent = a.agent_id[k];
    const int S = a.sfx_len[k];
    const uint64_t tok0 = (((uint64_t)agent * a.lc + lj) * a.hkv + g) * (uint64_t)a.sfx_cap;
    for (int r0 = 0; r0 < a.G; r0 += kSfxRows) {
        const int nr = min(kSfxRows, a.G - r0);
        // queries of this pass: bf16 pairs (BF16) or fp32 values, in LDS
        for (int idx = lane; idx < kSfxRows * D; idx += 64) {
            const int r = idx / D, i = idx % D;
            float x = 0.0f;
            if (r < nr) x = ld_elem(a.q, a.q_dtype, (((uint64_t)agent * a.lc + lj) * a.hq + g * a.G + r0 + r) * D + i);
            if (BF16) {
                // the bf16 query's bits (x is its exact fp32 widening)
                reinterpret_cast<uint16_t*>(qbuf)[r * D + i] = static_cast<uint16_t>(__float_as_uint(x) >> 16);
            } else {
                reinterpret_cast<float*>(qbuf)[r * D + i] = x;
            }
        }
        __builtin_amdgcn_wave_barrier();
        float m[kSfxRows], l[kSfxRows], acc[kSfxRows][EPL];
#pragma unroll
        for (int r = 0; r < kSfxRows; ++r) {
            m[r] = -INFINITY;
            l[r] = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[r][e] = 0.0f;
        }
        for (int c0 = 0; c0 < S; c0 += 64) {
            const int t = c0 + lane;
            const bool ok = t < S;
            float sc[kSfxRows];
#pragma unroll
            for (int r = 0; r < kSfxRows; ++r) sc[r] = 0.0f;
            if (ok) {
                if (BF16) {
                    const uint4* krow = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.sfx_k) + (tok0 + t) * D);
#pragma unroll 4
                    for (int c = 0; c < D / 8; ++c) {
                        const uint4 kv = krow[c];
#pragma unroll
                        for (int r = 0; r < kSfxRows; ++r) {
                            if (r < nr) {
                                const uint4 qv = reinterpret_cast<const uint4*>(qbuf)[(r * D) / 8 + c];
                                float s2 = sc[r];
                                s2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kv.x), __builtin_bit_cast(bf16x2_t, qv.x), s2, false);
                                s2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kv.y), __builtin_bit_cast(bf16x2_t, qv.y), s2, false);
                                s2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kv.z), __builtin_bit_cast(bf16x2_t, qv.z), s2, false);
                                s2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kv.w), __builtin_bit_cast(bf16x2_t, qv.w), s2, false);
                                sc[r] = s2;
                            }
                        }
                    }
                } else {
                    for (int c = 0; c < D; ++c) {
                        const float kv = ld_elem(a.sfx_k, a.sfx_dtype, (tok0 + t) * D + c);
#pragma unroll
                        for (int r = 0; r < kSfxRows; ++r)
                            if (r < nr) sc[r] += kv * reinterpret_cast<const float*>(qbuf)[r * D + c];
                    }
                }
            }
            // online softmax per row over this chunk (log2 units)
#pragma unroll
            for (int r = 0; r < kSfxRows; ++r) {
                if (r >= nr) break;
                const float x = ok ? sc[r] * a.sm_log2 : -INFINITY;
                float mx = x;
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
                const float mnew = fmaxf(m[r], mx);
                const float alpha = (m[r] == -INFINITY) ? 0.0f : exp2f(m[r] - mnew);
                const float p = ok ? exp2f(x - mnew) : 0.0f;
                float ps = p;
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off, 64);
                l[r] = l[r] * alpha + ps;
                m[r] = mnew;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[r][e] *= alpha;
                pbuf[lane * kSfxRows + r] = p;
            }
            __builtin_amdgcn_wave_barrier();
            const int nt = min(64, S - c0);
            for (int tt = 0; tt < nt; ++tt) {
                float v[EPL];
                const uint64_t vo = (tok0 + c0 + tt) * D + EPL * lane;
                if (BF16) {
                    if (EPL == 2) {
                        const uint32_t two = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.sfx_v) + vo)[0];
                        v[0] = __uint_as_float(two << 16);
                        v[EPL - 1] = __uint_as_float(two & 0xffff0000u);
                    } else {
                        v[0] = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.sfx_v)[vo]) << 16);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) v[e] = ld_elem(a.sfx_v, a.sfx_dtype, vo + e);
                }
                const float4 p03 = reinterpret_cast<const float4*>(pbuf)[tt * 2];
                const float4 p47 = reinterpret_cast<const float4*>(pbuf)[tt * 2 + 1];
                const float pr[kSfxRows] = {p03.x, p03.y, p03.z, p03.w, p47.x, p47.y, p47.z, p47.w};
#pragma unroll
                for (int r = 0; r < kSfxRows; ++r)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[r][e] += pr[r] * v[e];
            }
            __builtin_amdgcn_wave_barrier();
        }
        for (int r = 0; r < nr; ++r) {
            float* rec = a.part + a.sfx_part_off + (((uint64_t)k * a.lc + lj) * a.hq + g * a.G + r0 + r) * (2 + D);
            if (lane == 0) {
                rec[0] = m[r];
                rec[1] = l[r];
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) rec[2 + EPL * lane + e] = acc[r][e];
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// grid n_agents * lc * hkv: one single-wavefront workgroup per unit.  Workgroups of one
// wavefront spread the units evenly over the compute units (four-wavefront workgroups put
// 16 units on some and 12 on others at 3840 units, and the fuller ones set the time).
template <int D, int RS, bool PF>
__global__ void __launch_bounds__(64) k_sfx_fast(DecodeLaunch a) {
    __shared__ __align__(16) float sbuf[kSfxChunk * RS];
    const int unit = blockIdx.x;
    if (unit >= a.n_agents * a.lc * a.hkv) return;
    sfx_fast_wave<D, RS, PF>(a, unit, sbuf);
}

// ------------------------------------------------------------------ private segments
// A private segment (a pool of at most 8 rows: one agent's own older tokens) is decoded
// by one wavefront per (segment agent, layer, kv head), like the native suffix, with
// the pool's encoding: scores from int8 K as exact fp16 against fp16 query pairs
// (v_dot2_f32_f16; each query row pre-scaled by 2^-e so it fits fp16, the score scaled
// back by 2^e); V accumulated in the rotated domain, acc = sum p * Vn * c[code],
// from an fp32 centroid table in LDS.  The result is a partial record (m, l, acc) in
// the pool kernels' layout (one split), merged by k_merge with the shared pool's.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
constexpr int kSegChunk = 128;  // tokens per segment chunk (bounds the code fields held ahead)

__device__ __forceinline__ uint32_t pack_h2f(float lo, float hi) {
    const half2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// 4 int8 codes -> 4 fp16 values k, as two pairs: the byte k + 128 in the mantissa of 1024
// gives 1024 + (k + 128), and a packed fp16 subtraction of 1152 leaves k (all exact)
__device__ __forceinline__ void i8x4_to_h2x2(uint32_t w, uint32_t& lo, uint32_t& hi) {
    const uint32_t u = w ^ 0x80808080u;
    const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off);
    hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off);
}

template <int D, int RS, int BITS>
__device__ void seg_wave(const DecodeLaunch& a, const PoolEntry& P, int k, int jpos, int lj, int g, float* sbuf,
                         const float* cent) {
    // score sweep: LPT lanes per token, 16 dimensions (16 bytes of K) each
    constexpr int LPT = D / 16;
    constexpr int TPP = 64 / LPT;                  // tokens per load instruction
    constexpr int KG = RS >= 8 ? 32 : 64;          // tokens per score group
    constexpr int KU = KG / TPP;
    constexpr int RPL = RS / LPT > 1 ? RS / LPT : 1;
    constexpr int LB = LPT == 4 ? 2 : 3;           // log2 LPT
    constexpr int LS = RS / RPL == 1 ? 0 : RS / RPL == 2 ? 1 : RS / RPL == 4 ? 2 : 3;
    // value sweep: 4 dimensions per lane, LVG lanes per 8-token group, GP groups at once
    constexpr int LVG = D / 4;
    constexpr int GP = 64 / LVG;
    constexpr int FW = BITS;                       // field dwords of 4 dimensions (4 * 8 * BITS bits)
    constexpr int NGL = kSegChunk / 8 / GP;        // 8-token groups per lane per chunk (value sweep)
    static_assert((1 << LS) * RPL == RS && (GP == 2 || GP == 4), "segment tiling");

    const int lane = threadIdx.x & 63;
    const int l = a.l0 + lj;
    const int T = P.T;
    const int agent = P.agent_base >= 0 ? P.agent_base + jpos : a.agent_id[P.agent0 + jpos];
    const int8_t* kq = reinterpret_cast<const int8_t*>(P.base + P.off_kq) + ((uint64_t)l * a.hkv + g) * P.tc * D;
    const float* vn = reinterpret_cast<const float*>(P.base + P.off_vn) + ((uint64_t)l * a.hkv + g) * P.tc;
    const float* ks = reinterpret_cast<const float*>(P.base + P.off_ks) + ks_offset(P, l, g, a.hkv, D);
    const uint8_t* vc = P.base + P.off_vc0 + (uint64_t)a.hkv * P.tc * (D / 8) * layer_bits_prefix(P, l) +
                        (uint64_t)g * (P.tc / 8) * D * BITS;
    const int part = lane % LPT, tl = lane / LPT;
    int rb = 0;
    if constexpr (LS >= 1) rb += (lane & 1) * (RS / 2);
    if constexpr (LS >= 2) rb += ((lane >> 1) & 1) * (RS / 4);
    if constexpr (LS >= 3) rb += ((lane >> 2) & 1) * (RS / 8);
    const bool swriter = ((lane & (LPT - 1)) >> LS) == 0;
    const int gs = lane / LVG, db = lane % LVG;  // value sweep: group slot, dimension block

    for (int r0 = 0; r0 < a.G; r0 += RS) {
        const int nr = min(RS, a.G - r0);
        // query slices as fp16 pairs (dims 16 part .. 16 part + 15), each row times 2^-e so that
        // it stays below 2^15 (max|q| < 2^E, e = max(0, E - 15)); qsc = 2^e restores the score
        uint32_t qp[RS][8];
        float qsc[RS];
#pragma unroll
        for (int r = 0; r < RS; ++r) {
            const int rr = min(r0 + r, a.G - 1);
            const uint64_t qo = (((uint64_t)agent * a.lc + lj) * a.hq + g * a.G + rr) * D + 16 * part;
            float x[16];
            if (a.q_dtype == PKV_BF16) {
                const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qo);
                const uint4 w0 = src[0], w1 = src[1];
                const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    x[2 * i] = __uint_as_float(w[i] << 16);
                    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = static_cast<const float*>(a.q)[qo + i];
            }
            float mx = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(x[i]));
#pragma unroll
            for (int off = 1; off < LPT; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));  // the row's lanes
            int ex = 0;
            frexpf(mx, &ex);
            const int e = ex > 15 ? ex - 15 : 0;
            qsc[r] = ldexpf(1.0f, e);
            const float qinv = ldexpf(1.0f, -e);
#pragma unroll
            for (int i = 0; i < 8; ++i) qp[r][i] = pack_h2f(x[2 * i] * qinv, x[2 * i + 1] * qinv);
        }
        float M[RS], Lp[RS], acc[RS][4];
#pragma unroll
        for (int r = 0; r < RS; ++r) {
            M[r] = -INFINITY;
            Lp[r] = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[r][e] = 0.0f;
        }
        for (int c0 = 0; c0 < T; c0 += kSegChunk) {
            const int nc = min(kSegChunk, T - c0);
            const int ng = (nc + 7) / 8;
            // this lane's code fields of the chunk's groups gs, gs + GP, ..., loaded now so that
            // they arrive while the scores are computed
            uint32_t fw[NGL][FW];
#pragma unroll
            for (int q = 0; q < NGL; ++q) {
                const int gi = min(gs + q * GP, ng - 1);  // past the chunk: a valid group, not used
                const uint32_t* fp =
                    reinterpret_cast<const uint32_t*>(vc + (uint64_t)((c0 >> 3) + gi) * (D * BITS)) + FW * db;
#pragma unroll
                for (int i = 0; i < FW; ++i) fw[q][i] = fp[i];
            }
            // ---- scores (log2 units) into sbuf[t][r]
            float mloc[RPL];
#pragma unroll
            for (int i = 0; i < RPL; ++i) mloc[i] = -INFINITY;
            for (int g0 = 0; g0 < nc; g0 += KG) {
                uint4 kk[KU];
#pragma unroll
                for (int u = 0; u < KU; ++u) {
                    const int t = min(g0 + u * TPP + tl, nc - 1);
                    kk[u] = *reinterpret_cast<const uint4*>(kq + (uint64_t)(c0 + t) * D + 16 * part);
                }
#pragma unroll
                for (int u = 0; u < KU; ++u) {
                    const int t = g0 + u * TPP + tl;
                    const bool ok = t < nc;
                    uint32_t kh[8];
                    i8x4_to_h2x2(kk[u].x, kh[0], kh[1]);
                    i8x4_to_h2x2(kk[u].y, kh[2], kh[3]);
                    i8x4_to_h2x2(kk[u].z, kh[4], kh[5]);
                    i8x4_to_h2x2(kk[u].w, kh[6], kh[7]);
                    float sc[RS];
#pragma unroll
                    for (int r = 0; r < RS; ++r) {
                        sc[r] = 0.0f;
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            sc[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, kh[i]),
                                                           __builtin_bit_cast(half2_t, qp[r][i]), sc[r], false);
                        sc[r] *= qsc[r];
                    }
                    auto red = [&](auto bt) {
                        constexpr int b = decltype(bt)::value;
                        if constexpr (b < LS) scatter_add<(1 << b), (RS >> b)>(sc, lane & (1 << b));
                        else if constexpr (b < LB) all_add<(1 << b), RPL>(sc);
                    };
                    red(std::integral_constant<int, 0>{});
                    red(std::integral_constant<int, 1>{});
                    red(std::integral_constant<int, 2>{});
                    const float f = ks[c0 + min(t, nc - 1)] * a.sm_log2;
#pragma unroll
                    for (int i = 0; i < RPL; ++i) {
                        const float x = sc[i] * f;
                        if (ok) {
                            mloc[i] = fmaxf(mloc[i], x);
                            if (swriter) sbuf[t * RS + rb + i] = x;
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
#pragma unroll
                for (int off = LPT; off < 64; off <<= 1) mloc[i] = fmaxf(mloc[i], __shfl_xor(mloc[i], off, 64));
            }
#pragma unroll
            for (int r = 0; r < RS; ++r) {
                const int qq = r / RPL;
                int src = 0;
#pragma unroll
                for (int b = 0; b < LS; ++b) src |= ((qq >> (LS - 1 - b)) & 1) << b;
                const float mc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mloc[r % RPL]), src));
                const float mn = fmaxf(M[r], mc);
                const float alpha = (M[r] == -INFINITY) ? 0.0f : exp2f(M[r] - mn);
                M[r] = mn;
                Lp[r] *= alpha;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[r][e] *= alpha;
            }
            __builtin_amdgcn_wave_barrier();
            // ---- probabilities: l sums p, the value sweep uses w = p * Vn; tokens past the
            // chunk (to the end of its last 8-token group) get w = 0
            for (int t = lane; t < ((nc + 7) & ~7); t += 64) {
                const float n = t < nc ? vn[c0 + t] : 0.0f;
#pragma unroll
                for (int r = 0; r < RS; ++r) {
                    const float p = t < nc ? exp2f(sbuf[t * RS + r] - M[r]) : 0.0f;
                    Lp[r] += p;
                    sbuf[t * RS + r] = p * n;
                }
            }
            __builtin_amdgcn_wave_barrier();
            // ---- values: 8-token groups, 4 dimensions per lane, GP groups side by side
#pragma unroll
            for (int q = 0; q < NGL; ++q) {
                const int gi = gs + q * GP;
                if (gi >= ng) break;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int t = 8 * gi + i;
                    float w[RS];
                    if constexpr (RS >= 4) {
#pragma unroll
                        for (int r4 = 0; r4 < RS; r4 += 4) {
                            const float4 w4 = *reinterpret_cast<const float4*>(&sbuf[t * RS + r4]);
                            w[r4] = w4.x;
                            w[r4 + 1] = w4.y;
                            w[r4 + 2] = w4.z;
                            w[r4 + 3] = w4.w;
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < RS; ++r) w[r] = sbuf[t * RS + r];
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // dimension 4 db + e: bits [8 BITS e + BITS i, +BITS) of the 4 fields
                        const int bit = 8 * BITS * e + BITS * i;
                        const uint32_t lo = fw[q][bit >> 5] >> (bit & 31);
                        const uint32_t code =
                            ((bit & 31) + BITS > 32 ? (lo | (fw[q][(bit >> 5) + 1] << (32 - (bit & 31)))) : lo) &
                            ((1u << BITS) - 1u);
                        const float c = cent[code];
#pragma unroll
                        for (int r = 0; r < RS; ++r) acc[r][e] = fmaf(w[r], c, acc[r][e]);
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        // ---- records: l over all lanes; acc over the group slots
#pragma unroll
        for (int r = 0; r < RS; ++r) {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) Lp[r] += __shfl_xor(Lp[r], off, 64);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[r][e] += __shfl_xor(acc[r][e], LVG, 64);
                if constexpr (GP == 4) acc[r][e] += __shfl_xor(acc[r][e], 2 * LVG, 64);
            }
        }
        const int rho0 = jpos * a.G + r0;
        float* rec0 = a.part + P.part_off + (((uint64_t)lj * a.hkv + g) * P.rows) * (2 + D);
#pragma unroll
        for (int r = 0; r < RS; ++r) {
            if (r >= nr) break;
            float* rec = rec0 + (uint64_t)(rho0 + r) * (2 + D);
            if (gs == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) rec[2 + 4 * db + e] = acc[r][e];
            }
            if (lane == 0) {
                rec[0] = T > 0 ? M[r] : -INFINITY;
                rec[1] = Lp[r];
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// grid: ceil(segment units / 4), 256 threads; a unit is (segment pool, its agent, layer, kv head)
template <int D, int RS>
__global__ void __launch_bounds__(256) k_seg(DecodeLaunch a, Centroids cents) {
    __shared__ __align__(16) float sbuf[4][kSegChunk * RS];
    __shared__ float cent[3][16];
    if (threadIdx.x < 48) cent[threadIdx.x / 16][threadIdx.x % 16] = cents.c[threadIdx.x / 16][threadIdx.x % 16];
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int unit = blockIdx.x * 4 + wave;
    int p = -1;
    for (int i = 0; i < a.n_pools; ++i) {
        const PoolEntry& e = a.pools[i];
        if (e.seg_begin < 0) continue;
        const int n = (e.rows / a.G) * a.lc * a.hkv;
        if (unit >= e.seg_begin && unit < e.seg_begin + n) p = i;
    }
    if (p < 0) return;
    const PoolEntry& P = a.pools[p];
    unit -= P.seg_begin;
    const int g = unit % a.hkv;
    const int lj = (unit / a.hkv) % a.lc;
    const int jpos = unit / (a.hkv * a.lc);
    const int l = a.l0 + lj;
    switch (layer_bits(P, l)) {
        case 2: seg_wave<D, RS, 2>(a, P, P.agent0 + jpos, jpos, lj, g, sbuf[wave], cent[0]); break;
        case 3: seg_wave<D, RS, 3>(a, P, P.agent0 + jpos, jpos, lj, g, sbuf[wave], cent[1]); break;
        default: seg_wave<D, RS, 4>(a, P, P.agent0 + jpos, jpos, lj, g, sbuf[wave], cent[2]); break;
    }
}

// grid ceil(n_agents * lc * hkv / 4), 256 threads = 4 wavefronts, one unit each
template <int D>
__global__ void __launch_bounds__(256) k_sfx(DecodeLaunch a) {
    __shared__ __align__(16) float pbuf[4][64 * kSfxRows];
    __shared__ __align__(16) uint32_t qbuf[4][kSfxRows * D];
    const int wave = threadIdx.x >> 6;
    const int unit = blockIdx.x * 4 + wave;
    if (unit >= a.n_agents * a.lc * a.hkv) return;
    if (a.sfx_dtype == PKV_BF16 && a.q_dtype == PKV_BF16)
        sfx_wave<D, true>(a, unit, pbuf[wave], qbuf[wave]);
    else
        sfx_wave<D, false>(a, unit, pbuf[wave], qbuf[wave]);
}

// One wavefront per output row (launch agent, layer, q head): combine the
// pool's split records, apply the inverse FWHT (H / d) to the rotated-domain
// accumulator, fold in the suffix record and normalise.  Every load whose address
// is known up front is issued first, so the row costs about one memory round trip:
// the suffix record, the records' (m, l) spread over the lanes (record j on lane
// j % 64) and the accumulators of the first U records; further records (more than U
// splits) are summed U at a time, their loads issued before any is used.
template <int D>
__global__ void __launch_bounds__(kThreads) k_merge(DecodeLaunch a) {
    constexpr int EPL = D / 64;
    constexpr int U = 16;  // records whose accumulator loads are in flight together
    const int lane = threadIdx.x & 63;
    const uint64_t row = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const uint64_t n_rows = (uint64_t)a.n_agents * a.lc * a.hq;
    if (row >= n_rows) return;
    const int h = row % a.hq;
    const int lj = (row / a.hq) % a.lc;
    const int k = row / ((uint64_t)a.hq * a.lc);
    const int g = h / a.G;
    // the suffix record of the row
    float su_m = -INFINITY, su_l = 0.0f, su_v[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) su_v[e] = 0.0f;
    if (a.has_sfx) {
        const float* ru = a.part + a.sfx_part_off + (((uint64_t)k * a.lc + lj) * a.hq + h) * (2 + D);
        su_m = ru[0];
        su_l = ru[1];
#pragma unroll
        for (int e = 0; e < EPL; ++e) su_v[e] = ru[2 + EPL * lane + e];
    }
    // the agent's pool and, if it has one, its private pool: split records of both, all in
    // the rotated domain, merged before the one inverse transform (records 0 .. n0-1 the pool's)
    auto records = [&](int which, const float*& rec0, uint64_t& stride, int& splits) {
        const PoolEntry& P = a.pools[which == 0 ? a.agent_pool[k] : a.agent_pool2[k]];
        const int rho = (which == 0 ? a.agent_pos[k] : a.agent_pos2[k]) * a.G + h % a.G;
        rec0 = a.part + P.part_off + ((((uint64_t)lj * a.hkv + g) * P.splits) * P.rows + rho) * (2 + D);
        stride = (uint64_t)P.rows * (2 + D);
        splits = P.splits;
    };
    const float* base0;
    const float* base1 = nullptr;
    uint64_t st0, st1 = 0;
    int n0, n1 = 0;
    records(0, base0, st0, n0);
    if (a.agent_pool2[k] >= 0) records(1, base1, st1, n1);
    const int nrec = n0 + n1;
    auto rec = [&](int j) { return j < n0 ? base0 + (uint64_t)j * st0 : base1 + (uint64_t)(j - n0) * st1; };
    // this lane's record of the first 64 (m, l) and the first U records' accumulators
    float m0 = -INFINITY, l0 = 0.0f;
    if (lane < nrec) {
        const float* r = rec(lane);
        m0 = r[0];
        l0 = r[1];
    }
    float v[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float* r = rec(min(u, nrec - 1)) + 2 + EPL * lane;  // past the end: a valid record, weight 0
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[u][e] = r[e];
    }
    // M = max of the records' m; L = sum of 2^(m - M) l
    float M = m0;
    for (int j = lane + 64; j < nrec; j += 64) M = fmaxf(M, rec(j)[0]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float L = 0.0f, z[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) z[e] = 0.0f;
    if (M != -INFINITY) {
        for (int c = 0; c < nrec; c += 64) {
            // this lane's record c + lane: its weight (0 past the end and for empty records)
            float wt = 0.0f;
            if (c + lane < nrec) {
                float m = m0, lv = l0;
                if (c > 0) {
                    const float* r = rec(c + lane);
                    m = r[0];
                    lv = r[1];
                }
                wt = (m == -INFINITY) ? 0.0f : exp2f(m - M);
                L += wt * lv;
            }
            const int nc = min(64, nrec - c);
            for (int j0 = 0; j0 < nc; j0 += U) {
                if (c > 0 || j0 > 0) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const float* r = rec(c + min(j0 + u, nc - 1)) + 2 + EPL * lane;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) v[u][e] = r[e];
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float w = j0 + u < nc ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), j0 + u)) : 0.0f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) z[e] = fmaf(w, v[u][e], z[e]);
                }
            }
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) L += __shfl_xor(L, off, 64);
    }
    // inverse transform: H z / D (lane holds dims EPL*lane + e), then the rotation's signs
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
            const float pz = __shfl_xor(z[e], off, 64);
            z[e] = upper ? (pz - z[e]) : (z[e] + pz);
        }
    }
    {
        const uint32_t* vs = a.pools[a.agent_pool[k]].vsign;
        const int d0 = EPL * lane;
        const uint32_t sb = (vs[d0 >> 5] >> (d0 & 31)) & ((1u << EPL) - 1u);
#pragma unroll
        for (int e = 0; e < EPL; ++e) z[e] = __uint_as_float(__float_as_uint(z[e]) ^ (((sb >> e) & 1u) << 31));
    }
    const float inv_d = 1.0f / D;
    float o[EPL];
    float denom;
    if (a.has_sfx) {
        const float M2 = fmaxf(M, su_m);
        const float ap = (M == -INFINITY) ? 0.0f : exp2f(M - M2);
        const float au = (su_m == -INFINITY) ? 0.0f : exp2f(su_m - M2);
        denom = ap * L + au * su_l;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = ap * z[e] * inv_d + au * su_v[e];
    } else {
        denom = L;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = z[e] * inv_d;
    }
    const float rl = denom > 0.0f ? 1.0f / denom : 0.0f;
    float* out = a.out + (((uint64_t)a.agent_id[k] * a.lc + lj) * a.hq + h) * D + EPL * lane;
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = o[e] * rl;
}

// ------------------------------------------------------------------ host plan
struct Plan {
    std::vector<DecodeLaunch> launches;
    std::vector<int> pool_wg;  // workgroups of the pool kernel per launch
    size_t ws_floats = 0;
};

int make_plan(const pkv_decode_args* x, bool use_mfma, Plan* plan) {
    const pkv_pool* p0 = x->agent_pool[0];
    const int hkv = p0->cfg.n_kv_heads, d = p0->cfg.head_dim;
    const int G = x->n_q_heads / hkv;
    const float sigma = x->softmax_scale != 0.0f ? x->softmax_scale : 1.0f / std::sqrt((float)d);
    auto private_of = [&](int a) -> const pkv_pool* {
        return x->agent_private_pool ? x->agent_private_pool[a] : nullptr;
    };
    // fp32 queries, and queries that carry a per-channel pool's K scales, take the matrix-core
    // kernel's fp16 hi + lo operands: at most 48 rows per workgroup
    bool split_q = x->q_dtype == PKV_F32;
    for (int a = 0; a < x->n_agents; ++a) {
        split_q = split_q || x->agent_pool[a]->cfg.k_scale == PKV_KSCALE_CHANNEL;
        if (private_of(a)) split_q = split_q || private_of(a)->cfg.k_scale == PKV_KSCALE_CHANNEL;
    }

    // group agents by pool (first appearance order)
    std::vector<const pkv_pool*> order;
    std::map<const pkv_pool*, std::vector<int>> members;
    for (int a = 0; a < x->n_agents; ++a) {
        const pkv_pool* p = x->agent_pool[a];
        if (!members.count(p)) order.push_back(p);
        members[p].push_back(a);
    }
    // chunks of one pool's agents: at most kMaxAgentsPerLaunch agents and kMaxPoolsPerLaunch - 1
    // distinct private pools; within a chunk the agents of one private pool are consecutive
    // (agents without one first), so every pool entry's rows belong to consecutive launch agents
    struct Chunk {
        const pkv_pool* pool;
        std::vector<int> agents;
        std::vector<const pkv_pool*> privs;  // distinct private pools, first appearance order
    };
    std::vector<Chunk> chunks;
    for (const pkv_pool* p : order) {
        const std::vector<int>& m = members[p];
        size_t i = 0;
        while (i < m.size()) {
            Chunk c{p, {}, {}};
            while (i < m.size() && c.agents.size() < (size_t)kMaxAgentsPerLaunch) {
                const pkv_pool* q = private_of(m[i]);
                const bool seen = !q || std::find(c.privs.begin(), c.privs.end(), q) != c.privs.end();
                if (!seen && c.privs.size() + 1 >= (size_t)kMaxPoolsPerLaunch) break;
                if (!seen) c.privs.push_back(q);
                c.agents.push_back(m[i]);
                ++i;
            }
            std::stable_sort(c.agents.begin(), c.agents.end(), [&](int u, int v) {
                auto rank = [&](int a) {
                    const pkv_pool* q = private_of(a);
                    return q ? 1 + (int)(std::find(c.privs.begin(), c.privs.end(), q) - c.privs.begin()) : 0;
                };
                return rank(u) < rank(v);
            });
            chunks.push_back(std::move(c));
        }
    }
    size_t ci = 0;
    while (ci < chunks.size()) {
        DecodeLaunch L;
        std::memset(&L, 0, sizeof(L));
        L.sfx_wg_begin = -1;
        L.q = x->q;
        L.sfx_k = x->sfx_k;
        L.sfx_v = x->sfx_v;
        L.out = x->out;
        L.q_dtype = x->q_dtype;
        L.sfx_dtype = x->sfx_dtype;
        L.hq = x->n_q_heads;
        L.hkv = hkv;
        L.G = G;
        L.d = d;
        L.l0 = x->layer_begin;
        L.lc = x->layer_count;
        L.sfx_cap = x->sfx_cap;
        L.sm_log2 = sigma * 1.4426950408889634f;
        int n_agents = 0, wg = 0;
        uint64_t part = 0;
        // one pool entry: rows are (agents[i], head of the group) for the launch agents
        // agent0 .. agent0 + n - 1, which are call agents `agents`
        // seg: a private segment of at most 8 rows, decoded by k_seg instead of the pool kernel
        auto add_pool = [&](const pkv_pool* p, int agent0, const std::vector<int>& agents, bool seg = false) {
            PoolEntry& e = L.pools[L.n_pools];
            e.base = static_cast<const uint8_t*>(p->base);
            e.off_kq = p->off_kq;
            e.off_vn = p->off_vn;
            e.off_ks = p->off_ks;
            e.off_vmax = p->off_vmax;
            e.off_vc0 = p->off_vc[0];
            std::memcpy(e.vsign, p->cfg.v_signs, sizeof(e.vsign));
            e.kmode = p->cfg.k_scale;
            for (int l = 0; l < p->cfg.n_layers; ++l) {
                if (p->cfg.v_bits[l] >= 3) e.ge3[l >> 5] |= 1u << (l & 31);
                if (p->cfg.v_bits[l] == 4) e.eq4[l >> 5] |= 1u << (l & 31);
            }
            e.T = p->n_tokens[x->layer_begin];
            e.tc = p->tc;
            e.rows = (int)agents.size() * G;
            e.agent0 = agent0;
            const int units = x->layer_count * hkv;
            const int tiles = std::max(1, (e.T + kTile - 1) / kTile);
            // row blocks: the matrix-core kernel holds at most 64 rows per workgroup (48 with fp32
            // queries), balanced over the blocks; the vector kernel 32
            const int block_max = use_mfma ? (split_q ? 48 : 64) : kValuRows;
            e.rblocks = (e.rows + block_max - 1) / block_max;
            e.rb_rows = use_mfma ? (e.rows + e.rblocks - 1) / e.rblocks : kValuRows;
            int splits = x->splits;
            // default split: enough workgroups to cover the 256 compute units (MFMA: one
            // 4-wave workgroup per CU; VALU: two per CU).  A call with few (layer, kv head) units
            // (a single-layer call has 8) is bound by per-workgroup latency and the merge of the
            // splits' records: 128 matrix-core workgroups measured faster than 256 there
            const int target = use_mfma ? (units * e.rblocks < 32 ? 128 : 256) : 512;
            if (splits <= 0) splits = std::max(1, std::min(tiles, (target + units * e.rblocks - 1) / (units * e.rblocks)));
            splits = std::min(splits, tiles);
            e.chunk = (tiles + splits - 1) / splits * kTile;
            e.splits = std::max(1, (std::max(e.T, 1) + e.chunk - 1) / e.chunk);
            e.wg_begin = wg;
            e.seg_begin = -1;
            if (seg) {
                e.splits = 1;
                e.chunk = std::max(e.T, 1);
                e.rblocks = 1;
                e.rb_rows = e.rows;
                e.seg_begin = L.seg_units;
                L.seg_units += (int)agents.size() * units;
            }
            e.part_off = 0;  // assigned below, once the launch is known to finish its rows in the pool kernel or not
            if (!seg) wg += units * e.splits * e.rblocks;
            e.agent_base = agents[0];
            for (size_t i = 0; i < agents.size(); ++i)
                if (agents[i] != agents[0] + (int)i) e.agent_base = -1;
            return L.n_pools++;
        };
        while (ci < chunks.size() && L.n_pools + 1 + (int)chunks[ci].privs.size() <= kMaxPoolsPerLaunch &&
               n_agents + (int)chunks[ci].agents.size() <= kMaxAgentsPerLaunch) {
            const Chunk& c = chunks[ci];
            const int shared = add_pool(c.pool, n_agents, c.agents);
            for (size_t i = 0; i < c.agents.size(); ++i) {
                const int a = c.agents[i];
                const int k = n_agents + (int)i;
                L.agent_id[k] = (int16_t)a;
                L.agent_pool[k] = (int16_t)shared;
                L.agent_pos[k] = (int16_t)i;
                L.agent_pool2[k] = -1;
                L.agent_pos2[k] = 0;
                const int sl = x->sfx_len ? x->sfx_len[a] : 0;
                L.sfx_len[k] = sl;
                if (sl > 0) L.has_sfx = 1;
            }
            // private pools: their agents are consecutive within the chunk
            size_t i = 0;
            while (i < c.agents.size()) {
                const pkv_pool* q = private_of(c.agents[i]);
                size_t j = i;
                while (j < c.agents.size() && private_of(c.agents[j]) == q) ++j;
                if (q) {
                    const std::vector<int> grp(c.agents.begin() + i, c.agents.begin() + j);
                    const bool seg = x->q_dtype == PKV_BF16 && (int)grp.size() * G <= 8 &&
                                     q->cfg.k_scale != PKV_KSCALE_CHANNEL;
                    const int ent = add_pool(q, n_agents + (int)i, grp, seg);
                    for (size_t t = i; t < j; ++t) {
                        L.agent_pool2[n_agents + t] = (int16_t)ent;
                        L.agent_pos2[n_agents + t] = (int16_t)(t - i);
                    }
                    L.has_private = 1;
                }
                i = j;
            }
            n_agents += (int)c.agents.size();
            ++ci;
        }
        L.n_agents = n_agents;
        // The matrix-core kernel finishes the rows itself when every pool has one split and every
        // private pool is a segment (whose records k_seg writes); then only segments and suffixes
        // need partial records in the workspace, otherwise every pool does (read by k_merge).
        L.fused = use_mfma ? 1 : 0;
        for (int p = 0; p < L.n_pools; ++p)
            if (L.pools[p].seg_begin < 0 && L.pools[p].splits != 1) L.fused = 0;
        for (int k = 0; k < L.n_agents; ++k)
            if (L.agent_pool2[k] >= 0 && L.pools[L.agent_pool2[k]].seg_begin < 0) L.fused = 0;
        const int units = x->layer_count * hkv;
        for (int p = 0; p < L.n_pools; ++p) {
            PoolEntry& e = L.pools[p];
            if (L.fused && e.seg_begin < 0) continue;
            e.part_off = part;
            part += (uint64_t)units * e.splits * e.rows * record_floats(d);
        }
        if (L.has_sfx) {
            L.sfx_part_off = part;
            part += (uint64_t)n_agents * x->layer_count * x->n_q_heads * record_floats(d);
        }
        plan->ws_floats = std::max<size_t>(plan->ws_floats, part);
        plan->launches.push_back(L);
        plan->pool_wg.push_back(wg);
    }
    return PKV_OK;
}

int validate(const pkv_decode_args* x) {
    if (!x) return PKV_EINVAL;
    if (x->n_agents < 0 || x->layer_count < 0 || x->layer_begin < 0 || x->n_q_heads < 1) return PKV_EINVAL;
    if (x->n_agents == 0 || x->layer_count == 0) return PKV_OK;
    if (x->n_agents > 32767) return PKV_EINVAL;
    if (!x->agent_pool || !x->q || !x->out) return PKV_EINVAL;
    // the kernels read and write whole 16-byte chunks of these arrays
    auto misaligned = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; };
    if (misaligned(x->q) || misaligned(x->out) || misaligned(x->sfx_k) || misaligned(x->sfx_v)) return PKV_EINVAL;
    if (x->q_dtype != PKV_F32 && x->q_dtype != PKV_BF16) return PKV_EUNSUPPORTED;
    if (x->kernel < 0 || x->kernel > PKV_KERNEL_MFMA || x->splits < 0) return PKV_EINVAL;
    if (!(x->softmax_scale >= 0.0f) || std::isinf(x->softmax_scale)) return PKV_EINVAL;
    const pkv_pool* p0 = x->agent_pool[0];
    if (!p0) return PKV_EINVAL;
    for (int a = 0; a < x->n_agents; ++a) {
        const pkv_pool* p = x->agent_pool[a];
        if (!p || !p->base) return PKV_EINVAL;
        int err;
        if (!config_valid(&p->cfg, &err)) return err;
        if (p->cfg.n_kv_heads != p0->cfg.n_kv_heads || p->cfg.head_dim != p0->cfg.head_dim) return PKV_EINVAL;
        if (x->layer_begin + x->layer_count > p->cfg.n_layers) return PKV_EINVAL;
        const int T = p->n_tokens[x->layer_begin];
        for (int l = x->layer_begin; l < x->layer_begin + x->layer_count; ++l)
            if (p->n_tokens[l] != T) return PKV_EINVAL;
        if (T < 0 || T > p->cfg.capacity_tokens) return PKV_EINVAL;
    }
    if (x->agent_private_pool) {
        for (int a = 0; a < x->n_agents; ++a) {
            const pkv_pool* p = x->agent_private_pool[a];
            if (!p) continue;
            if (!p->base) return PKV_EINVAL;
            int err;
            if (!config_valid(&p->cfg, &err)) return err;
            if (p->cfg.n_kv_heads != p0->cfg.n_kv_heads || p->cfg.head_dim != p0->cfg.head_dim) return PKV_EINVAL;
            if (x->layer_begin + x->layer_count > p->cfg.n_layers) return PKV_EINVAL;
            const int T = p->n_tokens[x->layer_begin];
            for (int l = x->layer_begin; l < x->layer_begin + x->layer_count; ++l)
                if (p->n_tokens[l] != T) return PKV_EINVAL;
            if (T < 0 || T > p->cfg.capacity_tokens) return PKV_EINVAL;
            // a private pool is attended in addition to the shared one, never instead of it
            for (int b = 0; b < x->n_agents; ++b)
                if (x->agent_pool[b] == p) return PKV_EINVAL;
            // their rotated-domain sums are added before one inverse transform: same rotation
            if (std::memcmp(p->cfg.v_signs, x->agent_pool[a]->cfg.v_signs, sizeof(p->cfg.v_signs)) != 0)
                return PKV_EINVAL;
        }
    }
    if (x->n_q_heads % p0->cfg.n_kv_heads) return PKV_EINVAL;
    bool any_sfx = false;
    for (int a = 0; a < x->n_agents; ++a) {
        const int s = x->sfx_len ? x->sfx_len[a] : 0;
        if (s < 0 || s > x->sfx_cap) return PKV_EINVAL;
        any_sfx |= s > 0;
    }
    if (any_sfx) {
        if (!x->sfx_k || !x->sfx_v) return PKV_EINVAL;
        if (x->sfx_dtype != PKV_F32 && x->sfx_dtype != PKV_BF16) return PKV_EUNSUPPORTED;
    }
    return PKV_OK;
}

// Compute units of the current device (cached per device; 0 if the query fails, which keeps
// every launch on its own kernel)
int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int D, bool PF>
void launch_sfx_fast(const DecodeLaunch& L, int units, hipStream_t s) {
    const dim3 grid(units), block(64);
    if (L.G == 1) hipLaunchKernelGGL((k_sfx_fast<D, 1, PF>), grid, block, 0, s, L);
    else if (L.G == 2) hipLaunchKernelGGL((k_sfx_fast<D, 2, PF>), grid, block, 0, s, L);
    else if (L.G <= 4) hipLaunchKernelGGL((k_sfx_fast<D, 4, PF>), grid, block, 0, s, L);
    else hipLaunchKernelGGL((k_sfx_fast<D, 8, PF>), grid, block, 0, s, L);
}

template <int D>
int enqueue(const Plan& plan, bool use_mfma, float* ws, void* const* events, hipStream_t s) {
    Centroids cents;
    std::memcpy(cents.c, codebook_tables().cent, sizeof(cents.c));
    for (size_t i = 0; i < plan.launches.size(); ++i) {
        DecodeLaunch L = plan.launches[i];
        L.part = ws;
        int pool_wg = plan.pool_wg[i];
        if (L.has_sfx) {
            const int units = L.n_agents * L.lc * L.hkv;
            const dim3 grid((units + 3) / 4);
            // a split-record matrix-core launch that leaves compute units free takes the window's
            // workgroups itself: both run side by side, one launch fewer (k_merge joins them)
            const bool bf16 = L.q_dtype == PKV_BF16 && L.sfx_dtype == PKV_BF16;
            if (use_mfma && !L.fused && bf16 && pool_wg + (int)grid.x <= cu_count()) {
                L.sfx_wg_begin = pool_wg;
                pool_wg += (int)grid.x;
            } else if (bf16) {
                // rows per pass: the group size rounded up to a power of two, at most 8; with fewer
                // waves than SIMDs (e.g. a single-layer call) latency rules, so each wave keeps its
                // next load group in flight; with more, other waves hide it at the lower register count
                if (units < 1024) launch_sfx_fast<D, true>(L, units, s);
                else launch_sfx_fast<D, false>(L, units, s);
            } else {
                hipLaunchKernelGGL(k_sfx<D>, grid, dim3(kThreads), 0, s, L);
            }
        }
        // the event pair brackets the compressed-pool work of the call: private segments and the pool kernel
        if (events && i == 0 && hipEventRecord(static_cast<hipEvent_t>(events[0]), s) != hipSuccess) return PKV_EHIP;
        if (L.seg_units > 0) {
            const dim3 grid((L.seg_units + 3) / 4);
            if (L.G == 1) hipLaunchKernelGGL((k_seg<D, 1>), grid, dim3(kThreads), 0, s, L, cents);
            else if (L.G == 2) hipLaunchKernelGGL((k_seg<D, 2>), grid, dim3(kThreads), 0, s, L, cents);
            else if (L.G <= 4) hipLaunchKernelGGL((k_seg<D, 4>), grid, dim3(kThreads), 0, s, L, cents);
            else hipLaunchKernelGGL((k_seg<D, 8>), grid, dim3(kThreads), 0, s, L, cents);
        }
        if (use_mfma) {
            // L.fused (set by the plan): one split per (pool, layer, kv head) and every private pool
            // a segment, so the MFMA kernel finishes the rows itself
            const int st = launch_pool_mfma(L, pool_wg, s);
            if (st != PKV_OK) return st;
        } else {
            hipLaunchKernelGGL(k_pool_valu<D>, dim3(plan.pool_wg[i]), dim3(kThreads), 0, s, L, cents);
        }
        if (events && i + 1 == plan.launches.size() &&
            hipEventRecord(static_cast<hipEvent_t>(events[1]), s) != hipSuccess)
            return PKV_EHIP;
        if (!L.fused) {
            const uint64_t rows = (uint64_t)L.n_agents * L.lc * L.hq;
            hipLaunchKernelGGL(k_merge<D>, dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0, s, L);
        }
    }
    return launch_status();
}

}  // namespace
}  // namespace pkv

namespace pkv {
namespace {

// Validation, kernel choice and launch plan shared by both decode entry points.  Returns
// PKV_OK with *empty set for a call with no work.
int prepare(const pkv_decode_args* args, Plan* plan, bool* use_mfma, bool* empty) {
    *empty = false;
    const int v = validate(args);
    if (v != PKV_OK) return v;
    if (args->n_agents == 0 || args->layer_count == 0) {
        *empty = true;
        return PKV_OK;
    }
    // the matrix-core kernel takes any number of rows per pool (in row blocks of at most 64, 48
    // with fp32 queries); the vector kernel runs only when asked for
    *use_mfma = args->kernel != PKV_KERNEL_VALU;
    make_plan(args, *use_mfma, plan);
    if (args->pool_events && (!args->pool_events[0] || !args->pool_events[1])) return PKV_EINVAL;
    return PKV_OK;
}

int enqueue_plan(const pkv_decode_args* args, const Plan& plan, bool use_mfma, float* ws, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (args->agent_pool[0]->cfg.head_dim == 128) return enqueue<128>(plan, use_mfma, ws, args->pool_events, s);
    return enqueue<64>(plan, use_mfma, ws, args->pool_events, s);
}

}  // namespace
}  // namespace pkv

extern "C" int agent_decode_attention(const pkv_decode_args* args, void* workspace, size_t* workspace_bytes,
                                      void* stream) {
    using namespace pkv;
    if (!workspace_bytes) return PKV_EINVAL;
    Plan plan;
    bool use_mfma = false, empty = false;
    const int st = prepare(args, &plan, &use_mfma, &empty);
    if (st != PKV_OK) return st;
    if (empty) {
        if (!workspace) *workspace_bytes = 0;
        return PKV_OK;
    }
    const size_t need = plan.ws_floats * sizeof(float);
    if (!workspace) {
        *workspace_bytes = need;
        return PKV_OK;
    }
    if (*workspace_bytes < need) return PKV_ENOSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return PKV_EINVAL;
    return enqueue_plan(args, plan, use_mfma, static_cast<float*>(workspace), stream);
}

// ------------------------------------------------------------------ allocation-free variant
// The decode kernels' workspace (suffix, segment and split partial records) in a fixed device
// array instead of a caller buffer, for callers that cannot allocate (graph capture, tight
// serving loops).  Each device holds its own copy of the array until the process ends.  Host
// code never uses the array's name as an address: its device address is fetched once per device
// with hipGetSymbolAddress (with that device current) and kept in scratch_dev[].
static constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace pkv {
namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];  // device address of `scratch` per device, nullptr until fetched

int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PKV_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return PKV_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_EHIP;
        scratch_dev[dev] = p;
    }
    *out = scratch_dev[dev];
    return PKV_OK;
}
}  // namespace
}  // namespace pkv

extern "C" size_t pkv_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int agent_decode_attention_noalloc(const pkv_decode_args* args, void* stream) {
    using namespace pkv;
    Plan plan;
    bool use_mfma = false, empty = false;
    const int st = prepare(args, &plan, &use_mfma, &empty);
    if (st != PKV_OK || empty) return st;
    if (plan.ws_floats * sizeof(float) > kScratchBytes) return PKV_ENOSPACE;
    void* ws = nullptr;
    const int sa = scratch_address(&ws);
    if (sa != PKV_OK) return sa;
    return enqueue_plan(args, plan, use_mfma, static_cast<float*>(ws), stream);
}
