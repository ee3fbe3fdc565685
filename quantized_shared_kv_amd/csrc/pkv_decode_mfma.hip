// Matrix-core pool decode kernel for gfx950 (v_mfma_f32_16x16x32_f16).
//
// PolyKV explainer, section 2.A: every agent reads the one shared pool;
// section 2.B: K is int8 with a per-tensor scale, V is FWHT-rotated
// Lloyd-Max codes with a per-vector norm, dequantised by centroid lookup and
// an inverse FWHT.  With all agents' query heads of one kv head batched (R =
// agents * G rows, 60 for 15 agents of a 32/8-head model), each pool byte
// feeds 4 * R * d / (d + d*b/8 + 4) ~ 170 flop at d = 128, b = 3 -- far above
// the fp32 vector ridge of the chip -- so both contractions run on MFMA.
//
// One workgroup of 4 wavefronts handles one (pool, layer, kv head, token
// split); each wavefront streams every 4th 32-token step of the split and
// keeps all rows (up to 64, in RT tiles of 16) in registers:
//
//   S^T[32 tok][16 rows] = Kq (int8 -> exact fp16) x Q^T (fp16)   2*RT*(d/32) MFMAs
//   x = S * (Ks[t] * sigma * log2 e); lazy online softmax (rescale only when a
//   row max grows by more than 2^8); w = p * Vn[t] * 2^(7-e) with e from the
//   per-head max norm, so w < 2^15, split into fp16 hi + lo parts
//   acc[16 rows][16 dims] += (Wh + Wl)[16][32 tok] x C[32 tok][16 dims]   2*RT*(d/16) MFMAs
//
// Lane layout (16x16x32: A row / B column = lane & 15, k-group = lane >> 4,
// D rows 4*(lane>>4) + j): the S^T accumulator of lane (g, r) holds tokens
// 4g + j of each 16-token tile for row r, which is exactly the P.V A operand
// of k-slots 8g + i when tile u contributes slots i = 4u + j; the K rows are
// loaded in the matching order (A row 4g + j of tile u = token 8g + 4u + j).
// So lane group g owns tokens 8g .. 8g + 7 of a step, which is why V codes are
// stored in 8-token groups: the code chunk of lane (g, n) is dims
// NB*n .. NB*n + NB-1 (NB = d/16) of those 8 tokens, contiguous in memory.
// Code pairs (2 tokens, 2b bits) index a 2^(2b)-entry LUT of fp16 centroid
// pairs in LDS, replicated 32 times so the 32 lanes of a half-wave never hit
// the same bank; each LUT read is one B-operand register.
//
// The rotated-domain accumulator and (m, l) of every row are merged across the
// 4 wavefronts in LDS (in a fixed order, so results are deterministic) and
// written as partial records; k_merge applies the one inverse FWHT per row.
#include <cstring>

#include "pkv_decode.h"

namespace pkv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kStep = 32;         // tokens per wavefront step
constexpr float kLazy = 8.0f;     // log2 growth of a row max tolerated before rescaling
constexpr int kLutCopies = 32;
constexpr int kWeightExp = 7;     // weights are scaled into [0, 2^15)

struct CentArg {
    float c[3][16];
};

union H8 {
    half8 h;
    uint32_t u[4];
};

__device__ __forceinline__ int find_pool_m(const DecodeLaunch& a, int wg) {
    int p = 0;
    while (p + 1 < a.n_pools && wg >= a.pools[p + 1].wg_begin) ++p;
    return p;
}

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    const half2v v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// 4 int8 (two's complement) -> 4 exact fp16: bytes u = x + 128 are placed in the
// mantissa of 1024 (fp16 0x6400), giving 1024 + u, then 1152 is subtracted.
__device__ __forceinline__ void i8x4_to_h4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    const uint32_t u = w ^ 0x80808080u;
    const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    const half2v off = {(_Float16)(-1152.0f), (_Float16)(-1152.0f)};
    lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, a) + off);
    hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, b) + off);
}

template <int NBYTES>
struct Chunk {
    uint32_t w[NBYTES / 4];
};

// Load NBYTES (8, 12, 16, 24 or 32) of V codes; the address is NBYTES-multiple aligned
// within a 256-byte aligned region, so 8-byte pieces are 8-aligned when NBYTES % 8 == 0.
template <int NBYTES>
__device__ __forceinline__ Chunk<NBYTES> load_chunk(const uint8_t* p) {
    Chunk<NBYTES> c;
    if constexpr (NBYTES % 16 == 0) {
#pragma unroll
        for (int i = 0; i < NBYTES / 16; ++i) {
            const uint4 v = reinterpret_cast<const uint4*>(p)[i];
            c.w[4 * i] = v.x;
            c.w[4 * i + 1] = v.y;
            c.w[4 * i + 2] = v.z;
            c.w[4 * i + 3] = v.w;
        }
    } else if constexpr (NBYTES % 8 == 0) {
#pragma unroll
        for (int i = 0; i < NBYTES / 8; ++i) {
            const uint2 v = reinterpret_cast<const uint2*>(p)[i];
            c.w[2 * i] = v.x;
            c.w[2 * i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NBYTES / 4; ++i) c.w[i] = reinterpret_cast<const uint32_t*>(p)[i];
    }
    return c;
}

// 2b-bit field at bit position P of the chunk (P, b compile-time).
template <int NBYTES, int P, int W>
__device__ __forceinline__ uint32_t field(const Chunk<NBYTES>& c) {
    constexpr int wi = P >> 5, sh = P & 31;
    if constexpr (sh + W <= 32) {
        return (c.w[wi] >> sh) & ((1u << W) - 1u);
    } else {
        return __builtin_amdgcn_alignbit(c.w[wi + 1], c.w[wi], sh) & ((1u << W) - 1u);
    }
}

template <int NBYTES, int BITS, int NBI, int PI>
__device__ __forceinline__ uint32_t lut_pair(const Chunk<NBYTES>& c, const uint32_t* lut, uint32_t lane_off) {
    const uint32_t idx = field<NBYTES, 8 * BITS * NBI + 2 * BITS * PI, 2 * BITS>(c);
    return lut[idx * kLutCopies + lane_off];
}

template <int NBYTES, int BITS, int NBI>
__device__ __forceinline__ half8 decode_b(const Chunk<NBYTES>& c, const uint32_t* lut, uint32_t lane_off) {
    H8 r;
    r.u[0] = lut_pair<NBYTES, BITS, NBI, 0>(c, lut, lane_off);
    r.u[1] = lut_pair<NBYTES, BITS, NBI, 1>(c, lut, lane_off);
    r.u[2] = lut_pair<NBYTES, BITS, NBI, 2>(c, lut, lane_off);
    r.u[3] = lut_pair<NBYTES, BITS, NBI, 3>(c, lut, lane_off);
    return r.h;
}

template <int D, int RT, int BITS, int NBI = 0>
__device__ __forceinline__ void pv_all(f32x4 (&acc)[RT][D / 16], const half8 (&Wh)[RT], const half8 (&Wl)[RT],
                                       const Chunk<D / 16 * BITS>& c, const uint32_t* lut, uint32_t lane_off) {
    if constexpr (NBI < D / 16) {
        const half8 vb = decode_b<D / 16 * BITS, BITS, NBI>(c, lut, lane_off);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            acc[rt][NBI] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wh[rt], vb, acc[rt][NBI], 0, 0, 0);
            acc[rt][NBI] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wl[rt], vb, acc[rt][NBI], 0, 0, 0);
        }
        pv_all<D, RT, BITS, NBI + 1>(acc, Wh, Wl, c, lut, lane_off);
    }
}

struct Smem {
    union {
        uint32_t lut[256 * kLutCopies];  // fp16 centroid pairs, replicated
        float accbuf[64 * 128];          // cross-wave merge of the accumulators
    };
    float m[kWaves][64];
    float l[kWaves][64];
};

template <int D, int RT, int BITS, bool QSPLIT>
__device__ void pool_mfma_body(const DecodeLaunch& a, const CentArg& cents, Smem& sm) {
    constexpr int NB = D / 16;   // PV column tiles
    constexpr int KS = D / 32;   // QK k-steps
    constexpr int DL = D / 4;    // K bytes per lane per token
    constexpr int CB = NB * BITS;  // V code bytes per lane per step
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 15, lg = lane >> 4;

    const int p = find_pool_m(a, blockIdx.x);
    const PoolEntry& P = a.pools[p];
    int local = blockIdx.x - P.wg_begin;
    const int sp = local % P.splits;
    local /= P.splits;
    const int g = local % a.hkv;
    const int lj = local / a.hkv;
    const int l = a.l0 + lj;
    const int R = P.rows;

    const int8_t* kq = reinterpret_cast<const int8_t*>(P.base + P.off_kq) + ((uint64_t)l * a.hkv + g) * P.tc * D;
    const float* vn = reinterpret_cast<const float*>(P.base + P.off_vn) + ((uint64_t)l * a.hkv + g) * P.tc;
    const float* ks = reinterpret_cast<const float*>(P.base + P.off_ks) + (uint64_t)l * P.tc;
    const uint8_t* vc = P.base + P.off_vc0 + (uint64_t)a.hkv * P.tc * (D / 8) * layer_bits_prefix(P, l) +
                        (uint64_t)g * (P.tc / kGroupTokens) * D * BITS;
    const float vmax = reinterpret_cast<const float*>(P.base + P.off_vmax)[(uint64_t)l * a.hkv + g];
    int ex = 0;
    frexpf(vmax, &ex);
    // vn * nu < 2^7, so w = p * vn * nu < 2^15 fits fp16 while keeping the lo part of
    // small weights out of the fp16 subnormal range
    const float nu = ldexpf(1.0f, (vmax > 0.0f ? -ex : 0) + kWeightExp);

    // LUT of fp16 centroid pairs: entry e = c0 | c1 << BITS -> (c[c0], c[c1])
    {
        const float* c = cents.c[BITS - 2];
        constexpr int NE = 1 << (2 * BITS);
        for (int i = tid; i < NE * kLutCopies; i += 256) {
            const int e = i / kLutCopies;
            sm.lut[i] = pack_h2(c[e & ((1 << BITS) - 1)], c[e >> BITS]);
        }
    }

    // queries as B operands: lane (lg, rl) holds row 16 rt + rl, dims lg*DL + 8 ks + i
    half8 qb[RT][KS];
    half8 qlo[QSPLIT ? RT : 1][QSPLIT ? KS : 1];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int rho = 16 * rt + rl;
        const bool ok = rho < R;
        const int rr = ok ? rho : 0;
        const int agent = a.agent_id[P.agent0 + rr / a.G];
        const int head = g * a.G + rr % a.G;
        const uint64_t qoff = (((uint64_t)agent * a.lc + lj) * a.hq + head) * D + lg * DL;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            H8 hv, lv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x0 = 0.0f, x1 = 0.0f;
                if (ok) {
                    if (a.q_dtype == PKV_BF16) {
                        const uint32_t two = reinterpret_cast<const uint32_t*>(
                            static_cast<const uint16_t*>(a.q) + qoff + 8 * k)[i];
                        x0 = __uint_as_float(two << 16);
                        x1 = __uint_as_float(two & 0xffff0000u);
                    } else {
                        const float2 two = reinterpret_cast<const float2*>(static_cast<const float*>(a.q) + qoff + 8 * k)[i];
                        x0 = two.x;
                        x1 = two.y;
                    }
                }
                hv.u[i] = pack_h2(x0, x1);
                if constexpr (QSPLIT) {
                    const half2v hh = __builtin_bit_cast(half2v, hv.u[i]);
                    lv.u[i] = pack_h2(x0 - (float)hh[0], x1 - (float)hh[1]);
                }
            }
            qb[rt][k] = hv.h;
            if constexpr (QSPLIT) qlo[rt][k] = lv.h;
        }
    }
    __syncthreads();  // LUT ready

    float m[RT], lsum[RT];
    f32x4 acc[RT][NB];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m[rt] = -INFINITY;
        lsum[rt] = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[rt][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const int tb = sp * P.chunk;
    const int te = min(P.T, tb + P.chunk);
    const int nsteps = te > tb ? (te - tb + kStep - 1) / kStep : 0;
    const float fs = a.sm_log2;
    const uint32_t lane_off = lane & (kLutCopies - 1);
    const uint32_t* lut = sm.lut;
    // K row of this lane in tile u: token 8*(rl>>2) + 4u + (rl&3), bytes lg*DL .. lg*DL + DL
    const int ktok0 = 8 * (rl >> 2) + (rl & 3);

    for (int st = wave; st < nsteps; st += kWaves) {
        const int t0 = tb + st * kStep;
        // ---- loads
        uint4 kr[2][DL / 16];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint4* src = reinterpret_cast<const uint4*>(kq + (uint64_t)(t0 + ktok0 + 4 * u) * D + lg * DL);
#pragma unroll
            for (int i = 0; i < DL / 16; ++i) kr[u][i] = src[i];
        }
        const Chunk<CB> ch = load_chunk<CB>(vc + ((uint64_t)(t0 / kGroupTokens + lg) * 16 + rl) * CB);
        const float4 n0 = reinterpret_cast<const float4*>(vn + t0 + 8 * lg)[0];
        const float4 n1 = reinterpret_cast<const float4*>(vn + t0 + 8 * lg)[1];
        const float4 s0 = reinterpret_cast<const float4*>(ks + t0 + 8 * lg)[0];
        const float4 s1 = reinterpret_cast<const float4*>(ks + t0 + 8 * lg)[1];
        float nn[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
        float ff[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const bool tail = t0 + kStep > te;
        bool valid[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            valid[i] = !tail || (t0 + 8 * lg + i < te);
            nn[i] = valid[i] ? nn[i] * nu : 0.0f;
            ff[i] = valid[i] ? ff[i] * fs : 0.0f;
        }
        // ---- K -> fp16 A operands, S^T = K Q^T
        f32x4 S[RT][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            half8 ka[KS];
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const uint4 v = kr[u][k / 2];
                const uint32_t w0 = (k & 1) ? v.z : v.x;
                const uint32_t w1 = (k & 1) ? v.w : v.y;
                H8 h;
                i8x4_to_h4(w0, h.u[0], h.u[1]);
                i8x4_to_h4(w1, h.u[2], h.u[3]);
                ka[k] = h.h;
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[k], qb[rt][k], s, 0, 0, 0);
                    if constexpr (QSPLIT) s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[k], qlo[rt][k], s, 0, 0, 0);
                }
                S[rt][u] = s;
            }
        }
        // ---- scores (log2 units), lazy online softmax
        float x[RT][8];
        bool need = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float v = S[rt][i >> 2][i & 3] * ff[i];
                v = valid[i] ? v : -INFINITY;
                x[rt][i] = v;
                mx = fmaxf(mx, v);
            }
            need |= mx > m[rt] + kLazy;
            // stash the local max in lsum's neighbour slot via x[rt][*]: recomputed below if needed
        }
        if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 8; ++i) mx = fmaxf(mx, x[rt][i]);
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float mnew = fmaxf(m[rt], mx);
                const float alpha = (m[rt] == -INFINITY) ? 0.0f : exp2f(m[rt] - mnew);
                lsum[rt] *= alpha;
                m[rt] = mnew;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float aj = __shfl(alpha, 4 * lg + j, 64);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[rt][nb][j] *= aj;
                }
            }
        }
        // weights w = p * vn * nu as fp16 hi + lo (w - hi rounded again): ~2^-22 relative
        half8 Wh[RT], Wl[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float mr = (m[rt] == -INFINITY) ? 0.0f : m[rt];
            H8 wh, wl;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const float p0 = exp2f(x[rt][i] - mr);
                const float p1 = exp2f(x[rt][i + 1] - mr);
                lsum[rt] += p0 + p1;
                const float w0 = p0 * nn[i], w1 = p1 * nn[i + 1];
                const half2v hi = {(_Float16)w0, (_Float16)w1};
                const half2v lo = {(_Float16)(w0 - (float)hi[0]), (_Float16)(w1 - (float)hi[1])};
                wh.u[i / 2] = __builtin_bit_cast(uint32_t, hi);
                wl.u[i / 2] = __builtin_bit_cast(uint32_t, lo);
            }
            Wh[rt] = wh.h;
            Wl[rt] = wl.h;
        }
        // ---- acc += W x C  (C decoded per 16-dim column tile from the LUT)
        pv_all<D, RT, BITS>(acc, Wh, Wl, ch, lut, lane_off);
    }

    // ---- combine the 4 wavefronts in LDS (fixed order), write partial records
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        lsum[rt] += __shfl_xor(lsum[rt], 16, 64);
        lsum[rt] += __shfl_xor(lsum[rt], 32, 64);
        if (lg == 0) {
            sm.m[wave][16 * rt + rl] = m[rt];
            sm.l[wave][16 * rt + rl] = lsum[rt];
        }
    }
    __syncthreads();  // also: every wave is done with the LUT
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * rt + 4 * lg + j;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][row]);
            const float mw = sm.m[wave][row];
            const float al = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[rt][nb][j] *= al;
        }
    }
    for (int w = 0; w < kWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float* dst = &sm.accbuf[(16 * rt + 4 * lg + j) * D + NB * rl + nb];
                        *dst = (w == 0) ? acc[rt][nb][j] : *dst + acc[rt][nb][j];
                    }
        }
        __syncthreads();
    }
    const float inv_nu = 1.0f / nu;
    float* rec0 = a.part + P.part_off + (((uint64_t)lj * a.hkv + g) * P.splits + sp) * (uint64_t)R * (2 + D);
    for (int idx = tid; idx < R * D; idx += 256) {
        const int row = idx / D, i = idx % D;
        rec0[(uint64_t)row * (2 + D) + 2 + i] = sm.accbuf[row * D + i] * inv_nu;
    }
    for (int row = tid; row < R; row += 256) {
        float M = -INFINITY;
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][row]);
        float Lr = 0.0f;
        for (int w = 0; w < kWaves; ++w) {
            const float mw = sm.m[w][row];
            Lr += (mw == -INFINITY) ? 0.0f : exp2f(mw - M) * sm.l[w][row];
        }
        rec0[(uint64_t)row * (2 + D)] = M;
        rec0[(uint64_t)row * (2 + D) + 1] = Lr;
    }
}

template <int D, int RT, bool QSPLIT>
__global__ void __launch_bounds__(256) k_pool_mfma(DecodeLaunch a, CentArg cents) {
    __shared__ Smem sm;
    const PoolEntry& P = a.pools[find_pool_m(a, blockIdx.x)];
    int local = blockIdx.x - P.wg_begin;
    local /= P.splits;
    const int l = a.l0 + local / a.hkv;
    switch (layer_bits(P, l)) {
        case 2: pool_mfma_body<D, RT, 2, QSPLIT>(a, cents, sm); break;
        case 3: pool_mfma_body<D, RT, 3, QSPLIT>(a, cents, sm); break;
        default: pool_mfma_body<D, RT, 4, QSPLIT>(a, cents, sm); break;
    }
}

template <int D, bool QSPLIT>
int launch_d(const DecodeLaunch& a, int wg, hipStream_t s, const CentArg& c, int rt) {
    switch (rt) {
        case 1: hipLaunchKernelGGL((k_pool_mfma<D, 1, QSPLIT>), dim3(wg), dim3(256), 0, s, a, c); break;
        case 2: hipLaunchKernelGGL((k_pool_mfma<D, 2, QSPLIT>), dim3(wg), dim3(256), 0, s, a, c); break;
        case 3: hipLaunchKernelGGL((k_pool_mfma<D, 3, QSPLIT>), dim3(wg), dim3(256), 0, s, a, c); break;
        default: hipLaunchKernelGGL((k_pool_mfma<D, 4, QSPLIT>), dim3(wg), dim3(256), 0, s, a, c); break;
    }
    return PKV_OK;
}

}  // namespace

bool mfma_supported(const DecodeLaunch& a) {
    for (int p = 0; p < a.n_pools; ++p)
        if (a.pools[p].rows > 64) return false;
    return true;
}

int launch_pool_mfma(const DecodeLaunch& a, int total_wg, hipStream_t s) {
    if (!mfma_supported(a)) return PKV_EUNSUPPORTED;
    int rows = 1;
    for (int p = 0; p < a.n_pools; ++p) rows = rows > a.pools[p].rows ? rows : a.pools[p].rows;
    const int rt = (rows + 15) / 16;
    CentArg c;
    std::memcpy(c.c, codebook_tables().cent, sizeof(c.c));
    const bool split = a.q_dtype == PKV_F32;
    if (a.d == 128) return split ? launch_d<128, true>(a, total_wg, s, c, rt) : launch_d<128, false>(a, total_wg, s, c, rt);
    return split ? launch_d<64, true>(a, total_wg, s, c, rt) : launch_d<64, false>(a, total_wg, s, c, rt);
}

}  // namespace pkv
