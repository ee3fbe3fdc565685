// Native-window (suffix) attention for bf16 queries and a bf16 window, one wavefront per
// (launch agent, layer, kv head): the device code shared by the suffix kernel (pkv_decode.hip)
// and the split-record form of the matrix-core pool kernel, whose launch can carry the suffix
// work as extra workgroups (pkv_decode_mfma.h).
#pragma once

#include "pkv_decode.h"
#include "pkv_lanes.h"

namespace pkv {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Native suffix attention for bf16 queries and a bf16 suffix, one wavefront per
// (launch agent, layer, kv head), RS q heads per pass.  Per chunk of up to
// kSfxChunk tokens, two sweeps over groups of 64 tokens, each group's loads all
// issued before any is used:
//  1. scores: LPT lanes share a token, each holding D/LPT of its dimensions and
//     the pass's matching query slices in registers (bf16 pairs, dot2: exact
//     products, fp32 sums); a reduce-scatter across those lanes leaves each lane
//     RS/LPT rows, whose scores (log2 units) go to LDS;
//  2. values: p = 2^(s - m) replaces each score in LDS, then each lane, owning 8
//     dimensions of every 64/(D/8)-th token, accumulates p * v; a reduce-scatter
//     across the token lanes finishes the sums.
// The softmax reference moves only between chunks (accumulators rescaled once
// per chunk).
constexpr int kSfxChunk = 256;
constexpr int kSfxGroup = 64;

// Reduce-scatter step over the lane pairs that differ in bit M: on entry v[0, N)
// are per-lane values; on exit v[0, N/2) hold the pair's sums of v[0, N/2) on the
// lane with that bit clear and of v[N/2, N) on the other.
template <int M, int N>
__device__ __forceinline__ void scatter_add(float* v, bool hi) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const float send = hi ? v[i] : v[i + N / 2];
        const float keep = hi ? v[i + N / 2] : v[i];
        v[i] = keep + lane_xor<M>(send);
    }
}

template <int M, int N>
__device__ __forceinline__ void all_add(float* v) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += lane_xor<M>(v[i]);
}

// 16 bytes at base + off (base wave-uniform, off a per-lane byte offset)
__device__ __forceinline__ uint4 ld16(const void* base, uint32_t off) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(base) + off);
}

// The same for the window's keys and values, which a call reads once: a non-temporal load, so
// that streaming them does not push the shared pool, which every call reads again, out of the
// last-level cache
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* base, uint32_t off) {
    const u32x4_t v =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(static_cast<const uint8_t*>(base) + off));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int D, int RS, bool PF>
__device__ void sfx_fast_wave(const DecodeLaunch& a, int unit, float* sbuf) {
    // score sweep: LPT lanes per token, each reading KL 16-byte chunks of it (and holding the
    // matching query slices: RS * KL * 4 registers)
    constexpr int LPT = (RS * D / 64) > 2 ? RS * D / 64 : 2;
    constexpr int TPP = 64 / LPT;           // tokens per load instruction
    constexpr int KL = D / 8 / LPT;         // 16-byte chunks per lane per token
    constexpr int KG = TPP > (RS >= 4 ? 16 : 32) ? TPP : (RS >= 4 ? 16 : 32);  // tokens per score group
    constexpr int KU = KG / TPP;            // load instructions per chunk index per group
    constexpr int RPL = RS / LPT > 1 ? RS / LPT : 1;  // rows per lane after the reduction
    constexpr int LB = LPT == 2 ? 1 : LPT == 4 ? 2 : LPT == 8 ? 3 : 4;      // log2 LPT
    constexpr int LS = RS / RPL == 1 ? 0 : RS / RPL == 2 ? 1 : RS / RPL == 4 ? 2 : 3;  // scatter steps
    // value sweep: LV lanes per token, 8 dimensions each
    constexpr int LV = D / 8;
    constexpr int TV = 64 / LV;             // tokens per load instruction
    constexpr int VG = RS >= 4 ? 16 : 32;   // tokens per value group (bounds the probabilities held)
    constexpr int VU = VG / TV;             // load instructions per group
    constexpr int TB = TV == 4 ? 2 : 3;     // log2 TV
    static_assert(KL >= 1 && LPT <= 16 && (1 << LS) * RPL == RS && (TV == 4 || TV == 8), "suffix tiling");

    const int lane = threadIdx.x & 63;
    const int g = unit % a.hkv;
    const int lj = (unit / a.hkv) % a.lc;
    const int k = unit / (a.hkv * a.lc);
    const int agent = a.agent_id[k];
    const int S = a.sfx_len[k];
    const uint64_t tok0 = (((uint64_t)agent * a.lc + lj) * a.hkv + g) * (uint64_t)a.sfx_cap;
    const uint16_t* K = static_cast<const uint16_t*>(a.sfx_k) + tok0 * D;
    const uint16_t* V = static_cast<const uint16_t*>(a.sfx_v) + tok0 * D;

    const int part = lane % LPT;  // score sweep: chunks part, part + LPT, ... of token lane / LPT
    const int tl = lane / LPT;
    int rb = 0;                   // first row this lane keeps after the reduce-scatter
    if constexpr (LS >= 1) rb += (lane & 1) * (RS / 2);
    if constexpr (LS >= 2) rb += ((lane >> 1) & 1) * (RS / 4);
    if constexpr (LS >= 3) rb += ((lane >> 2) & 1) * (RS / 8);
    // the lane bits past the scatter steps are summed over: one lane of each copy writes
    const bool swriter = ((lane & (LPT - 1)) >> LS) == 0;
    const int dv = lane % LV;     // value sweep: dimensions 8 dv .. 8 dv + 7 of token lane / LV
    const int tv = lane / LV;

    for (int r0 = 0; r0 < a.G; r0 += RS) {
        const int nr = min(RS, a.G - r0);
        float M[RS], Lp[RS], acc[RS * 8];
#pragma unroll
        for (int r = 0; r < RS; ++r) {
            M[r] = -INFINITY;
            Lp[r] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < RS * 8; ++i) acc[i] = 0.0f;

        for (int c0 = 0; c0 < S; c0 += kSfxChunk) {
            const int nc = min(kSfxChunk, S - c0);
            const uint16_t* Kc = K + (uint64_t)c0 * D;
            const uint16_t* Vc = V + (uint64_t)c0 * D;
            // the pass's query slices, reloaded per chunk so that they are not held through the value sweep
            uint32_t qv[RS][KL * 4];
            uint32_t zero;
            asm volatile("v_mov_b32 %0, 0" : "=v"(zero));  // keeps the reload inside the chunk loop
#pragma unroll
            for (int r = 0; r < RS; ++r) {
                const int rr = min(r0 + r, a.G - 1);  // rows past G repeat the last one and are not stored
                const uint16_t* qrow =
                    static_cast<const uint16_t*>(a.q) + (((uint64_t)agent * a.lc + lj) * a.hq + g * a.G + rr) * D;
#pragma unroll
                for (int c = 0; c < KL; ++c) {
                    const uint4 w = ld16(qrow, zero + (uint32_t)(c * LPT + part) * 16);
                    qv[r][4 * c] = w.x;
                    qv[r][4 * c + 1] = w.y;
                    qv[r][4 * c + 2] = w.z;
                    qv[r][4 * c + 3] = w.w;
                }
            }
            // ---- 1. scores
            float mloc[RPL];
#pragma unroll
            for (int i = 0; i < RPL; ++i) mloc[i] = -INFINITY;
            // PF: each group's K loads are issued one group ahead (the next group's while this one
            // is scored), so a wave waits for one load latency per chunk, not one per group (for
            // launches too small to hide the latency with other waves; it costs registers)
            uint4 kn[KU][KL];
            auto load_k = [&](uint4 (&dst)[KU][KL], int gs) {
#pragma unroll
                for (int u = 0; u < KU; ++u) {
                    const int t = min(gs + u * TPP + tl, nc - 1);  // past the chunk: a valid token, score dropped
                    const uint32_t off = (uint32_t)t * (D * 2) + (uint32_t)part * 16;
#pragma unroll
                    for (int c = 0; c < KL; ++c) dst[u][c] = ld16_stream(Kc, off + c * LPT * 16);
                }
            };
            if constexpr (PF) load_k(kn, 0);
            for (int g0 = 0; g0 < nc; g0 += KG) {
                uint4 kk[KU][KL];
                if constexpr (PF) {
#pragma unroll
                    for (int u = 0; u < KU; ++u)
#pragma unroll
                        for (int c = 0; c < KL; ++c) kk[u][c] = kn[u][c];
                    load_k(kn, g0 + KG);
                } else {
                    load_k(kk, g0);
                }
#pragma unroll
                for (int u = 0; u < KU; ++u) {
                    const int t = g0 + u * TPP + tl;
                    float sc[RS];
#pragma unroll
                    for (int r = 0; r < RS; ++r) sc[r] = 0.0f;
#pragma unroll
                    for (int c = 0; c < KL; ++c) {
                        const uint32_t kw[4] = {kk[u][c].x, kk[u][c].y, kk[u][c].z, kk[u][c].w};
#pragma unroll
                        for (int r = 0; r < RS; ++r)
#pragma unroll
                            for (int w = 0; w < 4; ++w)
                                sc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kw[w]),
                                                                        __builtin_bit_cast(bf16x2_t, qv[r][4 * c + w]),
                                                                        sc[r], false);
                    }
                    // over lane bits 0 .. LB-1: scatter the rows while more than one is left, then sum
                    auto red = [&](auto bt) {
                        constexpr int b = decltype(bt)::value;
                        if constexpr (b < LS) scatter_add<(1 << b), (RS >> b)>(sc, lane & (1 << b));
                        else if constexpr (b < LB) all_add<(1 << b), RPL>(sc);
                    };
                    red(std::integral_constant<int, 0>{});
                    red(std::integral_constant<int, 1>{});
                    red(std::integral_constant<int, 2>{});
                    red(std::integral_constant<int, 3>{});
                    const bool ok = t < nc;
#pragma unroll
                    for (int i = 0; i < RPL; ++i) {
                        const float x = sc[i] * a.sm_log2;
                        if (ok) {
                            mloc[i] = fmaxf(mloc[i], x);
                            if (swriter) sbuf[t * RS + rb + i] = x;
                        }
                    }
                }
            }
            // chunk row maxima: over the token lanes, then each row read from a lane holding it
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
#pragma unroll
                for (int off = LPT; off < 64; off <<= 1) mloc[i] = fmaxf(mloc[i], __shfl_xor(mloc[i], off, 64));
            }
#pragma unroll
            for (int r = 0; r < RS; ++r) {
                // rows [rb, rb + RPL) sit on the lanes whose low LS bits, reversed, give rb / RPL
                const int q = r / RPL;
                int src = 0;
#pragma unroll
                for (int b = 0; b < LS; ++b) src |= ((q >> (LS - 1 - b)) & 1) << b;
                const float mc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mloc[r % RPL]), src));
                const float mn = fmaxf(M[r], mc);
                const float alpha = (M[r] == -INFINITY) ? 0.0f : exp2f(M[r] - mn);
                M[r] = mn;
                Lp[r] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r * 8 + e] *= alpha;
            }
            __builtin_amdgcn_wave_barrier();
            // PF: the first value group's loads (they do not depend on the scores)
            uint4 vn[VU];
            auto load_v = [&](uint4 (&dst)[VU], int gs) {
#pragma unroll
                for (int u = 0; u < VU; ++u) {
                    const int t = min(gs + u * TV + tv, nc - 1);  // past the chunk: a valid token, weight 0
                    dst[u] = ld16_stream(Vc, (uint32_t)t * (D * 2) + (uint32_t)dv * 16);
                }
            };
            if constexpr (PF) load_v(vn, 0);
            // ---- probabilities in place, per-lane partial sums
            for (int t = lane; t < nc; t += 64) {
#pragma unroll
                for (int r = 0; r < RS; ++r) {
                    const float p = exp2f(sbuf[t * RS + r] - M[r]);
                    sbuf[t * RS + r] = p;
                    Lp[r] += p;
                }
            }
            __builtin_amdgcn_wave_barrier();
            // ---- 2. values (PF: loads one group ahead, as the keys)
            for (int g0 = 0; g0 < nc; g0 += VG) {
                uint4 vv[VU];
                if constexpr (PF) {
#pragma unroll
                    for (int u = 0; u < VU; ++u) vv[u] = vn[u];
                    load_v(vn, g0 + VG);
                } else {
                    load_v(vv, g0);
                }
#pragma unroll
                for (int u = 0; u < VU; ++u) {
                    const int t = g0 + u * TV + tv;
                    const bool ok = t < nc;
                    float pr[RS];
                    if constexpr (RS >= 4) {
#pragma unroll
                        for (int r4 = 0; r4 < RS; r4 += 4) {
                            const float4 p4 = *reinterpret_cast<const float4*>(&sbuf[t * RS + r4]);
                            pr[r4] = p4.x;
                            pr[r4 + 1] = p4.y;
                            pr[r4 + 2] = p4.z;
                            pr[r4 + 3] = p4.w;
                        }
                    } else if constexpr (RS == 2) {
                        const float2 p2 = *reinterpret_cast<const float2*>(&sbuf[t * 2]);
                        pr[0] = p2.x;
                        pr[1] = p2.y;
                    } else {
                        pr[0] = sbuf[t];
                    }
#pragma unroll
                    for (int r = 0; r < RS; ++r) pr[r] = ok ? pr[r] : 0.0f;
                    const float v[8] = {bf16_lo(vv[u].x), bf16_hi(vv[u].x), bf16_lo(vv[u].y), bf16_hi(vv[u].y),
                                        bf16_lo(vv[u].z), bf16_hi(vv[u].z), bf16_lo(vv[u].w), bf16_hi(vv[u].w)};
#pragma unroll
                    for (int r = 0; r < RS; ++r)
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[r * 8 + e] = fmaf(pr[r], v[e], acc[r * 8 + e]);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        // ---- records: l over all lanes; acc over the token lanes, rows scattered
#pragma unroll
        for (int r = 0; r < RS; ++r) {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) Lp[r] += __shfl_xor(Lp[r], off, 64);
        }
        // steps over lane bits LV, 2 LV, ...: scatter rows while more than one is left
        constexpr int N1 = RS >= 2 ? RS / 2 : 1, N2 = RS >= 4 ? RS / 4 : 1, N3 = RS >= 8 ? RS / 8 : 1;
        int rv = 0;          // first row this lane holds afterwards
        bool writer = true;  // one lane per copy
        if constexpr (RS >= 2) { scatter_add<LV, RS * 8>(acc, lane & LV); rv += ((lane >> (6 - TB)) & 1) * (RS / 2); }
        else { all_add<LV, 8>(acc); writer = writer && !(lane & LV); }
        if constexpr (RS >= 4) { scatter_add<2 * LV, N1 * 8>(acc, lane & (2 * LV)); rv += ((lane >> (7 - TB)) & 1) * (RS / 4); }
        else { all_add<2 * LV, N1 * 8>(acc); writer = writer && !(lane & (2 * LV)); }
        if constexpr (TB == 3) {
            if constexpr (RS >= 8) { scatter_add<4 * LV, N2 * 8>(acc, lane & (4 * LV)); rv += ((lane >> 5) & 1) * (RS / 8); }
            else { all_add<4 * LV, N2 * 8>(acc); writer = writer && !(lane & (4 * LV)); }
        }
        constexpr int NF = TB == 3 ? N3 : N2;  // rows per lane at the end
        if (writer) {
#pragma unroll
            for (int i = 0; i < NF; ++i) {
                const int r = rv + i;
                if (r < nr) {
                    float* rec = a.part + a.sfx_part_off + (((uint64_t)k * a.lc + lj) * a.hq + g * a.G + r0 + r) * (2 + D);
#pragma unroll
                    for (int e = 0; e < 8; ++e) rec[2 + 8 * dv + e] = acc[i * 8 + e];
                }
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < RS; ++r) {
                if (r < nr) {
                    float* rec = a.part + a.sfx_part_off + (((uint64_t)k * a.lc + lj) * a.hq + g * a.G + r0 + r) * (2 + D);
                    rec[0] = M[r];
                    rec[1] = Lp[r];
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace
}  // namespace pkv
