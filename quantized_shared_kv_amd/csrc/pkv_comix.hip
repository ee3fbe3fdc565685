// CoMixKV controller: per-(agent, layer) sensitivity from recent queries and the
// native window, and joint 2/3/4-bit allocation under a byte budget.
//
// CoMixKV news article, abstract and method paragraphs: the controller builds
// a local attention-error bound from the recently seen queries, keys and
// values (no calibration data, no trial quantisation, no extra forward pass)
// and allocates 2 to 4 bits jointly over every resident agent and layer under
// one memory budget, with the real byte costs; new widths apply only to blocks
// quantised afterwards.
//
// Bound used here: with local attention p_t = softmax_t(sigma q . k_t) over the
// agent's native window and a V codec whose relative squared error has mean D_b
// (the Lloyd-Max distortion of N(0, 1)), ||sum_t p_t (v_t - v_hat_t)|| <=
// sum_t p_t ||v_t - v_hat_t||, whose mean is at most sqrt(D_b) sum_t p_t ||v_t||.
// The sensitivity of (agent, layer) is sum_t p_t ||v_t|| averaged over the
// agent's recent query rows (steps x query heads).
//
// k_comix_sens (fp32 operands; bf16 ones take k_comix_mfma, below): one workgroup
// of 4 wavefronts per (agent, layer); wavefront w
// takes kv heads w, w + 4, ...; for each, up to 32 query rows at a time are
// staged in LDS (fp32) and the window is swept 32 tokens at a time, two lanes
// per token: lane half h holds the 16-byte chunks 2i + h of its token's key row
// (fp32) and its ||v||, reads the same chunks of each query row from LDS (32
// lanes per address: a broadcast, the two halves on different banks), and one
// lane exchange completes the score; every lane keeps an online (max, sum p,
// sum p ||v||) per row over the tokens it has seen, and the 32 token slots'
// states are merged at the end.  Row values are summed in a fixed order,
// then the 4 wavefronts' sums in LDS, so the result is deterministic.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "pkv_internal.h"
#include "pkv_lanes.h"

namespace pkv {
namespace {

constexpr int kComixAgents = 256;  // agents per launch (their window lengths travel in the arguments)
constexpr int kComixRows = 32;     // query rows staged per pass

struct ComixLaunch {
    const void* q;
    const void* win_k;
    const void* win_v;
    float* out;
    int q_bf16, win_bf16;
    int n_agents, agent0, n_agents_total, lc, hq, hkv, G, cap, n_recent;
    float sm_log2;
    float inv_rows;
    int32_t len[kComixAgents];
};

__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// the 16-byte chunks 2i + h (i < D / 8) of row `t` of `base` (bf16 or fp32) as floats:
// x[4 i .. 4 i + 3] = elements 4 (2 i + h) .. 4 (2 i + h) + 3
template <int D>
__device__ __forceinline__ void load_half_row(const void* base, uint64_t t, int h, bool bf16, float (&x)[D / 2]) {
    if (bf16) {
        const uint2* p = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + t * D);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            const uint2 w = p[2 * i + h];
            x[4 * i] = __uint_as_float(w.x << 16);
            x[4 * i + 1] = __uint_as_float(w.x & 0xffff0000u);
            x[4 * i + 2] = __uint_as_float(w.y << 16);
            x[4 * i + 3] = __uint_as_float(w.y & 0xffff0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + t * D);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            const float4 f = p[2 * i + h];
            x[4 * i] = f.x;
            x[4 * i + 1] = f.y;
            x[4 * i + 2] = f.z;
            x[4 * i + 3] = f.w;
        }
    }
}

// (m, l, u) of one row: l = sum 2^(s - m), u = sum 2^(s - m) * ||v||; m = -inf: empty
__device__ __forceinline__ void merge_state(float& m, float& l, float& u, float m2, float l2, float u2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    const float a1 = exp2f(m - M), a2 = exp2f(m2 - M);  // exp2(-inf) = 0 for an empty side
    l = l * a1 + l2 * a2;
    u = u * a1 + u2 * a2;
    m = M;
}

template <int M>
__device__ __forceinline__ void merge_lanes(float& m, float& l, float& u) {
    const float m2 = lane_xor<M>(m), l2 = lane_xor<M>(l), u2 = lane_xor<M>(u);
    merge_state(m, l, u, m2, l2, u2);
}

template <int D>
__global__ void __launch_bounds__(256) k_comix_sens(ComixLaunch a) {
    __shared__ __align__(16) float qs[4][kComixRows][D];
    __shared__ float wsum[4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kl = blockIdx.x / a.lc;  // agent within the launch
    const int lj = blockIdx.x % a.lc;
    const int k = a.agent0 + kl;
    const int n = a.len[kl];
    const int NR = a.n_recent * a.G;

    float total = 0.0f;  // this wavefront's sum of row values, fixed order
    if (n > 0) {
        for (int g = wave; g < a.hkv; g += 4) {
            const uint64_t wrow = (((uint64_t)k * a.lc + lj) * a.hkv + g) * (uint64_t)a.cap;
            for (int rc = 0; rc < NR; rc += kComixRows) {
                const int nrc = min(kComixRows, NR - rc);
                // stage rows rc .. rc + nrc - 1 of this kv head: row j -> (step j / G, head g G + j % G)
                for (int e = lane; e < nrc * D; e += 64) {
                    const int j = rc + e / D, i = e % D;
                    const int r = j / a.G, h = g * a.G + j % a.G;
                    const uint64_t qo = ((((uint64_t)r * a.n_agents_total + k) * a.lc + lj) * a.hq + h) * D + i;
                    qs[wave][e / D][i] = a.q_bf16 ? bf16_to_f(static_cast<const uint16_t*>(a.q)[qo])
                                                  : static_cast<const float*>(a.q)[qo];
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

                float m[kComixRows], l[kComixRows], u[kComixRows];
#pragma unroll
                for (int j = 0; j < kComixRows; ++j) {
                    m[j] = -INFINITY;
                    l[j] = 0.0f;
                    u[j] = 0.0f;
                }
                const int hf = lane & 1, slot = lane >> 1;
                for (int t0 = 0; t0 < n; t0 += 32) {
                    const int t = t0 + slot;
                    const bool ok = t < n;
                    const uint64_t tt = wrow + (uint64_t)min(t, n - 1);  // past the window: a valid row, unused
                    float vn;
                    {
                        float vx[D / 2];
                        load_half_row<D>(a.win_v, tt, hf, a.win_bf16, vx);
                        float vv = 0.0f;
#pragma unroll
                        for (int i = 0; i < D / 2; ++i) vv = fmaf(vx[i], vx[i], vv);
                        vn = sqrtf(vv + lane_xor<1>(vv));
                    }
                    asm volatile("" ::: "memory");  // the value half-row is dead before the key half-row loads
                    float kx[D / 2];
                    load_half_row<D>(a.win_k, tt, hf, a.win_bf16, kx);
#pragma unroll
                    for (int j = 0; j < kComixRows; ++j) {
                        if (j < nrc) {
                            const float4* qr = reinterpret_cast<const float4*>(&qs[wave][j][0]);
                            float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
                            for (int i = 0; i < D / 8; i += 2) {
                                const float4 q0 = qr[2 * i + hf], q1 = qr[2 * i + 2 + hf];
                                s0 = fmaf(kx[4 * i], q0.x, s0);
                                s0 = fmaf(kx[4 * i + 1], q0.y, s0);
                                s0 = fmaf(kx[4 * i + 2], q0.z, s0);
                                s0 = fmaf(kx[4 * i + 3], q0.w, s0);
                                s1 = fmaf(kx[4 * i + 4], q1.x, s1);
                                s1 = fmaf(kx[4 * i + 5], q1.y, s1);
                                s1 = fmaf(kx[4 * i + 6], q1.z, s1);
                                s1 = fmaf(kx[4 * i + 7], q1.w, s1);
                            }
                            float s = s0 + s1;
                            s = (s + lane_xor<1>(s)) * a.sm_log2;
                            if (ok) {
                                const float mn = fmaxf(m[j], s);
                                const float al = exp2f(m[j] - mn), e = exp2f(s - mn);
                                l[j] = l[j] * al + e;
                                u[j] = u[j] * al + e * vn;
                                m[j] = mn;
                            }
                        }
                    }
                }
                // merge the 32 token slots' states (both lanes of a slot hold the same), then sum
                // the rows in order
#pragma unroll
                for (int j = 0; j < kComixRows; ++j) {
                    if (j < nrc) {
                        merge_lanes<2>(m[j], l[j], u[j]);
                        merge_lanes<4>(m[j], l[j], u[j]);
                        merge_lanes<8>(m[j], l[j], u[j]);
                        merge_lanes<16>(m[j], l[j], u[j]);
                        merge_lanes<32>(m[j], l[j], u[j]);
                        total += l[j] > 0.0f ? u[j] / l[j] : 0.0f;
                    }
                }
                // the next pass overwrites this wavefront's rows (LDS operations of a wavefront
                // complete in order; the fences keep the compiler from moving them)
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
    }
    if (lane == 0) wsum[wave] = total;
    __syncthreads();
    if (threadIdx.x == 0)
        a.out[(uint64_t)k * a.lc + lj] = n > 0 ? ((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) * a.inv_rows : 0.0f;
}

// k_comix_mfma: the same sums for bf16 queries and a bf16 window, with the scores on the matrix
// cores (v_mfma_f32_16x16x32_bf16: bf16 products are exact in fp32 and summed in fp32, as the
// vector kernel's fma chain does, in another order).  One workgroup per (agent, layer);
// wavefront w takes kv heads w, w + 4, ...; per kv head up to 64 query rows (4 tiles of 16) at a
// time are held as A operands, and the window is swept 16 tokens at a time: lane (kg, c) loads
// the B operands of token c of the tile (dimensions 32 s + 8 kg .. + 7 of every k-step s) and a
// quarter of its value row for ||v||, the next tile's loads in flight while the current one is
// used.  The lane keeps an online (max, sum p, sum p ||v||) of rows 4 kg + j of each tile over
// its tokens; the 16 token lanes' states are merged at the end and the rows summed in a fixed
// order, so the result is deterministic.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D>
__global__ void __launch_bounds__(256) k_comix_mfma(ComixLaunch a) {
    constexpr int KS = D / 32;  // k-steps of the scores
    constexpr int RTM = 4;      // row tiles of 16 per pass over the window
    constexpr int VQ = D / 4;   // value dimensions per lane (a quarter of the row)
    __shared__ float wsum[4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kl = blockIdx.x / a.lc;  // agent within the launch
    const int lj = blockIdx.x % a.lc;
    const int k = a.agent0 + kl;
    const int n = a.len[kl];
    const int NR = a.n_recent * a.G;
    const int c = lane & 15, kg = lane >> 4;
    const uint16_t* q16 = static_cast<const uint16_t*>(a.q);

    float total = 0.0f;  // this wavefront's sum of row values, fixed order
    if (n > 0) {
        for (int g = wave; g < a.hkv; g += 4) {
            const uint64_t wrow = (((uint64_t)k * a.lc + lj) * a.hkv + g) * (uint64_t)a.cap;
            const uint16_t* wk = static_cast<const uint16_t*>(a.win_k) + wrow * D;
            const uint16_t* wv = static_cast<const uint16_t*>(a.win_v) + wrow * D;
            for (int r0 = 0; r0 < NR; r0 += 16 * RTM) {
                // A operands: row r0 + 16 rt + c (step row / G, q head g G + row % G)
                bf16x8_t qa[RTM][KS];
#pragma unroll
                for (int rt = 0; rt < RTM; ++rt) {
                    const int row = r0 + 16 * rt + c;
                    const int rs = row / a.G, h = g * a.G + row % a.G;
                    const uint64_t qo = ((((uint64_t)rs * a.n_agents_total + k) * a.lc + lj) * a.hq + h) * D + 8 * kg;
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const uint4 v = row < NR ? *reinterpret_cast<const uint4*>(q16 + qo + 32 * s) : make_uint4(0, 0, 0, 0);
                        qa[rt][s] = __builtin_bit_cast(bf16x8_t, v);
                    }
                }
                float m[RTM][4], l[RTM][4], u[RTM][4];
#pragma unroll
                for (int rt = 0; rt < RTM; ++rt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        m[rt][j] = -INFINITY;
                        l[rt][j] = 0.0f;
                        u[rt][j] = 0.0f;
                    }
                auto load_tile = [&](int t0, uint4 (&kb)[KS], uint4 (&vb)[VQ / 8]) {
                    const uint64_t t = (uint64_t)min(t0 + c, n - 1);  // past the window: a valid row, unused
#pragma unroll
                    for (int s = 0; s < KS; ++s) kb[s] = *reinterpret_cast<const uint4*>(wk + t * D + 32 * s + 8 * kg);
#pragma unroll
                    for (int i = 0; i < VQ / 8; ++i) vb[i] = *reinterpret_cast<const uint4*>(wv + t * D + VQ * kg + 8 * i);
                };
                uint4 kb[KS], vb[VQ / 8];
                load_tile(0, kb, vb);
                for (int t0 = 0; t0 < n; t0 += 16) {
                    uint4 kn[KS], vnx[VQ / 8];
                    const bool more = t0 + 16 < n;
                    if (more) load_tile(t0 + 16, kn, vnx);
                    // ||v|| of token t0 + c: this lane's quarter of the row, then the four quarters
                    float vv = 0.0f;
#pragma unroll
                    for (int i = 0; i < VQ / 8; ++i) {
                        const uint32_t w4[4] = {vb[i].x, vb[i].y, vb[i].z, vb[i].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float lo = __uint_as_float(w4[e] << 16), hi = __uint_as_float(w4[e] & 0xffff0000u);
                            vv = fmaf(lo, lo, vv);
                            vv = fmaf(hi, hi, vv);
                        }
                    }
                    vv += lane_xor<16>(vv);
                    vv += lane_xor<32>(vv);
                    const float vn = sqrtf(vv);
                    const bool ok = t0 + c < n;
#pragma unroll
                    for (int rt = 0; rt < RTM; ++rt) {
                        if (r0 + 16 * rt >= NR) break;  // wave-uniform
                        f32x4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int s = 0; s < KS; ++s)
                            S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rt][s], __builtin_bit_cast(bf16x8_t, kb[s]), S, 0, 0, 0);
                        if (ok) {
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const float sc = S[j] * a.sm_log2;
                                const float mn = fmaxf(m[rt][j], sc);
                                const float al = exp2f(m[rt][j] - mn), e = exp2f(sc - mn);
                                l[rt][j] = l[rt][j] * al + e;
                                u[rt][j] = u[rt][j] * al + e * vn;
                                m[rt][j] = mn;
                            }
                        }
                    }
                    if (more) {
#pragma unroll
                        for (int s = 0; s < KS; ++s) kb[s] = kn[s];
#pragma unroll
                        for (int i = 0; i < VQ / 8; ++i) vb[i] = vnx[i];
                    }
                }
                // merge the 16 token lanes' states of each row, then sum this lane group's rows
                // (4 kg + j of each tile) in order and the four groups in a fixed tree
                float part = 0.0f;
#pragma unroll
                for (int rt = 0; rt < RTM; ++rt) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        merge_lanes<1>(m[rt][j], l[rt][j], u[rt][j]);
                        merge_lanes<2>(m[rt][j], l[rt][j], u[rt][j]);
                        merge_lanes<4>(m[rt][j], l[rt][j], u[rt][j]);
                        merge_lanes<8>(m[rt][j], l[rt][j], u[rt][j]);
                        const int row = r0 + 16 * rt + 4 * kg + j;
                        if (row < NR) part += l[rt][j] > 0.0f ? u[rt][j] / l[rt][j] : 0.0f;
                    }
                }
                part += lane_xor<16>(part);
                part += lane_xor<32>(part);
                total += part;
            }
        }
    }
    if (lane == 0) wsum[wave] = total;
    __syncthreads();
    if (threadIdx.x == 0)
        a.out[(uint64_t)k * a.lc + lj] = n > 0 ? ((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) * a.inv_rows : 0.0f;
}

}  // namespace
}  // namespace pkv

extern "C" {

int comix_sensitivity(const pkv_comix_args* x, void* stream) {
    using namespace pkv;
    if (!x) return PKV_EINVAL;
    if (x->n_agents < 0 || x->layer_count < 0 || x->n_kv_heads < 1 || x->n_q_heads < 1 || x->n_recent < 1)
        return PKV_EINVAL;
    if (x->n_q_heads % x->n_kv_heads) return PKV_EINVAL;
    if (x->head_dim != 64 && x->head_dim != 128) return PKV_EUNSUPPORTED;
    if ((x->q_dtype != PKV_F32 && x->q_dtype != PKV_BF16) || (x->win_dtype != PKV_F32 && x->win_dtype != PKV_BF16))
        return PKV_EUNSUPPORTED;
    if (!(x->softmax_scale >= 0.0f) || std::isinf(x->softmax_scale)) return PKV_EINVAL;
    if (x->n_agents == 0 || x->layer_count == 0) return PKV_OK;
    if (!x->q || !x->out || !x->win_len || x->win_cap < 0) return PKV_EINVAL;
    bool any = false;
    for (int a = 0; a < x->n_agents; ++a) {
        if (x->win_len[a] < 0 || x->win_len[a] > x->win_cap) return PKV_EINVAL;
        any |= x->win_len[a] > 0;
    }
    if (any && (!x->win_k || !x->win_v)) return PKV_EINVAL;
    // window rows are read in 16-byte pieces
    const uintptr_t mask = 15u;
    if ((reinterpret_cast<uintptr_t>(x->win_k) & mask) || (reinterpret_cast<uintptr_t>(x->win_v) & mask) ||
        (reinterpret_cast<uintptr_t>(x->out) & 3u))
        return PKV_EINVAL;
    ComixLaunch L;
    std::memset(&L, 0, sizeof(L));
    L.q = x->q;
    L.win_k = x->win_k;
    L.win_v = x->win_v;
    L.out = x->out;
    L.q_bf16 = x->q_dtype == PKV_BF16;
    L.win_bf16 = x->win_dtype == PKV_BF16;
    L.n_agents_total = x->n_agents;
    L.lc = x->layer_count;
    L.hq = x->n_q_heads;
    L.hkv = x->n_kv_heads;
    L.G = x->n_q_heads / x->n_kv_heads;
    L.cap = x->win_cap;
    L.n_recent = x->n_recent;
    const float sigma = x->softmax_scale > 0.0f ? x->softmax_scale : 1.0f / std::sqrt((float)x->head_dim);
    L.sm_log2 = sigma * 1.4426950408889634f;
    L.inv_rows = 1.0f / ((float)x->n_recent * (float)x->n_q_heads);
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int a0 = 0; a0 < x->n_agents; a0 += kComixAgents) {
        L.agent0 = a0;
        L.n_agents = std::min(kComixAgents, x->n_agents - a0);
        for (int i = 0; i < L.n_agents; ++i) L.len[i] = x->win_len[a0 + i];
        const dim3 grid((unsigned)(L.n_agents * L.lc));
        // bf16 operands: scores on the matrix cores; fp32 ones: the vector kernel
        const bool mfma = L.q_bf16 && L.win_bf16;
        if (x->head_dim == 128) {
            if (mfma) hipLaunchKernelGGL(k_comix_mfma<128>, grid, dim3(256), 0, s, L);
            else hipLaunchKernelGGL(k_comix_sens<128>, grid, dim3(256), 0, s, L);
        } else {
            if (mfma) hipLaunchKernelGGL(k_comix_mfma<64>, grid, dim3(256), 0, s, L);
            else hipLaunchKernelGGL(k_comix_sens<64>, grid, dim3(256), 0, s, L);
        }
    }
    return launch_status();
}

int comix_allocate_bits(int32_t n_items, const float* sensitivity, const uint64_t* cost, const double* error_factor,
                        uint64_t budget, uint8_t* bits) {
    if (n_items < 0) return PKV_EINVAL;
    if (n_items == 0) return PKV_OK;
    if (!sensitivity || !cost || !error_factor || !bits) return PKV_EINVAL;
    if (!(error_factor[0] > error_factor[1] && error_factor[1] > error_factor[2] && error_factor[2] >= 0.0) ||
        !std::isfinite(error_factor[0]))
        return PKV_EINVAL;
    uint64_t used = 0;
    for (int i = 0; i < n_items; ++i) {
        const float si = sensitivity[i];
        if (!(si >= 0.0f) || std::isinf(si)) return PKV_EINVAL;
        const uint64_t* c = cost + 3 * (size_t)i;
        if (!(c[0] < c[1] && c[1] < c[2])) return PKV_EINVAL;
        if (used > UINT64_MAX - c[2]) return PKV_EINVAL;  // totals must fit 64 bits
        used += c[0];
    }
    if (used > budget) return PKV_ENOSPACE;
    // repeatedly the upgrade b -> b + 1 with the largest error decrease per added byte (ties:
    // lower index); if it does not fit the remaining budget the item is not upgraded further.
    // A heap of each item's next upgrade, ordered by (ratio, then lower index), makes the same
    // choices as scanning every item each time.
    std::vector<uint8_t> b(n_items, 2);
    auto ratio = [&](int i) {
        const int k = b[i] - 2;
        const uint64_t* c = cost + 3 * (size_t)i;
        const double gain = (double)sensitivity[i] * (error_factor[k] - error_factor[k + 1]);
        return gain / (double)(c[k + 1] - c[k]);
    };
    typedef std::pair<double, int> Cand;
    auto worse = [](const Cand& x, const Cand& y) { return x.first < y.first || (x.first == y.first && x.second > y.second); };
    std::vector<Cand> heap;
    heap.reserve(n_items);
    for (int i = 0; i < n_items; ++i) heap.push_back({ratio(i), i});
    std::make_heap(heap.begin(), heap.end(), worse);
    while (!heap.empty()) {
        std::pop_heap(heap.begin(), heap.end(), worse);
        const int i = heap.back().second;
        heap.pop_back();
        const int k = b[i] - 2;
        const uint64_t dc = cost[3 * (size_t)i + k + 1] - cost[3 * (size_t)i + k];
        if (dc > budget - used) continue;  // stays at b[i]
        used += dc;
        if (++b[i] < 4) {
            heap.push_back({ratio(i), i});
            std::push_heap(heap.begin(), heap.end(), worse);
        }
    }
    std::memcpy(bits, b.data(), (size_t)n_items);
    return PKV_OK;
}

double pkv_lloyd_max_distortion(int32_t bits) {
    if (bits < 2 || bits > 4) return -1.0;
    // E[(X - Q(X))^2] for X ~ N(0, 1) over the fp32 table: on the cell (a, b] with
    // output c, the integral of (x - c)^2 phi(x) dx is
    // (1 + c^2)(Phi(b) - Phi(a)) - (b phi(b) - a phi(a)) + 2 c (phi(b) - phi(a))
    const pkv::CodebookTables& t = pkv::codebook_tables();
    const int n = 1 << bits;
    const double rs2 = 1.0 / std::sqrt(2.0), rs2pi = 1.0 / std::sqrt(2.0 * M_PI);
    auto phi = [&](double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) * rs2pi; };
    auto xphi = [&](double x) { return std::isinf(x) ? 0.0 : x * phi(x); };
    auto Phi = [&](double x) { return 0.5 * std::erfc(-x * rs2); };
    double d = 0.0;
    for (int j = 0; j < n; ++j) {
        const double lo = j == 0 ? -INFINITY : (double)t.thr[bits - 2][j - 1];
        const double hi = j == n - 1 ? INFINITY : (double)t.thr[bits - 2][j];
        const double c = (double)t.cent[bits - 2][j];
        d += (1.0 + c * c) * (Phi(hi) - Phi(lo)) - (xphi(hi) - xphi(lo)) + 2.0 * c * (phi(hi) - phi(lo));
    }
    return d;
}

}  // extern "C"
