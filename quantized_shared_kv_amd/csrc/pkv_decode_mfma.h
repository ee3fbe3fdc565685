// Matrix-core pool decode kernel templates, shared by the two translation units that
// instantiate its fused-finish form (pkv_decode_mfma.hip) and its split-record form
// (pkv_decode_mfma_split.hip), compiled in parallel.
#pragma once

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
// keeps all rows (up to 64, in RT tiles of 16) in its accumulators:
//
//   S^T[32 tok][16 rows] = (Kq as exact fp16) x Q'^T (fp16)          2*RT*(d/32) MFMAs
//   with Q' = Q * 2^-e per row (e > 0 only for rows past the fp16 range; the scores
//   are multiplied back by 2^e)
//   x = S * (Ks[t] * sigma * log2 e) - mref with a fixed per-row reference (see
//   below); w = p * Vn[t] * 2^(7-e) with e from the per-head max norm, so
//   w < 2^15, split into fp16 hi + lo parts
//   acc[16 rows][16 dims] += (Wh + Wl)[16][32 tok] x C[32 tok][16 dims]   2*RT*(d/16) MFMAs
//
// Memory: every wavefront owns a 4-stage ring in LDS filled by gfx950
// direct-to-LDS loads (global_load_lds, 16/12/4 bytes per lane; 12- and 16-byte
// loads place lane l's bytes at lane * 16), three steps ahead of use, so ~70 KB
// per CU are in flight without holding registers.
// The waits are explicit vmcnt counts and the ring is read by inline-asm
// ds_reads (the compiler would otherwise wait for every load before each
// LDS read).  K is fetched lane-owned (each lane's 16-byte pieces are exactly
// what it later reads), so those LDS reads are contiguous across the wave.
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
// 4 wavefronts in LDS in a fixed order (deterministic).  With one split per
// (layer, kv head) the workgroup then finishes the rows itself: one inverse
// FWHT per row, the agent's suffix record folded in, the output written.
// Otherwise it writes partial records for k_merge.
#include <cstring>
#include <type_traits>

#include "pkv_decode.h"
#include "pkv_lanes.h"
#include "pkv_sfx.h"

namespace pkv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kStep = 32;         // tokens per wavefront step
constexpr float kLazy = 8.0f;     // scores may exceed the reference by up to 2^8 (fp16 weights)
constexpr float kMargin = 8.0f;   // reference = first step's row max + this (log2 units)
constexpr int kLutCopies = 32;
constexpr int kWeightExp = 7;     // weights are scaled into [0, 2^15)
// LDS ring per wavefront: kStages slots (kStages - 1 steps in flight) of kStageBytes (K, V codes
// at 4 bits, norms and scales of one 32-token step).  At head_dim 64 a stage is half the size
// and three slots keep a workgroup under half the LDS, so two workgroups share a compute unit
// and one's set-up and finish overlap the other's stream (short pools run many workgroups).
template <int D>
struct Ring {
    static constexpr int kStages = D == 64 ? 3 : 4;
    static constexpr int kStageBytes = 32 * D + 16 * D + 256;
};

// Centroid tables of 2, 3 and 4 bits, each multiplied by its fp16 operand scale s (the LUT
// holds fp16 (s * c), much closer to s * c than fp16 (c) is to c), with ls = log2 s, which the
// weights' exponent takes off (w = p * Vn / s), and lsc = 2^ls, which puts the row sums back.
struct CentArg {
    float c[3][16];
    float ls[3];
    float lsc[3];
};

union H8 {
    half8 h;
    uint32_t u[4];
    uint4 v;
};

// Per-wavefront ring of the upcoming steps, filled by direct-to-LDS loads.
// During the token loop: the per-wavefront rings filled by direct-to-LDS loads and
// the LUT of centroid pairs.  After it: every wavefront's rotated-domain
// accumulator tile [64 rows][D], combined in a fixed order.
constexpr int kMaxRows = 64;
template <int D>
struct LoopLds {
    uint32_t lut[256 * kLutCopies];  // first, so its address has zero low 15 bits
    uint8_t ring[kWaves][Ring<D>::kStages][Ring<D>::kStageBytes];
};
template <int D>
union BigLds {
    LoopLds<D> loop;
    float accs[kWaves * kMaxRows * D];
};
__shared__ __align__(32768) BigLds<128> g_big128;
__shared__ __align__(32768) BigLds<64> g_big64;
template <int D>
__device__ __forceinline__ BigLds<D>& big_lds() {
    if constexpr (D == 128) return g_big128;
    else return g_big64;
}
__shared__ float g_m[kWaves][64];
__shared__ float g_l[kWaves][64];
__shared__ int g_flag;
// head_dim 128, fp16 query operands: each wavefront converts one 16-row tile and shares it
__shared__ uint4 g_qst[kWaves][4][64];
__shared__ float g_qsc[kWaves][16];
__shared__ int g_qany[kWaves];

// Accumulator tiles in LDS: lane x of a 16-lane group owns F floats of a row from F x on, in
// 16-byte slots.  Lanes x and x + 8 fall 128 floats apart, in the same banks, so from lane 8
// on a lane's slots are taken in swapped order (slot e4 at e4 ^ 4 when F = 8): the lanes of
// one access then cover all the banks.  Writers and readers use the same map.
template <int F>
__device__ __forceinline__ int acc_slot(int x, int e4) {
    return e4 ^ (4 * ((x >> 3) & (F / 4 - 1)));
}

// x summed over lanes l, l ^ 16, l ^ 32, l ^ 48 (the wavefront's four 16-lane rows), as
// (x_l + x_(l^16)) + (x_(l^32) + x_(l^48)) in every lane.  The lane index is computed here
// (and hidden from common-subexpression elimination), so no copy of it from the kernel's
// start stays live, or spilled, across the token loop.
__device__ __forceinline__ float sum_lane_rows(float x) {
    int lid;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lid));
    x += __int_as_float(__builtin_amdgcn_ds_bpermute((lid ^ 16) << 2, __float_as_int(x)));
    return x + __int_as_float(__builtin_amdgcn_ds_bpermute((lid ^ 32) << 2, __float_as_int(x)));
}

__device__ __forceinline__ int find_pool_m(const DecodeLaunch& a, int wg) {
    int p = 0;
    while (p + 1 < a.n_pools && wg >= a.pools[p + 1].wg_begin) ++p;
    return p;
}

// The set-up reads the kernel arguments as a chain (the pool's index, then its entry, then
// the rows' fields), and each first touch of a 64-byte argument line waits for memory.  One
// scalar load per line of the launch's scalar fields, pool entry 0 and the centroid table,
// waited for together, puts those lines in the scalar cache (and the L2) first.  The loads
// address the kernel-argument segment directly (DecodeLaunch at offset 0, CentArg after it):
// taking the address of a by-value argument would make the compiler copy it to scratch.
__device__ __forceinline__ void touch_kernel_args() {
    constexpr int kPool = sizeof(PoolEntry) - 4;            // last word of pool entry 0
    constexpr int kS0 = offsetof(DecodeLaunch, q);          // first scalar field
    constexpr int kS1 = offsetof(DecodeLaunch, sm_log2);    // last scalar field
    constexpr int kC0 = (sizeof(DecodeLaunch) + alignof(CentArg) - 1) / alignof(CentArg) * alignof(CentArg);
    constexpr int kC1 = kC0 + sizeof(CentArg) - 4;          // last word of the centroid table
    static_assert(kPool > 128 && kPool < 192 && kS1 - kS0 > 64 && kS1 - kS0 <= 128 && kC1 - kC0 > 192 &&
                      kC1 - kC0 < 256,
                  "the argument lines touched");
    const __attribute__((address_space(4))) uint32_t* k =
        (const __attribute__((address_space(4))) uint32_t*)__builtin_amdgcn_kernarg_segment_ptr();
    constexpr int offs[12] = {0, 64, 128, kPool, kS0, kS0 + 64, kS1, kC0, kC0 + 64, kC0 + 128, kC0 + 192, kC1};
    uint32_t x[12];
#pragma unroll
    for (int i = 0; i < 12; ++i) x[i] = k[offs[i] / 4];
    asm volatile("" ::"s"(x[0]), "s"(x[1]), "s"(x[2]), "s"(x[3]), "s"(x[4]), "s"(x[5]), "s"(x[6]), "s"(x[7]),
                 "s"(x[8]), "s"(x[9]), "s"(x[10]), "s"(x[11]));
}

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    const half2v v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 4 int8 (two's complement) -> 4 fp16 holding k exactly: the bytes u = k + 128 are
// placed in the mantissa of 1024 (fp16 0x6400), giving 1024 + u, and one packed fp16
// subtraction of 1152 leaves u - 128 = k (every step exact: integers below 2048).
// Exact operands keep the MFMA accumulator at the size of q . k itself, so its fp32
// rounding does not grow with the query's sum.
__device__ __forceinline__ void i8x4_to_h4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    const uint32_t u = w ^ 0x80808080u;
    const half2v off = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off);
    hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off);
}

// v_max3_f32 without the NaN-quieting the compiler adds around fmaxf of loaded or
// MFMA-produced values (the operands here are finite or -inf)
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// fp16 hi + lo parts of w0 = p0 * n0 and w1 = p1 * n1, packed (element 0 in the low
// halves): hi = fp16(p * n) and lo = fp16(p * n - hi), each one fused multiply-add
// with a single rounding (v_fma_mix with fp32 sources; the lo step reads hi as fp16)
__device__ __forceinline__ void weights_hilo(float p0, float n0, float p1, float n1, uint32_t& hi, uint32_t& lo) {
    asm("v_fma_mixlo_f16 %0, %2, %3, 0\n\t"
        "v_fma_mixhi_f16 %0, %4, %5, 0\n\t"
        "v_fma_mixlo_f16 %1, %2, %3, -%0 op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixhi_f16 %1, %4, %5, -%0 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
        : "=&v"(hi), "=&v"(lo)
        : "v"(p0), "v"(n0), "v"(p1), "v"(n1));
}

template <int NBYTES>
struct Chunk {
    uint32_t w[NBYTES / 4];
};

// LDS byte offset of LUT entry `field` (a W-bit field at bit P of the chunk, P and W
// compile-time) in this lane's copy: field * kLutCopies * 4 + lane_base.  The field
// is shifted straight into place and masked; with the LUT 32 KB-aligned, the sum
// with lane_base (< 128 above the LUT) has disjoint bits.
template <int NBYTES, int P, int W, int ES = 7>
__device__ __forceinline__ uint32_t lut_offset(const Chunk<NBYTES>& c, uint32_t lane_base) {
    constexpr int wi = P >> 5, sh = P & 31;
    constexpr uint32_t mask = ((1u << W) - 1u) << ES;  // entries of 2^ES bytes (pairs: kLutCopies * 4)
    uint32_t x;
    if constexpr (sh + W <= 32) {
        if constexpr (sh >= ES) x = (c.w[wi] >> (sh - ES)) & mask;
        else x = (c.w[wi] << (ES - sh)) & mask;
    } else {
        x = (__builtin_amdgcn_alignbit(c.w[wi + 1], c.w[wi], sh) << ES) & mask;
    }
    return x + lane_base;
}

template <int NBYTES, int BITS, int NBI, int PI>
__device__ __forceinline__ uint32_t lut_pair(const Chunk<NBYTES>& c, uint32_t lane_base) {
    const uint32_t off = lut_offset<NBYTES, 8 * BITS * NBI + 2 * BITS * PI, 2 * BITS>(c, lane_base);
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(static_cast<uintptr_t>(off));
}

// 3-bit codes: one 8-byte entry per 4 codes (a 12-bit field), a single copy of 4096
// entries at the start of LDS, so the offset is the field times 8
// 2-bit codes: 256 entries of 4 codes (an 8-bit field) in 16 copies, 128 bytes per entry
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int NBYTES, int BITS, int NBI, int QI>
__device__ __forceinline__ u32x2 lut_quad(const Chunk<NBYTES>& c, uint32_t lut_base) {
    constexpr int W = 4 * BITS;
    const uint32_t off = lut_offset<NBYTES, 8 * BITS * NBI + W * QI, W, BITS == 3 ? 3 : 7>(c, lut_base);
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(static_cast<uintptr_t>(off));
}

template <int NBYTES, int BITS, int NBI>
__device__ __forceinline__ half8 decode_b(const Chunk<NBYTES>& c, uint32_t lane_base) {
    H8 r;
    if constexpr (BITS <= 3) {
        const u32x2 q0 = lut_quad<NBYTES, BITS, NBI, 0>(c, lane_base), q1 = lut_quad<NBYTES, BITS, NBI, 1>(c, lane_base);
        r.u[0] = q0.x;
        r.u[1] = q0.y;
        r.u[2] = q1.x;
        r.u[3] = q1.y;
    } else {
        r.u[0] = lut_pair<NBYTES, BITS, NBI, 0>(c, lane_base);
        r.u[1] = lut_pair<NBYTES, BITS, NBI, 1>(c, lane_base);
        r.u[2] = lut_pair<NBYTES, BITS, NBI, 2>(c, lane_base);
        r.u[3] = lut_pair<NBYTES, BITS, NBI, 3>(c, lane_base);
    }
    return r.h;
}

template <int CB, int BITS, int NBI = 0>
__device__ __forceinline__ void decode_all(half8 (&vb)[CB / BITS], const Chunk<CB>& c, uint32_t lane_base) {
    if constexpr (NBI < CB / BITS) {
        vb[NBI] = decode_b<CB, BITS, NBI>(c, lane_base);
        decode_all<CB, BITS, NBI + 1>(vb, c, lane_base);
    }
}

// Workgroup barrier for LDS traffic only: global loads still in flight (the
// suffix records fetched ahead of the combine, the ring's direct-to-LDS loads,
// which every wave waits for on its own before reading its slots) are not
// waited for, as a full __syncthreads() would.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Direct-to-LDS load: every lane's `SIZE` bytes at base + off land at ldst + lane * SIZE
// (base wave-uniform, off per lane: the scalar-base form of the instruction).
typedef const __attribute__((address_space(1))) uint8_t* gptr_t;
template <int SIZE>
__device__ __forceinline__ void dma(const void* base, uint32_t off, void* ldst) {
    auto* l = reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(ldst));
    gptr_t g = reinterpret_cast<gptr_t>(reinterpret_cast<uintptr_t>(base)) + off;
    if constexpr (SIZE == 16) __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
    else if constexpr (SIZE == 12) __builtin_amdgcn_global_load_lds(g, l, 12, 0, 0);
    else __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
}

// Raw ring contents of one step for this lane: K pieces (kr[i] at ka + i * 1024), V code
// pieces (v[i] at va + i * VSTRIDE) and the norms (ns[0..1]) and scales (ns[2..3], 128
// bytes on) of its 8 tokens.  ring_read issues the LDS reads without waiting;
// ring_fence waits for them and passes every register through an asm output, so no
// instruction can read them before the data has arrived.
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <int CB> struct VPiece;
template <> struct VPiece<8> { typedef uint32_t type; static constexpr int n = 2; };
template <> struct VPiece<12> { typedef u32x3 type; static constexpr int n = 1; };
template <> struct VPiece<16> { typedef u32x4 type; static constexpr int n = 1; };
template <> struct VPiece<24> { typedef u32x3 type; static constexpr int n = 2; };
template <> struct VPiece<32> { typedef u32x4 type; static constexpr int n = 2; };

template <int NK, int CB>
struct RingRaw {
    u32x4 kr[NK];
    typename VPiece<CB>::type v[VPiece<CB>::n];
    u32x4 ns[4];
    // the CB code bytes as dwords
    __device__ __forceinline__ void code_words(uint32_t (&cw)[CB / 4]) const {
        constexpr int per = CB / 4 / VPiece<CB>::n;
#pragma unroll
        for (int i = 0; i < VPiece<CB>::n; ++i) {
            if constexpr (per == 1) cw[i] = v[i];
            else {
#pragma unroll
                for (int j = 0; j < per; ++j) cw[i * per + j] = v[i][j];
            }
        }
    }
};

template <int NK, int CB>
__device__ __forceinline__ void ring_read(uint32_t ka, uint32_t va, uint32_t na, RingRaw<NK, CB>& r);
template <int NK, int CB>
__device__ __forceinline__ void ring_fence(RingRaw<NK, CB>& r);
template <>
__device__ __forceinline__ void ring_read<2, 8>(uint32_t ka, uint32_t va, uint32_t na, RingRaw<2, 8>& r) {
    asm volatile("ds_read_b128 %0, %[ka] offset:0\n\tds_read_b128 %1, %[ka] offset:1024\n\tds_read_b32 %2, %[va] offset:0\n\tds_read_b32 %3, %[va] offset:256\n\tds_read_b128 %4, %[na] offset:0\n\tds_read_b128 %5, %[na] offset:16\n\tds_read_b128 %6, %[na] offset:128\n\tds_read_b128 %7, %[na] offset:144"
                 : "=&v"(r.kr[0]), "=&v"(r.kr[1]), "=&v"(r.v[0]), "=&v"(r.v[1]), "=&v"(r.ns[0]), "=&v"(r.ns[1]), "=&v"(r.ns[2]), "=&v"(r.ns[3])
                 : [ka] "v"(ka), [va] "v"(va), [na] "v"(na)
                 : "memory");
}
template <>
__device__ __forceinline__ void ring_fence<2, 8>(RingRaw<2, 8>& r) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r.kr[0]), "+v"(r.kr[1]), "+v"(r.v[0]), "+v"(r.v[1]), "+v"(r.ns[0]), "+v"(r.ns[1]), "+v"(r.ns[2]), "+v"(r.ns[3]) :: "memory");
}
template <>
__device__ __forceinline__ void ring_read<2, 12>(uint32_t ka, uint32_t va, uint32_t na, RingRaw<2, 12>& r) {
    asm volatile("ds_read_b128 %0, %[ka] offset:0\n\tds_read_b128 %1, %[ka] offset:1024\n\tds_read_b96 %2, %[va] offset:0\n\tds_read_b128 %3, %[na] offset:0\n\tds_read_b128 %4, %[na] offset:16\n\tds_read_b128 %5, %[na] offset:128\n\tds_read_b128 %6, %[na] offset:144"
                 : "=&v"(r.kr[0]), "=&v"(r.kr[1]), "=&v"(r.v[0]), "=&v"(r.ns[0]), "=&v"(r.ns[1]), "=&v"(r.ns[2]), "=&v"(r.ns[3])
                 : [ka] "v"(ka), [va] "v"(va), [na] "v"(na)
                 : "memory");
}
template <>
__device__ __forceinline__ void ring_fence<2, 12>(RingRaw<2, 12>& r) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r.kr[0]), "+v"(r.kr[1]), "+v"(r.v[0]), "+v"(r.ns[0]), "+v"(r.ns[1]), "+v"(r.ns[2]), "+v"(r.ns[3]) :: "memory");
}
template <>
__device__ __forceinline__ void ring_read<2, 16>(uint32_t ka, uint32_t va, uint32_t na, RingRaw<2, 16>& r) {
    asm volatile("ds_read_b128 %0, %[ka] offset:0\n\tds_read_b128 %1, %[ka] offset:1024\n\tds_read_b128 %2, %[va] offset:0\n\tds_read_b128 %3, %[na] offset:0\n\tds_read_b128 %4, %[na] offset:16\n\tds_read_b128 %5, %[na] offset:128\n\tds_read_b128 %6, %[na] offset:144"
                 : "=&v"(r.kr[0]), "=&v"(r.kr[1]), "=&v"(r.v[0]), "=&v"(r.ns[0]), "=&v"(r.ns[1]), "=&v"(r.ns[2]), "=&v"(r.ns[3])
                 : [ka] "v"(ka), [va] "v"(va), [na] "v"(na)
                 : "memory");
}
template <>
__device__ __forceinline__ void ring_fence<2, 16>(RingRaw<2, 16>& r) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r.kr[0]), "+v"(r.kr[1]), "+v"(r.v[0]), "+v"(r.ns[0]), "+v"(r.ns[1]), "+v"(r.ns[2]), "+v"(r.ns[3]) :: "memory");
}
template <>
__device__ __forceinline__ void ring_read<4, 16>(uint32_t ka, uint32_t va, uint32_t na, RingRaw<4, 16>& r) {
    asm volatile("ds_read_b128 %0, %[ka] offset:0\n\tds_read_b128 %1, %[ka] offset:1024\n\tds_read_b128 %2, %[ka] offset:2048\n\tds_read_b128 %3, %[ka] offset:3072\n\tds_read_b128 %4, %[va] offset:0\n\tds_read_b128 %5, %[na] offset:0\n\tds_read_b128 %6, %[na] offset:16\n\tds_read_b128 %7, %[na] offset:128\n\tds_read_b128 %8, %[na] offset:144"
                 : "=&v"(r.kr[0]), "=&v"(r.kr[1]), "=&v"(r.kr[2]), "=&v"(r.kr[3]), "=&v"(r.v[0]), "=&v"(r.ns[0]), "=&v"(r.ns[1]), "=&v"(r.ns[2]), "=&v"(r.ns[3])
                 : [ka] "v"(ka), [va] "v"(va), [na] "v"(na)
                 : "memory");
}
template <>
__device__ __forceinline__ void ring_fence<4, 16>(RingRaw<4, 16>& r) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r.kr[0]), "+v"(r.kr[1]), "+v"(r.kr[2]), "+v"(r.kr[3]), "+v"(r.v[0]), "+v"(r.ns[0]), "+v"(r.ns[1]), "+v"(r.ns[2]), "+v"(r.ns[3]) :: "memory");
}
template <>
__device__ __forceinline__ void ring_read<4, 24>(uint32_t ka, uint32_t va, uint32_t na, RingRaw<4, 24>& r) {
    asm volatile("ds_read_b128 %0, %[ka] offset:0\n\tds_read_b128 %1, %[ka] offset:1024\n\tds_read_b128 %2, %[ka] offset:2048\n\tds_read_b128 %3, %[ka] offset:3072\n\tds_read_b96 %4, %[va] offset:0\n\tds_read_b96 %5, %[va] offset:1024\n\tds_read_b128 %6, %[na] offset:0\n\tds_read_b128 %7, %[na] offset:16\n\tds_read_b128 %8, %[na] offset:128\n\tds_read_b128 %9, %[na] offset:144"
                 : "=&v"(r.kr[0]), "=&v"(r.kr[1]), "=&v"(r.kr[2]), "=&v"(r.kr[3]), "=&v"(r.v[0]), "=&v"(r.v[1]), "=&v"(r.ns[0]), "=&v"(r.ns[1]), "=&v"(r.ns[2]), "=&v"(r.ns[3])
                 : [ka] "v"(ka), [va] "v"(va), [na] "v"(na)
                 : "memory");
}
template <>
__device__ __forceinline__ void ring_fence<4, 24>(RingRaw<4, 24>& r) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r.kr[0]), "+v"(r.kr[1]), "+v"(r.kr[2]), "+v"(r.kr[3]), "+v"(r.v[0]), "+v"(r.v[1]), "+v"(r.ns[0]), "+v"(r.ns[1]), "+v"(r.ns[2]), "+v"(r.ns[3]) :: "memory");
}
template <>
__device__ __forceinline__ void ring_read<4, 32>(uint32_t ka, uint32_t va, uint32_t na, RingRaw<4, 32>& r) {
    asm volatile("ds_read_b128 %0, %[ka] offset:0\n\tds_read_b128 %1, %[ka] offset:1024\n\tds_read_b128 %2, %[ka] offset:2048\n\tds_read_b128 %3, %[ka] offset:3072\n\tds_read_b128 %4, %[va] offset:0\n\tds_read_b128 %5, %[va] offset:1024\n\tds_read_b128 %6, %[na] offset:0\n\tds_read_b128 %7, %[na] offset:16\n\tds_read_b128 %8, %[na] offset:128\n\tds_read_b128 %9, %[na] offset:144"
                 : "=&v"(r.kr[0]), "=&v"(r.kr[1]), "=&v"(r.kr[2]), "=&v"(r.kr[3]), "=&v"(r.v[0]), "=&v"(r.v[1]), "=&v"(r.ns[0]), "=&v"(r.ns[1]), "=&v"(r.ns[2]), "=&v"(r.ns[3])
                 : [ka] "v"(ka), [va] "v"(va), [na] "v"(na)
                 : "memory");
}
template <>
__device__ __forceinline__ void ring_fence<4, 32>(RingRaw<4, 32>& r) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r.kr[0]), "+v"(r.kr[1]), "+v"(r.kr[2]), "+v"(r.kr[3]), "+v"(r.v[0]), "+v"(r.v[1]), "+v"(r.ns[0]), "+v"(r.ns[1]), "+v"(r.ns[2]), "+v"(r.ns[3]) :: "memory");
}

template <int D, int BITS>
struct StageLayout {
    static constexpr int NK = D / 32;            // 16-byte K pieces per lane (2 tiles x D/64)
    static constexpr int CB = D / 16 * BITS;     // V code bytes per lane
    // V pieces per lane: 4-byte loads land lane-contiguous; 12- and 16-byte loads
    // land at lane * 16, so every piece of lane l sits at VOFF + i * VSTRIDE + l * VLANE
    static constexpr int NV = (CB == 12 || CB == 16) ? 1 : 2;
    static constexpr int VLANE = (CB == 8) ? 4 : 16;
    static constexpr int VSTRIDE = 64 * VLANE;
    static constexpr int KOFF = 0;
    static constexpr int VOFF = NK * 1024;
    static constexpr int NOFF = VOFF + NV * VSTRIDE;  // norms [32] then scales [32]
    static constexpr int NDMA = NK + NV + 1;          // direct-to-LDS instructions per stage
    static_assert(NOFF + 256 <= Ring<D>::kStageBytes, "stage overflow");
};

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Scheduling groups for the compiler (no instructions): N times one matrix-core instruction
// followed by V vector instructions, so the two units work side by side
template <int N, int V>
__device__ __forceinline__ void interleave() {
    if constexpr (N > 0) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // VALU
        interleave<N - 1, V>();
    }
}

// Always inlined: an out-of-line body would receive the launch struct by reference,
// which makes every lane copy it to scratch.
// FUSED: every (layer, kv head) is one workgroup, which finishes its rows itself; otherwise the
// workgroup writes partial records for k_merge.  Separate instantiations, so neither form's code
// shapes the other's register allocation.
template <int D, int RT, int BITS, bool QSPLIT, bool FUSED>
__device__ __forceinline__ void pool_mfma_body(const DecodeLaunch& a, const CentArg& cents) {
    using SL = StageLayout<D, BITS>;
    constexpr int NB = D / 16;   // PV column tiles
    constexpr int KS = D / 32;   // QK k-steps
    constexpr int DL = D / 4;    // K bytes per lane per token
    constexpr int CB = SL::CB;   // V code bytes per lane per step
    constexpr int kQK = 2 * KS * (QSPLIT ? 2 : 1);  // matrix-core instructions of one tile's scores
    constexpr int kPV = 2 * NB;                     // ... and of one tile's P.V products (hi + lo)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int rl = lane & 15, lg = lane >> 4;

    const int p = find_pool_m(a, blockIdx.x);
    const PoolEntry& P = a.pools[p];
    int rb = 0;
    int local = pool_item_of_wg(blockIdx.x - P.wg_begin, a.lc * a.hkv * P.splits, P.rblocks, &rb);
    const int sp = local % P.splits;
    local /= P.splits;
    const int g = local % a.hkv;
    const int lj = local / a.hkv;
    const int l = a.l0 + lj;
    // this workgroup's rows: pool rows r0 .. r0 + R - 1 (row block rb); row indices below are
    // local (LDS tiles, lanes) unless added to r0
    const int r0 = rb * P.rb_rows;
    const int R = min(P.rb_rows, P.rows - r0);

    const int8_t* kq = reinterpret_cast<const int8_t*>(P.base + P.off_kq) + ((uint64_t)l * a.hkv + g) * P.tc * D;
    const float* vn = reinterpret_cast<const float*>(P.base + P.off_vn) + ((uint64_t)l * a.hkv + g) * P.tc;
    // per-token K factors of the scores (Ks * sigma * log2 e, from the ring); a per-channel pool has
    // its scales folded into the queries instead, its ring slot reads the norms a second time
    const bool kchan = P.kmode == PKV_KSCALE_CHANNEL;
    const float* ks = kchan ? vn : reinterpret_cast<const float*>(P.base + P.off_ks) + ks_offset(P, l, g, a.hkv, D);
    const float* kch = reinterpret_cast<const float*>(P.base + P.off_ks) + ks_offset(P, l, g, a.hkv, D);
    const uint8_t* vc = P.base + P.off_vc0 + (uint64_t)a.hkv * P.tc * (D / 8) * layer_bits_prefix(P, l) +
                        (uint64_t)g * (P.tc / kGroupTokens) * D * BITS;
    const float vmax = reinterpret_cast<const float*>(P.base + P.off_vmax)[(uint64_t)l * a.hkv + g];
    int ex = 0;
    frexpf(vmax, &ex);
    // vn * nu < 2^7, so w = p * vn * nu < 2^15 fits fp16 while keeping the lo part of
    // small weights out of the fp16 subnormal range
    const int lnu0 = (vmax > 0.0f ? -ex : 0) + kWeightExp;
    // wave-uniform: the fused form holds it in a scalar register, so its combine needs no spilled
    // copy of it (the split form's code is different enough to keep it as it is)
    const int lnu = FUSED ? __builtin_amdgcn_readfirstlane(lnu0) : lnu0;
    const float nu = ldexpf(1.0f, lnu);

    const int tb = sp * P.chunk;
    const int te = min(P.T, tb + P.chunk);
    const int nsteps = te > tb ? (te - tb + kStep - 1) / kStep : 0;
    const int my_steps = nsteps > wave ? (nsteps - wave + kWaves - 1) / kWaves : 0;
    // K row of this lane in tile u: token 8*(rl>>2) + 4u + (rl&3), bytes lg*DL .. lg*DL + DL
    const int ktok0 = 8 * (rl >> 2) + (rl & 3);
    using RG = Ring<D>;
    BigLds<D>& g_big = big_lds<D>();
    uint8_t* ring = &g_big.loop.ring[wave][0][0];

    // Per-lane byte offsets of a step's pieces, fixed across steps: each load below is a
    // wave-uniform base (scalar) plus this 32-bit offset.
    uint32_t koff[SL::NK];
#pragma unroll
    for (int i = 0; i < SL::NK; ++i) {
        const int u = i / (DL / 16), h = i % (DL / 16);
        koff[i] = (uint32_t)((ktok0 + 4 * u) * D + lg * DL + 16 * h);
    }
    const uint32_t voff = (uint32_t)(CB * lane);  // this lane's code chunk in the step's 4 groups
    // norms (lanes 0-31) and K scales (lanes 32-63) of the step's 32 tokens
    const bool nlane = lane < 32;
    const uint32_t noff = 4u * (uint32_t)(lane & 31);
    auto issue = [&](int it) {  // DMA of this wavefront's it-th step into ring slot it % RG::kStages
        const int t0 = tb + (wave + it * kWaves) * kStep;
        uint8_t* st = ring + (it % RG::kStages) * RG::kStageBytes;
        const int8_t* kstep = kq + (uint64_t)t0 * D;
#pragma unroll
        for (int i = 0; i < SL::NK; ++i) dma<16>(kstep, koff[i], st + SL::KOFF + i * 1024);
        const uint8_t* vsrc = vc + (uint64_t)(t0 / kGroupTokens) * (D * BITS);
        if constexpr (CB == 8) {
            dma<4>(vsrc, voff, st + SL::VOFF);
            dma<4>(vsrc, voff + 4, st + SL::VOFF + SL::VSTRIDE);
        } else if constexpr (CB == 12) {
            dma<12>(vsrc, voff, st + SL::VOFF);
        } else if constexpr (CB == 16) {
            dma<16>(vsrc, voff, st + SL::VOFF);
        } else if constexpr (CB == 24) {
            dma<12>(vsrc, voff, st + SL::VOFF);
            dma<12>(vsrc, voff + 12, st + SL::VOFF + SL::VSTRIDE);
        } else {
            dma<16>(vsrc, voff, st + SL::VOFF);
            dma<16>(vsrc, voff + 16, st + SL::VOFF + SL::VSTRIDE);
        }
        // one load: lanes 0-31 read norms, 32-63 scales (per-lane base select, no 64-bit math)
        dma<4>(nlane ? (const void*)(vn + t0) : (const void*)(ks + t0), noff, st + SL::NOFF);
    };

    // ---- set-up loads first, all at once: this lane's query chunks (8 values per
    // (row tile, k-step): one 16-byte load for bf16, two for fp32) and one codebook
    // entry per lane; the ring's loads follow the query conversion
    const float cl = cents.c[BITS - 2][lane & 15];  // lane x holds centroid x (times the table's s)
    // log2 of the table's fp16 operand scale: every row reference below carries -lscale, so the
    // weights come out divided by s (the row maxima and records do not)
    const float lscale = cents.ls[BITS - 2];

    // QSHARE (head_dim 128, fp16 query operands): each wavefront loads and converts one 16-row
    // tile (wave w, tile w) into LDS, and every wavefront reads all of them after the barrier
    constexpr bool QSHARE = !QSPLIT && D == 128;
    half8 qreg[RT][KS];  // kept in registers for the whole unit
    half8 qlo[QSPLIT ? RT : 1][QSPLIT ? KS : 1];
    float qsc[RT];
    bool scaled_rows = false;
    if constexpr (QSHARE) {
        if (wave < RT) {
            const int rt = wave;
            const int rho = 16 * rt + rl;
            const bool ok = rho < R;
            const int rr = r0 + (ok ? rho : 0);
            const float rG = __builtin_amdgcn_rcpf((float)a.G);
            const int ka = (int)(((float)rr + 0.5f) * rG);  // rr / G, exact for rows < 2^20
            const int qa = P.agent_base >= 0 ? P.agent_base + ka : a.agent_id[P.agent0 + ka];
            const int qh = g * a.G + rr - ka * a.G;
            const uint64_t qo = (((uint64_t)qa * a.lc + lj) * a.hq + qh) * D + lg * DL;
            uint4 qr[KS];
#pragma unroll
            for (int k = 0; k < KS; ++k)
                qr[k] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qo + 8 * k);
            float xs[KS][8];
            float mx = 0.0f;
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const uint32_t h[4] = {qr[k].x, qr[k].y, qr[k].z, qr[k].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xs[k][2 * i] = ok ? __uint_as_float(h[i] << 16) : 0.0f;
                    xs[k][2 * i + 1] = ok ? __uint_as_float(h[i] & 0xffff0000u) : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(xs[k][i]));
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            int ex = 0;
            frexpf(mx, &ex);  // mx < 2^ex
            const int e = ex > 15 ? ex - 15 : 0;
            const float qinv = ldexpf(1.0f, -e);
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                H8 hv;
#pragma unroll
                for (int i = 0; i < 4; ++i) hv.u[i] = pack_h2(xs[k][2 * i] * qinv, xs[k][2 * i + 1] * qinv);
                g_qst[rt][k][lane] = hv.v;
            }
            if (lg == 0) g_qsc[rt][rl] = ldexpf(1.0f, e);
            const bool any = __builtin_amdgcn_ballot_w64(e > 0) != 0ull;
            if (lane == 0) g_qany[rt] = any ? 1 : 0;
        }
    } else {
        constexpr int QV = QSPLIT ? 2 : 1;
        // hi + lo query operands (QSPLIT) for fp32 queries, and for bf16 queries that carry a
        // per-channel pool's K scales
        const bool q32 = a.q_dtype == PKV_F32;
        uint4 qraw[RT][KS][QV];
        bool rok[RT];
        // the rows' agents and heads first (a table lookup only when the pool's agents are not
        // consecutive call agents), so that no wait for a lookup falls between the query loads
        int q_agent[RT], q_head[RT];
        const float rG = __builtin_amdgcn_rcpf((float)a.G);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int rho = 16 * rt + rl;
            rok[rt] = rho < R;
            const int rr = r0 + (rok[rt] ? rho : 0);        // pool row
            const int ka = (int)(((float)rr + 0.5f) * rG);  // rr / G, exact for rows < 2^20
            q_agent[rt] = P.agent0 + ka;
            q_head[rt] = g * a.G + rr - ka * a.G;
        }
        if (P.agent_base >= 0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) q_agent[rt] += P.agent_base - P.agent0;
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) q_agent[rt] = a.agent_id[q_agent[rt]];
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const uint64_t qo = (((uint64_t)q_agent[rt] * a.lc + lj) * a.hq + q_head[rt]) * D + lg * DL;
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                if (QSPLIT && q32) {
                    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(a.q) + qo + 8 * k);
                    qraw[rt][k][0] = src[0];
                    qraw[rt][k][QV - 1] = src[1];
                } else {
                    qraw[rt][k][0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qo + 8 * k);
                }
            }
        }
        // a per-channel pool's scales of this lane's query dimensions (lg*DL + 8 k + i), folded into q
        float4 chs[QSPLIT ? KS : 1][2];
        if constexpr (QSPLIT) {
            if (kchan) {
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    chs[k][0] = *reinterpret_cast<const float4*>(kch + lg * DL + 8 * k);
                    chs[k][1] = *reinterpret_cast<const float4*>(kch + lg * DL + 8 * k + 4);
                }
            }
        }
        // queries -> fp16 B operands (lane (lg, rl): row 16 rt + rl, dims lg*DL + 8 k + i).
        // Each row is first multiplied by 2^-e, e = max(0, E - 15) with max|q| < 2^E, so every
        // operand is below 2^15 (fp16 holds up to 65504); the power of two is exact and the
        // scores are multiplied back by qsc = 2^e.  bf16 values then convert exactly (8
        // significant bits; only values more than 2^39 below the row's largest reach fp16's
        // subnormal range), fp32 values are split into fp16 hi + lo operands.
        bool any_scaled = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float xs[KS][8];
            float mx = 0.0f;
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                uint32_t w[8];
                if (QSPLIT && q32) {
                    const uint4 r0 = qraw[rt][k][0], r1 = qraw[rt][k][QV - 1];
                    w[0] = r0.x; w[1] = r0.y; w[2] = r0.z; w[3] = r0.w;
                    w[4] = r1.x; w[5] = r1.y; w[6] = r1.z; w[7] = r1.w;
                } else {
                    const uint4 r0 = qraw[rt][k][0];
                    const uint32_t h[4] = {r0.x, r0.y, r0.z, r0.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        w[2 * i] = h[i] << 16;              // bf16 -> fp32 bits
                        w[2 * i + 1] = h[i] & 0xffff0000u;
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    xs[k][i] = rok[rt] ? __uint_as_float(w[i]) : 0.0f;
                    if constexpr (QSPLIT) {
                        if (kchan) {  // q'_i = q_i * s_i (fp32), split into fp16 hi + lo below
                            const float4 c = chs[k][i >> 2];
                            xs[k][i] *= (i & 3) == 0 ? c.x : (i & 3) == 1 ? c.y : (i & 3) == 2 ? c.z : c.w;
                        }
                    }
                    mx = fmaxf(mx, fabsf(xs[k][i]));
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            int ex = 0;
            frexpf(mx, &ex);  // mx < 2^ex
            const int e = ex > 15 ? ex - 15 : 0;
            qsc[rt] = ldexpf(1.0f, e);
            const float qinv = ldexpf(1.0f, -e);
            any_scaled |= e > 0;
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                H8 hv, lv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x0 = xs[k][2 * i] * qinv, x1 = xs[k][2 * i + 1] * qinv;
                    hv.u[i] = pack_h2(x0, x1);
                    if constexpr (QSPLIT) {
                        const half2v hh = __builtin_bit_cast(half2v, hv.u[i]);
                        lv.u[i] = pack_h2(x0 - (float)hh[0], x1 - (float)hh[1]);
                    }
                }
                qreg[rt][k] = hv.h;
                asm volatile("" : "+a"(qreg[rt][k]));  // a matrix-core operand only: kept in AGPRs
                if constexpr (QSPLIT) qlo[rt][k] = lv.h;
            }
        }
        // every wavefront of the workgroup holds all rows, so they all take the same branch below
        scaled_rows = __builtin_amdgcn_ballot_w64(any_scaled) != 0ull;
    }
    // the ring's first steps: issued once the query loads have landed, so those do not queue
    // behind the ring's burst of loads
#pragma unroll
    for (int it = 0; it < RG::kStages - 1; ++it)
        if (it < my_steps) issue(it);
    if constexpr (BITS == 3) {
        // LUT of fp16 centroid quads: entry e = c0 | c1 << 3 | c2 << 6 | c3 << 9 ->
        // (c[c0], c[c1], c[c2], c[c3]); this thread's entries tid + 256 k share the low pair
        const uint32_t lo = pack_h2(__shfl(cl, tid & 7, 64), __shfl(cl, (tid >> 3) & 7, 64));
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int hp = (tid >> 6) + 4 * k;  // the entry's high pair, c2 | c3 << 3
            const uint32_t hi = pack_h2(__shfl(cl, hp & 7, 64), __shfl(cl, hp >> 3, 64));
            reinterpret_cast<uint2*>(g_big.loop.lut)[tid + 256 * k] = make_uint2(lo, hi);
        }
    } else if constexpr (BITS == 2) {
        // 16 copies of the 256 quads: slot tid + 256 k holds entry (tid >> 4) + 16 k, whose
        // low pair (tid >> 4) & 15 is this thread's for every k
        const int lp = (tid >> 4) & 15;
        const uint32_t lo = pack_h2(__shfl(cl, lp & 3, 64), __shfl(cl, lp >> 2, 64));
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint32_t hi = pack_h2(__shfl(cl, k & 3, 64), __shfl(cl, k >> 2, 64));
            reinterpret_cast<uint2*>(g_big.loop.lut)[tid + 256 * k] = make_uint2(lo, hi);
        }
    } else {
        // LUT of fp16 centroid pairs: entry e = c0 | c1 << BITS -> (c[c0], c[c1])
        constexpr int NE = 1 << (2 * BITS);
#pragma unroll
        for (int i0 = 0; i0 < NE * kLutCopies; i0 += 256) {
            const int e = (i0 + tid) / kLutCopies;
            const float c0 = __shfl(cl, e & ((1 << BITS) - 1), 64);
            const float c1 = __shfl(cl, e >> BITS, 64);
            g_big.loop.lut[i0 + tid] = pack_h2(c0, c1);
        }
    }
    lds_barrier();  // LUT and query operands ready
    if constexpr (QSHARE) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                H8 h;
                h.v = g_qst[rt][k][lane];
                qreg[rt][k] = h.h;
                asm volatile("" : "+a"(qreg[rt][k]));  // a matrix-core operand only: kept in AGPRs
            }
            qsc[rt] = g_qsc[rt][rl];
            scaled_rows = scaled_rows || g_qany[rt] != 0;
        }
    }

    // this lane's LUT copy (pairs of 4-bit codes, quads of 2-bit ones), or the single 3-bit quad table
    const uint32_t lut_lane = lds_addr(g_big.loop.lut) +
                              (BITS == 3 ? 0u : BITS == 2 ? 8u * (lane & 15) : 4u * (lane & (kLutCopies - 1)));
    const uint32_t ring_a = lds_addr(ring);
    const float fs = a.sm_log2;
    const float fs_tok = kchan ? 0.0f : fs, fs_const = kchan ? fs : 0.0f;  // ff = Ks * fs_tok + fs_const

    // wait until at most `groups` steps' loads issued after the one needed are in
    // flight (each step is SL::NDMA load instructions, completed in order)
    auto wait_groups = [&](int groups) {
        if (groups >= 2) wait_vmcnt<2 * SL::NDMA>();
        else if (groups == 1) wait_vmcnt<SL::NDMA>();
        else wait_vmcnt<0>();
    };
    // ring slot of step `it` -> registers (no wait: see ring_fence)
    using Raw = RingRaw<SL::NK, CB>;
    auto ring_issue = [&](int it, Raw& r) {
        const uint32_t sa = ring_a + (it % RG::kStages) * RG::kStageBytes;
        ring_read<SL::NK, CB>(sa + SL::KOFF + lane * 16, sa + SL::VOFF + lane * SL::VLANE, sa + SL::NOFF + 32 * lg, r);
    };
    // K as exact fp16 operands
    auto convert_k = [&](const Raw& r, half8 (&ka)[2][KS]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const u32x4 v = r.kr[u * (DL / 16) + k / 2];
                H8 h;
                i8x4_to_h4((k & 1) ? v.z : v.x, h.u[0], h.u[1]);
                i8x4_to_h4((k & 1) ? v.w : v.y, h.u[2], h.u[3]);
                ka[u][k] = h.h;
            }
    };
    float cref[RT], lsum[RT], xmax[RT];
    f32x4 acc[RT][NB];
    // the token loop, compiled twice: SCALED multiplies every score tile by its rows' 2^e
    // (taken only when some row of the unit is past the fp16 range)
    auto unit_body = [&](auto scaled_tag) {
    constexpr bool SCALED = decltype(scaled_tag)::value;
    // S^T of row tile rt for the step's 32 tokens: lane (lg, rl) gets tokens
    // 8 lg + 4 u + j of row 16 rt + rl in S[u][j] (q . k for the int8 codes k)
    auto scores = [&](const half8 (&ka)[2][KS], int rt, f32x4 (&S)[2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) S[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // the two tiles' chains interleaved
#pragma unroll
        for (int k = 0; k < KS; ++k) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                S[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[u][k], qreg[rt][k], S[u], 0, 0, 0);
                if constexpr (QSPLIT) S[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[u][k], qlo[rt][k], S[u], 0, 0, 0);
            }
        }
        if constexpr (SCALED) {
#pragma unroll
            for (int u = 0; u < 2; ++u) S[u] *= qsc[rt];
        }
    };
    auto norms = [&](const u32x4 (&ns)[4], float (&nn)[8], float (&ff)[8]) {
        const uint32_t w[16] = {ns[0].x, ns[0].y, ns[0].z, ns[0].w, ns[1].x, ns[1].y, ns[1].z, ns[1].w,
                                ns[2].x, ns[2].y, ns[2].z, ns[2].w, ns[3].x, ns[3].y, ns[3].z, ns[3].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            nn[i] = __uint_as_float(w[i]);
            ff[i] = fmaf(__uint_as_float(w[8 + i]), fs_tok, fs_const);  // Ks * sigma * log2 e: log2 units
        }
    };

    // Softmax reference per row: p = exp2(score - mref).  mref is fixed before the
    // accumulation starts (this wavefront's first-step row max + kMargin), so the
    // accumulators are never rescaled inside the loop (they stay in AGPRs, touched
    // only by MFMAs).  The exponent also carries the weight scale nu = 2^lnu:
    // x = score - mref + lnu, p' = 2^x = p * nu, w = p' * vn.  If a score exceeds
    // mref + kLazy the weights could leave fp16 range: the workgroup then re-runs
    // the unit with the exact row maxima as references.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) cref[rt] = 0.0f;
    if (my_steps > 0) {
        wait_groups(min(my_steps, RG::kStages - 1) - 1);  // steps 0 .. RG::kStages - 2 were issued
        Raw r;
        ring_issue(0, r);
        ring_fence(r);
        half8 ka[2][KS];
        convert_k(r, ka);
        float nn[8], ff[8];
        norms(r.ns, nn, ff);
        const int t0 = tb + wave * kStep;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 S[2];
            scores(ka, rt, S);
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (t0 + 8 * lg + i < te) mx = fmaxf(mx, S[i >> 2][i & 3] * ff[i]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            cref[rt] = (float)lnu - (mx + kMargin) - lscale;
        }
    }

    // P.V of row tile rt with the weights (hi, lo): the eight hi products first, then the
    // lo ones, so no product waits for the one before it
    auto pv = [&](const half8 (&vb)[NB], int rt, const H8& wh, const H8& wl) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[rt][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh.h, vb[nb], acc[rt][nb], 0, 0, 0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[rt][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wl.h, vb[nb], acc[rt][nb], 0, 0, 0);
    };
    // softmax of row tile rt from its scores: exponents, row sum, running max, and the
    // weights w = p' * vn as fp16 hi + lo (w - hi, rounded once more): ~2^-22 relative
    auto weights = [&](const f32x4 (&S)[2], int rt, const float (&nn)[8], const float (&ff)[8], const bool (&ok)[8],
                       auto tail_tag, H8& wh, H8& wl) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = fmaf(S[i >> 2][i & 3], ff[i], cref[rt]);
            if (TAIL) x[i] = ok[i] ? x[i] : -INFINITY;
        }
        xmax[rt] = max3(max3(xmax[rt], x[0], x[1]), max3(x[2], x[3], x[4]), max3(x[5], x[6], x[7]));
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const float p0 = __builtin_amdgcn_exp2f(x[i]);
            const float p1 = __builtin_amdgcn_exp2f(x[i + 1]);
            lsum[rt] += p0 + p1;
            weights_hilo(p0, nn[i], p1, nn[i + 1], wh.u[i / 2], wl.u[i / 2]);
        }
    };

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            lsum[rt] = 0.0f;
            xmax[rt] = -INFINITY;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[rt][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        if (pass == 1) {
#pragma unroll
            for (int it = 0; it < RG::kStages - 1; ++it)
                if (it < my_steps) issue(it);
        }
        // The step loop is software-pipelined so that matrix-core and vector work of
        // different stages overlap.  Entering step it, the K operands (ka), V centroids (vb),
        // norms and score factors of step it are in registers and the scores of row tile 0
        // are issued.  Then, per row tile rt, the softmax of rt runs beside the scores of
        // rt + 1 and the P.V products of rt - 1; the last tile's P.V products run beside the
        // conversion of step it + 1's K, and its V decode beside the first scores of it + 1.
        // The ring reads of step it + 1 are issued before the last row tile's softmax and
        // waited for before the K conversion.
        // TAIL masks tokens at or past the end of the split; NEXT prepares step it + 1.
        const bool has_tail = my_steps > 0 && (te - tb) % kStep != 0 && wave == (nsteps - 1) % kWaves;
        if (my_steps > 0) {
            Raw raw;
            half8 ka[2][KS];
            half8 vb[NB];
            float nn[8], ff[8];
            f32x4 S0[2];
            wait_groups(min(my_steps - 1, RG::kStages - 2));
            ring_issue(0, raw);
            ring_fence(raw);
            {
                Chunk<CB> ch;
                raw.code_words(ch.w);
                decode_all<CB, BITS>(vb, ch, lut_lane);
            }
            convert_k(raw, ka);
            norms(raw.ns, nn, ff);
            scores(ka, 0, S0);
            // WAITG: load groups (steps) allowed in flight once step it + 1 has landed; ISSUE: step
            // it + kStages - 1 exists and is fetched now.  Both compile-time, so a step is one
            // branch-free block for the scheduler.
            auto step = [&](const int it, auto tail_tag, auto next_tag, auto waitg_tag, auto issue_tag) {
                constexpr bool TAIL = decltype(tail_tag)::value;
                constexpr bool NEXT = decltype(next_tag)::value;
                constexpr int WAITG = decltype(waitg_tag)::value;
                constexpr bool ISSUE = decltype(issue_tag)::value;
                const int t0 = tb + (wave + it * kWaves) * kStep;
                if constexpr (ISSUE) issue(it + RG::kStages - 1);  // into the slot of step it - 1, already read
                bool ok[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    ok[i] = !TAIL || (t0 + 8 * lg + i < te);
                    if (TAIL) nn[i] = ok[i] ? nn[i] : 0.0f;
                }
                H8 wh[2], wl[2];  // weights of tiles rt (index rt & 1) and rt - 1
                f32x4 S[2][2];    // scores of tiles rt and rt + 1 (index by parity)
                S[0][0] = S0[0];
                S[0][1] = S0[1];
                // per row tile rt: its softmax beside the scores of rt + 1 and the P.V products of
                // rt - 1 (all inputs produced before)
                static_for<0, RT>([&](auto rt_tag) {
                    constexpr int rt = decltype(rt_tag)::value;
                    if constexpr (NEXT && rt == RT - 1) {
                        // the ring reads of step it + 1 land during the last tile's softmax and
                        // P.V products (issued this late so their registers are not held all step)
                        wait_vmcnt<WAITG * SL::NDMA>();  // loads of step it + 1 landed
                        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LUT reads of this step are in
                        ring_issue(it + 1, raw);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if constexpr (rt + 1 < RT) scores(ka, rt + 1, S[(rt + 1) & 1]);
                    weights(S[rt & 1], rt, nn, ff, ok, tail_tag, wh[rt & 1], wl[rt & 1]);
                    if constexpr (rt >= 1) pv(vb, rt - 1, wh[(rt - 1) & 1], wl[(rt - 1) & 1]);
                });
                if constexpr (NEXT) {
                    __builtin_amdgcn_sched_barrier(0);  // the wait for the ring reads stays here
                    ring_fence(raw);
                    convert_k(raw, ka);
                }
                pv(vb, RT - 1, wh[(RT - 1) & 1], wl[(RT - 1) & 1]);
                if constexpr (NEXT) {
                    Chunk<CB> ch;
                    raw.code_words(ch.w);
                    decode_all<CB, BITS>(vb, ch, lut_lane);
                    norms(raw.ns, nn, ff);
                    scores(ka, 0, S0);
                    // the last tile's products and the first scores of step it + 1 beside the K
                    // conversion and V decode of step it + 1
                    interleave<kPV + kQK, 5>();
                }
            };
            using F = std::false_type;
            using T = std::true_type;
            using G0 = std::integral_constant<int, 0>;
            using G1 = std::integral_constant<int, 1>;
            using G2 = std::integral_constant<int, RG::kStages - 2>;
            static_assert(RG::kStages == 3 || RG::kStages == 4, "ring depth");
            // steady state: step it + 1 landed with kStages - 2 later steps in flight, and step
            // it + kStages - 1 to fetch; then the last steps of the ring, and the final step
            int it = 0;
            for (; it + RG::kStages <= my_steps; ++it) step(it, F{}, T{}, G2{}, T{});
            if constexpr (RG::kStages == 4) {
                if (it + 3 == my_steps) step(it++, F{}, T{}, G1{}, F{});
            }
            if (it + 2 == my_steps) step(it++, F{}, T{}, G0{}, F{});
            if (has_tail) step(my_steps - 1, T{}, F{}, G0{}, F{});
            else step(my_steps - 1, F{}, F{}, G0{}, F{});
        }
        // any row over the limit? then every wave re-runs with the exact row maxima
        if (tid == 0) g_flag = 0;
        lds_barrier();
        bool over = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float t = xmax[rt];
            t = fmaxf(t, __shfl_xor(t, 16, 64));
            t = fmaxf(t, __shfl_xor(t, 32, 64));
            over |= t > (float)lnu + kLazy;
            // this wave's max score of the row (log2 units)
            if (lg == 0) g_m[wave][16 * rt + rl] = my_steps > 0 ? t - cref[rt] : -INFINITY;
        }
        if (__builtin_amdgcn_ballot_w64(over) != 0ull && lane == 0) atomicOr(&g_flag, 1);
        lds_barrier();
        if (g_flag == 0) break;
        // re-run reference: the exact row max over the workgroup (no score exceeds it)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, g_m[w][16 * rt + rl]);
            cref[rt] = (float)lnu - M - lscale;
        }
        lds_barrier();
    }
    };
    if (scaled_rows) unit_body(std::true_type{});
    else unit_body(std::false_type{});
    const float inv_nu = 1.0f / nu;
    float m[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m[rt] = my_steps > 0 ? (float)lnu - (cref[rt] + lscale) : -INFINITY;
        lsum[rt] *= inv_nu * cents.lsc[BITS - 2];
    }

    // ---- combine the 4 wavefronts (fixed order, so results do not depend on timing)
    constexpr int RPW = kMaxRows / kWaves;  // rows finished per wavefront
    constexpr int FD = D / 16;              // fused finish: dimensions per lane (16 lanes per row)
    constexpr int FI = RPW / 4;             // fused finish: rows per lane (4 rows per wavefront pass)
    constexpr bool fused = FUSED;
    // fused finish: lane (fq, fl) handles rows wave + kWaves * (4 i + fq), i < FI, dims
    // FD fl .. FD fl + FD - 1.  Its rows' agents, heads and suffix records are fetched
    // now, so their latency overlaps the combine
    const int fq = lane >> 4, fl = lane & 15;
    float su_m[FI], su_l[FI], su_v[FI][FD];
    float se_m[FI], se_l[FI], se_v[FI][FD];  // the agent's private segment record (rotated domain), if any
    int f_row[FI], f_head[FI], f_agent[FI];
    if constexpr (fused) {
        // Every row's indices first, then each kind of load for all rows at once under one
        // wave-uniform branch: a per-row branch around a lookup would make each row wait for
        // the loads of the rows before it.
        const float rG = __builtin_amdgcn_rcpf((float)a.G);
        int f_ka[FI];  // the row's agent among the pool's agents
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            const int row = min(wave + kWaves * (4 * i + fq), R - 1);  // rows past R: computed, not stored
            const int prow = r0 + row;                                  // pool row
            const int ka = (int)(((float)prow + 0.5f) * rG);  // prow / G, exact for rows < 2^20
            f_row[i] = row;
            f_ka[i] = ka;
            f_head[i] = g * a.G + prow - ka * a.G;
            su_m[i] = -INFINITY;
            su_l[i] = 0.0f;
            se_m[i] = -INFINITY;
            se_l[i] = 0.0f;
#pragma unroll
            for (int e = 0; e < FD; ++e) {
                su_v[i][e] = 0.0f;
                se_v[i][e] = 0.0f;
            }
        }
        if (P.agent_base >= 0) {
#pragma unroll
            for (int i = 0; i < FI; ++i) f_agent[i] = P.agent_base + f_ka[i];
        } else {
#pragma unroll
            for (int i = 0; i < FI; ++i) f_agent[i] = a.agent_id[P.agent0 + f_ka[i]];
        }
        if (a.has_sfx) {
#pragma unroll
            for (int i = 0; i < FI; ++i) {
                const float* ru = a.part + a.sfx_part_off +
                                  (((uint64_t)(P.agent0 + f_ka[i]) * a.lc + lj) * a.hq + f_head[i]) * (2 + D);
                su_m[i] = ru[0];
                su_l[i] = ru[1];
#pragma unroll
                for (int e = 0; e < FD; ++e) su_v[i][e] = ru[2 + FD * fl + e];
            }
        }
        if (a.has_private) {
#pragma unroll
            for (int i = 0; i < FI; ++i) {
                const int e2 = a.agent_pool2[P.agent0 + f_ka[i]];
                if (e2 >= 0) {  // written by the segment kernel before this launch
                    const PoolEntry& Q = a.pools[e2];
                    const float* rs = a.part + Q.part_off +
                                      (((uint64_t)lj * a.hkv + g) * Q.rows + a.agent_pos2[P.agent0 + f_ka[i]] * a.G +
                                       (f_head[i] - g * a.G)) * (2 + D);
                    se_m[i] = rs[0];
                    se_l[i] = rs[1];
#pragma unroll
                    for (int e = 0; e < FD; ++e) se_v[i][e] = rs[2 + FD * fl + e];
                }
            }
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        lsum[rt] = sum_lane_rows(lsum[rt]);
        if (lg == 0) {
            g_m[wave][16 * rt + rl] = m[rt];
            g_l[wave][16 * rt + rl] = lsum[rt];
        }
    }
    lds_barrier();  // every wave is done with the ring and the LUT
    // this wave's tile: row 16 rt + 4 lg + j, dims NB * rl .. NB * rl + NB - 1
    float* mine = g_big.accs + wave * (kMaxRows * D);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float* dst = mine + (16 * rt + 4 * lg + j) * D + NB * rl;
#pragma unroll
            for (int h = 0; h < NB / 4; ++h)
                *reinterpret_cast<float4*>(dst + acc_slot<NB>(rl, 4 * h)) =
                    make_float4(acc[rt][4 * h][j], acc[rt][4 * h + 1][j], acc[rt][4 * h + 2][j], acc[rt][4 * h + 3][j]);
        }
    lds_barrier();
    // row combine: M = max of the waves' references, weights 2^(m_w - M)
    auto row_weights = [&](int row, float (&al)[kWaves], float& M, float& L) {
        M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, g_m[w][row]);
        L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = g_m[w][row];
            al[w] = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
            L += al[w] * g_l[w][row];
        }
    };
    if constexpr (!fused) {
        // partial records: lane (fq, fl) writes dims FD fl .. FD fl + FD - 1 of rows
        // wave + kWaves * (4 i + fq), all its loads issued before the stores (records are
        // 8-byte aligned: float2 stores)
        float* rec0 = a.part + P.part_off + (((uint64_t)lj * a.hkv + g) * P.splits + sp) * (uint64_t)P.rows * (2 + D) +
                      (uint64_t)r0 * (2 + D);
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            const int row = wave + kWaves * (4 * i + fq);
            if (row >= R) break;  // rows grow with i
            float al[kWaves], M, L;
            row_weights(row, al, M, L);
            float z[FD];
#pragma unroll
            for (int e = 0; e < FD; ++e) z[e] = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float* src = g_big.accs + w * (kMaxRows * D) + row * D + FD * fl;
#pragma unroll
                for (int e4 = 0; e4 < FD; e4 += 4) {
                    const float4 v = *reinterpret_cast<const float4*>(src + acc_slot<FD>(fl, e4));
                    z[e4] = fmaf(al[w], v.x, z[e4]);
                    z[e4 + 1] = fmaf(al[w], v.y, z[e4 + 1]);
                    z[e4 + 2] = fmaf(al[w], v.z, z[e4 + 2]);
                    z[e4 + 3] = fmaf(al[w], v.w, z[e4 + 3]);
                }
            }
            float* rec = rec0 + (uint64_t)row * (2 + D);
#pragma unroll
            for (int e = 0; e < FD; e += 2)
                *reinterpret_cast<float2*>(rec + 2 + FD * fl + e) = make_float2(z[e] * inv_nu, z[e + 1] * inv_nu);
            if (fl == 0) *reinterpret_cast<float2*>(rec) = make_float2(M, L);
        }
        return;
    }
    // ---- fused finish: per row, inverse FWHT (H / D), suffix record, normalise, store.
    // The Hadamard butterflies run over the dimension bits: the low log2 FD in-lane, the
    // high four across the row's 16 lanes (lane distance 1, 2, 4, 8: DPP moves only)
    // The rotation's signs of this lane's output dimensions FD fl .. FD fl + FD - 1, the same
    // for every row: picked from the four (scalar) mask words once, rather than indexed per
    // row, which is a vector load whose wait would also wait for the previous row's stores.
    // (The empty asm hands the selects the words in scalar registers, so that the compiler
    // does not fold them back into one indexed load.)
    const uint32_t sbits = [&] {
        const int d0 = FD * fl, w = d0 >> 5;
        uint32_t v0 = P.vsign[0], v1 = P.vsign[1], v2 = P.vsign[2], v3 = P.vsign[3];
        asm("" : "+s"(v0), "+s"(v1), "+s"(v2), "+s"(v3));
        const uint32_t word = w == 0 ? v0 : w == 1 ? v1 : w == 2 ? v2 : v3;
        return (word >> (d0 & 31)) & ((1u << FD) - 1u);
    }();
#pragma unroll
    for (int i = 0; i < FI; ++i) {
        if (wave + kWaves * 4 * i >= R) break;  // no row of this pass is stored
        const int row = f_row[i];
        float al[kWaves], M, L;
        row_weights(row, al, M, L);
        float z[FD];
#pragma unroll
        for (int e = 0; e < FD; ++e) z[e] = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float* src = g_big.accs + w * (kMaxRows * D) + row * D + FD * fl;
#pragma unroll
            for (int e4 = 0; e4 < FD; e4 += 4) {
                const float4 v = *reinterpret_cast<const float4*>(src + acc_slot<FD>(fl, e4));
                z[e4] = fmaf(al[w], v.x, z[e4]);
                z[e4 + 1] = fmaf(al[w], v.y, z[e4 + 1]);
                z[e4 + 2] = fmaf(al[w], v.z, z[e4 + 2]);
                z[e4 + 3] = fmaf(al[w], v.w, z[e4 + 3]);
            }
        }
        // the private segment's rotated-domain record joins before the transform (z loses its
        // weight scale nu here; M and L become those of pool + segment)
        float zscale = inv_nu;  // weight scale still on z
        if (a.has_private) {
            const float ms = se_m[i];
            const float M1 = fmaxf(M, ms);
            const float ap = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - M1);
            const float as = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - M1);
            const float zs = ap * inv_nu;
#pragma unroll
            for (int e = 0; e < FD; ++e) z[e] = fmaf(z[e], zs, as * se_v[i][e]);
            L = ap * L + as * se_l[i];
            M = M1;
            zscale = 1.0f;
        }
#pragma unroll
        for (int h = 1; h < FD; h <<= 1)
#pragma unroll
            for (int e = 0; e < FD; ++e)
                if (!(e & h)) {
                    const float u0 = z[e], u1 = z[e + h];
                    z[e] = u0 + u1;
                    z[e + h] = u0 - u1;
                }
        auto stage = [&](auto off_tag) {
            constexpr int OFF = decltype(off_tag)::value;
            const float sg = (lane & OFF) ? -1.0f : 1.0f;
#pragma unroll
            for (int e = 0; e < FD; ++e) z[e] = fmaf(sg, z[e], lane_xor_row<OFF>(z[e], lane));
        };
        stage(std::integral_constant<int, 1>{});
        stage(std::integral_constant<int, 2>{});
        stage(std::integral_constant<int, 4>{});
        stage(std::integral_constant<int, 8>{});
        // the rotation's signs: output dimension FD * fl + e negated where its bit is set
#pragma unroll
        for (int e = 0; e < FD; ++e) z[e] = __uint_as_float(__float_as_uint(z[e]) ^ (((sbits >> e) & 1u) << 31));
        const float mu = su_m[i];
        const float M2 = fmaxf(M, mu);
        const float ap = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - M2);
        const float au = (mu == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mu - M2);
        const float denom = ap * L + au * su_l[i];
        const float rinv = denom > 0.0f ? 1.0f / denom : 0.0f;
        const float sp_ = ap * zscale * (1.0f / D) * rinv;
        const float su_ = au * rinv;
        float o[FD];
#pragma unroll
        for (int e = 0; e < FD; ++e) o[e] = fmaf(z[e], sp_, su_v[i][e] * su_);
        const int rowi = wave + kWaves * (4 * i + fq);
        if (rowi < R) {
            float* out = a.out + (((uint64_t)f_agent[i] * a.lc + lj) * a.hq + f_head[i]) * D + FD * fl;
#pragma unroll
            for (int e4 = 0; e4 < FD; e4 += 4)
                *reinterpret_cast<float4*>(out + e4) = make_float4(o[e4], o[e4 + 1], o[e4 + 2], o[e4 + 3]);
        }
    }
}

// The native-window work a split-record launch carries beside the pool (workgroups from
// a.sfx_wg_begin on): 4 (agent, layer, kv head) units per workgroup, as the suffix kernel, with
// this launch's LDS (unused by such a workgroup otherwise) as each wave's score buffer.
template <int D>
__device__ __forceinline__ void pool_launch_sfx(const DecodeLaunch& a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int unit = ((int)blockIdx.x - a.sfx_wg_begin) * 4 + wave;
    if (unit >= a.n_agents * a.lc * a.hkv) return;
    float* sbuf = big_lds<D>().accs + wave * (kSfxChunk * 8);
    if (a.G == 1) sfx_fast_wave<D, 1, true>(a, unit, sbuf);
    else if (a.G == 2) sfx_fast_wave<D, 2, true>(a, unit, sbuf);
    else if (a.G <= 4) sfx_fast_wave<D, 4, true>(a, unit, sbuf);
    else sfx_fast_wave<D, 8, true>(a, unit, sbuf);
}
static_assert(kWaves * kSfxChunk * 8 <= kWaves * kMaxRows * 64, "window score buffers fit the LDS");

template <int D, int RT, bool QSPLIT, bool FUSED>
__global__ void __launch_bounds__(256) k_pool_mfma(DecodeLaunch a, CentArg cents) {
    touch_kernel_args();
    if constexpr (!FUSED) {
        if (a.sfx_wg_begin >= 0 && (int)blockIdx.x >= a.sfx_wg_begin) {
            pool_launch_sfx<D>(a);
            return;
        }
    }
    const PoolEntry& P = a.pools[find_pool_m(a, blockIdx.x)];
    int rb = 0;
    int local = pool_item_of_wg(blockIdx.x - P.wg_begin, a.lc * a.hkv * P.splits, P.rblocks, &rb);
    local /= P.splits;
    const int l = a.l0 + local / a.hkv;
    switch (layer_bits(P, l)) {
        case 2: pool_mfma_body<D, RT, 2, QSPLIT, FUSED>(a, cents); break;
        case 3: pool_mfma_body<D, RT, 3, QSPLIT, FUSED>(a, cents); break;
        default: pool_mfma_body<D, RT, 4, QSPLIT, FUSED>(a, cents); break;
    }
}

template <int D, bool QSPLIT, bool FUSED>
int launch_d(const DecodeLaunch& a, int wg, hipStream_t s, const CentArg& c, int rt) {
    switch (rt) {
        case 1: hipLaunchKernelGGL((k_pool_mfma<D, 1, QSPLIT, FUSED>), dim3(wg), dim3(256), 0, s, a, c); break;
        case 2: hipLaunchKernelGGL((k_pool_mfma<D, 2, QSPLIT, FUSED>), dim3(wg), dim3(256), 0, s, a, c); break;
        case 3: hipLaunchKernelGGL((k_pool_mfma<D, 3, QSPLIT, FUSED>), dim3(wg), dim3(256), 0, s, a, c); break;
        default:
            // split fp32 queries hold two operand sets in registers: at most 48 rows
            if constexpr (QSPLIT) return PKV_EUNSUPPORTED;
            else hipLaunchKernelGGL((k_pool_mfma<D, 4, QSPLIT, FUSED>), dim3(wg), dim3(256), 0, s, a, c);
            break;
    }
    return PKV_OK;
}

// Launch the kernel form (fused finish or split records) for rt row tiles of 16.
template <bool FUSED>
int launch_pool_mfma_form(const DecodeLaunch& a, int total_wg, hipStream_t s, int rt, bool split_q) {
    CentArg c;
    const CodebookTables& t = codebook_tables();
    for (int b = 0; b < 3; ++b) {
        for (int k = 0; k < 16; ++k) c.c[b][k] = t.fp16_scale[b] * t.cent[b][k];
        c.ls[b] = (float)std::log2((double)t.fp16_scale[b]);
        c.lsc[b] = (float)std::exp2((double)c.ls[b]);
    }
    if (a.d == 128) return split_q ? launch_d<128, true, FUSED>(a, total_wg, s, c, rt) : launch_d<128, false, FUSED>(a, total_wg, s, c, rt);
    return split_q ? launch_d<64, true, FUSED>(a, total_wg, s, c, rt) : launch_d<64, false, FUSED>(a, total_wg, s, c, rt);
}

}  // namespace

// The split-record form, compiled in its own translation unit.
int launch_pool_mfma_split(const DecodeLaunch& a, int total_wg, hipStream_t s, int rt, bool split_q);

}  // namespace pkv
