// A plain streaming read of a device buffer: the practical HBM read ceiling against
// which the decode kernels' achieved bandwidth is reported (the same run measures both).
// Every lane reads 16-byte words with a grid stride, eight loads in flight, and folds them
// with XOR, so no load can be optimised away; each wavefront writes one word of the result.
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace {

// 65536 workgroups with eight non-temporal 16-byte loads in flight per lane: the fastest of the
// grid sizes (1K-64K workgroups), unroll depths (4, 8, 16), temporal and non-temporal loads and
// strided and blocked orders measured on MI355X (6.38 TB/s over 2 GiB against 5.08 for four
// temporal loads in 2048 workgroups)
constexpr int kReadBlocks = 65536;
constexpr int kReadThreads = 256;
constexpr int kUnroll = 8;
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kReadThreads) k_stream_read(const u32x4v* __restrict__ src, uint64_t n16,
                                                              uint32_t* __restrict__ sink) {
    const uint64_t stride = (uint64_t)gridDim.x * kReadThreads;
    uint64_t i = (uint64_t)blockIdx.x * kReadThreads + threadIdx.x;
    uint32_t x = 0;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4v a[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) a[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4v a = __builtin_nontemporal_load(src + i);
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kReadThreads / 64) + (threadIdx.x >> 6)] = x;
}

}  // namespace

extern "C" size_t pkv_stream_read_sink_words(void) { return (size_t)kReadBlocks * (kReadThreads / 64); }

extern "C" int pkv_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(sink) % 4)
        return PKV_EINVAL;
    hipLaunchKernelGGL(k_stream_read, dim3(kReadBlocks), dim3(kReadThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4v*>(src), (uint64_t)(bytes / 16), sink);
    return pkv::launch_status();
}
