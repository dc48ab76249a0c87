// Streaming-read kernel: every workgroup reads one contiguous range of the
// buffer with 16-byte loads, 16 per thread in flight, and folds the words
// into one per wave so the loads stay live.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_probe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 16;
constexpr int kGrid = 512;
static_assert(kGrid * (kThreads / 64) * 4 <= MLA_PROBE_SINK_BYTES, "sink size");

__global__ __launch_bounds__(kThreads) void read_words(const u32x4* __restrict__ p, size_t n16,
                                                        size_t per, unsigned* __restrict__ sink) {
    const size_t lo = blockIdx.x * per;
    const size_t hi = lo + per < n16 ? lo + per : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    size_t i = lo + threadIdx.x;
    for (; i + (kUnroll - 1) * kThreads < hi; i += kUnroll * kThreads) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = p[i + u * kThreads];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < hi; i += kThreads) acc ^= p[i];
    unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = x;
}

}  // namespace

extern "C" int mla_probe_read(const void* buf, size_t bytes, void* sink, void* stream) {
    if (buf == nullptr || sink == nullptr) return 1;
    if (bytes % 16 != 0) return 2;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return 4;
    if (bytes == 0) return 0;
    const size_t n16 = bytes / 16;
    const size_t step = (size_t)kUnroll * kThreads;
    size_t per = (n16 + kGrid - 1) / kGrid;
    per = (per + step - 1) / step * step;
    hipLaunchKernelGGL(read_words, dim3(kGrid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(buf), n16, per, static_cast<unsigned*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 6;
}
