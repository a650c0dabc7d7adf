// Streaming-read probe: the HBM read bandwidth a kernel can reach on this
// device, the reference for the decode kernels, which are pure streams (every
// K and V byte read once, non-temporal).  Not part of libfa355: bench.py
// loads it from its own library to report decode against the measured rate
// as well as the published peak.
//
// Each workgroup reads one contiguous chunk of the buffer with 16-byte
// non-temporal loads, sixteen per thread in flight, and folds the words with
// XOR into one 32-bit value per thread, stored to `sink` so the loads stay
// live.  2048 workgroups and that depth were the fastest of a sweep over
// 2048-32768 workgroups and 4-16 loads in flight (4 GiB read): 6.90 TB/s,
// against 6.2 TB/s for the same kernel without the non-temporal hint.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 16;

__global__ __launch_bounds__(kThreads) void read_chunks(const u32x4 *__restrict__ src, size_t n, size_t per_wg,
                                                        unsigned *__restrict__ sink)
{
    const size_t lo = blockIdx.x * per_wg;
    const size_t hi = lo + per_wg < n ? lo + per_wg : n;
    unsigned acc = 0;
    size_t i = lo + threadIdx.x;
    for (; i + (kUnroll - 1) * kThreads < hi; i += kUnroll * kThreads) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < hi; i += kThreads) {
        const u32x4 x = __builtin_nontemporal_load(src + i);
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Workgroups of a launch; sink must hold this many * 256 uint32 values.
int fa_probe_read_blocks(void) { return 2048; }

// Read `bytes` bytes at `src` (16-byte aligned, a multiple of 16) once, on
// `stream`.  Returns 0, or a HIP error code (1 for invalid arguments, before
// any launch).
int fa_probe_read(const void *src, size_t bytes, unsigned *sink, hipStream_t stream)
{
    if (!src || !sink || bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return 1;
    const size_t n = bytes / 16;
    const int blocks = fa_probe_read_blocks();
    const size_t per_wg = (n + blocks - 1) / blocks;
    hipLaunchKernelGGL(read_chunks, dim3(blocks), dim3(kThreads), 0, stream, static_cast<const u32x4 *>(src), n,
                       per_wg, sink);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
