// Rounding of 16-bit tensors to FP8 (OCP E4M3) for the attention variant whose
// first product takes Q and K in 8 bits ("FlashAttention 1-2-3: The IO-Aware
// Revolution in LLM Inference", section "FlashAttention-3": Q and K quantised
// to FP8, V and O kept in 16 bits).  Each value is rounded on its own: nearest,
// ties to even, magnitudes beyond 448 saturated (the pages give no scaling
// factor).  The forward rounds Q itself as it loads it; a K that is not yet
// held in E4M3 is rounded once here, so the forward's K tiles arrive as 8-bit
// rows.  The pass streams 2 bytes in and 1 byte out per element.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa355 {
namespace {

constexpr int kQuantThreads = 256;
constexpr long long kQuantMaxBlocks = 8192;

template <typename T>
__global__ __launch_bounds__(kQuantThreads) void quantize_e4m3_kernel(const void *x, void *y, size_t n)
{
    // 8 elements per thread and step: 16 bytes in, 8 bytes out
    const size_t n8 = n / 8;
    const size_t stride = static_cast<size_t>(gridDim.x) * kQuantThreads;
    const u32x4 *src = static_cast<const u32x4 *>(x);
    u32x2 *dst = static_cast<u32x2 *>(y);
    for (size_t i = static_cast<size_t>(blockIdx.x) * kQuantThreads + threadIdx.x; i < n8; i += stride) {
        const u32x4 w = __builtin_nontemporal_load(src + i);  // each byte moves once
        __builtin_nontemporal_store(u32x2{e4m3x4(lo_f32<T>(w[0]), hi_f32<T>(w[0]), lo_f32<T>(w[1]), hi_f32<T>(w[1])),
                                          e4m3x4(lo_f32<T>(w[2]), hi_f32<T>(w[2]), lo_f32<T>(w[3]), hi_f32<T>(w[3]))},
                                    dst + i);
    }
    // the last n % 8 elements, one per thread of the first workgroup
    const size_t tail = n8 * 8 + threadIdx.x;
    if (blockIdx.x == 0 && tail < n) {
        const uint32_t bits = static_cast<const uint16_t *>(x)[tail];
        const uint32_t w = e4m3x4(lo_f32<T>(bits), 0.f, 0.f, 0.f);
        static_cast<uint8_t *>(y)[tail] = static_cast<uint8_t>(w & 0xff);
    }
}

}  // namespace

hipError_t launch_quantize_e4m3(const void *x, void *y, size_t n, Elem elem, hipStream_t stream)
{
    const long long n8 = static_cast<long long>(n / 8);
    long long blocks = (n8 + kQuantThreads - 1) / kQuantThreads;
    if (blocks > kQuantMaxBlocks) blocks = kQuantMaxBlocks;
    if (blocks < 1) blocks = 1;
    if (elem == Elem::F16)
        hipLaunchKernelGGL((quantize_e4m3_kernel<_Float16>), dim3(static_cast<unsigned>(blocks)), dim3(kQuantThreads),
                           0, stream, x, y, n);
    else
        hipLaunchKernelGGL((quantize_e4m3_kernel<__bf16>), dim3(static_cast<unsigned>(blocks)), dim3(kQuantThreads),
                           0, stream, x, y, n);
    return hipGetLastError();
}

}  // namespace fa355
