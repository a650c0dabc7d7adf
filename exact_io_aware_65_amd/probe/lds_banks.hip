// LDS bank probe: the evidence behind the kernels' LDS chunk permutations.
// Not part of libfa355; it builds into libfa355_probe.so beside the
// streaming-read probe, and bench.py --lds-probe runs it.
//
// One launch reads one access pattern: every lane of a 64-lane workgroup reads
// the LDS byte offset the pattern gives it, with ds_read_b128 (kind 0) or
// ds_read_b64_tr_b16 (kind 1), `iters` times.  Run under rocprofv3 with
// SQ_LDS_BANK_CONFLICT and SQ_INSTS_LDS, each dispatch gives its pattern's
// bank-conflict cycles per instruction.  A lane whose offset is 0xFFFFFFFF
// does not read (the instruction runs with it masked off), so two active
// lanes at two addresses of one bank tell whether the hardware serves those
// lanes in the same cycle.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
constexpr int kLdsBytes = 32768;
constexpr unsigned kSkip = 0xFFFFFFFFu;

struct LaneOffsets {
    unsigned v[64];
};

template <int KIND>
__global__ __launch_bounds__(64) void lds_pattern(LaneOffsets tab, int iters, unsigned zero, unsigned *__restrict__ sink)
{
    __shared__ u32x4 lds[kLdsBytes / 16];
    for (int i = threadIdx.x; i < kLdsBytes / 16; i += 64) {
        const unsigned u = static_cast<unsigned>(i);
        lds[i] = u32x4{u, u + 1, u + 2, u + 3};
    }
    __syncthreads();
    const unsigned off = tab.v[threadIdx.x];
    unsigned acc = 0;
    if (off != kSkip) {
        const char *base = reinterpret_cast<const char *>(lds);
        for (int it = 0; it < iters; ++it) {
            // zero is 0 at run time: the address stays the lane's own, but the
            // compiler cannot hoist the read out of the loop
            const unsigned o = off ^ (static_cast<unsigned>(it) & zero);
            if constexpr (KIND == 0) {
                const u32x4 x = *reinterpret_cast<const u32x4 *>(base + o);
                acc += x.x ^ x.w;
            } else {
                const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(base + o));
                acc += static_cast<unsigned>(x[0]) ^ static_cast<unsigned>(x[3]);
            }
        }
    }
    sink[static_cast<size_t>(blockIdx.x) * 64 + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Read one LDS access pattern.
//   kind     0: ds_read_b128 (offsets 16-byte aligned); 1: ds_read_b64_tr_b16
//            (offsets 8-byte aligned)
//   offsets  64 host values, one per lane: a byte offset into a 32 KiB LDS
//            buffer with room for the read, or 0xFFFFFFFF for a lane that does
//            not read; copied into the launch's arguments (the caller's array
//            is not used after the call returns)
//   blocks   workgroups of one wave each (1 .. 65536)
//   iters    reads per lane (1 .. 1 << 20)
//   sink     device buffer of blocks * 64 uint32, written (keeps the reads live)
// Returns 0, 1 for an invalid argument (checked before any launch), or the
// HIP error of the launch.
int fa_probe_lds(int kind, const unsigned *offsets, int blocks, int iters, unsigned *sink, hipStream_t stream)
{
    if ((kind != 0 && kind != 1) || !offsets || !sink || blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 20))
        return 1;
    const unsigned size = kind == 0 ? 16u : 8u;
    LaneOffsets tab;
    for (int l = 0; l < 64; ++l) {
        const unsigned o = offsets[l];
        if (o != kSkip && (o % size != 0 || o > static_cast<unsigned>(kLdsBytes) - size)) return 1;
        tab.v[l] = o;
    }
    if (kind == 0)
        hipLaunchKernelGGL(lds_pattern<0>, dim3(blocks), dim3(64), 0, stream, tab, iters, 0u, sink);
    else
        hipLaunchKernelGGL(lds_pattern<1>, dim3(blocks), dim3(64), 0, stream, tab, iters, 0u, sink);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
