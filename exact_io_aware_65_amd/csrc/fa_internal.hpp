// Internal interface between the C ABI layer (fa_abi.cpp) and the kernel
// launchers (fa_fwd.hip, fa_decode.hip).  Arguments arrive here already
// validated; launchers only pick a template instance, size the grid and launch.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace fa355 {

enum class Elem { F16 = 1, BF16 = 2 };

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;  // may be null
    int B, H, Nq, Nkv, d;
    bool causal;
    float scale;
    Elem elem;
    bool out_f32;
    bool k_e4m3 = false;  // k holds E4M3 bytes [B][H][Nkv][d]; q is quantised on the fly
};

struct DecodeArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;  // may be null
    int B, H, Nkv, d;
    float scale;
    Elem elem;
    bool out_f32;
    int splits;      // resolved split count, each split non-empty
    int chunk;       // keys per split (the last split may hold fewer)
    float *ws_o;     // [B*H][splits][d] normalised partial outputs
    float *ws_lse;   // [B*H][splits] partial log2-sum-exp values
    // paged cache (block_table non-null): k, v are pools of num_pages pages,
    // [page][H][slot][d] (layout 0) or [page][slot][H][d] (layout 1); Nkv is
    // then the bound on seq_lens that sized the splits
    const int *block_table = nullptr;  // [B][max_pages]
    const int *seq_lens = nullptr;     // [B]
    int num_pages = 0, page_size = 0, max_pages = 0, layout = 0;
};

struct BwdArgs {
    const void *q, *k, *v, *o, *dout;  // o: the forward output in the input type
    const float *lse;                   // [B*H][Nq], natural log
    void *dq, *dk, *dv;
    int B, H, Nq, Nkv, d;
    bool causal;
    float scale;
    Elem elem;
    bool out_f32;
    float *ws_l2;  // [B*H][Nq] LSE * log2(e)
    float *ws_dd;  // [B*H][Nq] rowsum(dO * O)
};

// Work-items (workgroups x threads) of the forward's launch for these
// arguments: HIP takes at most 2^32 - 1 in one grid dimension.
unsigned long long fwd_work_items(const FwdArgs &a);
constexpr unsigned long long kMaxWorkItems = 0xffffffffULL;

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream);
// x: n 16-bit values of type elem; y: n E4M3 bytes.  x 16-byte, y 8-byte aligned.
hipError_t launch_quantize_e4m3(const void *x, void *y, std::size_t n, Elem elem, hipStream_t stream);

// Workspace bytes of the backward: two fp32 values per query row.
inline std::size_t bwd_workspace_bytes(int B, int H, int Nq)
{
    return static_cast<std::size_t>(B) * H * Nq * 2 * sizeof(float);
}

// Split count used when the caller passes num_splits = 0.
int decode_auto_splits(int B, int H, int Nkv, int d);

// Size of the device-resident scratch fa_decode_noalloc uses in place of a
// workspace (4 MiB per device), and its device address on the current device
// (looked up once per device; no allocation).
constexpr std::size_t kDecodeScratchBytes = std::size_t(4) << 20;
hipError_t decode_scratch(void **ptr);

// Workspace bytes for a resolved split count.
inline std::size_t decode_workspace_bytes(int B, int H, int splits, int d)
{
    return static_cast<std::size_t>(B) * H * splits * (d + 1) * sizeof(float);
}

}  // namespace fa355
