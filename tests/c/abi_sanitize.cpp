// Drives every entry point of the C ABI (include/fa355.h) through valid calls
// and through each class of invalid argument, against the stub launchers of
// abi_sanitize_stubs.cpp, so that the validation code runs under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Pointers are fake, aligned,
// non-overlapping addresses: the ABI layer only checks them, and the stubs
// never touch them.  Extreme sizes exercise the overflow guards.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa355.h"

namespace {

int failures = 0;

void expect(int got, int want, const char *what)
{
    const char *msg = fa_last_error();
    if (got != want || (want != FA_OK && (!msg || !*msg))) {
        std::fprintf(stderr, "%s: got %s, want %s (%s)\n", what, fa_status_str(got), fa_status_str(want),
                     msg ? msg : "(null)");
        ++failures;
    }
}

void *at(std::uintptr_t gib) { return reinterpret_cast<void *>(gib << 36); }  // 64 GiB apart

}  // namespace

int main()
{
    void *q = at(1), *k = at(2), *v = at(3), *o = at(4), *ws = at(6), *dq = at(7), *dk = at(8), *dv = at(9);
    float *lse = static_cast<float *>(at(5));
    const auto *table = static_cast<const int32_t *>(at(10));
    const auto *lens = static_cast<const int32_t *>(at(11));
    void *dout = at(12);

    if (fa_version() != FA355_VERSION) ++failures;
    for (int s = -1; s <= 5; ++s)
        if (!fa_status_str(s) || !*fa_status_str(s)) ++failures;

    // forward
    expect(fa_fwd(q, k, v, o, lse, 2, 4, 300, 500, 128, 1, 0.1f, FA_F16, nullptr), FA_OK, "fwd");
    expect(fa_fwd(q, k, v, o, nullptr, 2, 4, 300, 500, 64, 0, 0.1f, FA_BF16 | FA_OUT_F32, nullptr), FA_OK, "fwd f32");
    expect(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 2, 4, 0, 500, 128, 1, 0.1f, FA_F16, nullptr), FA_OK,
           "fwd empty");
    expect(fa_fwd(nullptr, k, v, o, lse, 1, 1, 64, 64, 128, 0, 0.1f, FA_F16, nullptr), FA_ERR_INVALID, "fwd null q");
    expect(fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, 96, 0, 0.1f, FA_F16, nullptr), FA_ERR_UNSUPPORTED, "fwd d=96");
    expect(fa_fwd(q, k, v, o, lse, 1, 1, 65, 64, 128, 1, 0.1f, FA_F16, nullptr), FA_ERR_INVALID, "fwd causal");
    expect(fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, 128, 0, 1.f / 0.f, FA_F16, nullptr), FA_ERR_INVALID, "fwd scale");
    expect(fa_fwd(q, k, v, q, lse, 1, 1, 64, 64, 128, 0, 0.1f, FA_F16, nullptr), FA_ERR_INVALID, "fwd overlap");
    expect(fa_fwd(static_cast<char *>(q) + 8, k, v, o, lse, 1, 1, 64, 64, 128, 0, 0.1f, FA_F16, nullptr),
           FA_ERR_INVALID, "fwd misaligned");
    expect(fa_fwd(q, k, v, o, lse, INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128, 0, 0.1f, FA_F16, nullptr),
           FA_ERR_INVALID, "fwd 2^62");
    expect(fa_fwd(q, k, v, o, lse, 1, 1, 64, 1 << 24, 128, 0, 0.1f, FA_F16, nullptr), FA_ERR_UNSUPPORTED,
           "fwd 4 GiB head");
    expect(fa_fwd(q, k, v, o, lse, -1, 1, 64, 64, 128, 0, 0.1f, FA_F16, nullptr), FA_ERR_INVALID, "fwd negative");
    expect(fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, 128, 0, 0.1f, 0x7, nullptr), FA_ERR_INVALID, "fwd dtype");

    // FP8 forward and the quantiser
    expect(fa_fwd_fp8(q, k, v, o, lse, 2, 4, 300, 500, 128, 1, 0.1f, FA_F16, nullptr), FA_OK, "fwd_fp8");
    expect(fa_fwd_fp8(q, k, v, o, lse, 1, 1, 64, 64, 64, 0, 0.1f, 3, nullptr), FA_ERR_INVALID, "fwd_fp8 dtype");
    expect(fa_quantize_e4m3(q, k, 4099, FA_BF16, nullptr), FA_OK, "quantize");
    expect(fa_quantize_e4m3(nullptr, nullptr, 0, FA_F16, nullptr), FA_OK, "quantize empty");
    expect(fa_quantize_e4m3(q, static_cast<char *>(q) + 64, 100, FA_F16, nullptr), FA_ERR_INVALID,
           "quantize overlap");
    expect(fa_quantize_e4m3(q, k, SIZE_MAX, FA_F16, nullptr), FA_ERR_INVALID, "quantize 2^62");

    // decode
    const std::size_t need = fa_decode_workspace_size(3, 5, 7777, 128, 0);
    if (need == 0 || fa_decode_workspace_size(3, 5, 0, 128, 0) != 0) ++failures;
    expect(fa_decode(q, k, v, o, lse, 3, 5, 7777, 128, 0.1f, FA_F16, 0, ws, need, nullptr), FA_OK, "decode");
    expect(fa_decode(q, k, v, o, lse, 3, 5, 7777, 128, 0.1f, FA_F16, 0, ws, need - 16, nullptr), FA_ERR_WORKSPACE,
           "decode short workspace");
    expect(fa_decode(q, k, v, o, lse, 3, 5, 7777, 128, 0.1f, FA_F16, 0, k, need, nullptr), FA_ERR_WORKSPACE,
           "decode workspace overlap");
    expect(fa_decode(q, k, v, o, lse, 3, 5, 7777, 128, 0.1f, FA_F16, 70000, ws, 1 << 30, nullptr), FA_OK,
           "decode more splits than keys");
    expect(fa_decode(q, k, v, o, lse, 1, 1, 0, 128, 0.1f, FA_F16, 0, ws, need, nullptr), FA_ERR_INVALID,
           "decode no keys");
    expect(fa_decode(q, k, v, o, lse, INT_MAX, INT_MAX, INT_MAX, 128, 0.1f, FA_F16, 0, ws, need, nullptr),
           FA_ERR_INVALID, "decode 2^62");

    // decode without a workspace: partials in the library's device scratch
    expect(fa_decode_noalloc(q, k, v, o, lse, 3, 5, 7777, 128, 0.1f, FA_F16, 0, nullptr), FA_OK, "decode noalloc");
    expect(fa_decode_noalloc(q, k, v, o, lse, 64, 64, 100, 128, 0.1f, FA_F16, 1, nullptr), FA_OK,
           "decode noalloc one split (no scratch)");
    expect(fa_decode_noalloc(q, k, v, o, lse, 16, 32, 32768, 128, 0.1f, FA_F16, 64, nullptr), FA_ERR_WORKSPACE,
           "decode noalloc beyond the scratch");
    expect(fa_decode_noalloc(q, k, v, q, lse, 3, 5, 7777, 128, 0.1f, FA_F16, 0, nullptr), FA_ERR_INVALID,
           "decode noalloc overlap");
    expect(fa_decode_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 5, 7777, 128, 0.1f, FA_F16, 0, nullptr),
           FA_OK, "decode noalloc empty");
    // 2^24 heads of one key (one split each): 2^32 work-items, one beyond HIP's grid limit
    expect(fa_decode(q, k, v, o, lse, 1 << 12, 1 << 12, 1, 64, 0.1f, FA_F16, 1, ws, SIZE_MAX, nullptr),
           FA_ERR_UNSUPPORTED, "decode grid 2^32");

    // paged decode
    const std::size_t pneed = fa_decode_workspace_size(3, 5, 300, 64, 0);
    expect(fa_decode_paged(q, k, v, table, lens, o, lse, 3, 5, 64, 97, 16, 19, FA_PAGED_HND, 300, 0.1f, FA_F16, 0,
                           ws, pneed, nullptr),
           FA_OK, "paged");
    expect(fa_decode_paged(q, k, v, table, lens, o, lse, 3, 5, 64, 97, 16, 19, 7, 300, 0.1f, FA_F16, 0, ws, pneed,
                           nullptr),
           FA_ERR_INVALID, "paged layout");
    expect(fa_decode_paged(q, k, v, table, lens, o, lse, 3, 5, 64, 97, 1 << 16, 1 << 16, FA_PAGED_NHD, 300, 0.1f,
                           FA_F16, 0, ws, pneed, nullptr),
           FA_ERR_INVALID, "paged capacity");
    expect(fa_decode_paged(q, k, v, table, lens, o, lse, 3, 5, 64, 97, 16, 19, FA_PAGED_HND, 0, 0.1f, FA_F16, 0, ws,
                           pneed, nullptr),
           FA_ERR_INVALID, "paged max_seq_len");
    expect(fa_decode_paged(q, k, v, table, lens, o, lse, 3, 5, 64, INT_MAX, INT_MAX, 1, FA_PAGED_HND, 300, 0.1f,
                           FA_F16, 0, ws, pneed, nullptr),
           FA_ERR_INVALID, "paged huge pages");
    // 2^40 heads in 2^30 one-key splits: 2^70 workgroups, counted without overflow
    expect(fa_decode_paged(q, k, v, table, lens, o, lse, 1 << 20, 1 << 20, 64, 1, 1, 1 << 30, FA_PAGED_HND, 1 << 30,
                           0.1f, FA_F16, 1 << 30, ws, SIZE_MAX, nullptr),
           FA_ERR_UNSUPPORTED, "paged grid 2^70");

    // backward
    const std::size_t bneed = fa_bwd_workspace_size(2, 4, 300);
    expect(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, 2, 4, 300, 500, 128, 1, 0.1f, FA_F16, ws, bneed, nullptr), FA_OK,
           "bwd");
    expect(fa_bwd(nullptr, k, v, nullptr, nullptr, nullptr, nullptr, dk, dv, 2, 4, 0, 500, 64, 1, 0.1f,
                  FA_BF16 | FA_OUT_F32, nullptr, 0, nullptr),
           FA_OK, "bwd no query rows");
    expect(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, 2, 4, 300, 500, 128, 1, 0.1f, FA_F16, nullptr, 0, nullptr),
           FA_ERR_WORKSPACE, "bwd no workspace");
    expect(fa_bwd(q, k, v, o, dout, lse, dq, dq, dv, 2, 4, 300, 500, 128, 1, 0.1f, FA_F16, ws, bneed, nullptr),
           FA_ERR_INVALID, "bwd outputs overlap");
    expect(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128, 0, 0.1f, FA_F16, ws,
                  bneed, nullptr),
           FA_ERR_INVALID, "bwd 2^62");

    // 2^23 + 2^12 one-row heads: as many 8-wave workgroups of 512 threads
    // (forward), 2^32 + 2^21 work-items; 2^24 one-row heads in the backward's
    // 256-thread passes, 2^32: both beyond HIP's 2^32 - 1
    expect(fa_fwd(q, k, v, o, lse, 1 << 12, (1 << 11) + 1, 1, 1, 64, 0, 0.1f, FA_F16, nullptr), FA_ERR_UNSUPPORTED,
           "fwd grid 2^32 + 2^21");
    expect(fa_fwd(q, k, v, o, lse, 1 << 12, (1 << 11) - 1, 1, 1, 64, 0, 0.1f, FA_F16, nullptr), FA_OK,
           "fwd grid 2^32 - 2^21");
    expect(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, 1 << 12, 1 << 12, 1, 1, 64, 0, 0.1f, FA_F16, ws, SIZE_MAX,
                  nullptr),
           FA_ERR_UNSUPPORTED, "bwd grid 2^32");

    // size helpers at the extremes: no signed overflow, no wrapped sizes
    if (fa_decode_num_splits(INT_MAX, INT_MAX, INT_MAX, 64) < 1) ++failures;
    if (fa_decode_num_splits(1, 1, INT_MAX, 128) < 1) ++failures;
    // 2^24 - 1 one-key splits of one head, 256 threads each: just within HIP's
    // 2^32 - 1 work-items; one more split, or INT_MAX of them, is beyond it
    if (fa_decode_workspace_size(1, 1, ((1 << 24) - 1) * 128, 64, (1 << 24) - 1) !=
        static_cast<std::size_t>((1 << 24) - 1) * 65 * 4)
        ++failures;
    if (fa_decode_workspace_size(1, 1, INT_MAX, 64, 1 << 24) != 0) ++failures;
    if (fa_decode_workspace_size(1, 1, INT_MAX, 64, INT_MAX) != 0) ++failures;
    if (fa_decode_workspace_size(2, 1, INT_MAX, 64, INT_MAX) != 0) ++failures;
    if (fa_decode_workspace_size(INT_MAX, INT_MAX, INT_MAX, 128, INT_MAX) != 0) ++failures;
    if (fa_decode_workspace_size(4, 8, 1000, 64, INT_MAX) != static_cast<std::size_t>(4) * 8 * 1000 * 65 * 4)
        ++failures;
    if (fa_bwd_workspace_size(INT_MAX, INT_MAX, INT_MAX) != 0) ++failures;
    if (fa_bwd_workspace_size(1, 1, INT_MAX) != static_cast<std::size_t>(INT_MAX) * 8) ++failures;

    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::puts("ABI validation ran clean");
    return 0;
}
