// Stand-ins for the kernel launchers and the one HIP call of the ABI layer, so
// that fa_abi.cpp (argument validation, workspace layout, error reporting)
// can be linked into a host-only program and run under AddressSanitizer and
// UndefinedBehaviorSanitizer without a GPU.  Every "launch" succeeds without
// touching the pointers it is given; a launch with an empty grid is reported.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "fa_internal.hpp"

namespace fa355 {

// The forward's launch-shape rule, restated so that this host-only program
// links no device code: 8 waves x 256 rows when every CU gets one such
// workgroup (16-bit K), else two key groups on 128 (or, causal d = 64, 64)
// rows for small grids, else 4 waves x 128 rows.
unsigned long long fwd_work_items(const FwdArgs &a)
{
    const long long bh = static_cast<long long>(a.B) * a.H;
    int nw = 4, kg = 1;
    if (!a.k_e4m3 && bh * ((a.Nq + 255) / 256) >= 256) {
        nw = 8;
    } else if (bh * ((a.Nq + 127) / 128) <= 256 && a.Nkv > 192) {
        nw = a.causal && a.d == 64 && !a.k_e4m3 ? 4 : 8;
        kg = 2;
    }
    const long long rows = 32LL * nw / kg;
    return static_cast<unsigned long long>(bh) * ((a.Nq + rows - 1) / rows) * (64ULL * nw);
}

// A fake, aligned device address for the no-allocation decode's scratch.
hipError_t decode_scratch(void **ptr)
{
    *ptr = reinterpret_cast<void *>(std::uintptr_t(13) << 36);
    return hipSuccess;
}

// The library's rule for the automatic split count, restated so that this
// host-only program links no device code.
int decode_auto_splits(int B, int H, int Nkv, int)
{
    const long long n_bh = static_cast<long long>(B) * H;
    if (n_bh < 1 || Nkv < 1) return 1;
    long long s = std::max<long long>((256 + n_bh - 1) / n_bh, 4);
    s = std::min<long long>(s, std::max<long long>((2048 + n_bh - 1) / n_bh, 1));
    s = std::min<long long>(s, (static_cast<long long>(Nkv) + 127) / 128);
    return static_cast<int>(std::max<long long>(s, 1));
}

static void expect(bool ok, const char *what)
{
    if (!ok) {
        std::fprintf(stderr, "stub launcher: %s\n", what);
        std::abort();
    }
}

hipError_t launch_fwd(const FwdArgs &a, hipStream_t)
{
    expect(a.B > 0 && a.H > 0 && a.Nq > 0 && a.Nkv > 0 && a.q && a.k && a.v && a.o, "fwd launch with an empty grid");
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t)
{
    expect(a.B > 0 && a.H > 0 && a.splits > 0 && a.chunk > 0, "decode launch without splits");
    expect(a.splits == 1 || (a.ws_o && a.ws_lse), "split decode without partials");
    if (a.ws_o) {
        const std::size_t parts = static_cast<std::size_t>(a.B) * a.H * a.splits;
        expect(a.ws_lse == a.ws_o + parts * a.d, "decode partial LSEs misplaced");
    }
    return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t)
{
    expect(a.B > 0 && a.H > 0 && a.Nkv > 0 && a.k && a.v && a.dk && a.dv, "bwd launch with an empty grid");
    expect(a.Nq == 0 || (a.q && a.o && a.dout && a.lse && a.dq && a.ws_l2 && a.ws_dd), "bwd rows without buffers");
    return hipSuccess;
}

hipError_t launch_quantize_e4m3(const void *x, void *y, std::size_t n, Elem, hipStream_t)
{
    expect(x && y && n > 0, "quantize launch with nothing to do");
    return hipSuccess;
}

}  // namespace fa355

extern "C" const char *hipGetErrorString(hipError_t) { return "stub"; }
