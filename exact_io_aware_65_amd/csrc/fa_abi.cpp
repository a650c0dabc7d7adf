// C ABI of libfa355 (declared in include/fa355.h): argument validation,
// split-count resolution and dispatch to the kernel launchers.  Every check
// runs on the host before any HIP call, so a rejected call touches neither
// the device nor the outputs.
#include "fa355.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "fa_internal.hpp"

static_assert(FA_DECODE_NOALLOC_SCRATCH_BYTES == fa355::kDecodeScratchBytes, "the header states the scratch size");

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

bool log_enabled()
{
    static const bool on = [] {
        const char *e = std::getenv("FA355_LOG");
        return e && *e && *e != '0';
    }();
    return on;
}

struct Span {
    const char *name;
    std::uintptr_t lo, hi;
};

bool overlap(const Span &a, const Span &b) { return a.lo < b.hi && b.lo < a.hi; }

Span span(const char *name, const void *p, unsigned __int128 bytes)
{
    const auto lo = reinterpret_cast<std::uintptr_t>(p);
    return {name, lo, lo + static_cast<std::uintptr_t>(bytes)};
}

bool misaligned(const void *p, std::uintptr_t align)
{
    return reinterpret_cast<std::uintptr_t>(p) % align != 0;
}

// dtype = element type, optionally OR-ed with FA_OUT_F32.
int parse_dtype(const char *fn, int dtype, fa355::Elem *elem, bool *out_f32)
{
    const int base = dtype & 0xff, flags = dtype & ~0xff;
    if ((base != FA_F16 && base != FA_BF16) || (flags != 0 && flags != FA_OUT_F32))
        return fail(FA_ERR_INVALID, "%s: dtype 0x%x is not FA_F16 or FA_BF16 (optionally | FA_OUT_F32)",
                    fn, dtype);
    *elem = base == FA_F16 ? fa355::Elem::F16 : fa355::Elem::BF16;
    *out_f32 = flags == FA_OUT_F32;
    return FA_OK;
}

int check_head_dim(const char *fn, int d)
{
    if (d <= 0) return fail(FA_ERR_INVALID, "%s: head dimension d=%d must be positive", fn, d);
    if (d != 64 && d != 128)
        return fail(FA_ERR_UNSUPPORTED, "%s: head dimension d=%d is not supported (64 or 128)", fn, d);
    return FA_OK;
}

constexpr unsigned __int128 kMaxElems = static_cast<unsigned __int128>(1) << 62;

// Checks shared by fa_fwd and fa_decode once there is work to do.
int check_tensors(const char *fn, const void *q, const void *k, const void *v, const void *o,
                  const float *lse, int B, int H, int Nq, int Nkv, int d, bool out_f32, int k_elt = 2)
{
    if (!q || !k || !v || !o) return fail(FA_ERR_INVALID, "%s: q, k, v and o must be non-NULL", fn);
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16))
        return fail(FA_ERR_INVALID, "%s: q, k, v and o must be 16-byte aligned", fn);
    if (lse && misaligned(lse, 4)) return fail(FA_ERR_INVALID, "%s: lse must be 4-byte aligned", fn);
    const unsigned __int128 bh = static_cast<unsigned __int128>(B) * H;
    const unsigned __int128 nq_el = bh * Nq * d, nkv_el = bh * Nkv * d;
    if (nq_el >= kMaxElems || nkv_el >= kMaxElems)
        return fail(FA_ERR_INVALID, "%s: tensor sizes exceed 2^62 elements", fn);
    const Span in[3] = {span("q", q, nq_el * 2), span("k", k, nkv_el * k_elt), span("v", v, nkv_el * 2)};
    const Span out_o = span("o", o, nq_el * (out_f32 ? 4 : 2));
    for (const Span &s : in)
        if (overlap(out_o, s)) return fail(FA_ERR_INVALID, "%s: o overlaps %s", fn, s.name);
    if (lse) {
        const Span out_l = span("lse", lse, bh * Nq * 4);
        for (const Span &s : in)
            if (overlap(out_l, s)) return fail(FA_ERR_INVALID, "%s: lse overlaps %s", fn, s.name);
        if (overlap(out_l, out_o)) return fail(FA_ERR_INVALID, "%s: lse overlaps o", fn);
    }
    return FA_OK;
}

// Split count actually used for (Nkv >= 1, requested); each split holds >= 1
// key.  The sums are formed in 64 bits: Nkv and the request may both be near
// INT_MAX.
void resolve_splits(int B, int H, int Nkv, int d, int requested, int *splits, int *chunk)
{
    long long s = requested > 0 ? requested : fa355::decode_auto_splits(B, H, Nkv, d);
    if (s > Nkv) s = Nkv;
    const long long c = (static_cast<long long>(Nkv) + s - 1) / s;
    *chunk = static_cast<int>(c);
    *splits = static_cast<int>((Nkv + c - 1) / c);
}

// Work-items of a split decode's launches: the split kernel runs 256 threads
// per (b, h, split), the combine 512 per (b, h); each grid must stay within
// HIP's 2^32 - 1 work-items.
constexpr unsigned kDecodeSplitThreads = 256, kDecodeCombineThreads = 512;
bool decode_grid_fits(int B, int H, int splits)
{
    const unsigned __int128 bh = static_cast<unsigned __int128>(B) * H;
    return bh * splits * kDecodeSplitThreads <= fa355::kMaxWorkItems &&
           (splits == 1 || bh * kDecodeCombineThreads <= fa355::kMaxWorkItems);
}

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Nq,
           int Nkv, int d, int causal, float scale, int dtype, hipStream_t stream)
{
    static const char *fn = "fa_fwd";
    fa355::Elem elem;
    bool out_f32;
    int rc = parse_dtype(fn, dtype, &elem, &out_f32);
    if (rc) return rc;
    if ((rc = check_head_dim(fn, d))) return rc;
    if (B < 0 || H < 0 || Nq < 0 || Nkv < 0)
        return fail(FA_ERR_INVALID, "%s: negative size (B=%d H=%d Nq=%d Nkv=%d)", fn, B, H, Nq, Nkv);
    if (!std::isfinite(scale)) return fail(FA_ERR_INVALID, "%s: scale must be finite", fn);
    if (B == 0 || H == 0 || Nq == 0) return FA_OK;  // empty output: nothing to do
    if (Nkv == 0) return fail(FA_ERR_INVALID, "%s: Nkv=0: attention over no keys is undefined", fn);
    if (causal && Nq > Nkv)
        return fail(FA_ERR_INVALID, "%s: causal attention needs Nq <= Nkv (got %d > %d)", fn, Nq, Nkv);
    if ((rc = check_tensors(fn, q, k, v, o, lse, B, H, Nq, Nkv, d, out_f32))) return rc;
    if (static_cast<unsigned long long>(Nkv) * d * 2 > 0xffffffffULL ||
        static_cast<unsigned long long>(Nq) * d * (out_f32 ? 4 : 2) > 0xffffffffULL)
        return fail(FA_ERR_UNSUPPORTED, "%s: one head of q, k, v or o exceeds 4 GiB", fn);
    fa355::FwdArgs a{q, k, v, o, lse, B, H, Nq, Nkv, d, causal != 0, scale, elem, out_f32};
    const unsigned long long items = fa355::fwd_work_items(a);
    if (items > fa355::kMaxWorkItems)
        return fail(FA_ERR_UNSUPPORTED, "%s: %llu work-items exceed HIP's grid limit of 2^32 - 1", fn, items);
    if (log_enabled())
        std::fprintf(stderr, "fa355: fa_fwd B=%d H=%d Nq=%d Nkv=%d d=%d causal=%d dtype=0x%x work-items=%llu\n",
                     B, H, Nq, Nkv, d, causal != 0, dtype, items);
    const hipError_t err = fa355::launch_fwd(a, stream);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
    return FA_OK;
}

int fa_fwd_fp8(const void *q, const void *k8, const void *v, void *o, float *lse, int B, int H, int Nq, int Nkv,
               int d, int causal, float scale, int dtype, hipStream_t stream)
{
    static const char *fn = "fa_fwd_fp8";
    fa355::Elem elem;
    bool out_f32;
    int rc = parse_dtype(fn, dtype, &elem, &out_f32);
    if (rc) return rc;
    if ((rc = check_head_dim(fn, d))) return rc;
    if (B < 0 || H < 0 || Nq < 0 || Nkv < 0)
        return fail(FA_ERR_INVALID, "%s: negative size (B=%d H=%d Nq=%d Nkv=%d)", fn, B, H, Nq, Nkv);
    if (!std::isfinite(scale)) return fail(FA_ERR_INVALID, "%s: scale must be finite", fn);
    if (B == 0 || H == 0 || Nq == 0) return FA_OK;  // empty output: nothing to do
    if (Nkv == 0) return fail(FA_ERR_INVALID, "%s: Nkv=0: attention over no keys is undefined", fn);
    if (causal && Nq > Nkv)
        return fail(FA_ERR_INVALID, "%s: causal attention needs Nq <= Nkv (got %d > %d)", fn, Nq, Nkv);
    if ((rc = check_tensors(fn, q, k8, v, o, lse, B, H, Nq, Nkv, d, out_f32, 1))) return rc;
    if (static_cast<unsigned long long>(Nkv) * d * 2 > 0xffffffffULL ||
        static_cast<unsigned long long>(Nq) * d * (out_f32 ? 4 : 2) > 0xffffffffULL)
        return fail(FA_ERR_UNSUPPORTED, "%s: one head of q, v or o exceeds 4 GiB", fn);
    fa355::FwdArgs a{q, k8, v, o, lse, B, H, Nq, Nkv, d, causal != 0, scale, elem, out_f32};
    a.k_e4m3 = true;
    const unsigned long long items = fa355::fwd_work_items(a);
    if (items > fa355::kMaxWorkItems)
        return fail(FA_ERR_UNSUPPORTED, "%s: %llu work-items exceed HIP's grid limit of 2^32 - 1", fn, items);
    if (log_enabled())
        std::fprintf(stderr, "fa355: fa_fwd_fp8 B=%d H=%d Nq=%d Nkv=%d d=%d causal=%d dtype=0x%x work-items=%llu\n",
                     B, H, Nq, Nkv, d, causal != 0, dtype, items);
    const hipError_t err = fa355::launch_fwd(a, stream);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
    return FA_OK;
}

int fa_quantize_e4m3(const void *x, void *y, size_t n, int dtype, hipStream_t stream)
{
    static const char *fn = "fa_quantize_e4m3";
    if (dtype != FA_F16 && dtype != FA_BF16)
        return fail(FA_ERR_INVALID, "%s: dtype 0x%x is not FA_F16 or FA_BF16", fn, dtype);
    if (n == 0) return FA_OK;
    if (!x || !y || misaligned(x, 16) || misaligned(y, 16))
        return fail(FA_ERR_INVALID, "%s: x and y must be non-NULL and 16-byte aligned", fn);
    if (static_cast<unsigned __int128>(n) >= kMaxElems)
        return fail(FA_ERR_INVALID, "%s: n exceeds 2^62 elements", fn);
    if (overlap(span("x", x, static_cast<unsigned __int128>(n) * 2), span("y", y, n)))
        return fail(FA_ERR_INVALID, "%s: y overlaps x", fn);
    const hipError_t err = fa355::launch_quantize_e4m3(x, y, n, dtype == FA_F16 ? fa355::Elem::F16 : fa355::Elem::BF16,
                                                       stream);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
    return FA_OK;
}

size_t fa_decode_workspace_size(int B, int H, int Nkv, int d, int num_splits)
{
    if (B < 0 || H < 0 || Nkv < 1 || (d != 64 && d != 128) || num_splits < 0) return 0;
    if (B == 0 || H == 0) return 0;
    int splits, chunk;
    resolve_splits(B, H, Nkv, d, num_splits, &splits, &chunk);
    if (!decode_grid_fits(B, H, splits)) return 0;  // fa_decode rejects such a call
    return fa355::decode_workspace_bytes(B, H, splits, d);
}

int fa_decode_num_splits(int B, int H, int Nkv, int d)
{
    if (B < 0 || H < 0 || Nkv < 1 || (d != 64 && d != 128)) return 0;
    int splits, chunk;
    resolve_splits(B, H, Nkv, d, 0, &splits, &chunk);
    return splits;
}

}  // extern "C"

namespace {

// Validation shared by fa_decode and fa_decode_noalloc, up to (not including)
// the partials' storage.  Returns FA_OK with *work false when there is
// nothing to do, else fills *a (without workspace) and *need (bytes of
// partials the resolved split count uses; 0 with one split, which writes O
// and LSE directly).
int check_decode(const char *fn, const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                 int Nkv, int d, float scale, int dtype, int num_splits, fa355::DecodeArgs *a, size_t *need,
                 bool *work)
{
    *work = false;
    fa355::Elem elem;
    bool out_f32;
    int rc = parse_dtype(fn, dtype, &elem, &out_f32);
    if (rc) return rc;
    if ((rc = check_head_dim(fn, d))) return rc;
    if (B < 0 || H < 0 || Nkv < 0)
        return fail(FA_ERR_INVALID, "%s: negative size (B=%d H=%d Nkv=%d)", fn, B, H, Nkv);
    if (num_splits < 0) return fail(FA_ERR_INVALID, "%s: num_splits=%d must be >= 0", fn, num_splits);
    if (!std::isfinite(scale)) return fail(FA_ERR_INVALID, "%s: scale must be finite", fn);
    if (B == 0 || H == 0) return FA_OK;
    if (Nkv == 0) return fail(FA_ERR_INVALID, "%s: Nkv=0: attention over no keys is undefined", fn);
    if ((rc = check_tensors(fn, q, k, v, o, lse, B, H, 1, Nkv, d, out_f32))) return rc;

    if (static_cast<unsigned long long>(Nkv) * d * 2 > 0xffffffffULL)
        return fail(FA_ERR_UNSUPPORTED, "%s: one head of k or v exceeds 4 GiB", fn);
    int splits, chunk;
    resolve_splits(B, H, Nkv, d, num_splits, &splits, &chunk);
    if (!decode_grid_fits(B, H, splits))
        return fail(FA_ERR_UNSUPPORTED, "%s: B*H*splits = %d*%d*%d exceeds HIP's grid limit of 2^32 - 1 work-items",
                    fn, B, H, splits);
    *a = fa355::DecodeArgs{q, k, v, o, lse, B, H, Nkv, d, scale, elem, out_f32, splits, chunk, nullptr, nullptr};
    *need = splits > 1 ? fa355::decode_workspace_bytes(B, H, splits, d) : 0;
    *work = true;
    return FA_OK;
}

// The partials of a split decode at ws: [B*H][splits][d] outputs, then
// [B*H][splits] log-sum-exp values.
void place_partials(fa355::DecodeArgs *a, void *ws)
{
    a->ws_o = static_cast<float *>(ws);
    a->ws_lse = a->ws_o ? a->ws_o + static_cast<size_t>(a->B) * a->H * a->splits * a->d : nullptr;
}

}  // namespace

extern "C" {

int fa_decode(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Nkv,
              int d, float scale, int dtype, int num_splits, void *workspace, size_t workspace_bytes,
              hipStream_t stream)
{
    static const char *fn = "fa_decode";
    fa355::DecodeArgs a;
    size_t partials;
    bool work;
    int rc = check_decode(fn, q, k, v, o, lse, B, H, Nkv, d, scale, dtype, num_splits, &a, &partials, &work);
    if (rc || !work) return rc;
    const bool out_f32 = a.out_f32;
    const size_t need = fa355::decode_workspace_bytes(B, H, a.splits, d);
    if (!workspace || misaligned(workspace, 16) || workspace_bytes < need)
        return fail(FA_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned and hold %zu bytes (got %zu at %p)",
                    fn, need, workspace_bytes, workspace);
    const unsigned __int128 n_in = static_cast<unsigned __int128>(B) * H * d;
    const unsigned __int128 n_kv = static_cast<unsigned __int128>(B) * H * Nkv * d;
    const Span ws = span("workspace", workspace, need);
    const Span others[5] = {span("q", q, n_in * 2), span("k", k, n_kv * 2), span("v", v, n_kv * 2),
                            span("o", o, n_in * (out_f32 ? 4 : 2)),
                            span("lse", lse, lse ? static_cast<unsigned __int128>(B) * H * 4 : 0)};
    for (const Span &s : others)
        if (s.hi > s.lo && overlap(ws, s)) return fail(FA_ERR_WORKSPACE, "%s: workspace overlaps %s", fn, s.name);

    place_partials(&a, workspace);
    if (log_enabled())
        std::fprintf(stderr, "fa355: fa_decode B=%d H=%d Nkv=%d d=%d dtype=0x%x splits=%d chunk=%d\n", B, H,
                     Nkv, d, dtype, a.splits, a.chunk);
    const hipError_t err = fa355::launch_decode(a, stream);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
    return FA_OK;
}

int fa_decode_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Nkv,
                      int d, float scale, int dtype, int num_splits, hipStream_t stream)
{
    static const char *fn = "fa_decode_noalloc";
    fa355::DecodeArgs a;
    size_t need;
    bool work;
    int rc = check_decode(fn, q, k, v, o, lse, B, H, Nkv, d, scale, dtype, num_splits, &a, &need, &work);
    if (rc || !work) return rc;
    if (need > fa355::kDecodeScratchBytes)
        return fail(FA_ERR_WORKSPACE,
                    "%s: %d*%d heads x %d splits need %zu bytes of partials, beyond the %zu-byte device scratch "
                    "(call fa_decode with a workspace, or pass fewer splits)",
                    fn, B, H, a.splits, need, fa355::kDecodeScratchBytes);
    void *scratch = nullptr;
    if (need > 0) {
        const hipError_t err = fa355::decode_scratch(&scratch);
        if (err != hipSuccess)
            return fail(FA_ERR_HIP, "%s: device scratch lookup failed: %s", fn, hipGetErrorString(err));
    }
    place_partials(&a, scratch);
    if (log_enabled())
        std::fprintf(stderr, "fa355: fa_decode_noalloc B=%d H=%d Nkv=%d d=%d dtype=0x%x splits=%d chunk=%d\n", B, H,
                     Nkv, d, dtype, a.splits, a.chunk);
    const hipError_t err = fa355::launch_decode(a, stream);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
    return FA_OK;
}

int fa_decode_paged(const void *q, const void *k_pages, const void *v_pages, const int32_t *block_table,
                    const int32_t *seq_lens, void *o, float *lse, int B, int H, int d, int num_pages,
                    int page_size, int max_pages, int layout, int max_seq_len, float scale, int dtype,
                    int num_splits, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    static const char *fn = "fa_decode_paged";
    fa355::Elem elem;
    bool out_f32;
    int rc = parse_dtype(fn, dtype, &elem, &out_f32);
    if (rc) return rc;
    if ((rc = check_head_dim(fn, d))) return rc;
    if (B < 0 || H < 0 || num_pages < 0 || max_pages < 0)
        return fail(FA_ERR_INVALID, "%s: negative size (B=%d H=%d num_pages=%d max_pages=%d)", fn, B, H, num_pages,
                    max_pages);
    if (page_size < 1) return fail(FA_ERR_INVALID, "%s: page_size=%d must be >= 1", fn, page_size);
    if (layout != FA_PAGED_HND && layout != FA_PAGED_NHD)
        return fail(FA_ERR_INVALID, "%s: layout=%d is neither FA_PAGED_HND nor FA_PAGED_NHD", fn, layout);
    if (num_splits < 0) return fail(FA_ERR_INVALID, "%s: num_splits=%d must be >= 0", fn, num_splits);
    if (!std::isfinite(scale)) return fail(FA_ERR_INVALID, "%s: scale must be finite", fn);
    if (B == 0 || H == 0) return FA_OK;
    const long long capacity = static_cast<long long>(max_pages) * page_size;
    if (capacity >= (1LL << 31))
        return fail(FA_ERR_INVALID, "%s: max_pages * page_size = %lld must be below 2^31", fn, capacity);
    if (max_seq_len < 1 || max_seq_len > capacity)
        return fail(FA_ERR_INVALID, "%s: max_seq_len=%d must lie in [1, max_pages * page_size = %lld]", fn,
                    max_seq_len, capacity);
    if (num_pages < 1) return fail(FA_ERR_INVALID, "%s: the page pool is empty", fn);
    if (!q || !k_pages || !v_pages || !o)
        return fail(FA_ERR_INVALID, "%s: q, k_pages, v_pages and o must be non-NULL", fn);
    if (misaligned(q, 16) || misaligned(k_pages, 16) || misaligned(v_pages, 16) || misaligned(o, 16))
        return fail(FA_ERR_INVALID, "%s: q, k_pages, v_pages and o must be 16-byte aligned", fn);
    if (!block_table || !seq_lens || misaligned(block_table, 4) || misaligned(seq_lens, 4))
        return fail(FA_ERR_INVALID, "%s: block_table and seq_lens must be non-NULL and 4-byte aligned", fn);
    if (lse && misaligned(lse, 4)) return fail(FA_ERR_INVALID, "%s: lse must be 4-byte aligned", fn);
    const unsigned __int128 bh = static_cast<unsigned __int128>(B) * H;
    const unsigned __int128 pool_el = static_cast<unsigned __int128>(num_pages) * page_size * H * d;
    if (bh * d >= kMaxElems || pool_el >= kMaxElems)
        return fail(FA_ERR_INVALID, "%s: tensor sizes exceed 2^62 elements", fn);

    int splits, chunk;
    resolve_splits(B, H, max_seq_len, d, num_splits, &splits, &chunk);
    if (!decode_grid_fits(B, H, splits))
        return fail(FA_ERR_UNSUPPORTED, "%s: B*H*splits = %d*%d*%d exceeds HIP's grid limit of 2^32 - 1 work-items",
                    fn, B, H, splits);
    const size_t need = fa355::decode_workspace_bytes(B, H, splits, d);
    if (!workspace || misaligned(workspace, 16) || workspace_bytes < need)
        return fail(FA_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned and hold %zu bytes (got %zu at %p)",
                    fn, need, workspace_bytes, workspace);
    const Span ins[5] = {span("q", q, bh * d * 2), span("k_pages", k_pages, pool_el * 2),
                         span("v_pages", v_pages, pool_el * 2),
                         span("block_table", block_table, static_cast<unsigned __int128>(B) * max_pages * 4),
                         span("seq_lens", seq_lens, static_cast<unsigned __int128>(B) * 4)};
    const Span outs[2] = {span("o", o, bh * d * (out_f32 ? 4 : 2)), span("lse", lse, lse ? bh * 4 : 0)};
    for (const Span &os : outs) {
        if (os.hi <= os.lo) continue;
        for (const Span &is : ins)
            if (is.hi > is.lo && overlap(os, is)) return fail(FA_ERR_INVALID, "%s: %s overlaps %s", fn, os.name, is.name);
    }
    if (outs[1].hi > outs[1].lo && overlap(outs[0], outs[1])) return fail(FA_ERR_INVALID, "%s: lse overlaps o", fn);
    const Span ws = span("workspace", workspace, need);
    for (const Span &s : ins)
        if (s.hi > s.lo && overlap(ws, s)) return fail(FA_ERR_WORKSPACE, "%s: workspace overlaps %s", fn, s.name);
    for (const Span &s : outs)
        if (s.hi > s.lo && overlap(ws, s)) return fail(FA_ERR_WORKSPACE, "%s: workspace overlaps %s", fn, s.name);

    float *ws_o = static_cast<float *>(workspace);
    float *ws_lse = ws_o + static_cast<size_t>(B) * H * splits * d;
    fa355::DecodeArgs a{q, k_pages, v_pages, o, lse, B, H, max_seq_len, d, scale, elem, out_f32, splits, chunk,
                        ws_o, ws_lse};
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.num_pages = num_pages;
    a.page_size = page_size;
    a.max_pages = max_pages;
    a.layout = layout;
    if (log_enabled())
        std::fprintf(stderr,
                     "fa355: fa_decode_paged B=%d H=%d d=%d pages=%d page_size=%d max_pages=%d layout=%d "
                     "max_seq_len=%d dtype=0x%x splits=%d chunk=%d\n",
                     B, H, d, num_pages, page_size, max_pages, layout, max_seq_len, dtype, splits, chunk);
    const hipError_t err = fa355::launch_decode(a, stream);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
    return FA_OK;
}

size_t fa_bwd_workspace_size(int B, int H, int Nq)
{
    if (B < 0 || H < 0 || Nq < 0) return 0;
    // fa_bwd rejects B*H*Nq*d >= 2^62, so with d >= 64 no valid call has more rows
    if (static_cast<unsigned __int128>(B) * H * Nq >= (kMaxElems >> 6)) return 0;
    return fa355::bwd_workspace_bytes(B, H, Nq);
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
           void *dq, void *dk, void *dv, int B, int H, int Nq, int Nkv, int d, int causal, float scale,
           int dtype, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    static const char *fn = "fa_bwd";
    fa355::Elem elem;
    bool out_f32;
    int rc = parse_dtype(fn, dtype, &elem, &out_f32);
    if (rc) return rc;
    if ((rc = check_head_dim(fn, d))) return rc;
    if (B < 0 || H < 0 || Nq < 0 || Nkv < 0)
        return fail(FA_ERR_INVALID, "%s: negative size (B=%d H=%d Nq=%d Nkv=%d)", fn, B, H, Nq, Nkv);
    if (!std::isfinite(scale)) return fail(FA_ERR_INVALID, "%s: scale must be finite", fn);
    if (B == 0 || H == 0) return FA_OK;
    if (Nkv == 0) return fail(FA_ERR_INVALID, "%s: Nkv=0: attention over no keys is undefined", fn);
    if (causal && Nq > Nkv)
        return fail(FA_ERR_INVALID, "%s: causal attention needs Nq <= Nkv (got %d > %d)", fn, Nq, Nkv);
    // With no query rows only dk = dv = 0 is written: q, o, dout, lse and dq
    // are neither read nor written and may be NULL (as for fa_fwd).
    const bool rows = Nq > 0;
    const void *in16[5] = {q, k, v, o, dout};
    const bool in_needed[5] = {rows, true, true, rows, rows};
    void *outs[3] = {dq, dk, dv};
    const bool out_needed[3] = {rows, true, true};
    for (int i = 0; i < 5; ++i)
        if ((in_needed[i] && !in16[i]) || misaligned(in16[i], 16))
            return fail(FA_ERR_INVALID, "%s: q, k, v, o and dout must be non-NULL and 16-byte aligned", fn);
    for (int i = 0; i < 3; ++i)
        if ((out_needed[i] && !outs[i]) || misaligned(outs[i], 16))
            return fail(FA_ERR_INVALID, "%s: dq, dk and dv must be non-NULL and 16-byte aligned", fn);
    if ((rows && !lse) || misaligned(lse, 4))
        return fail(FA_ERR_INVALID, "%s: lse must be non-NULL and 4-byte aligned", fn);
    const unsigned __int128 bh = static_cast<unsigned __int128>(B) * H;
    const unsigned __int128 nq_el = bh * Nq * d, nkv_el = bh * Nkv * d;
    if (nq_el >= kMaxElems || nkv_el >= kMaxElems)
        return fail(FA_ERR_INVALID, "%s: tensor sizes exceed 2^62 elements", fn);
    const int oel = out_f32 ? 4 : 2;
    if (static_cast<unsigned long long>(Nkv) * d * oel > 0xffffffffULL ||
        static_cast<unsigned long long>(Nq) * d * oel > 0xffffffffULL)
        return fail(FA_ERR_UNSUPPORTED, "%s: one head of a tensor exceeds 4 GiB", fn);
    // the key-block and query-block passes: 256 threads per (b, h, 128-row
    // block); the row-statistics pass is grid-stride with a capped grid
    const unsigned long long items =
        static_cast<unsigned long long>(B) * H * ((std::max(Nq, Nkv) + 127) / 128) * 256ULL;
    if (items > fa355::kMaxWorkItems)
        return fail(FA_ERR_UNSUPPORTED, "%s: %llu work-items exceed HIP's grid limit of 2^32 - 1", fn, items);
    const size_t need = fa355::bwd_workspace_bytes(B, H, Nq);
    if (need && (!workspace || misaligned(workspace, 16) || workspace_bytes < need))
        return fail(FA_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned and hold %zu bytes (got %zu at %p)", fn,
                    need, workspace_bytes, workspace);
    const Span ins[6] = {span("q", q, nq_el * 2),    span("k", k, nkv_el * 2),      span("v", v, nkv_el * 2),
                         span("o", o, nq_el * 2),    span("dout", dout, nq_el * 2), span("lse", lse, bh * Nq * 4)};
    const Span outspans[3] = {span("dq", dq, nq_el * oel), span("dk", dk, nkv_el * oel), span("dv", dv, nkv_el * oel)};
    for (int i = 0; i < 3; ++i) {
        for (const Span &s : ins)
            if (outspans[i].hi > outspans[i].lo && s.hi > s.lo && overlap(outspans[i], s))
                return fail(FA_ERR_INVALID, "%s: %s overlaps %s", fn, outspans[i].name, s.name);
        for (int j = i + 1; j < 3; ++j)
            if (outspans[i].hi > outspans[i].lo && outspans[j].hi > outspans[j].lo && overlap(outspans[i], outspans[j]))
                return fail(FA_ERR_INVALID, "%s: %s overlaps %s", fn, outspans[i].name, outspans[j].name);
    }
    if (need) {
        const Span ws = span("workspace", workspace, need);
        for (const Span &s : ins)
            if (s.hi > s.lo && overlap(ws, s)) return fail(FA_ERR_WORKSPACE, "%s: workspace overlaps %s", fn, s.name);
        for (const Span &s : outspans)
            if (s.hi > s.lo && overlap(ws, s)) return fail(FA_ERR_WORKSPACE, "%s: workspace overlaps %s", fn, s.name);
    }

    float *ws_l2 = static_cast<float *>(workspace);
    float *ws_dd = ws_l2 ? ws_l2 + static_cast<size_t>(B) * H * Nq : nullptr;
    fa355::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nkv, d, causal != 0, scale, elem, out_f32,
                     ws_l2, ws_dd};
    if (log_enabled())
        std::fprintf(stderr, "fa355: fa_bwd B=%d H=%d Nq=%d Nkv=%d d=%d causal=%d dtype=0x%x\n", B, H, Nq, Nkv, d,
                     causal != 0, dtype);
    const hipError_t err = fa355::launch_bwd(a, stream);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
    return FA_OK;
}

const char *fa_status_str(int status)
{
    switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID: return "FA_ERR_INVALID";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_ERR_UNKNOWN";
    }
}

const char *fa_last_error(void) { return g_last_error.c_str(); }

int fa_version(void) { return FA355_VERSION; }

}  // extern "C"
