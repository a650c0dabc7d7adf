// Split-KV decode for gfx950: one query per (batch, head) against a long
// key/value cache ("Flash Attention -- Module 12.3", section "Prefill vs
// Decode").  A single query row leaves the matrix cores nothing to tile, so
// the path is a stream: its speed is the rate at which K and V leave HBM.
//
// Pass 1 (split kernel): the cache of every head is cut into `splits` chunks
// processed by independent workgroups ("FlashAttention 1-2-3: The IO-Aware
// Revolution in LLM Inference", section "Beyond FlashAttention: Future
// Directions and Alternatives": parallelise over the cache length, then
// reduce).  Inside a workgroup, each group of d/8 lanes owns a stream of
// keys; a lane holds 8 dimensions of q and reads the matching 16 bytes of
// every K and V row, so each wave-wide load covers whole consecutive rows.
// Scores come from packed 16-bit dot products with fp32 accumulation and a
// DPP reduction across the group; the group keeps its own online-softmax
// state (m, l, 8 accumulators per lane).  The groups are merged through LDS
// and the chunk's normalised partial output and base-2 log-sum-exp go to the
// workspace.
//
// The paged variant reads the cache through a block table: sequence b's key
// j sits in page block_table[b][j / page_size], slot j % page_size, of a pool
// of pages laid out [page][H][slot][d] or [page][slot][H][d] -- the cache of
// serving stacks that allocate it in fixed-size pages, each page one tile of
// the attention ("FlashAttention 1-2-3 ...", sections "Integration in Major
// Inference Engines" and "Beyond FlashAttention").  Each sequence has its own
// length (seq_lens[b], read on the device and clamped to the host's bound
// max_seq_len); chunks past it are empty and carry weight 0 into the combine.
//
// Pass 2 (combine kernel): per head, the partial results are merged exactly
// by their log-sum-exp values, the two-block merge of "FlashAttention 1-2-3
// ...", section "The Math Behind the Online Softmax Trick", applied to all
// chunks at once: O = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M).  With
// one split per head the split kernel writes O and LSE itself and pass 2 is
// not launched.
#include "fa_device.hpp"
#include "fa_internal.hpp"

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace fa355 {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecUnroll = 8;  // key rows in flight per lane group per iteration

struct SplitParams {
    const void *q, *k, *v;
    void *o;     // written directly when splits == 1
    float *lse;  // may be null
    float *ws_o, *ws_lse;
    int Nkv, chunk, splits, out_f32;
    float scale_log2;
    // paged cache only
    const int *block_table;  // [B][max_pages] page indices
    const int *seq_lens;     // [B] keys cached per sequence
    int H, num_pages, page_size, max_pages, max_len;
    unsigned div_magic;      // key / page_size == (key * div_magic) >> div_shift for key < 2^31
    int div_shift;
    size_t page_stride, head_stride, slot_stride;  // elements
};

// Key-row addressing of head bh, in two steps so that the memory reads of
// the first (the block table, for a paged cache) can be issued one iteration
// ahead of their use: ref(key) starts the lookup, offset(ref) gives the
// row's element offset in the cache.
//
// A contiguous [B*H][Nkv][D] cache needs no lookup.
template <int D> struct DenseRows {
    using Ref = int;
    size_t base;
    __device__ DenseRows(const SplitParams &p, int bh) : base(static_cast<size_t>(bh) * p.Nkv * D) {}
    __device__ Ref ref(int key) const { return key; }
    __device__ size_t offset(Ref key) const { return base + static_cast<size_t>(key) * D; }
};

// Element offset of key `key` of head bh in a paged cache: the page comes
// from the sequence's row of the block table, the slot is key mod page_size.
// Page indices are clamped to the pool, so a bad table reads wrong rows but
// never outside it.  The division by the page size is a multiply-high by a
// magic number (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): with l = ceil(log2 page_size) and
// m = ceil(2^(31+l) / page_size) < 2^32, floor(key * m / 2^(31+l)) is exact
// for every key < 2^31, because the rounding of m adds less than
// key / 2^(31+l) < 1 / page_size to key / page_size.
template <int D> struct PagedRows {
    struct Ref {
        int page, slot;
    };
    const int *table;
    size_t head_base, page_stride, slot_stride;
    unsigned magic;
    int shift, page_size, last_page;
    __device__ PagedRows(const SplitParams &p, int bh)
        : table(p.block_table + static_cast<size_t>(bh / p.H) * p.max_pages),
          head_base(static_cast<size_t>(bh % p.H) * p.head_stride), page_stride(p.page_stride),
          slot_stride(p.slot_stride), magic(p.div_magic), shift(p.div_shift), page_size(p.page_size),
          last_page(p.num_pages - 1)
    {
    }
    __device__ Ref ref(int key) const
    {
        const int t = static_cast<int>((static_cast<unsigned long long>(static_cast<unsigned>(key)) * magic) >> shift);
        return {table[t], key - t * page_size};
    }
    __device__ size_t offset(Ref r) const
    {
        const int page = min(max(r.page, 0), last_page);
        return head_base + static_cast<size_t>(page) * page_stride + static_cast<size_t>(r.slot) * slot_stride;
    }
};

template <int D, typename T, bool PAGED>
__global__ __launch_bounds__(64 * kDecWaves) void decode_split_kernel(SplitParams p)
{
    constexpr int LPK = D / 8;                 // lanes per key row
    constexpr int KPI = 64 / LPK;              // key rows per wave-wide load
    constexpr int GROUPS = kDecWaves * KPI;    // independent key streams per workgroup
    constexpr int STEP = GROUPS * kDecUnroll;  // keys per workgroup iteration

    const int split = blockIdx.x % p.splits;
    const int bh = blockIdx.x / p.splits;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane / LPK, r = lane % LPK;
    const int grp = w * KPI + g;
    const int ks = split * p.chunk;
    int n = p.Nkv;  // keys of this sequence
    if constexpr (PAGED) n = min(max(p.seq_lens[bh / p.H], 0), p.max_len);
    const int ke = min(n, ks + p.chunk);  // ke <= ks: a chunk past the sequence's end (empty)
    using Rows = typename std::conditional<PAGED, PagedRows<D>, DenseRows<D>>::type;
    const Rows row_of(p, bh);

    const T *Kg = static_cast<const T *>(p.k) + 8 * r;
    const T *Vg = static_cast<const T *>(p.v) + 8 * r;
    const u32x4 qv = *reinterpret_cast<const u32x4 *>(static_cast<const T *>(p.q) + static_cast<size_t>(bh) * D + 8 * r);

    float m = -INFINITY, l = 0.f;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;

    // Every lane reads a real row: a key past the chunk's end reads the
    // chunk's last row instead (and gets weight 0 below), so the loads need
    // no branch and the row lookups of the next iteration can be in flight
    // while this one computes.
    typename Rows::Ref ref[kDecUnroll];
    auto lookup = [&](int base) {
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) ref[u] = row_of.ref(min(base + u * GROUPS + grp, ke - 1));
    };
    if (ks < ke) lookup(ks);

    for (int base = ks; base < ke; base += STEP) {
        u32x4 kr[kDecUnroll], vr[kDecUnroll];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            // K and V are read once: non-temporal loads (measured on MI355X: a
            // plain streaming read reaches ~6.2 TB/s, a non-temporal one ~6.9)
            const size_t row = row_of.offset(ref[u]);
            kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(Kg + row));
            vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(Vg + row));
        }
        lookup(base + STEP);
        if (base + STEP > ke) {
            // the stand-in rows of keys past the end: zero values, so that a
            // weight of 0 contributes exactly 0 whatever the row holds
#pragma unroll
            for (int u = 0; u < kDecUnroll; ++u)
                if (base + u * GROUPS + grp >= ke) vr[u] = u32x4{0, 0, 0, 0};
        }
        float t[kDecUnroll];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) s = dot2<T>(qv[j], kr[u][j], s);
            s = group_sum<LPK>(s);
            const int key = base + u * GROUPS + grp;
            t[u] = key < ke ? s * p.scale_log2 : -INFINITY;
            mx = fmaxf(mx, t[u]);
        }
        const float m_new = fmaxf(m, mx);
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_ref);
        l *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= alpha;
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            const float pu = fast_exp2(t[u] - m_ref);
            l += pu;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[2 * j] += pu * lo_f32<T>(vr[u][j]);
                acc[2 * j + 1] += pu * hi_f32<T>(vr[u][j]);
            }
        }
        m = m_new;
    }

    // merge the workgroup's key streams
    __shared__ float s_m[GROUPS], s_l[GROUPS];
    __shared__ float s_acc[GROUPS][D];
    if constexpr (kPoisonLds) {
        // after the key loop, which uses no LDS: every thread is past it
        poison_lds(s_m, sizeof(s_m));
        poison_lds(s_l, sizeof(s_l));
        poison_lds(s_acc, sizeof(s_acc));
        __syncthreads();
    }
    if (r == 0) {
        s_m[grp] = m;
        s_l[grp] = l;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s_acc[grp][8 * r + j] = acc[j];
    __syncthreads();
    if (tid < D) {
        float M = -INFINITY;
        for (int G = 0; G < GROUPS; ++G) M = fmaxf(M, s_m[G]);
        float L = 0.f, o = 0.f;
        for (int G = 0; G < GROUPS; ++G) {
            const float wgt = fast_exp2(s_m[G] - M);  // 0 for a stream that saw no key
            L += s_l[G] * wgt;
            o += s_acc[G][tid] * wgt;
        }
        // an empty chunk (paged: past the sequence's end) contributes weight 0
        const float o_n = L > 0.f ? o / L : 0.f;
        const float lse2 = L > 0.f ? M + __builtin_amdgcn_logf(L) : -INFINITY;
        if (p.splits == 1) {
            // one chunk per head is the whole cache: its normalised output and
            // LSE are the result (the merge of one partial has weight 2^0 = 1)
            const size_t i = static_cast<size_t>(bh) * D + tid;
            if (p.out_f32)
                static_cast<float *>(p.o)[i] = o_n;
            else
                static_cast<T *>(p.o)[i] = static_cast<T>(o_n);
            if (tid == 0 && p.lse) p.lse[bh] = lse2 * kLn2;
        } else {
            const size_t slot = static_cast<size_t>(bh) * p.splits + split;
            p.ws_o[slot * D + tid] = o_n;
            if (tid == 0) p.ws_lse[slot] = lse2;
        }
    }
}

struct CombineParams {
    const float *ws_o, *ws_lse;
    void *o;
    float *lse;
    int splits;
};

// One workgroup per (batch, head).  All threads first take the largest
// partial LSE together; then group g of the kCombThreads / D groups of D
// threads (one per dimension) sums splits g, g + groups, ... with four loads
// in flight, and the groups' sums are added through LDS.  Few heads with many
// splits (a small batch over a long cache) thus cost a few microseconds
// instead of a serial walk over the splits.
constexpr int kCombThreads = 512;

template <int D, typename TO>
__global__ __launch_bounds__(kCombThreads) void decode_combine_kernel(CombineParams p)
{
    constexpr int G = kCombThreads / D;  // split groups
    constexpr int WAVES = kCombThreads / 64;
    __shared__ float s_max[WAVES];
    __shared__ float s_num[G][D];
    __shared__ float s_den[G];
    if constexpr (kPoisonLds) {
        poison_lds(s_max, sizeof(s_max));
        poison_lds(s_num, sizeof(s_num));
        poison_lds(s_den, sizeof(s_den));
        __syncthreads();
    }
    const int bh = blockIdx.x, t = threadIdx.x, d = t % D, g = t / D;
    const float *L = p.ws_lse + static_cast<size_t>(bh) * p.splits;
    const float *O = p.ws_o + static_cast<size_t>(bh) * p.splits * D + d;

    float m = -INFINITY;
    for (int s = t; s < p.splits; s += kCombThreads) m = fmaxf(m, L[s]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((t & 63) == 0) s_max[t >> 6] = m;
    __syncthreads();
    float M = s_max[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) M = fmaxf(M, s_max[w]);
    const float Mref = M == -INFINITY ? 0.f : M;  // every chunk empty: O = 0/0 below

    float den = 0.f, num = 0.f;
    int s = g;
    for (; s + 3 * G < p.splits; s += 4 * G) {
        float w[4], o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            w[u] = L[s + u * G];
            o[u] = O[static_cast<size_t>(s + u * G) * D];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float wu = fast_exp2(w[u] - Mref);
            den += wu;
            num += wu * o[u];
        }
    }
    for (; s < p.splits; s += G) {
        const float wu = fast_exp2(L[s] - Mref);
        den += wu;
        num += wu * O[static_cast<size_t>(s) * D];
    }
    s_num[g][d] = num;
    if (d == 0) s_den[g] = den;  // the same for every dimension of the group
    __syncthreads();
    if (g == 0) {
        num = s_num[0][d];
        den = s_den[0];
#pragma unroll
        for (int q = 1; q < G; ++q) {
            num += s_num[q][d];
            den += s_den[q];
        }
        // den == 0 only when every chunk was empty (a paged sequence of length
        // 0): attention over no key gives O = 0 and LSE = ln 0 = -inf
        static_cast<TO *>(p.o)[static_cast<size_t>(bh) * D + d] = static_cast<TO>(den > 0.f ? num / den : 0.f);
        if (d == 0 && p.lse) p.lse[bh] = den > 0.f ? (M + __builtin_amdgcn_logf(den)) * kLn2 : -INFINITY;
    }
}

template <int D, typename T, bool PAGED>
hipError_t launch(const DecodeArgs &a, hipStream_t stream)
{
    const int n_bh = a.B * a.H;
    SplitParams sp{};
    sp.q = a.q;
    sp.k = a.k;
    sp.v = a.v;
    sp.o = a.o;
    sp.lse = a.lse;
    sp.out_f32 = a.out_f32 ? 1 : 0;
    sp.ws_o = a.ws_o;
    sp.ws_lse = a.ws_lse;
    sp.Nkv = a.Nkv;
    sp.chunk = a.chunk;
    sp.splits = a.splits;
    sp.scale_log2 = a.scale * kLog2e;
    sp.block_table = a.block_table;
    sp.seq_lens = a.seq_lens;
    sp.H = a.H;
    sp.num_pages = a.num_pages;
    sp.page_size = a.page_size;
    sp.max_pages = a.max_pages;
    sp.max_len = a.Nkv;
    if (PAGED) {
        int l = 0;
        while ((1LL << l) < a.page_size) ++l;
        sp.div_magic = static_cast<unsigned>(((1ULL << (31 + l)) + a.page_size - 1) / a.page_size);
        sp.div_shift = 31 + l;
        const size_t ps = static_cast<size_t>(a.page_size), H = static_cast<size_t>(a.H);
        sp.page_stride = ps * H * D;
        sp.head_stride = a.layout == 0 ? ps * D : D;
        sp.slot_stride = a.layout == 0 ? D : H * D;
    }
    const dim3 grid1(static_cast<unsigned>(static_cast<long long>(n_bh) * a.splits));
    hipLaunchKernelGGL((decode_split_kernel<D, T, PAGED>), grid1, dim3(64 * kDecWaves), 0, stream, sp);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.splits == 1) return err;

    CombineParams cp;
    cp.ws_o = a.ws_o;
    cp.ws_lse = a.ws_lse;
    cp.o = a.o;
    cp.lse = a.lse;
    cp.splits = a.splits;
    if (a.out_f32)
        hipLaunchKernelGGL((decode_combine_kernel<D, float>), dim3(n_bh), dim3(kCombThreads), 0, stream, cp);
    else
        hipLaunchKernelGGL((decode_combine_kernel<D, T>), dim3(n_bh), dim3(kCombThreads), 0, stream, cp);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t stream)
{
    if (a.block_table)
        return a.elem == Elem::F16 ? launch<D, _Float16, true>(a, stream) : launch<D, __bf16, true>(a, stream);
    return a.elem == Elem::F16 ? launch<D, _Float16, false>(a, stream) : launch<D, __bf16, false>(a, stream);
}

}  // namespace

// Scratch of fa_decode_noalloc: the split partials of one call live in this
// file-scope device array instead of a caller workspace, so that callers that
// cannot allocate device memory can still run a split decode.  Each device
// holds its own copy for the life of the process.  In host code the array's
// name is only a stand-in: its device address comes from hipGetSymbolAddress,
// looked up once per device and kept below.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

int decode_auto_splits(int B, int H, int Nkv, int /*d*/)
{
    // Measured on MI355X (one process, interleaved): a long stream per
    // workgroup is cheapest, so the split count only has to give the chip
    // enough workgroups.  Four splits per head from 64 to 512 heads (the
    // 16 x 32 x 32K cache: 7.03 TB/s against 6.92 with 2K keys per split),
    // about 256 workgroups when there are fewer heads (one head of 1M keys:
    // 6.1 TB/s at 256 splits, 5.1 at 1024), one split once the heads alone
    // give about 2048 workgroups, and never fewer than ~128 keys per split.
    const long long n_bh = static_cast<long long>(B) * H;
    if (n_bh < 1 || Nkv < 1) return 1;
    long long s = std::max<long long>((256 + n_bh - 1) / n_bh, 4);
    s = std::min<long long>(s, std::max<long long>((2048 + n_bh - 1) / n_bh, 1));
    s = std::min<long long>(s, (static_cast<long long>(Nkv) + 127) / 128);
    return static_cast<int>(std::max<long long>(s, 1));
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    if (a.d == 64) return launch_d<64>(a, stream);
    if (a.d == 128) return launch_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa355
