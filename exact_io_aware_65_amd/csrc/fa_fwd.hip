// Fused exact attention forward (prefill) for gfx950.
//
// One workgroup owns one (batch*head, tile of BM query rows) pair and loops
// over key/value tiles of BN keys: Q-tiles outer and parallel, K/V tiles
// inner ("FlashAttention 1-2-3: The IO-Aware Revolution in LLM Inference",
// section "FlashAttention-2: Reducing Non-Matmul Overhead and Causal
// Efficiency").  Each K/V tile is copied once from HBM/L2 straight into LDS
// (global_load_lds, no register staging) while the previous tile is being
// consumed -- the double buffering of that page's section "FlashAttention-3"
// done with the gfx950 direct-to-LDS load.  The score tile lives only in
// registers and is consumed by an online softmax (running max m, running sum
// l, rescaled accumulator: "FlashAttention", section "Online softmax: the
// enabling trick"), so only O and the per-row log-sum-exp are written back.
// With a causal mask, tiles that no row of the workgroup can see are never
// loaded, and only tiles that straddle the diagonal (or the ragged end of
// the keys) pay for a mask.
//
// Per wave (32 query rows), per 32-key sub-tile, on the 32x32x16 MFMA:
//   S^T (32 keys x 32 queries) = K_sub (32 x d) * Q^T (d x 32)
// so every lane owns one query column: lane l holds query l % 32 and 16 of
// the 32 keys (half h = l / 32).  Row max and row sum are in-lane reductions
// plus one exchange with lane l ^ 32.  The K rows are fed to the MFMA in the
// order that makes a lane's 16 scores the keys {8h..8h+7} and {16+8h..16+8h+7},
// which is exactly the k-slot layout the second product needs, so P goes from
// the score accumulator to the MFMA operand without any lane movement:
//   O^T (32 dims x 32 queries) += V^T (32 dims x 16 keys) * P^T (16 keys x 32 queries)
// V stays [key][dim] in LDS; its transposed operand comes from two
// ds_read_b64_tr_b16 reads per MFMA.
//
// Softmax work per score: one max (three-input), one FMA (scale folded in,
// base-2 domain), one exp2, one add for the fp32 row sum and half a pack to
// 16 bits.  The accumulator is rescaled only when some row's
// maximum grows by more than 2^8 over the value in use; otherwise the stale
// maximum is kept, which bounds every probability by 2^8 and leaves the final
// O = acc / l exact, because numerator and denominator share the factor.
#include "fa_device.hpp"
#include "fa_internal.hpp"

#include <type_traits>

namespace fa355 {
namespace {

constexpr int kBN = 64;                // keys per tile
constexpr int kNW = 4;                 // waves per workgroup (32 query rows each)
constexpr float kRescaleSlack = 8.0f;  // log2 of the largest probability kept without rescaling

struct FwdParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int Nq, Nkv;
    int n_bh, n_qt;
    float c;         // |scale| * log2(e): scores are kept in the base-2 domain
    uint32_t qsign;  // 0x80008000 when scale < 0: Q is negated as it is loaded
};

// The MFMA row that lane l % 32 feeds is key swap23(l % 32) of the sub-tile
// (bits 2 and 3 exchanged); see the file comment.
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// XOR swizzles of the 16-byte chunk index of a row in LDS.  K: eight lanes
// reading one chunk column of rows swap23(0..7) hit eight bank groups.  V:
// the 16 lanes of a transposed read touch 4 consecutive rows x 2 adjacent
// chunks, which this spreads over all 32 banks.
__device__ __forceinline__ int kswz(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int vswz(int row) { return (row & 3) << 1; }

template <int D, typename T, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdParams p)
{
    constexpr int BN = kBN, BM = 32 * kNW, NT = 64 * kNW;
    constexpr int DC = D / 8;            // 16-byte chunks per row
    constexpr int TILE = BN * DC;        // chunks per K (or V) tile
    constexpr int LOADS = TILE / NT;     // direct loads per thread per tensor per tile
    constexpr int ROWB = D * 2;          // bytes per row
    static_assert(TILE % NT == 0 && LOADS >= 1, "tile must split evenly over the threads");
    using V8 = typename Vec<T>::v8;

    __shared__ u32x4 sk0[TILE], sk1[TILE];  // K tiles [key][dim], chunk-swizzled (two stages)
    __shared__ u32x4 sv0[TILE], sv1[TILE];  // V tiles [key][dim], chunk-swizzled

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform by construction
    const int c = lane & 31, h = lane >> 5;

    // Heaviest causal tiles (last query rows) are dispatched first.  Consecutive
    // workgroups cycle through heads, so when B*H is a multiple of the XCD count
    // every tile of one head lands on one XCD and shares its L2.
    const int bh = blockIdx.x % p.n_bh;
    const int qt = p.n_qt - 1 - static_cast<int>(blockIdx.x / p.n_bh);
    const int q0 = qt * BM;
    const int wq0 = q0 + 32 * wave;
    const int off = p.Nkv - p.Nq;  // causal: row i sees keys j <= i + off
    int kend = p.Nkv;
    if constexpr (CAUSAL) kend = min(p.Nkv, min(q0 + BM, p.Nq) + off);
    const int nkb = (kend + BN - 1) / BN;

    // Per-head buffer descriptors: reads past a head's last row return zeros,
    // which fills the ragged end of the last tile (those keys are masked) and
    // the query rows past Nq.
    const size_t q_head = static_cast<size_t>(bh) * p.Nq * ROWB;
    const size_t kv_head = static_cast<size_t>(bh) * p.Nkv * ROWB;
    const auto rq = make_rsrc(static_cast<const char *>(p.q) + q_head, static_cast<uint32_t>(p.Nq) * ROWB);
    const auto rk = make_rsrc(static_cast<const char *>(p.k) + kv_head, static_cast<uint32_t>(p.Nkv) * ROWB);
    const auto rv = make_rsrc(static_cast<const char *>(p.v) + kv_head, static_cast<uint32_t>(p.Nkv) * ROWB);

    // Q operand, loaded once: lane (c, h) holds query wq0 + c, dims 16 s + 8 h .. + 7.
    const int qrow = wq0 + c;
    V8 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        const u32x4 x = buffer_load16(rq, qrow * ROWB + (16 * s + 8 * h) * 2, 0) ^ p.qsign;
        qf[s] = as<V8>(x);
    }

    // Direct loads: the wave's i-th load fills LDS chunks [(wave*LOADS + i)*64, +64),
    // lane by lane; the lane fetches whichever global chunk the swizzle puts there.
    uint32_t koff[LOADS], voff[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int pch = (wave * LOADS + i) * 64 + lane;
        const int row = pch / DC, col = pch % DC;
        koff[i] = row * ROWB + (col ^ kswz(row)) * 16;
        voff[i] = row * ROWB + (col ^ vswz(row)) * 16;
    }
    auto issue = [&](auto stage_, int kb) {
        constexpr int S = decltype(stage_)::value;
        u32x4 *dk = S ? sk1 : sk0;
        u32x4 *dv = S ? sv1 : sv0;
        const uint32_t tile = static_cast<uint32_t>(kb) * BN * ROWB;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            buffer_to_lds16(rk, koff[i], tile, dk + (wave * LOADS + i) * 64);
            buffer_to_lds16(rv, voff[i], tile, dv + (wave * LOADS + i) * 64);
        }
    };

    // LDS byte addresses of this lane's MFMA operands, as a few bases plus
    // compile-time offsets.  K operand (kk, s): row 32 kk + swap23(c), chunk
    // (2 s + h) ^ kswz(row); s and s + 4 differ by 8 chunks, kk by 32 rows.
    uint32_t ka[4];
    {
        const int krow = swap23(c);
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[s] = krow * ROWB + (((2 * s + h) ^ kswz(krow)) << 4);
    }
    // V^T operand: lane 16 g + 4 j + q addresses key 8 (g / 2) + j (+4, +16 u,
    // +32 kk) and dims 32 dt + 16 (g % 2) + 4 q; with the swizzle the chunk is
    // 4 (dt ^ (j / 2)) + ((2 (g % 2) + q / 2) ^ 2 (j % 2)), so dt = 0, 1 need
    // their own base and dt = 2, 3 add 128 bytes.
    uint32_t va[2];
    {
        const int tg = lane >> 4, tj = (lane >> 2) & 3, tq = lane & 3;
        const int base = (8 * (tg >> 1) + tj) * ROWB + ((tq & 1) << 3);
        const int y = (2 * (tg & 1) + (tq >> 1)) ^ (2 * (tj & 1));
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) va[dt] = base + ((4 * (dt ^ (tj >> 1)) + y) << 4);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
    float m_run = -INFINITY;  // row max (base-2 scaled) the probabilities are taken against
    float l_run = 0.f;        // running sum over this lane's half of the keys

    auto compute = [&](auto stage_, int kv0) {
        constexpr int S = decltype(stage_)::value;
        const char *SK = reinterpret_cast<const char *>(S ? sk1 : sk0);
        const char *SV = reinterpret_cast<const char *>(S ? sv1 : sv0);

        // S^T = K Q^T for the two 32-key sub-tiles
        f32x16 sacc[BN / 32];
#pragma unroll
        for (int kk = 0; kk < BN / 32; ++kk) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kk][e] = 0.f;
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const u32x4 x = *reinterpret_cast<const u32x4 *>(SK + ka[s & 3] + (s >> 2) * 128 + kk * 32 * ROWB);
                sacc[kk] = mfma32(as<V8>(x), qf[s], sacc[kk]);
            }
        }

        // causal diagonal / ragged end: invisible keys get -inf
        const bool need_mask = (kv0 + BN > p.Nkv) || (CAUSAL && kv0 + BN - 1 > wq0 + off);
        if (need_mask) {
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = kv0 + 32 * kk + 16 * (e >> 3) + 8 * h + (e & 7);
                    if (key >= p.Nkv || (CAUSAL && key > qrow + off)) sacc[kk][e] = -INFINITY;
                }
        }

        // block max (raw scores; c >= 0), then the lazy rescale
        float mx = sacc[0][0];
#pragma unroll
        for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kk][e]);
        mx = max_with_other_half(mx);
        const float m_blk = mx == -INFINITY ? -INFINITY : mx * p.c;
        if (__builtin_amdgcn_ballot_w64(m_blk > m_run + kRescaleSlack)) {
            const float m_new = fmaxf(m_run, m_blk);
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
            m_run = m_new;
        }
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;

        // p = 2^(c s - m); the row sum is taken in fp32 before rounding P
        float rs = 0.f;
        if (need_mask) {
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float x = sacc[kk][e];
                    sacc[kk][e] = x == -INFINITY ? 0.f : fast_exp2(fmaf(x, p.c, neg_m));
                    rs += sacc[kk][e];
                }
        } else {
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    sacc[kk][e] = fast_exp2(fmaf(sacc[kk][e], p.c, neg_m));
                    rs += sacc[kk][e];
                }
        }
        l_run += rs;

        // P to the storage type: operand (kk, u) holds keys 32 kk + 16 u + 8 h .. + 7.
        V8 pf[BN / 32][2];
#pragma unroll
        for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                u32x4 w;
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = pack2<T>(sacc[kk][8 * u + 2 * j], sacc[kk][8 * u + 2 * j + 1]);
                pf[kk][u] = as<V8>(w);
            }

        // O^T += V^T P^T (two transposed reads per operand: keys +0..3 and +4..7)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const char *pa = SV + va[dt & 1] + (dt >> 1) * 128 + (32 * kk + 16 * u) * ROWB;
                    const u32x2 lo = lds_read_tr16(pa);
                    const u32x2 hi = lds_read_tr16(pa + 4 * ROWB);  // rows + 4: same swizzle
                    const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[dt] = mfma32(as<V8>(a), pf[kk][u], oacc[dt]);
                }
        }
    };

    auto step = [&](auto stage_, int kb) {
        constexpr int S = decltype(stage_)::value;
        if (kb + 1 < nkb) issue(std::integral_constant<int, S ^ 1>{}, kb + 1);
        const int kv0 = kb * BN;
        const bool active = wq0 < p.Nq && (!CAUSAL || kv0 <= wq0 + 31 + off);
        if (active) compute(stage_, kv0);
        wait_vmem();
        __syncthreads();
    };

    if (nkb > 0) issue(std::integral_constant<int, 0>{}, 0);
    wait_vmem();
    __syncthreads();
    for (int kb = 0; kb < nkb; kb += 2) {
        step(std::integral_constant<int, 0>{}, kb);
        if (kb + 1 < nkb) step(std::integral_constant<int, 1>{}, kb + 1);
    }

    // Epilogue: O = acc / l, LSE = ln 2 * (m + log2 l).
    const float l_tot = sum_with_other_half(l_run);
    if (qrow < p.Nq) {
        const float inv = 1.f / l_tot;
        const size_t orow = (static_cast<size_t>(bh) * p.Nq + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 32 * dt + 8 * j + 4 * h;
                const float a0 = oacc[dt][4 * j] * inv, a1 = oacc[dt][4 * j + 1] * inv;
                const float a2 = oacc[dt][4 * j + 2] * inv, a3 = oacc[dt][4 * j + 3] * inv;
                if constexpr (OUT_F32) {
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + orow + d0) = f32x4{a0, a1, a2, a3};
                } else {
                    *reinterpret_cast<u32x2 *>(static_cast<T *>(p.o) + orow + d0) =
                        u32x2{pack2<T>(a0, a1), pack2<T>(a2, a3)};
                }
            }
        if (h == 0 && p.lse) {
            const float m = m_run == -INFINITY ? 0.f : m_run;
            p.lse[static_cast<size_t>(bh) * p.Nq + qrow] = (m + __builtin_amdgcn_logf(l_tot)) * kLn2;
        }
    }
}

template <int D, typename T, bool CAUSAL, bool OUT_F32>
hipError_t launch(const FwdArgs &a, hipStream_t stream)
{
    constexpr int BM = 32 * kNW;
    FwdParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.o = a.o;
    p.lse = a.lse;
    p.Nq = a.Nq;
    p.Nkv = a.Nkv;
    p.n_bh = a.B * a.H;
    p.n_qt = (a.Nq + BM - 1) / BM;
    p.c = (a.scale < 0.f ? -a.scale : a.scale) * kLog2e;
    p.qsign = a.scale < 0.f ? 0x80008000u : 0u;
    const dim3 grid(static_cast<unsigned>(static_cast<long long>(p.n_bh) * p.n_qt));
    hipLaunchKernelGGL((fwd_kernel<D, T, CAUSAL, OUT_F32>), grid, dim3(64 * kNW), 0, stream, p);
    return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_dt(const FwdArgs &a, hipStream_t stream)
{
    if (a.causal)
        return a.out_f32 ? launch<D, T, true, true>(a, stream) : launch<D, T, true, false>(a, stream);
    return a.out_f32 ? launch<D, T, false, true>(a, stream) : launch<D, T, false, false>(a, stream);
}

template <int D>
hipError_t launch_d(const FwdArgs &a, hipStream_t stream)
{
    return a.elem == Elem::F16 ? launch_dt<D, _Float16>(a, stream) : launch_dt<D, __bf16>(a, stream);
}

}  // namespace

int fwd_rows_per_block(int) { return 32 * kNW; }

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream)
{
    if (a.d == 64) return launch_d<64>(a, stream);
    if (a.d == 128) return launch_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa355
