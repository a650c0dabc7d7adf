// Fused exact attention forward (prefill) for gfx950.
//
// One workgroup owns one (batch*head, tile of BM query rows) pair and loops
// over key/value tiles of BN keys: Q-tiles outer and parallel, K/V tiles
// inner ("FlashAttention 1-2-3: The IO-Aware Revolution in LLM Inference",
// section "FlashAttention-2: Reducing Non-Matmul Overhead and Causal
// Efficiency").  Each K/V tile is staged once in LDS and shared by the
// workgroup's waves; the score tile lives only in registers and is consumed
// by an online softmax (running max m, running sum l, rescaled accumulator:
// "FlashAttention", section "Online softmax: the enabling trick"), so only O
// and the per-row log-sum-exp are written back.  With a causal mask, tiles
// that no row of the workgroup can see are never loaded, and only tiles that
// straddle the diagonal (or the ragged end of the keys) pay for a mask.
//
// Per wave (32 query rows), per 32-key sub-tile, on the 32x32x16 MFMA:
//   S^T (32 keys x 32 queries) = K_sub (32 x d) * Q^T (d x 32)
// so every lane owns one query column: lane l holds query l % 32 and 16 of
// the 32 keys (half l / 32).  Row max and row sum are in-lane reductions plus
// one exchange with lane l ^ 32.  The K rows are fed to the MFMA in the order
// that makes a lane's 16 scores the keys {8h..8h+7} and {16+8h..16+8h+7},
// which is exactly the k-slot layout the second product needs, so P goes from
// the score accumulator to the MFMA operand without any lane movement:
//   O^T (32 dims x 32 queries) += V^T (32 dims x 16 keys) * P^T (16 keys x 32 queries)
// V is transposed into LDS as [dim][key] on its way in.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa355 {
namespace {

constexpr int kBN = 64;  // keys per tile
constexpr int kNW = 4;   // waves per workgroup (32 query rows each)

struct FwdParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int Nq, Nkv;
    int n_bh, n_qt;
    float scale_log2;  // scale * log2(e): scores are kept in the base-2 domain
};

// The MFMA row that lane l % 32 feeds is key swap23(l % 32) of the sub-tile
// (bits 2 and 3 exchanged); see the file comment.
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// XOR swizzle of the 16-byte chunk index of K row `row` in LDS.  Eight lanes
// that read one chunk column of rows swap23(0..7) (or swap23(8..15), ...) hit
// eight different bank groups.
__device__ __forceinline__ int kswz(int row) { return (row & 3) | ((row >> 1) & 4); }

template <int D, typename T, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(64 * kNW) void fwd_kernel(FwdParams p)
{
    constexpr int BN = kBN, BM = 32 * kNW, NT = 64 * kNW;
    constexpr int DC = D / 8;         // 16-byte chunks per K row
    constexpr int KC = BN / 8;        // 16-byte chunks per V^T row
    constexpr int NVB = KC * DC;      // V is loaded as 8x8 blocks, one per V-loading thread
    constexpr int NKT = BN * DC / 8;  // K-loading threads, 8 chunks each
    static_assert(NVB + NKT <= NT, "not enough threads to load a tile");
    static_assert(KC == 8, "V^T swizzle assumes 8 chunks per row");
    using V8 = typename Vec<T>::v8;

    __shared__ u32x4 sk[2][BN * DC];  // K tile [key][dim], chunk-swizzled, double-buffered
    __shared__ u32x4 sv[2][D * KC];   // V tile transposed [dim][key], chunk-swizzled

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

    const T *Q = static_cast<const T *>(p.q) + static_cast<size_t>(bh) * p.Nq * D;
    const T *Kg = static_cast<const T *>(p.k) + static_cast<size_t>(bh) * p.Nkv * D;
    const T *Vg = static_cast<const T *>(p.v) + static_cast<size_t>(bh) * p.Nkv * D;

    // Q operand, loaded once: lane (c, h) holds query wq0 + c, dims 16 s + 8 h .. + 7.
    const int qrow = wq0 + c;
    V8 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        u32x4 x = {0, 0, 0, 0};
        if (qrow < p.Nq) x = *reinterpret_cast<const u32x4 *>(Q + static_cast<size_t>(qrow) * D + 16 * s + 8 * h);
        qf[s] = as<V8>(x);
    }

    // Tile loading: threads [0, NVB) each move one 8-key x 8-dim block of V
    // (eight coalesced row reads, transposed in registers, eight LDS chunk
    // writes); threads [NVB, NVB + NKT) each move eight chunks of K.
    const bool v_loader = tid < NVB;
    const bool k_loader = !v_loader && tid < NVB + NKT;
    const int vg = tid % KC, vc = tid / KC;  // V block: key group, dim chunk
    const int kt = tid - NVB;
    u32x4 stage_regs[8];

    auto fetch = [&](int kb) {
        const int kv0 = kb * BN;
        if (v_loader) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = kv0 + 8 * vg + i;
                u32x4 x = {0, 0, 0, 0};
                if (row < p.Nkv) x = *reinterpret_cast<const u32x4 *>(Vg + static_cast<size_t>(row) * D + 8 * vc);
                stage_regs[i] = x;
            }
        } else if (k_loader) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = kt + i * NKT;
                const int row = kv0 + idx / DC, ch = idx % DC;
                u32x4 x = {0, 0, 0, 0};
                if (row < p.Nkv) x = *reinterpret_cast<const u32x4 *>(Kg + static_cast<size_t>(row) * D + 8 * ch);
                stage_regs[i] = x;
            }
        }
    };
    auto commit = [&](int stage) {
        if (v_loader) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u32x4 out;
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    const uint32_t a = stage_regs[2 * pp][e >> 1], b = stage_regs[2 * pp + 1][e >> 1];
                    out[pp] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
                }
                const int d = 8 * vc + e;
                sv[stage][d * KC + (vg ^ (d & 7))] = out;
            }
        } else if (k_loader) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = kt + i * NKT;
                const int row = idx / DC, ch = idx % DC;
                sk[stage][row * DC + (ch ^ kswz(row))] = stage_regs[i];
            }
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
    float m_run = -INFINITY;  // running row max of scale*log2(e)*score
    float l_run = 0.f;        // running sum over this lane's half of the keys

    if (nkb > 0) {
        fetch(0);
        commit(0);
    }
    __syncthreads();

    for (int kb = 0; kb < nkb; ++kb) {
        const int stage = kb & 1;
        if (kb + 1 < nkb) fetch(kb + 1);
        const int kv0 = kb * BN;
        const bool active = wq0 < p.Nq && (!CAUSAL || kv0 <= wq0 + 31 + off);
        if (active) {
            // S^T = K Q^T for the two 32-key sub-tiles
            f32x16 sacc[BN / 32];
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk) {
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[kk][e] = 0.f;
                const int krow = 32 * kk + swap23(c);
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
                    const V8 a = as<V8>(sk[stage][krow * DC + ((2 * s + h) ^ kswz(krow))]);
                    sacc[kk] = mfma32(a, qf[s], sacc[kk]);
                }
            }

            // mask (diagonal / ragged tiles only), scale, running max
            const bool need_mask = (kv0 + BN > p.Nkv) || (CAUSAL && kv0 + BN - 1 > wq0 + off);
            float mx = -INFINITY;
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float t = sacc[kk][e] * p.scale_log2;
                    if (need_mask) {
                        const int key = kv0 + 32 * kk + 16 * (e >> 3) + 8 * h + (e & 7);
                        if (key >= p.Nkv || (CAUSAL && key > qrow + off)) t = -INFINITY;
                    }
                    sacc[kk][e] = t;
                    mx = fmaxf(mx, t);
                }
            mx = max_with_other_half(mx);
            const float m_new = fmaxf(m_run, mx);
            const float m_ref = m_new == -INFINITY ? 0.f : m_new;  // row with no visible key yet
            const float alpha = fast_exp2(m_run - m_ref);
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[kk][e] = fast_exp2(sacc[kk][e] - m_ref);

            // P to the storage type: operand (kk, u) holds keys 32 kk + 16 u + 8 h .. + 7.
            // The row sum is taken over the rounded values, so the final division
            // normalises exactly the weights that multiply V.
            V8 pf[BN / 32][2];
            float rs = 0.f;
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    u32x4 w;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        w[j] = pack2<T>(sacc[kk][8 * u + 2 * j], sacc[kk][8 * u + 2 * j + 1]);
                        rs = dot2<T>(w[j], kOnePair<T>, rs);
                    }
                    pf[kk][u] = as<V8>(w);
                }
            l_run = l_run * alpha + rs;
            m_run = m_new;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;

            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const int d = 32 * dt + c;
#pragma unroll
                for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int kc = 4 * kk + 2 * u + h;
                        const V8 a = as<V8>(sv[stage][d * KC + (kc ^ (d & 7))]);
                        oacc[dt] = mfma32(a, pf[kk][u], oacc[dt]);
                    }
            }
        }
        if (kb + 1 < nkb) commit(stage ^ 1);
        __syncthreads();
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
        if (h == 0 && p.lse)
            p.lse[static_cast<size_t>(bh) * p.Nq + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
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
    p.scale_log2 = a.scale * kLog2e;
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
