// Attention backward for gfx950: dQ, dK, dV given dL/dO, from the forward's
// inputs, its output O and its per-row log-sum-exp.
//
// The forward keeps only one statistic per query row (LSE) instead of the
// softmax matrix, and the backward recomputes P tile by tile from it ("FlashAttention
// 1-2-3: The IO-Aware Revolution in LLM Inference", section "FlashAttention-1:
// Tiling, Recomputation, and Online Softmax"); like the forward it never
// writes an Nq x Nkv matrix to HBM ("Flash Attention -- Module 12.3", section
// "Training").  With z = scale * q.k, P = exp(z - LSE) and the chain rule:
//
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO[i][c] O[i][c] (= sum_j P_ij dP_ij),
//   dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Three kernels, all on one stream:
//   bwd_prep_kernel   per query row: D_i and the base-2 LSE, into the workspace;
//   bwd_dkdv_kernel   key blocks outer (each wave owns 32 keys, K and V in
//                     registers), query tiles streamed through LDS; accumulates
//                     dV^T += dO^T P and dK^T += Q^T dS in registers;
//   bwd_dq_kernel     query blocks outer (each wave owns 32 queries, Q and dO
//                     in registers), key tiles streamed through LDS;
//                     accumulates dQ^T += K^T dS^T.
// The two passes come in two forms: bwd_dkdv16_kernel and bwd_dq16_kernel on
// the 16x16x32 MFMA (d = 128, and d = 64 once the grid gives every CU two
// workgroups), and the 32x32x16 kernels named above for the small d = 64
// grids.  Recomputing S and dP in both passes costs 7 products instead of 5,
// but no partial sums cross workgroups: no atomics, results are
// deterministic.
//
// MFMA layouts (32x32x16, lane l holds column l % 32 of the accumulator):
//   dK/dV kernel: S = Q K^T with the Q rows fed in swap23 order, so a lane
//     holds, for its key, the queries {8h..8h+7, 16+8h..16+8h+7}: exactly the
//     B-operand k-slots of dV^T = dO^T P and dK^T = Q^T dS, so P and dS go to
//     the second products without lane movement (as P does in the forward).
//   dQ kernel: S^T = K Q^T, as in the forward; dS^T is the B operand of
//     dQ^T = K^T dS^T.
// Tiles read both as rows (b128) and transposed (ds_read_b64_tr_b16) -- Q and
// dO in the dK/dV kernel, K in the dQ kernel -- use a chunk permutation that
// is conflict-free for both reads (see dswz).
#include "fa_device.hpp"
#include "fa_internal.hpp"

#include <algorithm>
#include <type_traits>

namespace fa355 {
namespace {

#ifndef FA355_DKDV16
#define FA355_DKDV16 1
#endif
#ifndef FA355_DQ16
#define FA355_DQ16 1
#endif
#ifndef FA355_BWD16_D64
#define FA355_BWD16_D64 1
#endif
constexpr long long kPrepMaxBlocks = 65536;  // prep grid cap (grid-stride beyond)
// At d = 64 the 16x16x32 passes are faster once the grid gives every CU two
// workgroups (8K causal fp16: 679 -> 710 TFLOP/s, 16K bf16: 736 -> 763, at two
// waves per SIMD), and slower below that (2K, B H = 16, one workgroup per CU:
// 258 -> 235), where the 32x32 passes, whose key-block pass covers 64-row
// query tiles, stay.
constexpr long long kBwd16MinBlocksD64 = 2 * 256;
// Waves per SIMD of the 16x16x32 passes: at d = 64 they fit 168 registers, so
// three workgroups share a CU (8K fp16: 721 -> 772 TFLOP/s, 4K: 645 -> 717,
// against two); at d = 128 they need 218-250.
template <int D> constexpr int kBwd16Waves = D == 64 ? 3 : 2;
constexpr float kBwdMinC = 1e-30f;  // as the forward: a zero scale keeps -inf * c = -inf

struct BwdParams {
    const void *q, *k, *v, *dout;
    void *dq, *dk, *dv;
    const float *l2;   // [BH][Nq] LSE * log2(e)
    const float *dd;   // [BH][Nq] D_i = rowsum(dO * O)
    int Nq, Nkv, n_bh, n_tiles;
    float c;           // max(|scale| * log2(e), kBwdMinC)
    float scale;       // signed scale: the dQ and dK factor
    uint32_t sign;     // 0x80008000 when scale < 0: K (dK/dV kernel) or Q (dQ kernel) is negated on load
};

struct PrepParams {
    const void *o, *dout;
    const float *lse;
    float *l2, *dd;
    long long rows;
};

// The MFMA row that lane l % 32 feeds is row swap23(l % 32) of the tile.
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// Chunk permutations (XOR on the 16-byte chunk index of a row).
// kswz: rows read as 16-byte runs only (a b128 group of 16 lanes holds rows
// swap23 of its lanes, 16 rows with distinct low four bits).
// dswz: rows read both as 16-byte runs and transposed (32 lanes covering 4
// consecutive rows x 64 bytes).  d = 128: the row's low nibble with its two
// halves exchanged; d = 64: bit 1 of the row to chunk bit 2, bits 2-3 to
// chunk bits 0-1 (two rows share a 256-byte bank line).
template <int D> __device__ __forceinline__ int kswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D> __device__ __forceinline__ int dswz(int row)
{
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// ---------------------------------------------------------------------------
// Per query row: D = sum_c dO * O (fp32 from the 16-bit values) and LSE in
// base 2.  D/8 lanes per row, 16 bytes each.

template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(PrepParams p)
{
    constexpr int LPR = D / 8, RPB = 256 / LPR;
    const int tid = threadIdx.x, part = tid % LPR;
    // grid-stride over blocks of RPB rows (the grid is capped on the host);
    // the bound is the same for every lane of a row group, so the DPP sum
    // below always runs with whole groups
    const long long stride = static_cast<long long>(gridDim.x) * RPB;
    for (long long row = static_cast<long long>(blockIdx.x) * RPB + tid / LPR; row - tid / LPR < p.rows;
         row += stride) {
        float acc = 0.f;
        if (row < p.rows) {
            const size_t off = static_cast<size_t>(row) * D * 2 + part * 16;
            const u32x4 o = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.o) + off);
            const u32x4 g = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.dout) + off);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = dot2<T>(o[j], g[j], acc);
        }
        acc = group_sum<LPR>(acc);
        if (part == 0 && row < p.rows) {
            p.dd[row] = acc;
            p.l2[row] = p.lse[row] * kLog2e;
        }
    }
}

// ---------------------------------------------------------------------------
// dK, dV: key blocks of 128 (4 waves x 32 keys), query tiles through a
// two-stage LDS ring.  Two waves per SIMD, so that one wave's softmax runs
// beside the other's MFMAs: K and the dK, dV accumulators stay in registers,
// and for d = 128 V moves to LDS (read as the forward reads K) and the query
// tiles shrink to 32 rows, which keeps a workgroup's LDS within half a CU's.

template <int D, typename T, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdParams p)
{
    constexpr bool VLDS = D == 128;  // V operand from LDS rather than registers
    constexpr int NW = 4, BK = 32 * NW, BQ = VLDS ? 32 : 64, NQQ = BQ / 32, NT = 64 * NW;
    constexpr int DC = D / 8, TILE = BQ * DC, LOADS = TILE / NT, ROWB = 2 * D, KS = D / 16, DT = D / 32;
    static_assert(TILE % NT == 0 && (BK * DC) % NT == 0, "tiles must split evenly over the threads");
    using V8 = typename Vec<T>::v8;

    __shared__ u32x4 sq[2][TILE];   // Q tiles [query][dim], dswz-permuted
    __shared__ u32x4 sdo[2][TILE];  // dO tiles [query][dim], dswz-permuted
    // base-2 LSE and D of the tile's queries; wave 0 fills them with one
    // 64-lane dword load each, so each stage holds 64 entries (with BQ = 32
    // the second half is the next tile's, unused)
    constexpr int LQ = BQ < 64 ? 64 : BQ;
    static_assert(LQ == 64, "one wave-wide dword load per stage");
    __shared__ float sl2[2][LQ];
    __shared__ float sdd[2][LQ];
    __shared__ u32x4 sv[VLDS ? BK * DC : 1];  // the block's V [key][dim], kswz-permuted
    if constexpr (kPoisonLds) {
        poison_lds(sq, sizeof(sq));
        poison_lds(sdo, sizeof(sdo));
        poison_lds(sl2, sizeof(sl2));
        poison_lds(sdd, sizeof(sdd));
        poison_lds(sv, sizeof(sv));
        __syncthreads();
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, h = lane >> 5;

    // Causal: key blocks near the start see the most queries; they go first.
    const int bh = blockIdx.x % p.n_bh;
    const int kt = static_cast<int>(blockIdx.x / p.n_bh);
    const int k0 = kt * BK;
    const int kw0 = k0 + 32 * wave;
    const int key = kw0 + c;
    const int off = p.Nkv - p.Nq;  // row i sees keys j <= i + off
    const int nqt = (p.Nq + BQ - 1) / BQ;
    // first query tile any key of the block can be seen from; a wave's own first query row
    const int t0 = CAUSAL ? max(0, k0 - off) / BQ : 0;
    const int wfirst = CAUSAL ? kw0 - off : 0;

    const size_t qh = static_cast<size_t>(bh) * p.Nq * ROWB, kh = static_cast<size_t>(bh) * p.Nkv * ROWB;
    const u32x4 rq = make_rsrc_words(static_cast<const char *>(p.q) + qh, static_cast<uint32_t>(p.Nq) * ROWB);
    const u32x4 rdo = make_rsrc_words(static_cast<const char *>(p.dout) + qh, static_cast<uint32_t>(p.Nq) * ROWB);
    const u32x4 rl2 = make_rsrc_words(p.l2 + static_cast<size_t>(bh) * p.Nq, static_cast<uint32_t>(p.Nq) * 4);
    const u32x4 rdd = make_rsrc_words(p.dd + static_cast<size_t>(bh) * p.Nq, static_cast<uint32_t>(p.Nq) * 4);

    // K and V as B operands of S = Q K^T and dP = dO V^T: lane (c, h) holds key
    // kw0 + c, dims 16 s + 8 h .. + 7 (zeros past Nkv).  K carries the sign of
    // the scale.  With VLDS the block's V goes to LDS instead, each chunk
    // permuted by kswz of its row; the lane then reads row 32 wave + c, logical
    // chunk 2 s + h, conflict-free as the forward's K reads.
    V8 kf[KS], vf[VLDS ? 1 : KS];
    uint32_t va0 = 0;
    {
        const auto rk = make_rsrc(static_cast<const char *>(p.k) + kh, static_cast<uint32_t>(p.Nkv) * ROWB);
        const auto rv = make_rsrc(static_cast<const char *>(p.v) + kh, static_cast<uint32_t>(p.Nkv) * ROWB);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            kf[s] = as<V8>(buffer_load16(rk, static_cast<uint32_t>(key) * ROWB + (16 * s + 8 * h) * 2, 0) ^ p.sign);
            if constexpr (!VLDS) vf[s] = as<V8>(buffer_load16(rv, static_cast<uint32_t>(key) * ROWB + (16 * s + 8 * h) * 2, 0));
        }
        if constexpr (VLDS) {
#pragma unroll
            for (int i = 0; i < BK * DC / NT; ++i) {
                const int ch = i * NT + tid, row = ch / DC, col = ch % DC;
                sv[row * DC + (col ^ kswz<D>(row))] = buffer_load16(rv, static_cast<uint32_t>(k0 + row) * ROWB + col * 16, 0);
            }
            const int vrow = 32 * wave + c;
            va0 = vrow * ROWB + ((h ^ kswz<D>(vrow)) << 4);
        }
    }
    const char *SV = reinterpret_cast<const char *>(sv);

    auto ld_off = [&](int i) {
        const int pch = (wave * LOADS + i) * 64 + lane;
        const int row = pch / DC, col = pch % DC;
        return static_cast<uint32_t>(row * ROWB + ((col ^ dswz<D>(row)) << 4));
    };
    auto issue = [&](int st, int t) {
        const uint32_t tq = static_cast<uint32_t>(t) * BQ * ROWB;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            dma_to_lds16(rq, ld_off(i), tq, &sq[st][(wave * LOADS + i) * 64]);
            dma_to_lds16(rdo, ld_off(i), tq, &sdo[st][(wave * LOADS + i) * 64]);
        }
        if (wave == 0) {
            dma_to_lds4(rl2, lane * 4, static_cast<uint32_t>(t) * BQ * 4, &sl2[st][0]);
            dma_to_lds4(rdd, lane * 4, static_cast<uint32_t>(t) * BQ * 4, &sdd[st][0]);
        }
    };

    // Row reads of Q and dO (A operands of S and dP): row swap23(c) (+ 32 per
    // sub-tile), logical chunk 2 s + h.
    uint32_t ra0;
    {
        const int r = swap23(c);
        ra0 = r * ROWB + ((h ^ dswz<D>(r)) << 4);
    }
    // Transposed reads (A operands of dV^T = dO^T P and dK^T = Q^T dS): lane
    // 16 g + 4 j + q addresses query 8 (g / 2) + j + 4 half (+ 16 u + 32 per
    // sub-tile) and dims 32 dt + 16 (g % 2) + 4 q .. + 3.  The permutation
    // depends on half; dt enters as an XOR on bits 6.. of the offset.
    uint32_t ta0[2];
    {
        const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int r = 8 * (g >> 1) + j + 4 * half;
            ta0[half] = r * ROWB + (((2 * (g & 1) + (q >> 1)) ^ dswz<D>(r)) << 4) + ((q & 1) << 3);
        }
    }

    f32x16 dvacc[DT], dkacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) dvacc[dt][e] = dkacc[dt][e] = 0.f;
    const float cs = p.c;

    auto subtile = [&](auto stc, int t, int qq) {
        constexpr int st = decltype(stc)::value;
        const char *SQ = reinterpret_cast<const char *>(sq[st]);
        const char *SDO = reinterpret_cast<const char *>(sdo[st]);
        const int qs0 = t * BQ + 32 * qq;  // first query of the sub-tile
        // S = Q K^T and dP = dO V^T (rows: queries in swap23 order; columns: keys)
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint32_t a = (ra0 ^ (ks << 5)) + qq * 32 * ROWB;
            s = mfma32(as<V8>(*reinterpret_cast<const u32x4 *>(SQ + a)), kf[ks], s);
            V8 vb;
            if constexpr (VLDS)
                vb = as<V8>(*reinterpret_cast<const u32x4 *>(SV + (va0 ^ (ks << 5))));
            else
                vb = vf[ks];
            dp = mfma32(as<V8>(*reinterpret_cast<const u32x4 *>(SDO + a)), vb, dp);
        }
        // Causal: hidden pairs get s = -inf, so that p = 2^(c s - l2) = 0: a
        // pass over the scores that only sub-tiles crossing the diagonal or the
        // ragged end take; the common path has no per-score test.  Element e
        // is query qs0 + 8 h + r(e), r(e) = 16 (e / 8) + e % 8, visible iff
        // lo <= r(e) < hi.
        // Without the causal mask the only hidden rows are those past Nq, and
        // they need no test: their Q, dO, l2 and D are read as zeros, so p = 1
        // there but dO = 0 and dS = p (dP - D) = 0, and they add nothing to
        // dV or dK.
        if constexpr (CAUSAL) {
            if (qs0 + 32 > p.Nq || kw0 + 31 > qs0 + off) {
                const int base = qs0 + 8 * h;
                const int lo = key - off - base;
                const int hi = max(p.Nq - base, lo);
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (static_cast<unsigned>(16 * (e / 8) + e % 8 - lo) >= static_cast<unsigned>(hi - lo))
                        s[e] = -INFINITY;
            }
        }
        // this lane's queries: element e <-> query 8 h + e (e < 8), 16 + 8 h + e - 8
        const f32x4 *l2v = reinterpret_cast<const f32x4 *>(&sl2[st][32 * qq + 8 * h]);
        const f32x4 *ddv = reinterpret_cast<const f32x4 *>(&sdd[st][32 * qq + 8 * h]);
        const f32x4 l2a[4] = {l2v[0], l2v[1], l2v[4], l2v[5]};
        const f32x4 dda[4] = {ddv[0], ddv[1], ddv[4], ddv[5]};
        u32x4 pw[2], dw[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float pr[2], dr[2];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int e = 8 * u + 2 * j + b;
                    const float l2 = l2a[e / 4][e % 4], dd = dda[e / 4][e % 4];
                    const float pe = fast_exp2(fmaf(s[e], cs, -l2));
                    pr[b] = pe;
                    dr[b] = pe * (dp[e] - dd);
                }
                pw[u][j] = pack2<T>(pr[0], pr[1]);
                dw[u][j] = pack2<T>(dr[0], dr[1]);
            }
        // dV^T += dO^T P, dK^T += Q^T dS
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint32_t rowoff = (qq * 32 + 16 * u) * ROWB;
                const uint32_t a0 = (ta0[0] ^ (dt << 6)) + rowoff, a1 = (ta0[1] ^ (dt << 6)) + rowoff;
                const u32x2 do_lo = lds_read_tr16(SDO + a0), do_hi = lds_read_tr16(SDO + a1);
                const u32x2 q_lo = lds_read_tr16(SQ + a0), q_hi = lds_read_tr16(SQ + a1);
                dvacc[dt] = mfma32(as<V8>(u32x4{do_lo[0], do_lo[1], do_hi[0], do_hi[1]}), as<V8>(pw[u]), dvacc[dt]);
                dkacc[dt] = mfma32(as<V8>(u32x4{q_lo[0], q_lo[1], q_hi[0], q_hi[1]}), as<V8>(dw[u]), dkacc[dt]);
            }
    };

    // tile t sits in stage (t - t0) & 1; the loop takes two tiles per pass so
    // that the stage is a constant of each copy
    auto step = [&](auto stc, int t) {
        constexpr int st = decltype(stc)::value;
        wait_vmcnt<0>();
        __syncthreads();  // tile t visible to every wave; tile t - 1's stage free
        if (t + 1 < nqt) issue(st ^ 1, t + 1);
#pragma unroll
        for (int qq = 0; qq < NQQ; ++qq) {
            const int qs0 = t * BQ + 32 * qq;
            // some (query, key) pair of the sub-tile is visible to this wave
            if (qs0 < p.Nq && (!CAUSAL || qs0 + 31 >= wfirst)) subtile(stc, t, qq);
        }
    };
    if (t0 < nqt) issue(0, t0);
    for (int t = t0; t < nqt; t += 2) {
        step(std::integral_constant<int, 0>{}, t);
        if (t + 1 < nqt) step(std::integral_constant<int, 1>{}, t + 1);
    }

    // Epilogue: lane (c, h) writes key kw0 + c, dims 32 dt + 8 j + 4 h .. + 3.
    if (key < p.Nkv) {
        const size_t orow = (static_cast<size_t>(bh) * p.Nkv + key) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 32 * dt + 8 * j + 4 * h;
                const f32x4 v4 = {dvacc[dt][4 * j], dvacc[dt][4 * j + 1], dvacc[dt][4 * j + 2], dvacc[dt][4 * j + 3]};
                const f32x4 k4 = {dkacc[dt][4 * j] * p.scale, dkacc[dt][4 * j + 1] * p.scale,
                                  dkacc[dt][4 * j + 2] * p.scale, dkacc[dt][4 * j + 3] * p.scale};
                if constexpr (OUT_F32) {
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dv) + orow + d0) = v4;
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dk) + orow + d0) = k4;
                } else {
                    *reinterpret_cast<u32x2 *>(static_cast<T *>(p.dv) + orow + d0) =
                        u32x2{pack2<T>(v4[0], v4[1]), pack2<T>(v4[2], v4[3])};
                    *reinterpret_cast<u32x2 *>(static_cast<T *>(p.dk) + orow + d0) =
                        u32x2{pack2<T>(k4[0], k4[1]), pack2<T>(k4[2], k4[3])};
                }
            }
    }
}

// ---------------------------------------------------------------------------
// dQ: query blocks of 128 (4 waves x 32 queries), key tiles of 64 through a
// two-stage LDS ring, as in the forward.

template <int D, typename T, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p)
{
    constexpr int NW = 4, BM = 32 * NW, BN = 64, NT = 64 * NW;
    constexpr int DC = D / 8, TILE = BN * DC, LOADS = TILE / NT, ROWB = 2 * D, KS = D / 16, DT = D / 32;
    static_assert(TILE % NT == 0, "tile must split evenly over the threads");
    using V8 = typename Vec<T>::v8;

    __shared__ u32x4 sk[2][TILE];  // K tiles, dswz (row and transposed reads)
    __shared__ u32x4 sv[2][TILE];  // V tiles, kswz (row reads)
    if constexpr (kPoisonLds) {
        poison_lds(sk, sizeof(sk));
        poison_lds(sv, sizeof(sv));
        __syncthreads();
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, h = lane >> 5;

    const int bh = blockIdx.x % p.n_bh;
    const int qt = p.n_tiles - 1 - static_cast<int>(blockIdx.x / p.n_bh);  // heavy causal tiles first
    const int q0 = qt * BM;
    const int wq0 = q0 + 32 * wave;
    const int qrow = wq0 + c;
    const int off = p.Nkv - p.Nq;
    int kend = p.Nkv;
    if constexpr (CAUSAL) kend = min(p.Nkv, min(q0 + BM, p.Nq) + off);
    const int nkb = (kend + BN - 1) / BN;

    const size_t qh = static_cast<size_t>(bh) * p.Nq * ROWB, kh = static_cast<size_t>(bh) * p.Nkv * ROWB;
    const u32x4 rk = make_rsrc_words(static_cast<const char *>(p.k) + kh, static_cast<uint32_t>(p.Nkv) * ROWB);
    const u32x4 rv = make_rsrc_words(static_cast<const char *>(p.v) + kh, static_cast<uint32_t>(p.Nkv) * ROWB);

    // Q (sign of the scale folded in) and dO as B operands: lane (c, h) holds
    // query qrow, dims 16 s + 8 h .. + 7.
    V8 qf[KS], gf[KS];
    {
        const auto rq = make_rsrc(static_cast<const char *>(p.q) + qh, static_cast<uint32_t>(p.Nq) * ROWB);
        const auto rdo = make_rsrc(static_cast<const char *>(p.dout) + qh, static_cast<uint32_t>(p.Nq) * ROWB);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[s] = as<V8>(buffer_load16(rq, static_cast<uint32_t>(qrow) * ROWB + (16 * s + 8 * h) * 2, 0) ^ p.sign);
            gf[s] = as<V8>(buffer_load16(rdo, static_cast<uint32_t>(qrow) * ROWB + (16 * s + 8 * h) * 2, 0));
        }
    }
    const bool live = qrow < p.Nq;
    const float l2 = live ? p.l2[static_cast<size_t>(bh) * p.Nq + qrow] : 0.f;
    const float dd = live ? p.dd[static_cast<size_t>(bh) * p.Nq + qrow] : 0.f;

    auto ld_off = [&](int i, bool dual) {
        const int pch = (wave * LOADS + i) * 64 + lane;
        const int row = pch / DC, col = pch % DC;
        return static_cast<uint32_t>(row * ROWB + ((col ^ (dual ? dswz<D>(row) : kswz<D>(row))) << 4));
    };
    auto issue = [&](int st, int kb) {
        const uint32_t tk = static_cast<uint32_t>(kb) * BN * ROWB;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            dma_to_lds16(rk, ld_off(i, true), tk, &sk[st][(wave * LOADS + i) * 64]);
            dma_to_lds16(rv, ld_off(i, false), tk, &sv[st][(wave * LOADS + i) * 64]);
        }
    };

    // Row reads of K (dswz) and V (kswz): row 32 kk + swap23(c), chunk 2 s + h.
    uint32_t ka0, va0;
    {
        const int r = swap23(c);
        ka0 = r * ROWB + ((h ^ dswz<D>(r)) << 4);
        va0 = r * ROWB + ((h ^ kswz<D>(r)) << 4);
    }
    // Transposed reads of K (A operand of dQ^T = K^T dS^T), as in the dK/dV kernel.
    uint32_t ta0[2];
    {
        const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int r = 8 * (g >> 1) + j + 4 * half;
            ta0[half] = r * ROWB + (((2 * (g & 1) + (q >> 1)) ^ dswz<D>(r)) << 4) + ((q & 1) << 3);
        }
    }

    f32x16 dqacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) dqacc[dt][e] = 0.f;
    const float cs = p.c;

    // One 64-key tile, as two 32-key halves each taken through S, dP, dS and
    // its dQ products before the next (half the score registers live at once).
    auto tile = [&](auto stc, int kv0) {
        constexpr int st = decltype(stc)::value;
        const char *SK = reinterpret_cast<const char *>(sk[st]);
        const char *SV = reinterpret_cast<const char *>(sv[st]);
        const bool edge = (kv0 + BN > p.Nkv) || (CAUSAL && kv0 + BN - 1 > wq0 + off);
        // the last key this lane's row sees, relative to the lane's first key of the tile
        const int lim = (CAUSAL ? min(qrow + off, p.Nkv - 1) : p.Nkv - 1) - kv0 - 8 * h;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // keep the next half's operand loads out of this half (register pressure)
            __builtin_amdgcn_sched_barrier(0);
            // S^T = K Q^T and dP^T = V dO^T (rows: keys in swap23 order; columns: queries)
            f32x16 s = {}, dp = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 xk = *reinterpret_cast<const u32x4 *>(SK + (ka0 ^ (ks << 5)) + kk * 32 * ROWB);
                const u32x4 xv = *reinterpret_cast<const u32x4 *>(SV + (va0 ^ (ks << 5)) + kk * 32 * ROWB);
                s = mfma32(as<V8>(xk), qf[ks], s);
                dp = mfma32(as<V8>(xv), gf[ks], dp);
            }
            // hidden pairs: s = -inf before the exponential, in a pass that
            // only tiles crossing the diagonal or the ragged end take
            if (edge) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (32 * kk + 16 * (e / 8) + e % 8 > lim) s[e] = -INFINITY;
            }
            u32x4 dw[2];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float dr[2];
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        const int e = 8 * u + 2 * j + b;
                        const float pe = fast_exp2(fmaf(s[e], cs, -l2));
                        dr[b] = pe * (dp[e] - dd);
                    }
                    dw[u][j] = pack2<T>(dr[0], dr[1]);
                }
            // dQ^T += K^T dS^T
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const uint32_t rowoff = (32 * kk + 16 * u) * ROWB;
                    const u32x2 lo = lds_read_tr16(SK + ((ta0[0] ^ (dt << 6)) + rowoff));
                    const u32x2 hi = lds_read_tr16(SK + ((ta0[1] ^ (dt << 6)) + rowoff));
                    dqacc[dt] = mfma32(as<V8>(u32x4{lo[0], lo[1], hi[0], hi[1]}), as<V8>(dw[u]), dqacc[dt]);
                }
        }
    };

    // key tile kb sits in stage kb & 1; two tiles per pass, so that the stage
    // is a constant of each copy
    auto step = [&](auto stc, int kb) {
        constexpr int st = decltype(stc)::value;
        wait_vmcnt<0>();
        __syncthreads();
        if (kb + 1 < nkb) issue(st ^ 1, kb + 1);
        const int kv0 = kb * BN;
        // wave-uniform: the products mix operands across lanes, so a wave runs
        // them whole; columns of rows past Nq are formed and never stored
        if (wq0 < p.Nq && (!CAUSAL || kv0 <= wq0 + 31 + off)) tile(stc, kv0);
    };
    if (nkb > 0) issue(0, 0);
    for (int kb = 0; kb < nkb; kb += 2) {
        step(std::integral_constant<int, 0>{}, kb);
        if (kb + 1 < nkb) step(std::integral_constant<int, 1>{}, kb + 1);
    }

    if (live) {
        const size_t orow = (static_cast<size_t>(bh) * p.Nq + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 32 * dt + 8 * j + 4 * h;
                const f32x4 v4 = {dqacc[dt][4 * j] * p.scale, dqacc[dt][4 * j + 1] * p.scale,
                                  dqacc[dt][4 * j + 2] * p.scale, dqacc[dt][4 * j + 3] * p.scale};
                if constexpr (OUT_F32)
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dq) + orow + d0) = v4;
                else
                    *reinterpret_cast<u32x2 *>(static_cast<T *>(p.dq) + orow + d0) =
                        u32x2{pack2<T>(v4[0], v4[1]), pack2<T>(v4[2], v4[3])};
            }
    }
}

// ---------------------------------------------------------------------------
// dQ on the 16x16x32 MFMA (d = 128, and d = 64 on wide grids): the forward's
// fragment layout.  Per wave 32 queries as two 16-query blocks qb; per 64-key
// tile
//
//   S^T  (16 keys x 16 queries) = K (16 keys x 32 dims) Q^T     (A: K rows)
//   dP^T (16 keys x 16 queries) = V (16 keys x 32 dims) dO^T    (A: V rows)
//   dQ^T (16 dims x 16 queries) += K^T (16 dims x 32 keys) dS^T (A: K read transposed)
//
// Lane l = 16 g + i receives, per 16-key block kb, query i and keys 4 g .. + 3;
// a k-step of the third product takes key blocks 2 s and 2 s + 1, whose keys
// 4 g .. + 3 are the lane's k-slots, so dS goes to its B operand without
// moving between lanes (the forward's P).  The K tile is read both as rows
// and transposed; its chunk permutation dswz16 is conflict-free for both
// patterns.  A ds_read_b128 is served in four groups of 16 lanes: in each
// half-wave, the lane quads whose three index bits have even parity form one
// group and the odd ones the other (measured: lane 0 shares banks with lanes
// 1-3, 12-15 and 20-27 only).  For rows i = lane % 16 at chunk g ^ p(i), a
// group holds rows {0-3, 12-15} of one g and rows {4-11} of the other, so p
// must separate those two sets from each other under XOR by 1; row & 15 and
// the p below do, ((row & 7) << 1) | (row >> 3) does not (2-way conflicts).
// A transposed read covers 8 consecutive rows x 32 bytes per 32 lanes, so
// p / 2 must be a bijection on rows 0-7 and on rows 8-15: here it is
// (row & 7) XOR 4 (row >> 3).
__host__ __device__ __forceinline__ constexpr int dswz16(int row) { return (((row & 7) ^ ((row >> 1) & 4)) << 1) | ((row >> 3) & 1); }
__host__ __device__ __forceinline__ constexpr int kswz16(int row) { return row & 15; }

// d = 64: rows of 128 bytes, two to a bank line (row parity picks the half).
// The same two conditions hold for row & 6 (rows read both ways) and
// (row >> 1) & 7 (rows read as rows only): in a row read each parity's eight
// rows of a group take distinct chunks, and in a transposed read the four
// rows of each parity among 8 consecutive rows take distinct 32-byte runs.
__host__ __device__ __forceinline__ constexpr int dswz16h(int row) { return row & 6; }
__host__ __device__ __forceinline__ constexpr int kswz16h(int row) { return (row >> 1) & 7; }
template <int ROWB> __host__ __device__ __forceinline__ constexpr int dual16(int row)
{
    return ROWB == 256 ? dswz16(row) : dswz16h(row);
}
template <int ROWB> __host__ __device__ __forceinline__ constexpr int rows16(int row)
{
    return ROWB == 256 ? kswz16(row) : kswz16h(row);
}

// The b128 condition above for a row permutation p, checked lane by lane: two
// lanes of one group (same half-wave, same quad parity) never read the same
// 16-byte slot of the bank line at different addresses.  Lane 16 g + i reads
// row i at logical chunk g.
template <int (*P)(int), int ROWB> constexpr bool b128_conflict_free()
{
    auto slot = [](int lane) {
        const int row = lane & 15, chunk = (lane >> 4) ^ P(row);
        return ROWB == 256 ? chunk : (8 * (row & 1) + chunk) & 15;
    };
    for (int a = 0; a < 64; ++a)
        for (int b = a + 1; b < 64; ++b) {
            const int qa = (a >> 2) & 7, qb = (b >> 2) & 7;
            const bool same_group = (a >> 5) == (b >> 5) && (__builtin_popcount(qa) & 1) == (__builtin_popcount(qb) & 1);
            if (same_group && (a & 15) != (b & 15) && slot(a) == slot(b)) return false;
        }
    return true;
}
// Transposed reads: 8 consecutive rows x 32 bytes per half-wave; each row's
// 32-byte run (chunk pair P(row) / 2) must land in its own run of the line.
template <int (*P)(int), int ROWB> constexpr bool tr_conflict_free()
{
    auto run = [](int row) { return ROWB == 256 ? (P(row) >> 1) : 4 * (row & 1) + ((P(row) >> 1) & 3); };
    for (int a = 0; a < 16; ++a)
        for (int b = a + 1; b < 16; ++b)
            if ((a >> 3) == (b >> 3) && run(a) == run(b)) return false;
    return true;
}
static_assert(b128_conflict_free<dswz16, 256>() && tr_conflict_free<dswz16, 256>(), "dswz16: conflict-free row and transposed reads");
static_assert(b128_conflict_free<kswz16, 256>(), "kswz16: conflict-free row reads");
static_assert(b128_conflict_free<dswz16h, 128>() && tr_conflict_free<dswz16h, 128>(), "dswz16h: conflict-free row and transposed reads");
static_assert(b128_conflict_free<kswz16h, 128>(), "kswz16h: conflict-free row reads");

template <int D, typename T, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kBwd16Waves<D>, kBwd16Waves<D>)))
void bwd_dq16_kernel(BwdParams p)
{
    static_assert(D == 64 || D == 128, "d = 64 or 128");
    constexpr int NW = 4, BM = 32 * NW, BN = 64, NT = 64 * NW;
    constexpr int DC = D / 8, TILE = BN * DC, LOADS = TILE / NT, ROWB = 2 * D, KS = D / 32, DB = D / 16;
    static_assert(TILE % NT == 0, "tile must split evenly over the threads");
    using V8 = typename Vec<T>::v8;

    __shared__ u32x4 sk[2][TILE];  // K tiles, dual16 (row and transposed reads)
    __shared__ u32x4 sv[2][TILE];  // V tiles, rows16 (row reads)
    if constexpr (kPoisonLds) {
        poison_lds(sk, sizeof(sk));
        poison_lds(sv, sizeof(sv));
        __syncthreads();
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;

    const int bh = blockIdx.x % p.n_bh;
    const int qt = p.n_tiles - 1 - static_cast<int>(blockIdx.x / p.n_bh);  // heavy causal tiles first
    const int q0 = qt * BM;
    const int wq0 = q0 + 32 * wave;
    const int off = p.Nkv - p.Nq;
    int kend = p.Nkv;
    if constexpr (CAUSAL) kend = min(p.Nkv, min(q0 + BM, p.Nq) + off);
    const int nkb = (kend + BN - 1) / BN;

    const size_t qh = static_cast<size_t>(bh) * p.Nq * ROWB, kh = static_cast<size_t>(bh) * p.Nkv * ROWB;
    const u32x4 rk = make_rsrc_words(static_cast<const char *>(p.k) + kh, static_cast<uint32_t>(p.Nkv) * ROWB);
    const u32x4 rv = make_rsrc_words(static_cast<const char *>(p.v) + kh, static_cast<uint32_t>(p.Nkv) * ROWB);

    // Q (sign of the scale folded in) and dO as B operands: lane (g, i) holds
    // query wq0 + 16 qb + i, dims 32 s + 8 g .. + 7.
    V8 qf[2][KS], gf[2][KS];
    float l2[2], dd[2];
    {
        const auto rq = make_rsrc(static_cast<const char *>(p.q) + qh, static_cast<uint32_t>(p.Nq) * ROWB);
        const auto rdo = make_rsrc(static_cast<const char *>(p.dout) + qh, static_cast<uint32_t>(p.Nq) * ROWB);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int qrow = wq0 + 16 * qb + li;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const uint32_t o = static_cast<uint32_t>(qrow) * ROWB + (32 * s + 8 * g) * 2;
                qf[qb][s] = as<V8>(buffer_load16(rq, o, 0) ^ p.sign);
                gf[qb][s] = as<V8>(buffer_load16(rdo, o, 0));
            }
            const bool live = qrow < p.Nq;
            l2[qb] = live ? p.l2[static_cast<size_t>(bh) * p.Nq + qrow] : 0.f;
            dd[qb] = live ? p.dd[static_cast<size_t>(bh) * p.Nq + qrow] : 0.f;
        }
    }

    // Direct loads: load i of the wave fills LDS chunks [(wave LOADS + i) 64, + 64).
    auto issue = [&](int st, int kb) {
        const uint32_t tk = static_cast<uint32_t>(kb) * BN * ROWB;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int pch = (wave * LOADS + i) * 64 + lane;
            const int row = pch / DC, col = pch % DC;
            dma_to_lds16(rk, static_cast<uint32_t>(row * ROWB + ((col ^ dual16<ROWB>(row)) << 4)), tk,
                         &sk[st][(wave * LOADS + i) * 64]);
            dma_to_lds16(rv, static_cast<uint32_t>(row * ROWB + ((col ^ rows16<ROWB>(row)) << 4)), tk,
                         &sv[st][(wave * LOADS + i) * 64]);
        }
    };

    // Row reads (A of S^T and dP^T): row 16 kb + i, logical chunk 4 s + g; the
    // permutation depends on i only.
    const uint32_t ka0 = li * ROWB + ((g ^ dual16<ROWB>(li)) << 4);
    const uint32_t va0 = li * ROWB + ((g ^ rows16<ROWB>(li)) << 4);
    // Transposed reads of K (A of dQ^T): the in-group lane i addresses row
    // 4 g + i / 4 (+ 32 s + 16 h) and bytes 32 db + 8 (i % 4) .. + 7, receiving
    // dims 16 db + i of the four rows; db enters as an XOR on the chunk index.
    uint32_t ta0;
    {
        const int row = 4 * g + (li >> 2);
        ta0 = row * ROWB + ((((li & 3) >> 1) ^ dual16<ROWB>(row)) << 4) + ((li & 1) << 3);
    }

    f32x4 dqacc[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) dqacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float cs = p.c;

    // One 64-key tile as two 32-key halves (key blocks 2 h and 2 h + 1), each
    // taken through S^T, dP^T, dS and its dQ products before the next: half
    // the score registers live at once.
    auto tile = [&](auto stc, int kv0) {
        constexpr int st = decltype(stc)::value;
        const char *SK = reinterpret_cast<const char *>(sk[st]);
        const char *SV = reinterpret_cast<const char *>(sv[st]);
        const bool edge = (kv0 + BN > p.Nkv) || (CAUSAL && kv0 + BN - 1 > wq0 + off);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // keep the next half's operand reads out of this half (registers)
            __builtin_amdgcn_sched_barrier(0);
            f32x4 sa[2][2], pa[2][2];
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) sa[b][qb] = pa[b][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int kb = 2 * h + b;
                    const u32x4 xk = *reinterpret_cast<const u32x4 *>(SK + (ka0 ^ ((4 * s) << 4)) + kb * 16 * ROWB);
                    const u32x4 xv = *reinterpret_cast<const u32x4 *>(SV + (va0 ^ ((4 * s) << 4)) + kb * 16 * ROWB);
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        sa[b][qb] = mfma16(as<V8>(xk), qf[qb][s], sa[b][qb]);
                        pa[b][qb] = mfma16(as<V8>(xv), gf[qb][s], pa[b][qb]);
                    }
                }
            // hidden pairs (past Nkv, or above the diagonal) get s = -inf, on
            // tiles that cross the diagonal or the ragged end only: element
            // (b, r) is key kv0 + 16 (2 h + b) + 4 g + r
            if (edge) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    int lim = p.Nkv - 1;
                    if constexpr (CAUSAL) lim = min(lim, wq0 + 16 * qb + li + off);
                    const int t = lim - kv0 - 4 * g;
#pragma unroll
                    for (int b = 0; b < 2; ++b)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (16 * (2 * h + b) + r > t) sa[b][qb][r] = -INFINITY;
                }
            }
            // dS = P (dP - D) in the storage type, the B operand of k-step h
            V8 dsf[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                u32x4 w;
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    float e[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        e[r] = fast_exp2(fmaf(sa[b][qb][r], cs, -l2[qb])) * (pa[b][qb][r] - dd[qb]);
                    w[2 * b] = pack2<T>(e[0], e[1]);
                    w[2 * b + 1] = pack2<T>(e[2], e[3]);
                }
                dsf[qb] = as<V8>(w);
            }
            // dQ^T += K^T dS^T
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const char *pa0 = SK + (ta0 ^ (db << 5)) + 32 * h * ROWB;
                const u32x2 lo = lds_read_tr16(pa0), hi = lds_read_tr16(pa0 + 16 * ROWB);
                const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) dqacc[db][qb] = mfma16(as<V8>(a), dsf[qb], dqacc[db][qb]);
            }
        }
    };

    // key tile kb sits in stage kb & 1; two tiles per pass, so that the stage
    // is a constant of each copy
    auto step = [&](auto stc, int kb) {
        constexpr int st = decltype(stc)::value;
        wait_vmcnt<0>();
        __syncthreads();
        if (kb + 1 < nkb) issue(st ^ 1, kb + 1);
        const int kv0 = kb * BN;
        // wave-uniform: columns of rows past Nq are formed and never stored
        if (wq0 < p.Nq && (!CAUSAL || kv0 <= wq0 + 31 + off)) tile(stc, kv0);
    };
    if (nkb > 0) issue(0, 0);
    for (int kb = 0; kb < nkb; kb += 2) {
        step(std::integral_constant<int, 0>{}, kb);
        if (kb + 1 < nkb) step(std::integral_constant<int, 1>{}, kb + 1);
    }

    // Epilogue: lane (g, i) holds dims 16 db + 4 g .. + 3 of query wq0 + 16 qb + i.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int qrow = wq0 + 16 * qb + li;
        if (qrow < p.Nq) {
            const size_t orow = (static_cast<size_t>(bh) * p.Nq + qrow) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d0 = 16 * db + 4 * g;
                const f32x4 v4 = dqacc[db][qb] * p.scale;
                if constexpr (OUT_F32)
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dq) + orow + d0) = v4;
                else
                    *reinterpret_cast<u32x2 *>(static_cast<T *>(p.dq) + orow + d0) =
                        u32x2{pack2<T>(v4[0], v4[1]), pack2<T>(v4[2], v4[3])};
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dK, dV on the 16x16x32 MFMA (d = 128, and d = 64 on wide grids).  Per wave
// 32 keys as two 16-key blocks kb; per 32-query sub-tile (two 16-query blocks
// qb)
//
//   S   (16 queries x 16 keys) = Q (16 queries x 32 dims) K^T    (A: Q rows)
//   dP  (16 queries x 16 keys) = dO (16 queries x 32 dims) V^T   (A: dO rows)
//   dV^T (16 dims x 16 keys) += dO^T (16 dims x 32 queries) P    (A: dO read transposed)
//   dK^T (16 dims x 16 keys) += Q^T (16 dims x 32 queries) dS    (A: Q read transposed)
//
// Lane l = 16 g + i receives, per query block qb, key i and queries 4 g .. + 3;
// the 32 queries of a sub-tile are one k-step of the last two products, whose
// k-slots for the lane are those queries of qb = 0 and 1, so P and dS go to
// their B operands without moving between lanes.  K^T (the B operand of S)
// stays in registers; the block's V sits in LDS (read as rows), Q and dO
// stream through a two-stage ring and are read both as rows and transposed
// (dswz16).
template <int D, typename T, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kBwd16Waves<D>, kBwd16Waves<D>)))
void bwd_dkdv16_kernel(BwdParams p)
{
    static_assert(D == 64 || D == 128, "d = 64 or 128");
    constexpr int NW = 4, BK = 32 * NW, BQ = 32, NT = 64 * NW;
    constexpr int DC = D / 8, TILE = BQ * DC, LOADS = TILE / NT, ROWB = 2 * D, KS = D / 32, DB = D / 16;
    static_assert(TILE % NT == 0 && (BK * DC) % NT == 0, "tiles must split evenly over the threads");
    using V8 = typename Vec<T>::v8;

    // base-2 LSE and D of the tile's queries: wave 0 fills each stage with one
    // 64-lane dword load (the second half is the next tile's, unused)
    __shared__ u32x4 sq[2][TILE];   // Q tiles [query][dim], dual16
    __shared__ u32x4 sdo[2][TILE];  // dO tiles [query][dim], dual16
    __shared__ float sl2[2][64];
    __shared__ float sdd[2][64];
    __shared__ u32x4 sv[BK * DC];   // the block's V [key][dim], rows16
    if constexpr (kPoisonLds) {
        poison_lds(sq, sizeof(sq));
        poison_lds(sdo, sizeof(sdo));
        poison_lds(sl2, sizeof(sl2));
        poison_lds(sdd, sizeof(sdd));
        poison_lds(sv, sizeof(sv));
        __syncthreads();
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;

    // Causal: key blocks near the start see the most queries; they go first.
    const int bh = blockIdx.x % p.n_bh;
    const int kt = static_cast<int>(blockIdx.x / p.n_bh);
    const int k0 = kt * BK;
    const int kw0 = k0 + 32 * wave;
    const int off = p.Nkv - p.Nq;  // row i sees keys j <= i + off
    const int nqt = (p.Nq + BQ - 1) / BQ;
    const int t0 = CAUSAL ? max(0, k0 - off) / BQ : 0;
    const int wfirst = CAUSAL ? kw0 - off : 0;  // the wave's first query row that sees one of its keys

    const size_t qh = static_cast<size_t>(bh) * p.Nq * ROWB, kh = static_cast<size_t>(bh) * p.Nkv * ROWB;
    const u32x4 rq = make_rsrc_words(static_cast<const char *>(p.q) + qh, static_cast<uint32_t>(p.Nq) * ROWB);
    const u32x4 rdo = make_rsrc_words(static_cast<const char *>(p.dout) + qh, static_cast<uint32_t>(p.Nq) * ROWB);
    const u32x4 rl2 = make_rsrc_words(p.l2 + static_cast<size_t>(bh) * p.Nq, static_cast<uint32_t>(p.Nq) * 4);
    const u32x4 rdd = make_rsrc_words(p.dd + static_cast<size_t>(bh) * p.Nq, static_cast<uint32_t>(p.Nq) * 4);

    // K^T as the B operand of S: lane (g, i) holds key kw0 + 16 kb + i, dims
    // 32 s + 8 g .. + 7 (zeros past Nkv), with the sign of the scale.  The
    // block's V goes to LDS, each chunk permuted by kswz16 of its row.
    V8 kf[2][KS];
    {
        const auto rk = make_rsrc(static_cast<const char *>(p.k) + kh, static_cast<uint32_t>(p.Nkv) * ROWB);
        const auto rv = make_rsrc(static_cast<const char *>(p.v) + kh, static_cast<uint32_t>(p.Nkv) * ROWB);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s = 0; s < KS; ++s)
                kf[kb][s] = as<V8>(buffer_load16(rk, static_cast<uint32_t>(kw0 + 16 * kb + li) * ROWB + (32 * s + 8 * g) * 2, 0) ^
                                   p.sign);
#pragma unroll
        for (int i = 0; i < BK * DC / NT; ++i) {
            const int ch = i * NT + tid, row = ch / DC, col = ch % DC;
            sv[row * DC + (col ^ rows16<ROWB>(row))] = buffer_load16(rv, static_cast<uint32_t>(k0 + row) * ROWB + col * 16, 0);
        }
    }
    const char *SV = reinterpret_cast<const char *>(sv);

    auto issue = [&](int st, int t) {
        const uint32_t tq = static_cast<uint32_t>(t) * BQ * ROWB;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int pch = (wave * LOADS + i) * 64 + lane;
            const int row = pch / DC, col = pch % DC;
            const uint32_t o = static_cast<uint32_t>(row * ROWB + ((col ^ dual16<ROWB>(row)) << 4));
            dma_to_lds16(rq, o, tq, &sq[st][(wave * LOADS + i) * 64]);
            dma_to_lds16(rdo, o, tq, &sdo[st][(wave * LOADS + i) * 64]);
        }
        if (wave == 0) {
            dma_to_lds4(rl2, lane * 4, static_cast<uint32_t>(t) * BQ * 4, &sl2[st][0]);
            dma_to_lds4(rdd, lane * 4, static_cast<uint32_t>(t) * BQ * 4, &sdd[st][0]);
        }
    };

    // Row reads of Q and dO (A of S and dP): row 16 qb + i, logical chunk 4 s + g.
    const uint32_t ra0 = li * ROWB + ((g ^ dual16<ROWB>(li)) << 4);
    // Row reads of V (B of dP): row 32 wave + 16 kb + i, logical chunk 4 s + g.
    const uint32_t va0 = (32 * wave + li) * ROWB + ((g ^ rows16<ROWB>(li)) << 4);
    // Transposed reads of dO and Q (A of dV^T and dK^T): the in-group lane i
    // addresses row 4 g + i / 4 (+ 16 for the second half of the k-step) and
    // bytes 32 db + 8 (i % 4) .. + 7, receiving dims 16 db + i of the four rows.
    uint32_t ta0;
    {
        const int row = 4 * g + (li >> 2);
        ta0 = row * ROWB + ((((li & 3) >> 1) ^ dual16<ROWB>(row)) << 4) + ((li & 1) << 3);
    }

    f32x4 dvacc[DB][2], dkacc[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dvacc[db][kb] = dkacc[db][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float cs = p.c;

    auto subtile = [&](auto stc, int t) {
        constexpr int st = decltype(stc)::value;
        const char *SQ = reinterpret_cast<const char *>(sq[st]);
        const char *SDO = reinterpret_cast<const char *>(sdo[st]);
        const int qs0 = t * BQ;
        // S and dP: [qb][kb]
        f32x4 sa[2][2], pa[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) sa[qb][kb] = pa[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            V8 vb[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                vb[kb] = as<V8>(*reinterpret_cast<const u32x4 *>(SV + (va0 ^ ((4 * s) << 4)) + kb * 16 * ROWB));
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const uint32_t a = (ra0 ^ ((4 * s) << 4)) + qb * 16 * ROWB;
                const V8 xq = as<V8>(*reinterpret_cast<const u32x4 *>(SQ + a));
                const V8 xd = as<V8>(*reinterpret_cast<const u32x4 *>(SDO + a));
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    sa[qb][kb] = mfma16(xq, kf[kb][s], sa[qb][kb]);
                    pa[qb][kb] = mfma16(xd, vb[kb], pa[qb][kb]);
                }
            }
        }
        // Causal: hidden pairs get s = -inf, on sub-tiles that cross the
        // diagonal or the ragged end only; element (qb, kb, r) is query
        // qs0 + 16 qb + 4 g + r and key kw0 + 16 kb + i.  Without the causal
        // mask the only hidden rows are those past Nq, and they need no test:
        // their Q, dO, l2 and D are read as zeros, so p = 1 there but dO = 0
        // and dS = p (dP - D) = 0, and they add nothing to dV or dK.
        if constexpr (CAUSAL) {
            if (qs0 + BQ > p.Nq || kw0 + 31 > qs0 + off) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    // query q sees the key iff q >= key - off, and q < Nq
                    const int lo = kw0 + 16 * kb + li - off - qs0 - 4 * g, hi = p.Nq - qs0 - 4 * g;
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int q = 16 * qb + r;
                            if (q < lo || q >= hi) sa[qb][kb][r] = -INFINITY;
                        }
                }
            }
        }
        // P and dS into the B operands of the last two products: operand kb
        // holds, for key 16 kb + i, queries 4 g .. + 3 of qb = 0 then qb = 1
        const f32x4 l2a[2] = {*reinterpret_cast<const f32x4 *>(&sl2[st][4 * g]),
                              *reinterpret_cast<const f32x4 *>(&sl2[st][16 + 4 * g])};
        const f32x4 dda[2] = {*reinterpret_cast<const f32x4 *>(&sdd[st][4 * g]),
                              *reinterpret_cast<const f32x4 *>(&sdd[st][16 + 4 * g])};
        V8 pw[2], dw[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            u32x4 wp, wd;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float pe[4], de[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pe[r] = fast_exp2(fmaf(sa[qb][kb][r], cs, -l2a[qb][r]));
                    de[r] = pe[r] * (pa[qb][kb][r] - dda[qb][r]);
                }
                wp[2 * qb] = pack2<T>(pe[0], pe[1]);
                wp[2 * qb + 1] = pack2<T>(pe[2], pe[3]);
                wd[2 * qb] = pack2<T>(de[0], de[1]);
                wd[2 * qb + 1] = pack2<T>(de[2], de[3]);
            }
            pw[kb] = as<V8>(wp);
            dw[kb] = as<V8>(wd);
        }
        // dV^T += dO^T P, dK^T += Q^T dS (their transposed reads stay below
        // the VALU block)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint32_t a = ta0 ^ (db << 5);
            const u32x2 dlo = lds_read_tr16(SDO + a), dhi = lds_read_tr16(SDO + a + 16 * ROWB);
            const u32x2 qlo = lds_read_tr16(SQ + a), qhi = lds_read_tr16(SQ + a + 16 * ROWB);
            const V8 ad = as<V8>(u32x4{dlo[0], dlo[1], dhi[0], dhi[1]});
            const V8 aq = as<V8>(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]});
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                dvacc[db][kb] = mfma16(ad, pw[kb], dvacc[db][kb]);
                dkacc[db][kb] = mfma16(aq, dw[kb], dkacc[db][kb]);
            }
        }
    };

    // tile t sits in stage (t - t0) & 1; two tiles per pass
    auto step = [&](auto stc, int t) {
        constexpr int st = decltype(stc)::value;
        wait_vmcnt<0>();
        __syncthreads();  // tile t visible to every wave; tile t - 1's stage free
        if (t + 1 < nqt) issue(st ^ 1, t + 1);
        const int qs0 = t * BQ;
        // some (query, key) pair of the sub-tile is visible to this wave
        if (qs0 < p.Nq && (!CAUSAL || qs0 + BQ - 1 >= wfirst)) subtile(stc, t);
    };
    if (t0 < nqt) issue(0, t0);
    for (int t = t0; t < nqt; t += 2) {
        step(std::integral_constant<int, 0>{}, t);
        if (t + 1 < nqt) step(std::integral_constant<int, 1>{}, t + 1);
    }

    // Epilogue: lane (g, i) holds dims 16 db + 4 g .. + 3 of key kw0 + 16 kb + i.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int key = kw0 + 16 * kb + li;
        if (key < p.Nkv) {
            const size_t orow = (static_cast<size_t>(bh) * p.Nkv + key) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d0 = 16 * db + 4 * g;
                const f32x4 v4 = dvacc[db][kb];
                const f32x4 k4 = dkacc[db][kb] * p.scale;
                if constexpr (OUT_F32) {
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dv) + orow + d0) = v4;
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dk) + orow + d0) = k4;
                } else {
                    *reinterpret_cast<u32x2 *>(static_cast<T *>(p.dv) + orow + d0) =
                        u32x2{pack2<T>(v4[0], v4[1]), pack2<T>(v4[2], v4[3])};
                    *reinterpret_cast<u32x2 *>(static_cast<T *>(p.dk) + orow + d0) =
                        u32x2{pack2<T>(k4[0], k4[1]), pack2<T>(k4[2], k4[3])};
                }
            }
        }
    }
}

template <int D, typename T, bool CAUSAL, bool OUT_F32>
hipError_t launch(const BwdArgs &a, hipStream_t stream)
{
    // With Nq = 0 only the key pass runs: it writes dK = dV = 0.
    const long long rows = static_cast<long long>(a.B) * a.H * a.Nq;
    hipError_t err;
    if (rows > 0) {
        PrepParams pp{a.o, a.dout, a.lse, a.ws_l2, a.ws_dd, rows};
        constexpr int RPB = 256 / (D / 8);
        const long long blocks = std::min<long long>((rows + RPB - 1) / RPB, kPrepMaxBlocks);
        hipLaunchKernelGGL((bwd_prep_kernel<D, T>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, pp);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }

    BwdParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.dout = a.dout;
    p.dq = a.dq;
    p.dk = a.dk;
    p.dv = a.dv;
    p.l2 = a.ws_l2;
    p.dd = a.ws_dd;
    p.Nq = a.Nq;
    p.Nkv = a.Nkv;
    p.n_bh = a.B * a.H;
    const float c = (a.scale < 0.f ? -a.scale : a.scale) * kLog2e;
    p.c = c < kBwdMinC ? kBwdMinC : c;
    p.scale = a.scale;
    p.sign = a.scale < 0.f ? 0x80008000u : 0u;

    p.n_tiles = (a.Nkv + 127) / 128;
    const dim3 gk(static_cast<unsigned>(static_cast<long long>(p.n_bh) * p.n_tiles));
    if constexpr (D == 128 && FA355_DKDV16) {
        hipLaunchKernelGGL((bwd_dkdv16_kernel<D, T, CAUSAL, OUT_F32>), gk, dim3(256), 0, stream, p);
    } else {
        if (FA355_DKDV16 && FA355_BWD16_D64 && static_cast<long long>(gk.x) >= kBwd16MinBlocksD64)
            hipLaunchKernelGGL((bwd_dkdv16_kernel<D, T, CAUSAL, OUT_F32>), gk, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, T, CAUSAL, OUT_F32>), gk, dim3(256), 0, stream, p);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;

    p.n_tiles = (a.Nq + 127) / 128;
    if (p.n_tiles == 0) return hipSuccess;
    const dim3 gq(static_cast<unsigned>(static_cast<long long>(p.n_bh) * p.n_tiles));
    if constexpr (D == 128 && FA355_DQ16) {
        hipLaunchKernelGGL((bwd_dq16_kernel<D, T, CAUSAL, OUT_F32>), gq, dim3(256), 0, stream, p);
    } else {
        if (FA355_DQ16 && FA355_BWD16_D64 && static_cast<long long>(gq.x) >= kBwd16MinBlocksD64)
            hipLaunchKernelGGL((bwd_dq16_kernel<D, T, CAUSAL, OUT_F32>), gq, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((bwd_dq_kernel<D, T, CAUSAL, OUT_F32>), gq, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_dt(const BwdArgs &a, hipStream_t stream)
{
    if (a.causal)
        return a.out_f32 ? launch<D, T, true, true>(a, stream) : launch<D, T, true, false>(a, stream);
    return a.out_f32 ? launch<D, T, false, true>(a, stream) : launch<D, T, false, false>(a, stream);
}

template <int D>
hipError_t launch_d(const BwdArgs &a, hipStream_t stream)
{
    return a.elem == Elem::F16 ? launch_dt<D, _Float16>(a, stream) : launch_dt<D, __bf16>(a, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream)
{
    if (a.d == 64) return launch_d<64>(a, stream);
    if (a.d == 128) return launch_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa355
