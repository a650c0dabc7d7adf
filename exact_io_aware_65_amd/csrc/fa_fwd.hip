// Fused exact attention forward (prefill) for gfx950.
//
// One workgroup owns one (batch*head, tile of BM query rows) pair and loops
// over key/value tiles of BN keys: Q-tiles outer and parallel, K/V tiles
// inner ("FlashAttention 1-2-3: The IO-Aware Revolution in LLM Inference",
// section "FlashAttention-2: Reducing Non-Matmul Overhead and Causal
// Efficiency").  Each K/V tile is copied once from HBM/L2 straight into LDS
// (buffer_load ... lds, no register staging) while earlier tiles are being
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
// Software pipeline (per wave, per key tile j):
//   phase 1: the 16 MFMAs of S_{j+1} = K_{j+1} Q^T are issued while the VALU
//            turns S_j into probabilities (FMA + exp2, row sum, pack to 16 bits);
//   phase 2: the 16 MFMAs of O += V_j P_j are issued while the VALU takes the
//            row maximum of S_{j+1}.
// A wave's own VALU work runs beside its MFMAs when the two are independent,
// which is what this ordering gives the scheduler.  K therefore runs one tile
// ahead of V in the LDS ring.
//
// LDS layout: rows of d 16-bit elements (row stride 2d bytes; d bytes for an
// E4M3 K) with the 16-byte chunks of each row permuted by an XOR with a
// function of the row.  gfx950 serves a ds_read_b128 in four groups of 16
// lanes (in each half-wave, the lane quads whose three index bits have even
// parity, then the odd ones) and a ds_read_b64 / ds_read_b64_tr_b16 in groups
// of 32, each group over 64 four-byte banks (address bits 2-7); the
// permutations below make every K and V operand read conflict-free.
//
// Variants (template parameters): E4M3 Q and K for the first product (KF8),
// and two key groups per query tile for grids too small to fill the chip
// (KG = 2); both are described at the kernel.
//
// Softmax work per score: half a three-input max, one FMA (scale folded in,
// base-2 domain), one exp2, half a pack to 16 bits, and for the row sum one
// fp32 add (bf16) or half a v_dot2 of the rounded P (fp16); the per-tile sums
// enter the running sum through a compensated (Kahan) add.  The accumulator
// is rescaled only when some row's maximum grows by more than 2^8 over the
// value in use; otherwise the stale maximum is kept, which bounds every
// probability by 2^8 and leaves the final O = acc / l exact, because
// numerator and denominator share the factor.
#include "fa_device.hpp"
#include "fa_internal.hpp"

#include <type_traits>
#include <utility>

namespace fa355 {
namespace {

constexpr int kBN = 64;                // keys per tile
constexpr float kRescaleSlack = 8.0f;  // log2 of the largest probability kept without rescaling
constexpr float kMinC = 1e-30f;        // lower bound of the exponent scale (see launch)

struct FwdParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int Nq, Nkv;
    int n_bh, n_qt;
    float c;         // max(|scale| * log2(e), kMinC): scores are kept in the base-2 domain
    uint32_t qsign;  // 0x80008000 when scale < 0: Q is negated as it is loaded
};

template <int N> using IC = std::integral_constant<int, N>;

// The MFMA row that lane l % 32 feeds is key swap23(l % 32) of the sub-tile
// (bits 2 and 3 exchanged); see the file comment.
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// XOR permutations of the 16-byte chunk index within a row, as functions of
// the row.  K is read as 16-byte runs, one logical chunk per half-wave: a
// b128 group of 16 lanes (lanes {0-3, 12-15, 20-27} and the like, see the
// file comment) holds rows swap23 of those lanes, i.e. rows {0-3, 12-15,
// 20-27} mod 32, whose low four bits are all distinct: the permutation must
// send those 16 rows to 16 distinct 16-byte bank groups.  V is read
// transposed: 32 lanes cover 4 consecutive rows (starting at a multiple of 4)
// x 64 bytes, so the 4 rows must land in 4 distinct 64-byte bank segments.
// For d = 64 two rows share one 256-byte bank line, hence the extra shift by
// one row bit.
//
// K rows are 2d bytes (16-bit K) or d bytes (E4M3 K): 256, 128 or 64 bytes,
// i.e. one, a half or a quarter of a 256-byte bank line.  The 16 rows read
// together differ in their low four bits, so the row bits below the line take
// the low bits of the bank-group index and the rest of the XOR spreads the
// rows that share them.
template <int ROWB> __host__ __device__ constexpr int kswz(int row)
{
    static_assert(ROWB == 256 || ROWB == 128 || ROWB == 64, "K rows of 256, 128 or 64 bytes");
    return ROWB == 256 ? (row & 15) : ROWB == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
template <int D> __host__ __device__ constexpr int vswz(int row)
{
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// Wait until at most n direct loads of this wave are in flight, n a multiple
// of L in [0, K L] (s_waitcnt takes an immediate, so the few possible values
// are dispatched).
template <int L, int K> __device__ __forceinline__ void wait_loads(int n)
{
    if constexpr (K > 0) {
        if (n >= K * L) {
            wait_vmcnt<K * L>();
            return;
        }
        wait_loads<L, K - 1>(n);
    } else {
        wait_vmcnt<0>();
    }
}

constexpr int lcm2(int n) { return n % 2 ? 2 * n : n; }

// Direct K loads: a wave's load i fills the LDS chunks 64 i .. 64 i + 63 after
// those of its load 0, which hold the rows 1024 i / ROWB further on, so its
// global offset is load 0's with the row advanced (the instruction offset,
// 1024 i bytes) and the chunk permutation changed.  The change is the XOR
// kswz(1024 i / ROWB) on the chunk index when, for every lane, the rows of
// load 0 keep clear of the permutation bits that the advance flips.  This
// checks that for every lane of every wave of a key group (the wave's loads
// start at chunk w * LOADS_K * 64).
template <int ROWB> constexpr int k_load_xor(int i) { return kswz<ROWB>(i * (1024 / ROWB)); }
template <int ROWB, int LOADS_K, int WGW> constexpr bool k_load_xor_holds()
{
    constexpr int KDC = ROWB / 16;
    for (int w = 0; w < WGW; ++w)
        for (int lane = 0; lane < 64; ++lane) {
            const int row = (w * LOADS_K * 64 + lane) / KDC;
            for (int i = 0; i < LOADS_K; ++i)
                if (kswz<ROWB>(row + i * (1024 / ROWB)) != (kswz<ROWB>(row) ^ k_load_xor<ROWB>(i))) return false;
        }
    return true;
}

// NW waves in KG key groups, each wave of a group owning 32 query rows
// (BM = 32 NW / KG rows per workgroup), and a ring of NS K/V stages per group.  KF8: Q and K enter the first product as E4M3 ("FlashAttention
// 1-2-3 ...", section "FlashAttention-3": Q and K in FP8, V and O in 16 bits,
// fp32 accumulation).  K then arrives already quantised (d bytes per row, half
// the LDS bytes of the 16-bit tile), Q is quantised here as it is loaded, and
// S^T = K Q^T runs on the 32x32x64 E4M3 MFMA; everything after the scores is
// unchanged.
//
// KG = 2 (key groups) serves grids too small to fill the chip: the waves form
// two groups that take the same query rows and alternate key tiles (group g
// takes tiles g, g + 2, ...), each with its own LDS ring, and the two partial
// results are merged exactly at the end through LDS, with the two-block merge
// of "FlashAttention 1-2-3 ...", section "The Math Behind the Online Softmax
// Trick".  That halves the serial chain of key tiles behind each query tile.
template <int D, typename T, bool CAUSAL, bool OUT_F32, int NW, int NS, bool KF8, int KG>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdParams p)
{
    static_assert(KG == 1 || KG == 2, "one or two key groups");
    constexpr int WGW = NW / KG;            // waves per key group
    constexpr int BN = kBN, BM = 32 * WGW;  // keys per tile, query rows per workgroup
    constexpr int NT = 64 * WGW;            // threads of a key group (they fill its ring)
    constexpr int DC = D / 8;               // 16-byte chunks per Q, V or O row
    constexpr int TILE = BN * DC;           // chunks per V tile
    constexpr int LOADS = TILE / NT;        // direct loads per thread per V tile
    constexpr int ROWB = D * 2;             // bytes per Q, V or O row
    constexpr int KROWB = KF8 ? D : 2 * D;  // bytes per K row
    constexpr int KDC = KROWB / 16;         // chunks per K row
    constexpr int KTILE = BN * KDC;         // chunks per K tile
    constexpr int LOADS_K = KTILE / NT;     // direct loads per thread per K tile
    constexpr int KS = KF8 ? D / 64 : D / 16;  // k-steps of the first product
    constexpr int DT = D / 32;              // 32-dim blocks of the output
    constexpr int U = lcm2(NS);             // steps per loop iteration (stage and score-set periods)
    static_assert(NS >= 2 && TILE % NT == 0 && LOADS >= 1 && LOADS <= 4, "tile must split evenly over the threads");
    static_assert(KTILE % NT == 0 && LOADS_K >= 1 && LOADS_K <= 4, "K tile must split evenly, 4 loads at most");
    static_assert(k_load_xor_holds<KROWB, LOADS_K, WGW>(), "K load i is load 0 advanced and re-permuted");
    static_assert(NS * TILE * 16 <= 65536, "stage offsets must fit the 16-bit LDS immediate");
    using V8 = typename Vec<T>::v8;
    using QOp = typename std::conditional<KF8, i32x8, V8>::type;

    // K and V rings of each key group, [key][dim] tiles, chunk-permuted; with
    // two key groups the same memory holds the partial results at the end.
    __shared__ u32x4 lds_rings[KG * NS * (KTILE + TILE)];
    u32x4(*const sk)[NS][KTILE] = reinterpret_cast<u32x4(*)[NS][KTILE]>(lds_rings);
    u32x4(*const sv)[NS][TILE] = reinterpret_cast<u32x4(*)[NS][TILE]>(lds_rings + KG * NS * KTILE);
    static_assert(KG == 1 || (WGW * (DT * 16 + 2) * 64 * 4 <= KG * NS * (KTILE + TILE) * 16),
                  "the partial results of a key group fit the rings");
    if constexpr (kPoisonLds) {
        poison_lds(lds_rings, sizeof(lds_rings));
        __syncthreads();
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform by construction
    const int grp = KG == 1 ? 0 : wave / WGW;                   // key group of the wave
    const int rw = KG == 1 ? wave : wave % WGW;                 // its block of 32 query rows
    const int c = lane & 31, h = lane >> 5;

    // Heaviest causal tiles (last query rows) are dispatched first.  Consecutive
    // workgroups cycle through heads, so when B*H is a multiple of the XCD count
    // every tile of one head lands on one XCD and shares its L2.
    const int bh = blockIdx.x % p.n_bh;
    const int qt = p.n_qt - 1 - static_cast<int>(blockIdx.x / p.n_bh);
    const int q0 = qt * BM;
    const int wq0 = q0 + 32 * rw;
    const int off = p.Nkv - p.Nq;  // causal: row i sees keys j <= i + off
    int kend = p.Nkv;
    if constexpr (CAUSAL) kend = min(p.Nkv, min(q0 + BM, p.Nq) + off);
    const int nkb = (kend + BN - 1) / BN;  // >= 1: every row sees key 0
    // key tiles this wave's rows can see; 0 for a wave wholly past Nq
    int nkw = 0;
    if (wq0 < p.Nq) {
        nkw = nkb;
        if constexpr (CAUSAL) nkw = min(nkb, (min(wq0 + 31, p.Nq - 1) + off) / BN + 1);
    }
    // This group's share: local tile t is key tile KG t + grp.  Both groups run
    // ntl steps (group 0's count), so every wave reaches every barrier.
    const int ntl = (nkb + KG - 1) / KG;
    const int nkb_g = (nkb - grp + KG - 1) / KG;  // tiles of the group's ring
    const int nkw_g = (nkw - grp + KG - 1) / KG;  // of them, tiles this wave's rows can see

    // Per-head buffer descriptors: reads past a head's last row return zeros,
    // which fills the ragged end of the last tile (those keys are masked) and
    // the query rows past Nq.  Offsets are unsigned 32-bit: every row of a head
    // (< 4 GiB) fits, and for a head within a tile of 4 GiB the rows past its
    // end wrap to rows of the same head instead.  Either way those keys get
    // s = -inf before the row max and those query rows are never stored.
    const size_t q_head = static_cast<size_t>(bh) * p.Nq * ROWB;
    const size_t k_head = static_cast<size_t>(bh) * p.Nkv * KROWB;
    const size_t v_head = static_cast<size_t>(bh) * p.Nkv * ROWB;
    const auto rq = make_rsrc(static_cast<const char *>(p.q) + q_head, static_cast<uint32_t>(p.Nq) * ROWB);
    const u32x4 rk = make_rsrc_words(static_cast<const char *>(p.k) + k_head, static_cast<uint32_t>(p.Nkv) * KROWB);
    const u32x4 rv = make_rsrc_words(static_cast<const char *>(p.v) + v_head, static_cast<uint32_t>(p.Nkv) * ROWB);

    // Q operand, loaded once: lane (c, h) holds query wq0 + c, dims 16 s + 8 h .. + 7
    // (16-bit), or dims 64 s + 32 h .. + 31 rounded to E4M3 (KF8).
    const int qrow = wq0 + c;
    QOp qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        if constexpr (KF8) {
            i32x8 w;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x4 x = buffer_load16(rq, static_cast<uint32_t>(qrow) * ROWB + (64 * s + 32 * h + 8 * t) * 2, 0) ^ p.qsign;
                w[2 * t] = static_cast<int>(e4m3x4(lo_f32<T>(x[0]), hi_f32<T>(x[0]), lo_f32<T>(x[1]), hi_f32<T>(x[1])));
                w[2 * t + 1] = static_cast<int>(e4m3x4(lo_f32<T>(x[2]), hi_f32<T>(x[2]), lo_f32<T>(x[3]), hi_f32<T>(x[3])));
            }
            qf[s] = w;
        } else {
            const u32x4 x = buffer_load16(rq, static_cast<uint32_t>(qrow) * ROWB + (16 * s + 8 * h) * 2, 0) ^ p.qsign;
            qf[s] = as<V8>(x);
        }
    }

    // Direct loads: the wave's i-th load of a tensor fills LDS chunks
    // [(wave*LOADS + i)*64, +64) lane by lane; the lane fetches whichever
    // global chunk the permutation puts there.  Load i sits 1024 bytes after
    // load 0 both in memory and in LDS (the instruction offset), and only the
    // K permutation changes with i, as the XOR k_load_xor(i) on the chunk
    // index (checked for this shape by the static_assert above).
    uint32_t koff0, voff0;
    {
        const int pch = rw * LOADS_K * 64 + lane;
        const int row = pch / KDC, col = pch % KDC;
        koff0 = row * KROWB + ((col ^ kswz<KROWB>(row)) << 4);
    }
    {
        const int pch = rw * LOADS * 64 + lane;
        const int row = pch / DC, col = pch % DC;
        voff0 = row * ROWB + ((col ^ vswz<D>(row)) << 4);
    }
    // kb: the group's local tile index
    auto issue_k = [&](auto st, int kb) {
        const uint32_t tile = static_cast<uint32_t>(KG * kb + grp) * BN * KROWB;
        const u32x4 *dst = &sk[grp][decltype(st)::value][rw * LOADS_K * 64];
        dma_to_lds16<0>(rk, koff0, tile, dst);
        if constexpr (LOADS_K > 1) dma_to_lds16<1024>(rk, koff0 ^ (k_load_xor<KROWB>(1) << 4), tile, dst);
        if constexpr (LOADS_K > 2) dma_to_lds16<2048>(rk, koff0 ^ (k_load_xor<KROWB>(2) << 4), tile, dst);
        if constexpr (LOADS_K > 3) dma_to_lds16<3072>(rk, koff0 ^ (k_load_xor<KROWB>(3) << 4), tile, dst);
    };
    auto issue_v = [&](auto st, int kb) {
        const uint32_t tile = static_cast<uint32_t>(KG * kb + grp) * BN * ROWB;
        const u32x4 *dst = &sv[grp][decltype(st)::value][rw * LOADS * 64];
        dma_to_lds16<0>(rv, voff0, tile, dst);
        if constexpr (LOADS > 1) dma_to_lds16<1024>(rv, voff0, tile, dst);
        if constexpr (LOADS > 2) dma_to_lds16<2048>(rv, voff0, tile, dst);
        if constexpr (LOADS > 3) dma_to_lds16<3072>(rv, voff0, tile, dst);
    };
    // Step j requests V_{j+NS-1} and K_{j+NS}; the prologue acts as steps
    // 1 - NS .. -1.  At the end of step j, K_{j+2} and V_{j+1} must have
    // landed, so the loads of steps j + 3 - NS .. j may stay in flight.
    auto allowance = [&](int j) {
        int n = 0;
#pragma unroll
        for (int i = j + 3 - NS; i <= j; ++i)
            if (i >= 1 - NS) n += LOADS * (i + NS - 1 < nkb_g) + LOADS_K * (i + NS < nkb_g);
        return n;
    };
    // LOADS is a multiple of LOADS_K, so every allowance is one too
    constexpr int kMaxWait = (NS - 2) * (LOADS + LOADS_K) / LOADS_K;

    // LDS byte offsets of this lane's MFMA operands within a tile.
    // K operand (kk, s): row 32 kk + swap23(c), logical chunk 2 s + h (16-bit)
    // or the two chunks 4 s + 2 h and 4 s + 2 h + 1 (E4M3).  The permutation is
    // an XOR on the chunk index and these chunk numbers are the step-0 chunk
    // with disjoint higher bits set, so every operand is the step-0 offset
    // XOR-ed by a constant; kk adds 32 rows, which leaves the permutation
    // unchanged.
    uint32_t ka0;
    {
        const int krow = swap23(c);
        ka0 = krow * KROWB + (((KF8 ? 2 * h : h) ^ kswz<KROWB>(krow)) << 4);
    }
    // V^T operand (dt, kk, u, half): lane 16 g + 4 j + q addresses key
    // 32 kk + 16 u + 8 (g / 2) + j + 4 half and dims 32 dt + 16 (g % 2) + 4 q .. + 3,
    // i.e. logical chunk 4 dt + 2 (g % 2) + q / 2, byte 8 (q % 2) within it.
    // dt enters as an XOR on bits 6.. of the in-row offset; kk, u and half move
    // the row by multiples of 4, which leaves the permutation unchanged, so
    // they are compile-time offsets.
    uint32_t va0;
    {
        const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
        const int row = 8 * (g >> 1) + j;
        va0 = row * ROWB + (((2 * (g & 1) + (q >> 1)) ^ vswz<D>(row)) << 4) + ((q & 1) << 3);
    }

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
    float m_run = -INFINITY;  // row max (base-2 scaled) the probabilities are taken against
    float l_run = 0.f;        // running sum over this lane's half of the keys
    float l_cmp = 0.f;        // minus the low-order part the last add dropped
    const float cs = p.c;

    // Compensated (Kahan) row sum.  With millions of keys a row's per-tile
    // sums fall near half an ulp of the running sum and plain adds round them
    // away, always downwards; the compensation carries each add's loss into
    // the next one.
    auto add_l = [&](float x) {
        const float y = x - l_cmp;
        const float t = l_run + y;
        l_cmp = (t - l_run) - y;
        l_run = t;
    };

    // S^T = K Q^T for the K tile in stage st (two 32-key sub-tiles).
    auto scores = [&](auto st, f32x16 (&sn)[2]) {
        const char *SK = reinterpret_cast<const char *>(sk[grp][decltype(st)::value]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 16; ++e) sn[kk][e] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if constexpr (KF8) {
                    const char *base = SK + kk * 32 * KROWB;
                    const u32x4 x0 = *reinterpret_cast<const u32x4 *>(base + (ka0 ^ ((4 * s) << 4)));
                    const u32x4 x1 = *reinterpret_cast<const u32x4 *>(base + (ka0 ^ ((4 * s + 1) << 4)));
                    const i32x8 a = {static_cast<int>(x0[0]), static_cast<int>(x0[1]), static_cast<int>(x0[2]),
                                     static_cast<int>(x0[3]), static_cast<int>(x1[0]), static_cast<int>(x1[1]),
                                     static_cast<int>(x1[2]), static_cast<int>(x1[3])};
                    sn[kk] = mfma32_e4m3(a, qf[s], sn[kk]);
                } else {
                    const u32x4 x = *reinterpret_cast<const u32x4 *>(SK + (ka0 ^ (s << 5)) + kk * 32 * KROWB);
                    sn[kk] = mfma32(as<V8>(x), qf[s], sn[kk]);
                }
            }
    };

    // causal diagonal / ragged end: invisible keys get -inf
    auto needs_mask = [&](int kv0) { return (kv0 + BN > p.Nkv) || (CAUSAL && kv0 + BN - 1 > wq0 + off); };
    auto mask = [&](f32x16 (&sn)[2], int kv0) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = kv0 + 32 * kk + 16 * (e >> 3) + 8 * h + (e & 7);
                if (key >= p.Nkv || (CAUSAL && key > qrow + off)) sn[kk][e] = -INFINITY;
            }
    };

    // Row maximum of a score tile, scaled to the base-2 domain (c > 0); two
    // chains of three-input maxima.
    auto rowmax = [&](const f32x16 (&sn)[2]) {
        float m0 = fmaxf(sn[0][0], sn[0][1]), m1 = fmaxf(sn[1][0], sn[1][1]);
#pragma unroll
        for (int e = 2; e < 16; e += 2) {
            m0 = fmaxf(fmaxf(m0, sn[0][e]), sn[0][e + 1]);
            m1 = fmaxf(fmaxf(m1, sn[1][e]), sn[1][e + 1]);
        }
        return max_with_other_half(fmaxf(m0, m1)) * cs;
    };

    // Lazy rescale: only when some row's block max exceeds the max in use by
    // more than the slack (a wave-uniform branch).
    auto rescale = [&](float m_blk) {
        if (__builtin_amdgcn_ballot_w64(m_blk > m_run + kRescaleSlack)) {
            const float m_new = fmaxf(m_run, m_blk);
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
            l_run *= alpha;
            l_cmp *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
            m_run = m_new;
        }
    };

    // p = 2^(c s - m) (exactly 0 for masked keys) and P in the storage type:
    // operand (kk, u) holds keys 32 kk + 16 u + 8 h .. + 7.  The row sum:
    //  - fp16: the rounded P that the second product uses, summed in fp32 by
    //    v_dot2 (rowsum_p, in phase 2); P's rounding error is at most 2^-11 of
    //    each term, so the normalisation stays consistent with the numerator;
    //  - bf16: the fp32 values before rounding (2^-9 per term would be too
    //    coarse for the log-sum-exp).
    constexpr bool kSumP = std::is_same<T, _Float16>::value;
    auto softmax = [&](f32x16 (&sc)[2], V8 (&pf)[2][2]) {
        // m_run is finite once a row has seen a key; with one key group every
        // row sees key 0 in the first tile.  The second group's first tiles
        // may hide every key from a row: then m_run is -inf and p must be 0.
        float neg_m = -m_run;
        if constexpr (KG > 1) neg_m = m_run == -INFINITY ? 0.f : neg_m;
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                u32x4 w;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float a = fast_exp2(fmaf(sc[kk][8 * u + 2 * j], cs, neg_m));
                    const float b = fast_exp2(fmaf(sc[kk][8 * u + 2 * j + 1], cs, neg_m));
                    if constexpr (!kSumP) {
                        rs0 += a;
                        rs1 += b;
                    }
                    w[j] = pack2<T>(a, b);
                }
                pf[kk][u] = as<V8>(w);
            }
        if constexpr (!kSumP) {
            add_l(rs0 + rs1);
            asm volatile("" : "+v"(l_run), "+v"(l_cmp));  // keep the adds beside the exps
        }
    };
    auto rowsum_p = [&](const V8 (&pf)[2][2]) {
        if constexpr (kSumP) {
            const uint32_t ones = 0x3C003C00u;  // (1.0, 1.0) in binary16
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const u32x4 w = __builtin_bit_cast(u32x4, pf[kk][u]);
                    r0 = dot2<T>(w[0], ones, r0);
                    r1 = dot2<T>(w[1], ones, r1);
                    r0 = dot2<T>(w[2], ones, r0);
                    r1 = dot2<T>(w[3], ones, r1);
                }
            add_l(r0 + r1);
        }
    };
    // An empty asm statement that claims to read and rewrite P: the compiler
    // must form P before it, in the same block as the score MFMAs.
    auto pin = [](V8 (&pf)[2][2]) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                u32x4 w = __builtin_bit_cast(u32x4, pf[kk][u]);
                asm volatile("" : "+v"(w));
                pf[kk][u] = as<V8>(w);
            }
    };

    // O^T += V^T P^T for the V tile in stage st (two transposed reads per operand).
    auto pv = [&](auto st, const V8 (&pf)[2][2]) {
        const char *SV = reinterpret_cast<const char *>(sv[grp][decltype(st)::value]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const char *pa = SV + (va0 ^ (dt << 6)) + (32 * kk + 16 * u) * ROWB;
                    const u32x2 lo = lds_read_tr16(pa);
                    const u32x2 hi = lds_read_tr16(pa + 4 * ROWB);
                    const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[dt] = mfma32(as<V8>(a), pf[kk][u], oacc[dt]);
                }
    };

    // One pipeline step for key tile j (stage S = j % NS): V_j sits in sv[S],
    // K_{j+1} in sk[(S + 1) % NS].  The two score sets alternate with j % 2.
    // Waves skip the arithmetic of tiles none of their rows can see but take
    // part in every load and barrier.  On a wave's last tile the scores of the
    // next tile are still formed (from whatever the stage holds, always in
    // bounds) and never used: one branch fewer keeps the step spill-free.
    f32x16 sa[2], sb[2];
    V8 pf[2][2];
    float mx = -INFINITY;
    auto step = [&](auto st, f32x16 (&sc)[2], f32x16 (&sn)[2], int j) {
        constexpr int S = decltype(st)::value % NS;
        if (j + NS - 1 < nkb_g) issue_v(IC<(S + NS - 1) % NS>{}, j + NS - 1);
        if (j + NS < nkb_g) issue_k(IC<S>{}, j + NS);
        if (j < nkw_g) {
            rescale(mx);
            // phase 1: MFMAs of the next scores beside the softmax of the current ones
            scores(IC<(S + 1) % NS>{}, sn);
            softmax(sc, pf);
            pin(pf);  // P is formed here, not sunk past the mask branch
            const int kv1 = (KG * (j + 1) + grp) * BN;
            if (needs_mask(kv1)) mask(sn, kv1);
            // phase 2: MFMAs of O += V P beside the row max of the next scores
            pv(IC<S>{}, pf);
            rowsum_p(pf);
            mx = rowmax(sn);
        }
        wait_loads<LOADS_K, kMaxWait>(allowance(j));
        __syncthreads();
    };

    // Prologue: K_0, then the requests of steps 1 - NS .. -1 (V_0 .. V_{NS-2},
    // K_1 .. K_{NS-1}); wait for K_0, V_0 and K_1, form S_0 and its row max.
    if (nkb_g > 0) issue_k(IC<0>{}, 0);
    [&]<int... I>(std::integer_sequence<int, I...>) {
        ((I < nkb_g ? (issue_v(IC<I>{}, I), 0) : 0, I + 1 < nkb_g ? (issue_k(IC<I + 1>{}, I + 1), 0) : 0), ...);
    }(std::make_integer_sequence<int, NS - 1>{});
    wait_loads<LOADS_K, kMaxWait>(allowance(-1));
    __syncthreads();
    if (nkw_g > 0) {
        scores(IC<0>{}, sa);
        if (needs_mask(grp * BN)) mask(sa, grp * BN);
        mx = rowmax(sa);
    }
    __syncthreads();  // every wave is done with sk[0] before K_NS refills it

    for (int j = 0; j < ntl; j += U) {
        [&]<int... I>(std::integer_sequence<int, I...>) {
            ((j + I < ntl ? (I % 2 == 0 ? step(IC<I>{}, sa, sb, j + I) : step(IC<I>{}, sb, sa, j + I)), 0 : 0), ...);
        }(std::make_integer_sequence<int, U>{});
    }

    // Epilogue: O = acc / l, LSE = ln 2 * (m + log2 l).
    float l_tot = sum_with_other_half(l_run - l_cmp);
    if constexpr (KG == 2) {
        // Group 1 hands its partial result (accumulator, reference max, row
        // sum; lane by lane, so the same lane of the partner wave holds the
        // same query and dims) to group 0 through the rings' memory, which the
        // last step's barrier has freed.  Group 0 merges:
        //   M = max(m0, m1), O = (2^(m0-M) O0 + 2^(m1-M) O1) / (2^(m0-M) l0 + 2^(m1-M) l1).
        float *xo = reinterpret_cast<float *>(lds_rings);  // [WGW][DT * 16][64]
        float *xm = xo + WGW * DT * 16 * 64;              // [WGW][2][64]
        if (grp == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) xo[((rw * DT + dt) * 16 + e) * 64 + lane] = oacc[dt][e];
            xm[(rw * 2) * 64 + lane] = m_run;
            xm[(rw * 2 + 1) * 64 + lane] = l_tot;
        }
        __syncthreads();
        if (grp == 0) {
            const float m1 = xm[(rw * 2) * 64 + lane], l1 = xm[(rw * 2 + 1) * 64 + lane];
            const float mm = fmaxf(m_run, m1);  // finite: group 0 holds key 0
            const float a0 = fast_exp2(m_run - mm), a1 = fast_exp2(m1 - mm);
            l_tot = a0 * l_tot + a1 * l1;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    oacc[dt][e] = a0 * oacc[dt][e] + a1 * xo[((rw * DT + dt) * 16 + e) * 64 + lane];
            m_run = mm;
        }
    }
    if (qrow < p.Nq && grp == 0) {
        const float inv = 1.f / l_tot;
        const size_t orow = (static_cast<size_t>(bh) * p.Nq + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
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
        if (h == 0 && p.lse) p.lse[static_cast<size_t>(bh) * p.Nq + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// The same algorithm on the 16x16x32 MFMA, for 16-bit K.
//
// Measured on MI355X with random fp16 operands at two waves per SIMD, a stream
// of v_mfma_f32_16x16x32_f16 sustains about 18% more FLOP/s than one of
// v_mfma_f32_32x32x16_f16 (1876 against 1592 TFLOP/s), while on all-zero
// operands the two are equal (2352 / 2322): the smaller instruction moves a
// quarter of the accumulator per issue, and under the chip's power limit the
// energy per FLOP sets the rate.  This kernel keeps the 32x32 kernel's
// structure -- 32 query rows per wave, 64-key tiles through a direct-to-LDS
// ring, heavy tiles first -- and changes the fragment layout and the
// schedule (below):
//
//   S^T (16 keys x 16 queries) += K (16 keys x 32 dims) * Q^T (32 dims x 16 queries)
//   O^T (16 dims x 16 queries) += V^T (16 dims x 32 keys) * P^T (32 keys x 16 queries)
//
// Lane l = 16 g + i supplies row / column i of an operand and the eight
// k-slots of group g; it receives column i (a query) and rows 4g .. 4g + 3 of
// the result.  A wave's 32 rows are two query blocks, so a lane holds two
// queries and, per 64-key tile, the keys {16 kb + 4 g + r : kb < 4, r < 4} of
// each.  Each K or V^T operand read from LDS feeds both query blocks (the same
// LDS bytes per FLOP as the 32x32 kernel).  A k-step of the second product
// takes key blocks 2s and 2s + 1, and a lane's k-slots are keys 4g .. 4g + 3 of
// each -- the keys its score fragments already hold -- so P goes from the
// score accumulators to the MFMA operand without moving between lanes.
//
// Row maxima are taken on demand.  Probabilities are formed against the
// reference maximum in use (m_run, the same for the four lanes of a query);
// the tile is redone against the running maximum only when some lane's sum
// over its keys exceeds kSumLimit or is not finite (a wave-uniform branch:
// the first tile of every row, and a row whose scores later rise by more than
// about 2^15 over the reference).  So every probability of a 16-bit P operand
// is at most kSumLimit, far inside its range, and the common step has no
// cross-lane reduction at all: the four lanes' partial row sums meet only in
// the epilogue.  O = acc / l is exact whatever the reference, as numerator and
// denominator share it.
//
// Schedule of the eight-wave shape (two waves per SIMD).  A wave's work per
// key tile splits into an MFMA block M (the next tile's scores and this
// tile's O += V P: 64 MFMAs at d = 128, no VALU beyond addressing) and a VALU
// block (softmax of the scores just formed: about 110 instructions, a third
// of them v_exp_f32).  A single wave issues at most one VALU instruction per
// ~8 cycles, while an MFMA stream of another wave on the same SIMD keeps
// running beside it at nearly full rate (measured: 17 cycles per 16x16x32
// MFMA beside a stream of FMAs, 19 beside exps, 16 alone).  So the two waves
// of a SIMD are kept half a step apart: waves 0..3 pass the step's barrier
// after their softmax block and waves 4..7 after their MFMA block, and each
// SIMD's MFMA block of one wave runs beside the softmax block of the other.
// Measured 4-6% faster than running both waves through the same phases on
// the causal 8K and 16K d = 128 workloads; the M block requests its LDS
// operands a fixed distance ahead of the MFMAs that take them (K one k-step,
// V six MFMA pairs ahead): another 2-7%.
constexpr float kSumLimit = 32768.0f;

// V rows are read transposed: a 32-lane group covers 8 consecutive rows x 32
// bytes; the permutation puts those 8 runs into 8 distinct 32-byte segments of
// the 256-byte bank line (two rows share a line at d = 64).
template <int D> __host__ __device__ constexpr int vswz16(int row)
{
    return D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3);
}
template <int ROWB, int LOADS, int NW, int (*SWZ)(int)> constexpr bool load_xor_holds(int (*xor_of)(int))
{
    constexpr int DCH = ROWB / 16;
    for (int w = 0; w < NW; ++w)
        for (int lane = 0; lane < 64; ++lane) {
            const int row = (w * LOADS * 64 + lane) / DCH;
            for (int i = 0; i < LOADS; ++i)
                if (SWZ(row + i * (1024 / ROWB)) != (SWZ(row) ^ xor_of(i))) return false;
        }
    return true;
}
// E4M3 K rows (128 bytes at d = 128, two to a bank line) under the 16x16x128
// read: lane l = 16 g + i takes row i at chunks 2 g and 2 g + 1 (two b128
// reads).  A ds_read_b128 is served in four groups of 16 lanes: in each
// half-wave the lane quads whose three index bits have even parity form one
// group and the odd ones the other, so a group reads rows {0-3, 12-15} of one
// g and rows {4-11} of the other.  (row & 6) | (row >> 3) puts every group's
// 16 reads in distinct 16-byte slots of the bank line; kswz<128> = (row >> 1)
// & 7 would put them 2 to a slot.
__host__ __device__ constexpr int k8swz16(int row) { return (row & 6) | ((row >> 3) & 1); }
constexpr bool k8_reads_conflict_free()
{
    for (int rd = 0; rd < 2; ++rd)
        for (int a = 0; a < 64; ++a)
            for (int b = a + 1; b < 64; ++b) {
                const int qa = (a >> 2) & 7, qb = (b >> 2) & 7;
                if ((a >> 5) != (b >> 5) || (__builtin_popcount(qa) & 1) != (__builtin_popcount(qb) & 1)) continue;
                const int ra = a & 15, rb = b & 15;
                const int sa = (8 * (ra & 1) + ((2 * (a >> 4) + rd) ^ k8swz16(ra))) & 15;
                const int sb = (8 * (rb & 1) + ((2 * (b >> 4) + rd) ^ k8swz16(rb))) & 15;
                if (ra != rb && sa == sb) return false;
            }
    return true;
}
static_assert(k8_reads_conflict_free(), "E4M3 K reads of the 16x16x128 MFMA are conflict-free");

template <int ROWB> constexpr int k16_xor(int i) { return kswz<ROWB>(i * (1024 / ROWB)); }
template <int D> constexpr int v16_xor(int i) { return vswz16<D>(i * (1024 / (2 * D))); }
template <int ROWB> constexpr int kswz_fn(int row) { return kswz<ROWB>(row); }
template <int D> constexpr int vswz16_fn(int row) { return vswz16<D>(row); }

template <int D, typename T, bool CAUSAL, bool OUT_F32, int NW, int NS, bool KF8 = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd16_kernel(FwdParams p)
{
    constexpr int BN = kBN, BM = 32 * NW;  // keys per tile, query rows per workgroup
    constexpr int NT = 64 * NW;            // threads (they fill the ring)
    constexpr int DC = D / 8;              // 16-byte chunks per row
    constexpr int TILE = BN * DC;          // chunks per K or V tile
    constexpr int LOADS = TILE / NT;       // direct loads per thread per tile
    constexpr int ROWB = D * 2;            // bytes per row
    constexpr int KS = D / 32;             // k-steps of the first product
    constexpr int DB = D / 16;             // 16-dim blocks of the output
    constexpr int U = lcm2(NS);
    // KF8: K arrives as E4M3 bytes (d bytes per row) and Q is rounded to E4M3
    // as it is loaded; S^T = K Q^T then takes one 16x16x128 E4M3 MFMA per
    // (key block, query block) at d = 128, the rest is unchanged.
    static_assert(!KF8 || (D == 128 && NW == 8 && NS == 2), "E4M3 K: d = 128, eight waves");
    constexpr int KROWB = KF8 ? D : ROWB;  // bytes per K row
    constexpr int KTILE = BN * KROWB / 16; // chunks per K tile
    constexpr int LOADS_K = KTILE / NT;    // direct loads per thread per K tile
    static_assert(NS >= 2 && TILE % NT == 0 && LOADS >= 1 && LOADS <= 4, "tile must split evenly over the threads");
    static_assert(KTILE % NT == 0 && LOADS_K >= 1, "K tile must split evenly over the threads");
    static_assert(KF8 || load_xor_holds<ROWB, LOADS, NW, kswz_fn<ROWB>>(k16_xor<ROWB>), "K load i is load 0 re-permuted");
    static_assert(load_xor_holds<ROWB, LOADS, NW, vswz16_fn<D>>(v16_xor<D>), "V load i is load 0 re-permuted");
    static_assert(NS * (KTILE + TILE) * 16 <= 65536, "stage offsets must fit the 16-bit LDS immediate");
    using V8 = typename Vec<T>::v8;

    // K and V rings; the O stage of the epilogue reuses them (hence the size)
    constexpr int RING = NS * (KTILE + TILE), OSTAGE = NW * 32 * ROWB / 16;
    __shared__ u32x4 lds_rings[RING > OSTAGE ? RING : OSTAGE];
    u32x4(*const sk)[KTILE] = reinterpret_cast<u32x4(*)[KTILE]>(lds_rings);
    u32x4(*const sv)[TILE] = reinterpret_cast<u32x4(*)[TILE]>(lds_rings + NS * KTILE);
    if constexpr (kPoisonLds) {
        poison_lds(lds_rings, sizeof(lds_rings));
        __syncthreads();
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;

    const int bh = blockIdx.x % p.n_bh;
    const int qt = p.n_qt - 1 - static_cast<int>(blockIdx.x / p.n_bh);
    const int q0 = qt * BM;
    const int wq0 = q0 + 32 * wave;
    const int off = p.Nkv - p.Nq;
    int kend = p.Nkv;
    if constexpr (CAUSAL) kend = min(p.Nkv, min(q0 + BM, p.Nq) + off);
    const int nkb = (kend + BN - 1) / BN;
    int nkw = 0;
    if (wq0 < p.Nq) {
        nkw = nkb;
        if constexpr (CAUSAL) nkw = min(nkb, (min(wq0 + 31, p.Nq - 1) + off) / BN + 1);
    }

    const size_t q_head = static_cast<size_t>(bh) * p.Nq * ROWB;
    const size_t kv_head = static_cast<size_t>(bh) * p.Nkv * ROWB;
    const auto rq = make_rsrc(static_cast<const char *>(p.q) + q_head, static_cast<uint32_t>(p.Nq) * ROWB);
    const u32x4 rk = make_rsrc_words(static_cast<const char *>(p.k) + (KF8 ? kv_head / 2 : kv_head),
                                     static_cast<uint32_t>(p.Nkv) * KROWB);
    const u32x4 rv = make_rsrc_words(static_cast<const char *>(p.v) + kv_head, static_cast<uint32_t>(p.Nkv) * ROWB);

    // Q operand, loaded once: lane (g, i) holds query wq0 + 16 qb + i, dims
    // 32 s + 8 g .. + 7.
    // KF8: dims 32 g .. + 31 rounded to E4M3 (qf8), the B operand of the one
    // 128-deep k-step.
    V8 qf[2][KF8 ? 1 : KS];
    i32x8 qf8[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        if constexpr (KF8) {
            i32x8 w;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x4 x =
                    buffer_load16(rq, static_cast<uint32_t>(wq0 + 16 * qb + li) * ROWB + (32 * g + 8 * t) * 2, 0) ^ p.qsign;
                w[2 * t] = static_cast<int>(e4m3x4(lo_f32<T>(x[0]), hi_f32<T>(x[0]), lo_f32<T>(x[1]), hi_f32<T>(x[1])));
                w[2 * t + 1] = static_cast<int>(e4m3x4(lo_f32<T>(x[2]), hi_f32<T>(x[2]), lo_f32<T>(x[3]), hi_f32<T>(x[3])));
            }
            qf8[qb] = w;
        } else {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4 x =
                    buffer_load16(rq, static_cast<uint32_t>(wq0 + 16 * qb + li) * ROWB + (32 * s + 8 * g) * 2, 0) ^ p.qsign;
                qf[qb][s] = as<V8>(x);
            }
        }
    }

    // Direct loads (as in the 32x32 kernel): the wave's load i fills LDS chunks
    // [(wave LOADS + i) 64, + 64); load i is load 0 moved by 1024 i bytes in
    // memory and in LDS, with the chunk permutation changed by an XOR (checked
    // above for this shape).
    uint32_t koff0, voff0;
    {
        const int pch = wave * LOADS * 64 + lane;
        const int row = pch / DC, col = pch % DC;
        koff0 = row * ROWB + ((col ^ kswz<ROWB>(row)) << 4);
        voff0 = row * ROWB + ((col ^ vswz16<D>(row)) << 4);
        if constexpr (KF8) {  // one load per thread: 8 rows of 8 chunks per wave
            const int kch = wave * 64 + lane, krow = kch / (KROWB / 16), kcol = kch % (KROWB / 16);
            koff0 = krow * KROWB + ((kcol ^ k8swz16(krow)) << 4);
        }
    }
    constexpr int kx1 = k16_xor<ROWB>(1), kx2 = k16_xor<ROWB>(2), kx3 = k16_xor<ROWB>(3);
    constexpr int vx1 = v16_xor<D>(1), vx2 = v16_xor<D>(2), vx3 = v16_xor<D>(3);
    auto issue = [&](const u32x4 &rsrc, uint32_t off0, auto x1, auto x2, auto x3, const u32x4 *dst_tile, int kb) {
        const uint32_t tile = static_cast<uint32_t>(kb) * BN * ROWB;
        const u32x4 *dst = dst_tile + wave * LOADS * 64;
        dma_to_lds16<0>(rsrc, off0, tile, dst);
        if constexpr (LOADS > 1) dma_to_lds16<1024>(rsrc, off0 ^ (decltype(x1)::value << 4), tile, dst);
        if constexpr (LOADS > 2) dma_to_lds16<2048>(rsrc, off0 ^ (decltype(x2)::value << 4), tile, dst);
        if constexpr (LOADS > 3) dma_to_lds16<3072>(rsrc, off0 ^ (decltype(x3)::value << 4), tile, dst);
    };
    auto issue_k8 = [&](const u32x4 *dst_tile, int kb) {
        dma_to_lds16<0>(rk, koff0, static_cast<uint32_t>(kb) * BN * KROWB, dst_tile + wave * 64);
    };
    auto issue_k = [&](auto st, int kb) {
        if constexpr (KF8)
            issue_k8(sk[decltype(st)::value], kb);
        else
            issue(rk, koff0, IC<kx1>{}, IC<kx2>{}, IC<kx3>{}, sk[decltype(st)::value], kb);
    };
    auto issue_v = [&](auto st, int kb) {
        issue(rv, voff0, IC<vx1>{}, IC<vx2>{}, IC<vx3>{}, sv[decltype(st)::value], kb);
    };
    // Step j requests V_{j+NS-1} and K_{j+NS}; at the end of step j, K_{j+2}
    // and V_{j+1} must have landed.
    auto allowance = [&](int j) {
        int n = 0;
#pragma unroll
        for (int i = j + 3 - NS; i <= j; ++i)
            if (i >= 1 - NS) n += LOADS * (i + NS - 1 < nkb) + LOADS * (i + NS < nkb);
        return n;
    };
    constexpr int kMaxWait = 2 * (NS - 2);

    // LDS byte offsets of this lane's operands within a tile.
    // K (kb, s): row 16 kb + i, logical chunk 4 s + g; the permutation depends
    // on i only, and chunk 4 s + g is chunk g XOR 4 s.
    const uint32_t ka0 = li * ROWB + ((g ^ kswz<ROWB>(li)) << 4);
    // KF8: row 16 kb + i, logical chunks 2 g and 2 g + 1 (the 32 k-slots of
    // group g); the permutation (k8swz16) again depends on i only.
    const uint32_t ka8 = li * KROWB + (((2 * g) ^ k8swz16(li)) << 4);
    // V^T (db, s, h): the in-group lane i addresses row 4 g + i / 4 (+ 32 s +
    // 16 h) and bytes 32 db + 8 (i % 4) .. + 7, so that lane i receives dims
    // 16 db + i of the four rows; db enters as an XOR on the chunk index, and
    // the row offsets leave the permutation unchanged.
    uint32_t va0;
    {
        const int row = 4 * g + (li >> 2);
        va0 = row * ROWB + ((((li & 3) >> 1) ^ vswz16<D>(row)) << 4) + ((li & 1) << 3);
    }

    f32x4 oacc[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};  // reference maximum (base 2), per query block
    float l_run[2] = {0.f, 0.f}, l_cmp[2] = {0.f, 0.f};
    const float cs = p.c;

    auto add_l = [&](int qb, float x) {
        const float y = x - l_cmp[qb];
        const float t = l_run[qb] + y;
        l_cmp[qb] = (t - l_run[qb]) - y;
        l_run[qb] = t;
    };

    using Frag = f32x4[4][2];  // [key block][query block]
    // S^T = K Q^T for the K tile in stage st.
    auto kop = [&](const char *SK, int s, int kb) {
        return *reinterpret_cast<const u32x4 *>(SK + (ka0 ^ ((4 * s) << 4)) + kb * 16 * ROWB);
    };
    auto kop8 = [&](const char *SK, int kb) {
        const u32x4 x0 = *reinterpret_cast<const u32x4 *>(SK + ka8 + kb * 16 * KROWB);
        const u32x4 x1 = *reinterpret_cast<const u32x4 *>(SK + (ka8 ^ 16) + kb * 16 * KROWB);
        return i32x8{static_cast<int>(x0[0]), static_cast<int>(x0[1]), static_cast<int>(x0[2]), static_cast<int>(x0[3]),
                     static_cast<int>(x1[0]), static_cast<int>(x1[1]), static_cast<int>(x1[2]), static_cast<int>(x1[3])};
    };
    auto scores = [&](auto st, Frag &sn) {
        const char *SK = reinterpret_cast<const char *>(sk[decltype(st)::value]);
        if constexpr (KF8) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const i32x8 a = kop8(SK, kb);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) sn[kb][qb] = mfma16_e4m3(a, qf8[qb], f32x4{0.f, 0.f, 0.f, 0.f});
            }
            return;
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) sn[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const u32x4 x = kop(SK, s, kb);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) sn[kb][qb] = mfma16(as<V8>(x), qf[qb][s], sn[kb][qb]);
            }
    };

    // A key is hidden from a query when key > min(query + off, Nkv - 1) (or
    // past Nkv alone without the causal mask).  With t = that bound - kv0 - 4 g
    // per query block, element (kb, r) is hidden iff 16 kb + r > t; the select
    // is a bitfield insert on the sign of t - 16 kb - r, so no per-element
    // compare result has to live in a scalar register pair.
    auto needs_mask = [&](int kv0) { return (kv0 + BN > p.Nkv) || (CAUSAL && kv0 + BN - 1 > wq0 + off); };
    auto mask = [&](Frag &sn, int kv0) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            int lim = p.Nkv - 1;
            if constexpr (CAUSAL) lim = min(lim, wq0 + 16 * qb + li + off);
            const int t = lim - kv0 - 4 * g;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                // whole-vector bit casts (a bit cast of one vector element is
                // lowered as a read of element 0)
                u32x4 bits = __builtin_bit_cast(u32x4, sn[kb][qb]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t hide = static_cast<uint32_t>((t - 16 * kb - r) >> 31);  // all ones when hidden
                    bits[r] = (hide & 0xff800000u) | (~hide & bits[r]);
                }
                sn[kb][qb] = __builtin_bit_cast(f32x4, bits);
            }
        }
    };

    // P of tile sc against m_run, in the storage type: operand (qb, s) holds
    // key blocks 2 s and 2 s + 1.  Returns this lane's sums over its keys:
    // for fp16, of the rounded P that the second product takes, so that
    // O = acc / l is a weighted mean whose weights sum to one exactly as
    // rounded (each widened by v_fma_mix; v_dot2c would take half the
    // instructions but shares the matrix pipeline and waits behind the other
    // wave's MFMAs: measured 25 cycles each beside an MFMA stream, against 12
    // for v_fma_mix); for bf16, of the fp32 values (widening a bf16 half
    // costs an extra instruction, and the bf16 bar is eight times wider).
    V8 pf[2][2];
    auto probs = [&](const Frag &sc, float (&rs)[2]) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float neg_m = -m_run[qb];
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                u32x4 w;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f32x4 v = sc[2 * s + h][qb];
                    const float a = fast_exp2(fmaf(v[0], cs, neg_m)), b = fast_exp2(fmaf(v[1], cs, neg_m));
                    const float c = fast_exp2(fmaf(v[2], cs, neg_m)), d = fast_exp2(fmaf(v[3], cs, neg_m));
                    w[2 * h] = pack2<T>(a, b);
                    w[2 * h + 1] = pack2<T>(c, d);
                    if constexpr (std::is_same<T, _Float16>::value) {
                        r0 = add_lo_f16(add_lo_f16(r0, w[2 * h]), w[2 * h + 1]);
                        r1 = add_hi_f16(add_hi_f16(r1, w[2 * h]), w[2 * h + 1]);
                    } else {
                        r0 += a + c;
                        r1 += b + d;
                    }
                }
                pf[qb][s] = as<V8>(w);
            }
            rs[qb] = r0 + r1;
        }
    };
    // The softmax step of tile sc, with the maximum taken on demand.
    auto softmax = [&](const Frag &sc) {
        float rs[2];
        probs(sc, rs);
        if (__builtin_amdgcn_ballot_w64(!(rs[0] <= kSumLimit && rs[1] <= kSumLimit))) {
            // the four lanes of a query (i, i + 16, i + 32, i + 48) agree on
            // the new reference: the tile's maximum across them, or m_run
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float m = sc[0][qb][0];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m = fmaxf(m, sc[kb][qb][r]);
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                const float m_new = fmaxf(m_run[qb], m * cs);
                // m_new is finite: the tile's first step of a row sees key 0,
                // and m_run stays finite after it
                const float alpha = fast_exp2(m_run[qb] - m_new);
                l_run[qb] *= alpha;
                l_cmp[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
                m_run[qb] = m_new;
            }
            probs(sc, rs);
        }
        add_l(0, rs[0]);
        add_l(1, rs[1]);
    };
    auto pin = [](V8 (&pfr)[2][2]) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                u32x4 w = __builtin_bit_cast(u32x4, pfr[qb][s]);
                asm volatile("" : "+v"(w));
                pfr[qb][s] = as<V8>(w);
            }
    };

    // O^T += V^T P^T for the V tile in stage st.
    auto vop = [&](const char *SV, int s, int db) {
        const char *pa = SV + (va0 ^ (db << 5)) + 32 * s * ROWB;
        const u32x2 lo = lds_read_tr16(pa);
        const u32x2 hi = lds_read_tr16(pa + 16 * ROWB);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    auto pv = [&](auto st) {
        const char *SV = reinterpret_cast<const char *>(sv[decltype(st)::value]);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4 a = vop(SV, s, db);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = mfma16(as<V8>(a), pf[qb][s], oacc[db][qb]);
            }
    };

    // Eight waves alternate MFMA and softmax blocks (below); other shapes
    // overlap them within each wave.
    constexpr bool kAlternate = NW == 8 && NS == 2;

    // One pipeline step for key tile j (stage S = j % NS): V_j in sv[S],
    // K_{j+1} in sk[(S + 1) % NS]; the two score sets alternate with j % 2.
    Frag sa, sb;
    auto step = [&](auto st, Frag &sc, Frag &sn, int j) {
        constexpr int S = decltype(st)::value % NS;
        if (j + NS - 1 < nkb) issue_v(IC<(S + NS - 1) % NS>{}, j + NS - 1);
        if (j + NS < nkb) issue_k(IC<S>{}, j + NS);
        if (j < nkw) {
            // phase 1: MFMAs of the next scores beside the softmax of the current ones
            scores(IC<(S + 1) % NS>{}, sn);
            softmax(sc);
            pin(pf);
            const int kv1 = (j + 1) * BN;
            if (needs_mask(kv1)) mask(sn, kv1);
            // phase 2: MFMAs of O += V P
            pv(IC<S>{});
        }
        wait_loads<LOADS, kMaxWait>(allowance(j));
        __syncthreads();
    };

    if (nkb > 0) issue_k(IC<0>{}, 0);
    [&]<int... I>(std::integer_sequence<int, I...>) {
        ((I < nkb ? (issue_v(IC<I>{}, I), 0) : 0, I + 1 < nkb ? (issue_k(IC<I + 1>{}, I + 1), 0) : 0), ...);
    }(std::make_integer_sequence<int, NS - 1>{});
    wait_loads<LOADS, kMaxWait>(allowance(-1));
    __syncthreads();
    if (nkw > 0) {
        scores(IC<0>{}, sa);
        if (!kAlternate && needs_mask(0)) mask(sa, 0);
    }
    __syncthreads();  // every wave is done with sk[0] before K_NS refills it

    if constexpr (kAlternate) {
        // Alternating blocks.  Every wave runs the same sequence
        //   M_j: S_{j+1} = K_{j+1} Q^T and O += V_j P_j (MFMA only),
        //   V_{j+1}: softmax of S_{j+1} into P_{j+1} (VALU only),
        // and the step's barrier falls after V for waves 0..3 and after M for
        // waves 4..7, so that each SIMD starts a step with one wave on its
        // MFMA block and the other on its softmax.  Between barriers j - 1 and
        // j every wave runs M_j, so the ring protocol is the plain step's.
        const bool lead = wave < NW / 2;
        auto loads = [&](int j) __attribute__((always_inline)) {
            const int S = j & 1;
            if (j + 1 < nkb) issue(rv, voff0, IC<vx1>{}, IC<vx2>{}, IC<vx3>{}, sv[S ^ 1], j + 1);
            if (j + 2 < nkb) {
                if constexpr (KF8)
                    issue_k8(sk[S], j + 2);
                else
                    issue(rk, koff0, IC<kx1>{}, IC<kx2>{}, IC<kx3>{}, sk[S], j + 2);
            }
        };
        auto end_step = [&](int j) __attribute__((always_inline)) {
            wait_loads<LOADS, kMaxWait>(allowance(j));
            __syncthreads();
        };
        auto vblock = [&](int j) __attribute__((always_inline)) {
            const int kv = j * BN;
            if (needs_mask(kv)) mask(sa, kv);
            softmax(sa);
            pin(pf);
        };
        // M with its LDS operands requested ahead of the MFMAs that take
        // them: K k-step s + 1 while k-step s multiplies (8 MFMAs, 128
        // cycles), and the V operands kVAhead groups (2 MFMAs each) ahead.
        constexpr int kVAhead = 6;
        auto mblock = [&](auto st) __attribute__((always_inline)) {
            constexpr int S = decltype(st)::value;
            const char *SK = reinterpret_cast<const char *>(sk[S ^ 1]);
            const char *SV = reinterpret_cast<const char *>(sv[S]);
            constexpr int NG = 2 * DB;  // V groups: (s, db)
            u32x4 kx[2][4], vx[kVAhead + 1];
            auto kread = [&](int s) __attribute__((always_inline)) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) kx[s & 1][kb] = kop(SK, s, kb);
            };
            auto vread = [&](int gi) __attribute__((always_inline)) { vx[gi % (kVAhead + 1)] = vop(SV, gi / DB, gi % DB); };
            if constexpr (KF8) {
                // the four K operands, then the first V operands, before the
                // eight score MFMAs (256 cycles: too short to cover the V reads)
                i32x8 k8[4];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) k8[kb] = kop8(SK, kb);
#pragma unroll
                for (int gi = 0; gi < kVAhead && gi < NG; ++gi) vread(gi);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        sa[kb][qb] = mfma16_e4m3(k8[kb], qf8[qb], f32x4{0.f, 0.f, 0.f, 0.f});
                __builtin_amdgcn_sched_barrier(0);
            } else {
            kread(0);
            if constexpr (KS > 1) kread(1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        sa[kb][qb] = mfma16(as<V8>(kx[s & 1][kb]), qf[qb][s],
                                            s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sa[kb][qb]);
                __builtin_amdgcn_sched_barrier(0);
                if (s + 2 < KS) kread(s + 2);
                if (s == KS - 2 || (KS == 1 && s == 0)) {
#pragma unroll
                    for (int gi = 0; gi < kVAhead && gi < NG; ++gi) vread(gi);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            }
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const u32x4 a = vx[gi % (kVAhead + 1)];
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    oacc[gi % DB][qb] = mfma16(as<V8>(a), pf[qb][gi / DB], oacc[gi % DB][qb]);
                __builtin_amdgcn_sched_barrier(0);
                if (gi + kVAhead < NG) vread(gi + kVAhead);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // a step of a wave that has tile j + 1 after tile j
        auto full = [&](auto st, int j) __attribute__((always_inline)) {
            loads(j);
            mblock(st);
            if (!lead) end_step(j);
            vblock(j + 1);
            if (lead) end_step(j);
        };
        if (0 < nkw) vblock(0);
        int j = 0;
        for (; j + 2 < nkw; j += 2) {
            full(IC<0>{}, j);
            full(IC<1>{}, j + 1);
        }
        if (j + 1 < nkw) full(IC<0>{}, j++);
        if (j < nkw) {  // the wave's last tile
            loads(j);
            if (j & 1)
                pv(IC<1>{});
            else
                pv(IC<0>{});
            end_step(j++);
        }
        for (; j < nkb; ++j) {  // tiles of the workgroup's later rows only
            loads(j);
            end_step(j);
        }
    } else {
        for (int j = 0; j < nkb; j += U) {
            [&]<int... I>(std::integer_sequence<int, I...>) {
                ((j + I < nkb ? (I % 2 == 0 ? step(IC<I>{}, sa, sb, j + I) : step(IC<I>{}, sb, sa, j + I)), 0 : 0),
                 ...);
            }(std::make_integer_sequence<int, U>{});
        }
    }

    // Epilogue: the four lanes' partial sums of a query, then O = acc / l and
    // LSE = ln 2 (m + log2 l).
    float inv[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float l = l_run[qb] - l_cmp[qb];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        inv[qb] = 1.f / l;
        const int qrow = wq0 + 16 * qb + li;
        if (g == 0 && p.lse && qrow < p.Nq)
            p.lse[static_cast<size_t>(bh) * p.Nq + qrow] = (m_run[qb] + __builtin_amdgcn_logf(l)) * kLn2;
    }
    if constexpr (!OUT_F32) {
        // 16-bit O leaves through LDS: the wave's 32 rows are written to its
        // slice of the (now idle) ring, row-major with the 16-byte chunks of
        // row r permuted by r mod (chunks per row), and read back so that
        // every store writes whole rows (1 KB per instruction) rather than
        // 32-byte pieces of 16 rows.  The loop's last barrier ended every
        // wave's use of the ring and every load into it.
        constexpr int CPR = ROWB / 16;  // 16-byte chunks per row
        constexpr int RPI = 1024 / ROWB;  // rows per 1 KB instruction
        static_assert(NW * 32 * ROWB <= static_cast<int>(sizeof(lds_rings)), "O stage fits the ring");
        char *const stage = reinterpret_cast<char *>(lds_rings) + wave * 32 * ROWB;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = 16 * qb + li;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const f32x4 o = oacc[db][qb] * inv[qb];
                const int byte = 32 * db + 8 * g;
                *reinterpret_cast<u32x2 *>(stage + row * ROWB + ((((byte >> 4) ^ (row % CPR)) << 4) | (byte & 8))) =
                    u32x2{pack2<T>(o[0], o[1]), pack2<T>(o[2], o[3])};
            }
        }
        char *const obase = static_cast<char *>(p.o) + static_cast<size_t>(bh) * p.Nq * ROWB;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int row = i * RPI + lane / CPR, chunk = lane % CPR;
            const u32x4 x = *reinterpret_cast<const u32x4 *>(stage + row * ROWB + ((chunk ^ (row % CPR)) << 4));
            if (wq0 + row < p.Nq)
                *reinterpret_cast<u32x4 *>(obase + static_cast<size_t>(wq0 + row) * ROWB + chunk * 16) = x;
        }
    } else {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int qrow = wq0 + 16 * qb + li;
            if (qrow < p.Nq) {
                const size_t orow = (static_cast<size_t>(bh) * p.Nq + qrow) * D;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int d0 = 16 * db + 4 * g;
                    const f32x4 o = oacc[db][qb] * inv[qb];
                    if constexpr (OUT_F32) {
                        *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + orow + d0) = o;
                    } else {
                        *reinterpret_cast<u32x2 *>(static_cast<T *>(p.o) + orow + d0) =
                            u32x2{pack2<T>(o[0], o[1]), pack2<T>(o[2], o[3])};
                    }
                }
            }
        }
    }
}

// Launch shapes: 8 waves (256 rows per workgroup, one workgroup per CU) when
// the grid gives every CU such a workgroup; two 4-wave key groups on 128 rows
// when even 128-row tiles leave CUs idle; else 4 waves (128 rows, two
// workgroups per CU); all with a 2-stage ring.  Measured on the 8K d=128
// causal workload, deeper rings (3 or 4 stages) were no faster: a step's
// loads already land within the step, and the chip is power-bound there.
constexpr int kCUs = 256;
#ifndef FA355_FP8_16
#define FA355_FP8_16 1
#endif

template <int D, typename T, bool CAUSAL, bool OUT_F32, int NW, int NS, bool KF8, int KG = 1>
hipError_t launch_shape(const FwdArgs &a, hipStream_t stream)
{
    constexpr int BM = 32 * NW / KG;
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
    // A zero scale would make a masked score (-inf) times c a NaN; any c up to
    // kMinC leaves every finite score's 2^(c s - m) equal to 1 in fp32, which
    // is the uniform weighting a zero scale asks for.
    const float c = (a.scale < 0.f ? -a.scale : a.scale) * kLog2e;
    p.c = c < kMinC ? kMinC : c;
    p.qsign = a.scale < 0.f ? 0x80008000u : 0u;
    const dim3 grid(static_cast<unsigned>(static_cast<long long>(p.n_bh) * p.n_qt));
    hipLaunchKernelGGL((fwd_kernel<D, T, CAUSAL, OUT_F32, NW, NS, KF8, KG>), grid, dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

// The launch shape of a call: waves per workgroup and key groups.
struct Shape {
    int nw, kg;
};

Shape pick_shape(const FwdArgs &a)
{
    // E4M3 K: the 4-wave shape only.  Its first product is a quarter of the
    // 16-bit one, so phase 1 is VALU-bound, and two workgroups per CU (whose
    // waves do not share barriers) overlap one wave's softmax with the other's
    // MFMAs better than one 8-wave workgroup: measured 4% faster at 8K d=128.
    // (A d = 64 E4M3 K tile is also exactly one load per thread of 4 waves.)
    const long long wide_blocks = static_cast<long long>(a.B) * a.H * ((a.Nq + 255) / 256);
    // Causal at d = 64 with one 256-row tile per CU: each CU's time is its
    // tile's, so the heaviest sets the kernel's; 128-row tiles two to a CU
    // balance better (4K, B H = 16: 498 -> 589 TFLOP/s).  From two tiles per
    // CU, and at d = 128 at any size, the 8-wave shape is faster.
    if (!a.k_e4m3 && a.causal && a.d == 64 && wide_blocks >= kCUs && wide_blocks < 2 * kCUs) return {4, 1};
    if ((!a.k_e4m3 || (FA355_FP8_16 && a.d == 128)) && wide_blocks >= kCUs) return {8, 1};
    // Too few 128-row tiles to give every CU one: two key groups per tile
    // halve the serial chain of key tiles (worth it from 4 key tiles on).
    // Causal at d = 64 (16-bit K): 64-row tiles of two 2-wave key groups.
    // The last query tiles then carry half the work, and twice as many
    // workgroups let the heavy-first order give each CU a heavy tile and a
    // light one; measured 17-35% faster from 1K to 16K keys.  Without the
    // mask the tiles are even, and the 128-row shape is 4-5% faster.
    const long long tiles = static_cast<long long>(a.B) * a.H * ((a.Nq + 127) / 128);
    if (tiles <= kCUs && a.Nkv > 3 * kBN) {
        if (a.causal && a.d == 64 && !a.k_e4m3) return {4, 2};
        return {8, 2};
    }
    return {4, 1};
}

// The 16x16x32 kernel for 16-bit K in the one-group shapes, and for E4M3 K
// in the eight-wave shape at d = 128.
template <int D, typename T, bool CAUSAL, bool OUT_F32, int NW, bool KF8 = false>
hipError_t launch16(const FwdArgs &a, hipStream_t stream)
{
    constexpr int BM = 32 * NW;
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
    const float c = (a.scale < 0.f ? -a.scale : a.scale) * kLog2e;
    p.c = c < kMinC ? kMinC : c;
    p.qsign = a.scale < 0.f ? 0x80008000u : 0u;
    const dim3 grid(static_cast<unsigned>(static_cast<long long>(p.n_bh) * p.n_qt));
    hipLaunchKernelGGL((fwd16_kernel<D, T, CAUSAL, OUT_F32, NW, 2, KF8>), grid, dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

// 16-bit K in the one-group shapes runs the 16x16x32 kernel; the two-group
// shapes and E4M3 K run the 32x32x16 one.
template <int D, typename T, bool CAUSAL, bool OUT_F32, bool KF8>
hipError_t launch_k(const FwdArgs &a, hipStream_t stream)
{
    const Shape s = pick_shape(a);
    if constexpr (KF8 && D == 128)
        if (s.nw == 8 && s.kg == 1) return launch16<D, T, CAUSAL, OUT_F32, 8, true>(a, stream);
    if constexpr (!KF8)
        if (s.kg == 1) return s.nw == 8 ? launch16<D, T, CAUSAL, OUT_F32, 8>(a, stream)
                                        : launch16<D, T, CAUSAL, OUT_F32, 4>(a, stream);
    if constexpr (CAUSAL && D == 64 && !KF8)
        if (s.nw == 4 && s.kg == 2) return launch_shape<D, T, CAUSAL, OUT_F32, 4, 2, KF8, 2>(a, stream);
    if (s.nw == 8 && s.kg == 2) return launch_shape<D, T, CAUSAL, OUT_F32, 8, 2, KF8, 2>(a, stream);
    return launch_shape<D, T, CAUSAL, OUT_F32, 4, 2, KF8>(a, stream);
}

template <int D, typename T, bool CAUSAL, bool OUT_F32>
hipError_t launch(const FwdArgs &a, hipStream_t stream)
{
    return a.k_e4m3 ? launch_k<D, T, CAUSAL, OUT_F32, true>(a, stream)
                    : launch_k<D, T, CAUSAL, OUT_F32, false>(a, stream);
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

unsigned long long fwd_work_items(const FwdArgs &a)
{
    const Shape s = pick_shape(a);
    const long long rows = 32LL * s.nw / s.kg;
    return static_cast<unsigned long long>(a.B) * a.H * ((a.Nq + rows - 1) / rows) * (64ULL * s.nw);
}

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream)
{
    if (a.d == 64) return launch_d<64>(a, stream);
    if (a.d == 128) return launch_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa355
