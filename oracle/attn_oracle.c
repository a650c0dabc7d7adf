/*
 * attn_oracle.c -- plain, slow fp64 CPU reference for exact softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark are the only code that loads this library.
 * The GPU library neither links nor includes anything from here, and nothing
 * here comes from the GPU library.
 *
 * What it computes, for every batch b, head h and query row i:
 *
 *   S[i][j] = scale * sum_c q[i][c] * k[j][c]   for every key j visible to i,
 *             -infinity                          for keys that are not visible.
 *       Standard attention S = Q K^T, P = softmax(S), O = P V ("FlashAttention",
 *       section "The problem: the n x n score matrix"), with the 1/sqrt(d)
 *       factor of "Flash Attention -- Module 12.3", section "Definition",
 *       generalised to a caller-supplied scale.
 *
 *   m_i     = max_j S[i][j]
 *   l_i     = sum_j exp(S[i][j] - m_i)
 *   P[i][j] = exp(S[i][j] - m_i) / l_i
 *       The two-pass stable softmax of "FlashAttention 1-2-3: The IO-Aware
 *       Revolution in LLM Inference", section "The Math Behind the Online
 *       Softmax Trick" (find the max, exponentiate the shifted values, sum,
 *       divide).
 *
 *   O[i][c] = sum_j P[i][j] * v[j][c]
 *   LSE_i   = m_i + ln(l_i)
 *       LSE is not named on the pages; it is the natural logarithm of
 *       sum_j exp(S[i][j]), i.e. the row's (m, l) pair folded into one number.
 *
 * Causal visibility: key j is visible to row i iff j <= i + (Nkv - Nq).  With
 * Nq == Nkv this is the lower triangle including the diagonal; for Nq < Nkv the
 * last query row sees every key (the alignment is a reading: the pages show
 * only square causal masks).  Causal with Nq > Nkv is rejected.
 *
 * Inputs are row-major [B][H][N][d] arrays of doubles; 16-bit inputs are first
 * widened exactly by fa_oracle_widen.  For each head the full Nq x Nkv score
 * matrix is materialised, softmaxed in place into P, and multiplied by V: the
 * three passes of standard attention, nothing blocked, fused or reordered.
 * Rows are spread over OpenMP threads; every row's arithmetic is sequential in
 * key order, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16: sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double fa_oracle_f16_to_f64(uint16_t bits)
{
    int sign = bits >> 15;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);              /* subnormal: frac * 2^-14 * 2^-10 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(frac | 0x400), expo - 25); /* 1.frac * 2^(expo-15) */
    return sign ? -mag : mag;
}

/* bfloat16: sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double fa_oracle_bf16_to_f64(uint16_t bits)
{
    int sign = bits >> 15;
    int expo = (bits >> 7) & 0xff;
    int frac = bits & 0x7f;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -133);             /* subnormal: frac * 2^-126 * 2^-7 */
    else if (expo == 255)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(frac | 0x80), expo - 134); /* 1.frac * 2^(expo-127) */
    return sign ? -mag : mag;
}

/* kind 1 = binary16, kind 2 = bfloat16.  Returns 0, or -1 for an unknown kind. */
int fa_oracle_widen(const uint16_t *bits, double *out, int64_t n, int kind)
{
    if (kind != 1 && kind != 2)
        return -1;
    for (int64_t t = 0; t < n; ++t)
        out[t] = kind == 1 ? fa_oracle_f16_to_f64(bits[t]) : fa_oracle_bf16_to_f64(bits[t]);
    return 0;
}

int fa_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int is_visible(int64_t i, int64_t j, int64_t Nq, int64_t Nkv, int causal)
{
    return !causal || j <= i + (Nkv - Nq);
}

/* Row i of S: scaled dot products with every visible key, -inf elsewhere. */
static void score_row(const double *qi, const double *k, int64_t i, int64_t Nq, int64_t Nkv,
                      int64_t d, int causal, double scale, double *s_row)
{
    for (int64_t j = 0; j < Nkv; ++j) {
        if (!is_visible(i, j, Nq, Nkv, causal)) {
            s_row[j] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += qi[c] * k[j * d + c];
        s_row[j] = scale * dot;
    }
}

/* Two-pass stable softmax of one row, in place (S row -> P row).  Returns LSE. */
static double softmax_row(double *s_row, int64_t Nkv)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < Nkv; ++j)
        if (s_row[j] > m)
            m = s_row[j];
    double l = 0.0;
    for (int64_t j = 0; j < Nkv; ++j) {
        s_row[j] = exp(s_row[j] - m);
        l += s_row[j];
    }
    for (int64_t j = 0; j < Nkv; ++j)
        s_row[j] = s_row[j] / l;
    return m + log(l);
}

/* Row i of O = P V (sum over keys in ascending order for every column). */
static void pv_row(const double *p_row, const double *v, int64_t Nkv, int64_t d, double *oi)
{
    for (int64_t c = 0; c < d; ++c)
        oi[c] = 0.0;
    for (int64_t j = 0; j < Nkv; ++j) {
        double p = p_row[j];
        for (int64_t c = 0; c < d; ++c)
            oi[c] += p * v[j * d + c];
    }
}

static int check_shape(int64_t Nq, int64_t Nkv, int64_t d, int causal)
{
    if (Nq < 0 || Nkv < 1 || d < 1)
        return -1;
    if (causal && Nq > Nkv)
        return -1;
    return 0;
}

/* One head: S materialised (Nq x Nkv), then P in place, then O.  -2 if out of memory. */
static int head_attention(const double *q, const double *k, const double *v, double *o,
                          double *lse, int64_t Nq, int64_t Nkv, int64_t d, int causal,
                          double scale)
{
    double *S = (double *)malloc((size_t)Nq * (size_t)Nkv * sizeof(double));
    if (!S)
        return -2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < Nq; ++i)
        score_row(q + i * d, k, i, Nq, Nkv, d, causal, scale, S + i * Nkv);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < Nq; ++i)
        lse[i] = softmax_row(S + i * Nkv, Nkv);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < Nq; ++i)
        pv_row(S + i * Nkv, v, Nkv, d, o + i * d);
    free(S);
    return 0;
}

/*
 * Full attention over [B][H][N][d] inputs.  o: [B][H][Nq][d], lse: [B][H][Nq].
 * Returns 0, -1 for an invalid shape, -2 if the score matrix cannot be allocated.
 */
int fa_oracle_attention(const double *q, const double *k, const double *v, double *o, double *lse,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, int causal,
                        double scale)
{
    if (B < 0 || H < 0 || check_shape(Nq, Nkv, d, causal))
        return -1;
    for (int64_t bh = 0; bh < B * H; ++bh) {
        int rc = head_attention(q + bh * Nq * d, k + bh * Nkv * d, v + bh * Nkv * d,
                                o + bh * Nq * d, lse + bh * Nq, Nq, Nkv, d, causal, scale);
        if (rc)
            return rc;
    }
    return 0;
}

/*
 * Selected rows of one head, for spot checks at sizes where a whole head's S is
 * too large to hold: the same three passes on a one-row S.  q, k, v are one
 * head ([Nq][d], [Nkv][d], [Nkv][d]); rows lists query indices; o gets
 * [nrows][d], lse [nrows].
 */
int fa_oracle_attention_rows(const double *q, const double *k, const double *v, int64_t Nq,
                             int64_t Nkv, int64_t d, int causal, double scale,
                             const int64_t *rows, int64_t nrows, double *o, double *lse)
{
    if (check_shape(Nq, Nkv, d, causal))
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= Nq)
            return -1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        double *s_row = (double *)malloc((size_t)Nkv * sizeof(double));
        if (!s_row) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        int64_t i = rows[r];
        score_row(q + i * d, k, i, Nq, Nkv, d, causal, scale, s_row);
        lse[r] = softmax_row(s_row, Nkv);
        pv_row(s_row, v, Nkv, d, o + r * d);
        free(s_row);
    }
    return failed ? -2 : 0;
}

/*
 * Backward of the same attention for a loss L with dL/dO = dO ("FlashAttention
 * 1-2-3", section "FlashAttention-1: Tiling, Recomputation, and Online Softmax":
 * the backward keeps per-row statistics instead of the softmax matrix;
 * "Flash Attention -- Module 12.3", section "Training": the backward is IO-aware
 * too).  The pages give no formulas; these are the chain rule through the
 * definition above, written out per head with P materialised:
 *
 *   dV[j][c] = sum_i P[i][j] * dO[i][c]
 *   dP[i][j] = sum_c dO[i][c] * v[j][c]
 *   D_i      = sum_j P[i][j] * dP[i][j]       (softmax Jacobian: row-wise)
 *            = sum_c dO[i][c] * O[i][c]       (the same number, as O = P v)
 *   dS[i][j] = P[i][j] * (dP[i][j] - D_i)
 *   dQ[i][c] = scale * sum_j dS[i][j] * k[j][c]
 *   dK[j][c] = scale * sum_i dS[i][j] * q[i][c]
 *
 * Invisible keys have P = 0 and so dS = 0.  P is recomputed from q and k here
 * (the oracle stores nothing between calls).
 *
 * The backward of a training step is handed the forward's output O as the
 * caller holds it (rounded to the 16-bit input type), and forms D from it
 * ("Flash Attention -- Module 12.3", section "Training": the backward works
 * from what the forward kept).  Reading taken here: when oD is given, D_i is
 * the second form above evaluated on that O, D_i = sum_c dO[i][c] * oD[i][c];
 * when oD is NULL, D_i is the first form, from P itself.  With oD = P v
 * exactly the two agree.
 */
static int head_attention_bwd(const double *q, const double *k, const double *v, const double *dO,
                              const double *oD, double *dq, double *dk, double *dv, int64_t Nq, int64_t Nkv,
                              int64_t d, int causal, double scale)
{
    double *P = (double *)malloc((size_t)Nq * (size_t)Nkv * sizeof(double));
    double *dS = (double *)malloc((size_t)Nq * (size_t)Nkv * sizeof(double));
    if (!P || !dS) {
        free(P);
        free(dS);
        return -2;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < Nq; ++i) {
        double *p_row = P + i * Nkv, *ds_row = dS + i * Nkv;
        score_row(q + i * d, k, i, Nq, Nkv, d, causal, scale, p_row);
        softmax_row(p_row, Nkv);
        double Di = 0.0;
        for (int64_t j = 0; j < Nkv; ++j) {
            double dp = 0.0;
            for (int64_t c = 0; c < d; ++c)
                dp += dO[i * d + c] * v[j * d + c];
            ds_row[j] = dp;
            Di += p_row[j] * dp;
        }
        if (oD) {
            Di = 0.0;
            for (int64_t c = 0; c < d; ++c)
                Di += dO[i * d + c] * oD[i * d + c];
        }
        for (int64_t j = 0; j < Nkv; ++j)
            ds_row[j] = p_row[j] * (ds_row[j] - Di);
        for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < Nkv; ++j)
                acc += ds_row[j] * k[j * d + c];
            dq[i * d + c] = scale * acc;
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < Nkv; ++j) {
        for (int64_t c = 0; c < d; ++c) {
            double acc_v = 0.0, acc_k = 0.0;
            for (int64_t i = 0; i < Nq; ++i) {
                acc_v += P[i * Nkv + j] * dO[i * d + c];
                acc_k += dS[i * Nkv + j] * q[i * d + c];
            }
            dv[j * d + c] = acc_v;
            dk[j * d + c] = scale * acc_k;
        }
    }
    free(P);
    free(dS);
    return 0;
}

/*
 * Gradients over [B][H][N][d] inputs: dO like o, dq like q, dk and dv like k;
 * oD (like o, or NULL) is the forward output D is formed from (see above).
 * Returns 0, -1 for an invalid shape, -2 if a score matrix cannot be allocated.
 */
int fa_oracle_attention_bwd(const double *q, const double *k, const double *v, const double *dO,
                            const double *oD, double *dq, double *dk, double *dv, int64_t B, int64_t H,
                            int64_t Nq, int64_t Nkv, int64_t d, int causal, double scale)
{
    if (B < 0 || H < 0 || check_shape(Nq, Nkv, d, causal))
        return -1;
    for (int64_t bh = 0; bh < B * H; ++bh) {
        int rc = head_attention_bwd(q + bh * Nq * d, k + bh * Nkv * d, v + bh * Nkv * d,
                                    dO + bh * Nq * d, oD ? oD + bh * Nq * d : NULL, dq + bh * Nq * d,
                                    dk + bh * Nkv * d, dv + bh * Nkv * d, Nq, Nkv, d, causal, scale);
        if (rc)
            return rc;
    }
    return 0;
}

/*
 * Selected gradients of one head, for spot checks where the whole P does not
 * fit: the same formulas as head_attention_bwd, evaluated row by row.  A first
 * pass over every query row i forms LSE_i and D_i (both need the full row of
 * S and dP); dq rows and dk/dv columns are then sums over one row or one
 * column of P and dS, each entry recomputed from LSE_i and D_i as
 * P_ij = exp(S_ij - LSE_i), dS_ij = P_ij * (dP_ij - D_i).
 * q, dO: [Nq][d]; k, v: [Nkv][d]; qrows / kcols list indices; dq gets
 * [nq][d], dk and dv [nk][d]; oD ([Nq][d] or NULL) as for the full entry.
 * Returns 0, -1 for bad arguments, -2 if out of memory.
 */
int fa_oracle_attention_bwd_sampled(const double *q, const double *k, const double *v, const double *dO,
                                    const double *oD, int64_t Nq, int64_t Nkv, int64_t d, int causal, double scale,
                                    const int64_t *qrows, int64_t nq, const int64_t *kcols, int64_t nk,
                                    double *dq, double *dk, double *dv)
{
    if (check_shape(Nq, Nkv, d, causal))
        return -1;
    for (int64_t r = 0; r < nq; ++r)
        if (qrows[r] < 0 || qrows[r] >= Nq)
            return -1;
    for (int64_t r = 0; r < nk; ++r)
        if (kcols[r] < 0 || kcols[r] >= Nkv)
            return -1;
    double *lse = (double *)malloc((size_t)(Nq > 0 ? Nq : 1) * sizeof(double));
    double *Dv = (double *)malloc((size_t)(Nq > 0 ? Nq : 1) * sizeof(double));
    if (!lse || !Dv) {
        free(lse);
        free(Dv);
        return -2;
    }
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < Nq; ++i) {
        double *row = (double *)malloc((size_t)Nkv * 2 * sizeof(double));
        if (!row) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double *p_row = row, *dp_row = row + Nkv;
        score_row(q + i * d, k, i, Nq, Nkv, d, causal, scale, p_row);
        lse[i] = softmax_row(p_row, Nkv);
        double Di = 0.0;
        for (int64_t j = 0; j < Nkv; ++j) {
            double dp = 0.0;
            for (int64_t c = 0; c < d; ++c)
                dp += v[j * d + c] * dO[i * d + c];
            dp_row[j] = dp;
            Di += p_row[j] * dp;
        }
        if (oD) {
            Di = 0.0;
            for (int64_t c = 0; c < d; ++c)
                Di += dO[i * d + c] * oD[i * d + c];
        }
        Dv[i] = Di;
        free(row);
    }
    if (failed) {
        free(lse);
        free(Dv);
        return -2;
    }
    /* one entry of P and dS from the row statistics */
#define P_AT(i, j, pij, dsij)                                                      \
    do {                                                                           \
        double s_ = 0.0, dp_ = 0.0;                                                \
        for (int64_t c_ = 0; c_ < d; ++c_) {                                       \
            s_ += q[(i) * d + c_] * k[(j) * d + c_];                               \
            dp_ += dO[(i) * d + c_] * v[(j) * d + c_];                             \
        }                                                                          \
        pij = is_visible((i), (j), Nq, Nkv, causal) ? exp(scale * s_ - lse[i]) : 0.0; \
        dsij = pij * (dp_ - Dv[i]);                                                \
    } while (0)
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nq; ++r) {
        int64_t i = qrows[r];
        for (int64_t c = 0; c < d; ++c)
            dq[r * d + c] = 0.0;
        for (int64_t j = 0; j < Nkv; ++j) {
            double pij, dsij;
            P_AT(i, j, pij, dsij);
            (void)pij;
            for (int64_t c = 0; c < d; ++c)
                dq[r * d + c] += dsij * k[j * d + c];
        }
        for (int64_t c = 0; c < d; ++c)
            dq[r * d + c] *= scale;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nk; ++r) {
        int64_t j = kcols[r];
        for (int64_t c = 0; c < d; ++c)
            dk[r * d + c] = dv[r * d + c] = 0.0;
        for (int64_t i = 0; i < Nq; ++i) {
            double pij, dsij;
            P_AT(i, j, pij, dsij);
            for (int64_t c = 0; c < d; ++c) {
                dv[r * d + c] += pij * dO[i * d + c];
                dk[r * d + c] += dsij * q[i * d + c];
            }
        }
        for (int64_t c = 0; c < d; ++c)
            dk[r * d + c] *= scale;
    }
#undef P_AT
    free(lse);
    free(Dv);
    return 0;
}

/*
 * Decode over a paged key/value cache, for one query per (batch, head).
 *
 * A serving stack keeps the cache in fixed-size pages and a per-sequence block
 * table; attention treats each page of the cache as a tile ("FlashAttention 1-2-3:
 * The IO-Aware Revolution in LLM Inference", sections "Integration in Major
 * Inference Engines" and "Beyond FlashAttention: Future Directions and
 * Alternatives").  Reading taken here: key j of sequence b is row
 * (j mod page_size) of page table[b][j / page_size], for j < lens[b]; the
 * result is the ordinary softmax attention of the sequence's query over those
 * lens[b] keys, i.e. exactly the dense attention over the gathered cache.
 *
 * kpool, vpool hold num_pages pages; layout 0 stores them [page][H][page_size][d]
 * (one head's slots contiguous), layout 1 [page][page_size][H][d] (one slot's
 * heads contiguous).  q: [B][H][d]; table: [B][max_pages]; o: [B][H][d];
 * lse: [B][H].  A sequence with lens[b] == 0 attends to nothing: its o is 0 and
 * its lse is -infinity (the empty sum's logarithm).
 *
 * The pages that sequence b uses are gathered row by row into a dense
 * [lens[b]][d] copy, then the three passes of standard attention run on it.
 * Returns 0, -1 for invalid arguments (a length outside [0, max_pages *
 * page_size], a used page outside the pool), -2 if out of memory.
 */
int fa_oracle_paged_decode(const double *q, const double *kpool, const double *vpool,
                           const int32_t *table, const int32_t *lens, double *o, double *lse,
                           int64_t B, int64_t H, int64_t num_pages, int64_t page_size,
                           int64_t max_pages, int64_t d, int layout, double scale)
{
    if (B < 0 || H < 0 || num_pages < 0 || page_size < 1 || max_pages < 0 || d < 1 ||
        (layout != 0 && layout != 1))
        return -1;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t n = lens[b];
        if (n < 0 || n > max_pages * page_size)
            return -1;
        for (int64_t t = 0; t * page_size < n; ++t)
            if (table[b * max_pages + t] < 0 || table[b * max_pages + t] >= num_pages)
                return -1;
    }
    for (int64_t b = 0; b < B; ++b) {
        const int64_t n = lens[b];
        double *kd = (double *)malloc((size_t)(n > 0 ? n : 1) * (size_t)d * sizeof(double));
        double *vd = (double *)malloc((size_t)(n > 0 ? n : 1) * (size_t)d * sizeof(double));
        if (!kd || !vd) {
            free(kd);
            free(vd);
            return -2;
        }
        for (int64_t h = 0; h < H; ++h) {
            double *oh = o + (b * H + h) * d;
            if (n == 0) {
                for (int64_t c = 0; c < d; ++c)
                    oh[c] = 0.0;
                lse[b * H + h] = -INFINITY;
                continue;
            }
            for (int64_t j = 0; j < n; ++j) {
                const int64_t page = table[b * max_pages + j / page_size];
                const int64_t slot = j % page_size;
                const int64_t row = layout == 0 ? (page * H + h) * page_size + slot
                                                : (page * page_size + slot) * H + h;
                memcpy(kd + j * d, kpool + row * d, (size_t)d * sizeof(double));
                memcpy(vd + j * d, vpool + row * d, (size_t)d * sizeof(double));
            }
            int rc = head_attention(q + (b * H + h) * d, kd, vd, oh, lse + b * H + h, 1, n, d, 0, scale);
            if (rc) {
                free(kd);
                free(vd);
                return rc;
            }
        }
        free(kd);
        free(vd);
    }
    return 0;
}

/*
 * FP8 (OCP E4M3, "e4m3fn") for the forward with Q and K in 8 bits.
 *
 * The variant quantises Q and K to FP8 for the first product while V, P and
 * O keep their 16-bit type, with fp32 accumulation ("FlashAttention 1-2-3:
 * The IO-Aware Revolution in LLM Inference", section "FlashAttention-3: FP8,
 * Async Warp Overlap, and Hopper-Specific Optimizations"; FP32 accumulation
 * of the exponentials in "The Math Behind the Online Softmax Trick").  The
 * pages name no scaling factor, so the reading taken is a direct cast of each
 * value: round to the nearest E4M3 value, ties to even, and saturate
 * magnitudes above the largest finite value 448 (infinities included) to
 * +-448; NaN stays NaN.  The attention is then the ordinary definition above
 * evaluated on the quantised Q and K.
 *
 * E4M3: sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent field
 * 0 holds the subnormals m * 2^-9; field e in 1..15 holds (8 + m) * 2^(e - 10);
 * field 15 with mantissa 7 is NaN, and there is no infinity.
 */
double fa_oracle_e4m3_to_f64(uint8_t code)
{
    const int e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return (code & 0x80) ? -v : v;
}

uint8_t fa_oracle_f64_to_e4m3(double x)
{
    if (isnan(x))
        return 0x7F;
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    const double a = fabs(x);
    if (a >= 448.0)
        return sign | 0x7E;            /* the largest finite value; beyond it saturate */
    if (a < ldexp(1.0, -6)) {
        /* subnormal grid, step 2^-9; a result of 8 is the smallest normal (code 0x08) */
        const double q = nearbyint(ldexp(a, 9));
        return sign | (uint8_t)q;
    }
    int E;
    frexp(a, &E);                      /* a = f * 2^E, f in [0.5, 1): a in [2^(E-1), 2^E) */
    int e = E - 1;                     /* a in [2^e, 2^(e+1)), e >= -6 */
    double q = nearbyint(ldexp(a, 3 - e)); /* multiples of the step 2^(e-3): q in [8, 16] */
    if (q == 16.0) {
        q = 8.0;
        e += 1;
    }
    /* a < 448 = 14 * 2^5 keeps the result at or below 448 (field 15, mantissa 6) */
    return sign | (uint8_t)(((e + 7) << 3) | (int)(q - 8.0));
}

int fa_oracle_quantize_e4m3(const double *x, uint8_t *codes, int64_t n)
{
    if (n < 0)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        codes[i] = fa_oracle_f64_to_e4m3(x[i]);
    return 0;
}

/* The values the quantised tensor holds: x rounded to E4M3 and read back. */
static void quantised_copy(const double *x, double *y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = fa_oracle_e4m3_to_f64(fa_oracle_f64_to_e4m3(x[i]));
}

/*
 * Attention with Q and K quantised to E4M3 (see above) and V as given:
 * quantise, then the three passes of standard attention in fp64.  Shapes and
 * return codes as fa_oracle_attention.
 */
int fa_oracle_attention_fp8qk(const double *q, const double *k, const double *v, double *o, double *lse,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, int causal,
                              double scale)
{
    if (B < 0 || H < 0 || check_shape(Nq, Nkv, d, causal))
        return -1;
    const int64_t nq = B * H * Nq * d, nk = B * H * Nkv * d;
    double *q8 = (double *)malloc((size_t)(nq > 0 ? nq : 1) * sizeof(double));
    double *k8 = (double *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(double));
    if (!q8 || !k8) {
        free(q8);
        free(k8);
        return -2;
    }
    quantised_copy(q, q8, nq);
    quantised_copy(k, k8, nk);
    const int rc = fa_oracle_attention(q8, k8, v, o, lse, B, H, Nq, Nkv, d, causal, scale);
    free(q8);
    free(k8);
    return rc;
}
