/*
 * Calls every entry point of the fp64 reference (oracle/attn_oracle.c) once
 * on small, ragged inputs, so that the test suite can run the reference's C
 * code under AddressSanitizer and UndefinedBehaviorSanitizer.  The values
 * are checked elsewhere; here every call must succeed and every output must
 * be written (finite, or -inf where an empty paged sequence asks for it).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int fa_oracle_widen(const uint16_t *bits, double *out, int64_t n, int kind);
int fa_oracle_attention(const double *q, const double *k, const double *v, double *o, double *lse, int64_t B,
                        int64_t H, int64_t Nq, int64_t Nkv, int64_t d, int causal, double scale);
int fa_oracle_attention_rows(const double *q, const double *k, const double *v, int64_t Nq, int64_t Nkv, int64_t d,
                             int causal, double scale, const int64_t *rows, int64_t nrows, double *o, double *lse);
int fa_oracle_attention_bwd(const double *q, const double *k, const double *v, const double *dO, const double *oD,
                            double *dq, double *dk, double *dv, int64_t B, int64_t H, int64_t Nq, int64_t Nkv,
                            int64_t d, int causal, double scale);
int fa_oracle_attention_bwd_sampled(const double *q, const double *k, const double *v, const double *dO,
                                    const double *oD, int64_t Nq, int64_t Nkv, int64_t d, int causal, double scale,
                                    const int64_t *qrows, int64_t nq, const int64_t *kcols, int64_t nk, double *dq,
                                    double *dk, double *dv);
int fa_oracle_paged_decode(const double *q, const double *kpool, const double *vpool, const int32_t *table,
                           const int32_t *lens, double *o, double *lse, int64_t B, int64_t H, int64_t num_pages,
                           int64_t page_size, int64_t max_pages, int64_t d, int layout, double scale);
int fa_oracle_quantize_e4m3(const double *x, uint8_t *codes, int64_t n);
double fa_oracle_e4m3_to_f64(uint8_t code);
int fa_oracle_attention_fp8qk(const double *q, const double *k, const double *v, double *o, double *lse, int64_t B,
                              int64_t H, int64_t Nq, int64_t Nkv, int64_t d, int causal, double scale);

static double *normals(size_t n, unsigned *state)
{
    double *x = malloc(n * sizeof *x);
    for (size_t i = 0; i < n; ++i) {
        *state = *state * 1664525u + 1013904223u;
        x[i] = ((double)(*state >> 8) / (double)(1u << 24) - 0.5) * 3.0;
    }
    return x;
}

static int finite_all(const double *x, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i]))
            return 0;
    return 1;
}

#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
            return 1;                                                 \
        }                                                             \
    } while (0)

int main(void)
{
    unsigned st = 12345u;
    const int64_t B = 2, H = 3, Nq = 37, Nkv = 53, d = 16;
    const size_t nq = B * H * Nq * d, nk = B * H * Nkv * d;
    double *q = normals(nq, &st), *k = normals(nk, &st), *v = normals(nk, &st), *dO = normals(nq, &st);
    double *o = malloc(nq * sizeof *o), *lse = malloc(B * H * Nq * sizeof *lse);
    double *dq = malloc(nq * sizeof *dq), *dk = malloc(nk * sizeof *dk), *dv = malloc(nk * sizeof *dv);

    uint16_t bits[512];
    double wide[512];
    for (int i = 0; i < 512; ++i)
        bits[i] = (uint16_t)(i * 131u);
    CHECK(fa_oracle_widen(bits, wide, 512, 1) == 0 && fa_oracle_widen(bits, wide, 512, 2) == 0);

    for (int causal = 0; causal < 2; ++causal) {
        CHECK(fa_oracle_attention(q, k, v, o, lse, B, H, Nq, Nkv, d, causal, 0.3) == 0);
        CHECK(finite_all(o, nq) && finite_all(lse, B * H * Nq));
        CHECK(fa_oracle_attention_fp8qk(q, k, v, o, lse, B, H, Nq, Nkv, d, causal, 0.3) == 0);
        CHECK(finite_all(o, nq) && finite_all(lse, B * H * Nq));
        CHECK(fa_oracle_attention_bwd(q, k, v, dO, NULL, dq, dk, dv, B, H, Nq, Nkv, d, causal, 0.3) == 0);
        CHECK(finite_all(dq, nq) && finite_all(dk, nk) && finite_all(dv, nk));
        CHECK(fa_oracle_attention_bwd(q, k, v, dO, o, dq, dk, dv, B, H, Nq, Nkv, d, causal, 0.3) == 0);
        CHECK(finite_all(dq, nq) && finite_all(dk, nk) && finite_all(dv, nk));
        const int64_t rows[3] = {0, 18, Nq - 1}, cols[3] = {0, 1, Nkv - 1};
        double ro[3 * 16], rl[3], sdq[3 * 16], sdk[3 * 16], sdv[3 * 16];
        CHECK(fa_oracle_attention_rows(q, k, v, Nq, Nkv, d, causal, 0.3, rows, 3, ro, rl) == 0);
        CHECK(finite_all(ro, 3 * 16) && finite_all(rl, 3));
        CHECK(fa_oracle_attention_bwd_sampled(q, k, v, dO, NULL, Nq, Nkv, d, causal, 0.3, rows, 3, cols, 3, sdq,
                                              sdk, sdv) == 0);
        CHECK(finite_all(sdq, 3 * 16) && finite_all(sdk, 3 * 16) && finite_all(sdv, 3 * 16));
        CHECK(fa_oracle_attention_bwd_sampled(q, k, v, dO, o, Nq, Nkv, d, causal, 0.3, rows, 3, cols, 3, sdq, sdk,
                                              sdv) == 0);
        CHECK(finite_all(sdq, 3 * 16) && finite_all(sdk, 3 * 16) && finite_all(sdv, 3 * 16));
    }

    /* paged decode: 3 sequences (one empty) over a shuffled pool of 5-key pages */
    const int64_t PB = 3, ps = 5, max_pages = 4, num_pages = 9;
    const int32_t table[12] = {7, 2, 5, 0, 1, 8, -1, -1, 3, 6, 4, -1};
    const int32_t lens[3] = {20, 7, 0};
    for (int layout = 0; layout < 2; ++layout) {
        double *pq = normals(PB * H * d, &st), *kp = normals(num_pages * H * ps * d, &st);
        double *vp = normals(num_pages * H * ps * d, &st);
        double po[3 * 3 * 16], pl[3 * 3];
        CHECK(fa_oracle_paged_decode(pq, kp, vp, table, lens, po, pl, PB, H, num_pages, ps, max_pages, d, layout,
                                     0.25) == 0);
        CHECK(finite_all(po, 2 * H * d) && finite_all(pl, 2 * H));
        for (int i = 0; i < H; ++i)
            CHECK(pl[2 * H + i] == -INFINITY && po[(2 * H + i) * d] == 0.0);
        free(pq);
        free(kp);
        free(vp);
    }

    uint8_t codes[300];
    double xs[300];
    for (int i = 0; i < 300; ++i)
        xs[i] = (i - 150) * 4.1;
    xs[0] = INFINITY;
    xs[1] = -INFINITY;
    CHECK(fa_oracle_quantize_e4m3(xs, codes, 300) == 0);
    for (int i = 0; i < 256; ++i) {
        const double x = fa_oracle_e4m3_to_f64((uint8_t)i);
        CHECK(isnan(x) == ((i & 0x7f) == 0x7f));
    }

    free(q);
    free(k);
    free(v);
    free(dO);
    free(o);
    free(lse);
    free(dq);
    free(dk);
    free(dv);
    puts("oracle entry points ran clean");
    return 0;
}
