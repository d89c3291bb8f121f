/*
 * Every entry point of the CPU oracle (oracle/csa_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer, on seeded small problems
 * that cover its edge cases: empty rows and caches (W = 0), rows that see no
 * entry, offsets, segment ids, compress rates 1..4, row and entry samples,
 * statistics on and off, top-k larger than the row, -inf and NaN scores, KL
 * rows without target mass.  Every buffer is allocated at its exact size, so
 * that a read or write past an array's end is reported.  Checks a few
 * invariants on the way; exit status 0 when all hold and no sanitizer fires.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void csa_oracle_scores_f32(int64_t B, int64_t S, int64_t H, int64_t D, int64_t W, int64_t m, float scale,
                           const uint16_t *q, const uint16_t *k, const uint16_t *w, const int32_t *q_offset,
                           const int32_t *q_seg, const int32_t *k_seg, int64_t n_rows, const int64_t *rows, float *out);
void csa_oracle_scores_f64(int64_t B, int64_t S, int64_t H, int64_t D, int64_t W, int64_t m, double scale,
                           const uint16_t *q, const uint16_t *k, const uint16_t *w, const int32_t *q_offset,
                           const int32_t *q_seg, const int32_t *k_seg, int64_t n_rows, const int64_t *rows,
                           double *out);
void csa_oracle_valid(int64_t S, int64_t W, int64_t m, const int32_t *q_offset, const int32_t *q_seg,
                      const int32_t *k_seg, int64_t n_rows, const int64_t *rows, uint8_t *out);
void csa_oracle_topk(int64_t rows, int64_t W, int64_t top_k, const float *scores, int32_t *idx);
void csa_oracle_backward_f64(int64_t B, int64_t S, int64_t H, int64_t D, int64_t W, int64_t m, double scale,
                             const uint16_t *q, const uint16_t *k, const uint16_t *w, const int32_t *q_offset,
                             const int32_t *q_seg, const int32_t *k_seg, const float *g, double *dq, double *dk,
                             double *dw, double *sq, double *sk, double *sw);
void csa_oracle_backward_sample_f64(int64_t B, int64_t S, int64_t H, int64_t D, int64_t W, int64_t m,
                                    double scale, const uint16_t *q, const uint16_t *k, const uint16_t *w,
                                    const int32_t *q_offset, const int32_t *q_seg, const int32_t *k_seg,
                                    const float *g, int64_t n_rows, const int64_t *rows, int64_t n_entries,
                                    const int64_t *entries, double *dq, double *dw, double *dk, double *sq,
                                    double *sw, double *sk);
void csa_oracle_kl_from_scores(int64_t rows, int64_t W, const double *scores, const float *target, double *kl,
                               double *grad, double *mag);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void)
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int64_t below(int64_t n) { return n > 0 ? (int64_t)(next_u64() % (uint64_t)n) : 0; }
static float unit(void) { return (float)((next_u64() >> 40) * (1.0 / 16777216.0)) * 2.0f - 1.0f; }
static uint16_t bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16); /* truncation: any bf16 value will do */
}

/* exact-size allocation (at least one byte, so that an empty array is not NULL) */
static void *xalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int g_fail = 0;
#define CHECK(c)                                                                                                      \
    do {                                                                                                              \
        if (!(c)) {                                                                                                   \
            fprintf(stderr, "line %d: %s\n", __LINE__, #c);                                                          \
            ++g_fail;                                                                                                 \
        }                                                                                                             \
    } while (0)

static void one_problem(void)
{
    const int64_t B = 1 + below(2), S = 1 + below(9), H = 1 + below(5), D = 8 * (1 + below(2));
    const int64_t W = below(14), m = 1 + below(4), rows_all = B * S;
    const int with_off = (int)below(2), with_seg = (int)below(2), with_stats = (int)below(2);
    uint16_t *q = xalloc(sizeof(uint16_t) * (size_t)(B * H * S * D));
    uint16_t *k = xalloc(sizeof(uint16_t) * (size_t)(B * W * D));
    uint16_t *w = xalloc(sizeof(uint16_t) * (size_t)(B * S * H));
    for (int64_t x = 0; x < B * H * S * D; ++x)
        q[x] = bf16_bits(unit());
    for (int64_t x = 0; x < B * W * D; ++x)
        k[x] = bf16_bits(unit());
    for (int64_t x = 0; x < B * S * H; ++x)
        w[x] = bf16_bits(unit());
    int32_t *off = NULL, *qs = NULL, *ks = NULL;
    if (with_off) {
        off = xalloc(sizeof(int32_t) * (size_t)B);
        for (int64_t b = 0; b < B; ++b)
            off[b] = (int32_t)below(3 * W + 2);
    }
    if (with_seg) {
        qs = xalloc(sizeof(int32_t) * (size_t)(B * S));
        ks = xalloc(sizeof(int32_t) * (size_t)(B * W));
        for (int64_t x = 0; x < B * S; ++x)
            qs[x] = (int32_t)below(3);
        for (int64_t x = 0; x < B * W; ++x)
            ks[x] = (int32_t)below(3);
    }
    /* all rows, then a sample in random order with repeats */
    const int64_t n_s = 1 + below(rows_all + 2);
    int64_t *rs = xalloc(sizeof(int64_t) * (size_t)n_s);
    for (int64_t r = 0; r < n_s; ++r)
        rs[r] = below(rows_all);
    float *sc = xalloc(sizeof(float) * (size_t)(rows_all * W));
    double *sd = xalloc(sizeof(double) * (size_t)(rows_all * W));
    uint8_t *vd = xalloc((size_t)(rows_all * W));
    csa_oracle_scores_f32(B, S, H, D, W, m, 0.5f, q, k, w, off, qs, ks, rows_all, NULL, sc);
    csa_oracle_scores_f64(B, S, H, D, W, m, 0.5, q, k, w, off, qs, ks, rows_all, NULL, sd);
    csa_oracle_valid(S, W, m, off, qs, ks, rows_all, NULL, vd);
    for (int64_t x = 0; x < rows_all * W; ++x) {
        CHECK(vd[x] == (sc[x] != -INFINITY)); /* masked exactly where invalid */
        CHECK(vd[x] == (sd[x] != -INFINITY));
    }
    float *ss = xalloc(sizeof(float) * (size_t)(n_s * W));
    csa_oracle_scores_f32(B, S, H, D, W, m, 0.5f, q, k, w, off, qs, ks, n_s, rs, ss);
    for (int64_t r = 0; r < n_s; ++r)
        for (int64_t j = 0; j < W; ++j)
            CHECK(memcmp(&ss[r * W + j], &sc[rs[r] * W + j], sizeof(float)) == 0);
    /* top-k, including k above the row length and -inf / NaN holes */
    for (int64_t x = 0; x < rows_all * W; ++x)
        if (below(17) == 0)
            sc[x] = below(2) ? NAN : -INFINITY;
    const int64_t top_k = 1 + below(W + 3);
    int32_t *idx = xalloc(sizeof(int32_t) * (size_t)(rows_all * top_k));
    csa_oracle_topk(rows_all, W, top_k, sc, idx);
    for (int64_t x = 0; x < rows_all * top_k; ++x)
        CHECK(idx[x] >= -1 && idx[x] < W);
    /* backward, full and sampled */
    float *g = xalloc(sizeof(float) * (size_t)(rows_all * W));
    for (int64_t x = 0; x < rows_all * W; ++x)
        g[x] = unit();
    double *dq = xalloc(sizeof(double) * (size_t)(B * H * S * D));
    double *dk = xalloc(sizeof(double) * (size_t)(B * W * D));
    double *dw = xalloc(sizeof(double) * (size_t)(B * S * H));
    double *sq = NULL, *sk = NULL, *sw = NULL;
    if (with_stats) {
        sq = xalloc(sizeof(double) * (size_t)(B * H * S * D * 3));
        sk = xalloc(sizeof(double) * (size_t)(B * W * D * 3));
        sw = xalloc(sizeof(double) * (size_t)(B * S * H * 3));
    }
    csa_oracle_backward_f64(B, S, H, D, W, m, 0.5, q, k, w, off, qs, ks, g, dq, dk, dw, sq, sk, sw);
    const int64_t n_e = 1 + below(B * W + 1);
    int64_t *es = xalloc(sizeof(int64_t) * (size_t)n_e);
    for (int64_t e = 0; e < n_e; ++e)
        es[e] = below(B * W);
    double *pq = xalloc(sizeof(double) * (size_t)(n_s * H * D));
    double *pw = xalloc(sizeof(double) * (size_t)(n_s * H));
    double *pk = xalloc(sizeof(double) * (size_t)(n_e * D));
    double *tq = NULL, *tw = NULL, *tk = NULL;
    if (with_stats) {
        tq = xalloc(sizeof(double) * (size_t)(n_s * H * D * 3));
        tw = xalloc(sizeof(double) * (size_t)(n_s * H * 3));
        tk = xalloc(sizeof(double) * (size_t)(n_e * D * 3));
    }
    /* entries of an empty cache: none to sample */
    csa_oracle_backward_sample_f64(B, S, H, D, W, m, 0.5, q, k, w, off, qs, ks, g, n_s, rs, B * W > 0 ? n_e : 0,
                                   es, pq, pw, pk, tq, tw, tk);
    for (int64_t r = 0; r < n_s; ++r) {
        const int64_t b = rs[r] / S, i = rs[r] % S;
        for (int64_t h = 0; h < H; ++h) {
            CHECK(pw[r * H + h] == dw[(b * S + i) * H + h]);
            for (int64_t t = 0; t < D; ++t)
                CHECK(pq[(r * H + h) * D + t] == dq[((b * H + h) * S + i) * D + t]);
        }
    }
    /* KL: rows with and without target mass */
    float *tg = xalloc(sizeof(float) * (size_t)(rows_all * W));
    for (int64_t x = 0; x < rows_all * W; ++x)
        tg[x] = (x / (W > 0 ? W : 1)) % 3 == 0 ? 0.0f : fabsf(unit());
    double *kl = xalloc(sizeof(double) * (size_t)rows_all);
    double *kg = xalloc(sizeof(double) * (size_t)(rows_all * W));
    double *mg = xalloc(sizeof(double) * (size_t)(rows_all * 3));
    csa_oracle_kl_from_scores(rows_all, W, sd, tg, kl, below(2) ? kg : NULL, below(2) ? mg : NULL);
    for (int64_t r = 0; r < rows_all; ++r)
        CHECK(kl[r] >= -1e-12 && kl[r] == kl[r]);

    free(q); free(k); free(w); free(off); free(qs); free(ks); free(rs); free(sc); free(sd); free(vd); free(ss);
    free(idx); free(g); free(dq); free(dk); free(dw); free(sq); free(sk); free(sw); free(es); free(pq); free(pw);
    free(pk); free(tq); free(tw); free(tk); free(tg); free(kl); free(kg); free(mg);
}

int main(int argc, char **argv)
{
    const int n = argc > 1 ? atoi(argv[1]) : 400;
    for (int it = 0; it < n; ++it)
        one_problem();
    if (g_fail) {
        fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    printf("oracle driver: %d problems, all checks hold\n", n);
    return 0;
}
