/*
 * csa_oracle.c -- plain CPU oracle for the CSA indexer score and top-k path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this code.  It shares nothing with
 * the HIP library: no headers, no helpers, no tables.
 *
 * What it computes (one query row i of batch b, compressed entry j):
 *
 *   logit[h]   = sum_t q[b,h,i,t] * k[b,j,t]            bf16 inputs, fp32 sums
 *   score[i,j] = scale * sum_h w[b,i,h] * ReLU(logit[h])  fp32
 *
 * following the fused StreamIndex score (MaxText PR #5079 "Add StreamIndex
 * Kernel for CSA": head-major q [B,H,S,D], compressed keys [B,W,D], weights
 * [B,S,H], scores [B,S,W]; bf16 einsums with float32 accumulation per the
 * commit that chunks the head accumulation).  Masks follow MaxText PR #4915
 * ("DSV4: Add indexer_save_selection and indexer_sharded_topk", inline review
 * of the indexer's future mask): entry j is a future entry of row i when
 * j >= causal_threshold(i); with absolute row position p = q_offset[b] + i,
 * causal_threshold = floor((p + 1) / m) clamped to [0, W].  When segment ids
 * are given, entries of another segment are masked as well.  Masked entries
 * are never selected and read -inf in the score output.
 *
 * The selection keeps, per row, the top_k valid entries ordered by score
 * descending with ties going to the lower entry index, and pads with -1 when
 * fewer than top_k entries are valid.
 *
 * Every loop runs in the order written: t from 0 to D-1 inside h from 0 to
 * H-1, one rounding per operation (built with -ffp-contract=off, so no fused
 * multiply-add).  The products of two bf16 values are exact in fp32; w times
 * ReLU(logit) is rounded before it is added.  A float64 twin of the score
 * (same loops in double) bounds the fp32 version's own rounding error.
 *
 * Pins: see tests/test_oracle.py (closed forms, a library special case,
 * invariants, brute-force selection, the float64 twin).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static float bf16_value(uint16_t bits)
{
    /* A bfloat16 value is the upper half of the float32 with the same value. */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static int64_t floor_div(int64_t a, int64_t b)
{
    int64_t q = a / b;
    if ((a % b) != 0 && ((a < 0) != (b < 0)))
        q -= 1;
    return q;
}

/* Number of visible compressed entries for a row at absolute position pos. */
static int64_t causal_threshold(int64_t pos, int64_t m, int64_t W)
{
    int64_t t = floor_div(pos + 1, m);
    if (t < 0)
        t = 0;
    if (t > W)
        t = W;
    return t;
}

static int entry_is_valid(int64_t b, int64_t i, int64_t j, int64_t S, int64_t W, int64_t m,
                          const int32_t *q_offset, const int32_t *q_seg, const int32_t *k_seg)
{
    int64_t pos = (q_offset ? (int64_t)q_offset[b] : 0) + i;
    if (j >= causal_threshold(pos, m, W))
        return 0;
    if (q_seg && q_seg[b * S + i] != k_seg[b * W + j])
        return 0;
    return 1;
}

/*
 * Scores of n_rows rows, fp32.  rows[r] = b*S + i names the row (rows == NULL
 * means rows 0..n_rows-1).  out is [n_rows, W].  q is [B,H,S,D], k is
 * [B,W,D], w is [B,S,H], all dense bf16 bit patterns.
 */
void csa_oracle_scores_f32(int64_t B, int64_t S, int64_t H, int64_t D, int64_t W, int64_t m,
                           float scale, const uint16_t *q, const uint16_t *k, const uint16_t *w,
                           const int32_t *q_offset, const int32_t *q_seg, const int32_t *k_seg,
                           int64_t n_rows, const int64_t *rows, float *out)
{
    (void)B;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t row = rows ? rows[r] : r;
        int64_t b = row / S, i = row % S;
        for (int64_t j = 0; j < W; ++j) {
            float *o = &out[r * W + j];
            if (!entry_is_valid(b, i, j, S, W, m, q_offset, q_seg, k_seg)) {
                *o = -INFINITY;
                continue;
            }
            float s = 0.0f;
            for (int64_t h = 0; h < H; ++h) {
                float logit = 0.0f;
                for (int64_t t = 0; t < D; ++t) {
                    float qv = bf16_value(q[((b * H + h) * S + i) * D + t]);
                    float kv = bf16_value(k[(b * W + j) * D + t]);
                    logit = logit + qv * kv;
                }
                float relu = logit > 0.0f ? logit : 0.0f;
                float wv = bf16_value(w[(b * S + i) * H + h]);
                float term = wv * relu;
                s = s + term;
            }
            s = scale * s;
            *o = s + 0.0f; /* -0 becomes +0 */
        }
    }
}

/* The same scores computed in float64 throughout (inputs widened exactly). */
void csa_oracle_scores_f64(int64_t B, int64_t S, int64_t H, int64_t D, int64_t W, int64_t m,
                           double scale, const uint16_t *q, const uint16_t *k, const uint16_t *w,
                           const int32_t *q_offset, const int32_t *q_seg, const int32_t *k_seg,
                           int64_t n_rows, const int64_t *rows, double *out)
{
    (void)B;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t row = rows ? rows[r] : r;
        int64_t b = row / S, i = row % S;
        for (int64_t j = 0; j < W; ++j) {
            double *o = &out[r * W + j];
            if (!entry_is_valid(b, i, j, S, W, m, q_offset, q_seg, k_seg)) {
                *o = -INFINITY;
                continue;
            }
            double s = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                double logit = 0.0;
                for (int64_t t = 0; t < D; ++t) {
                    double qv = (double)bf16_value(q[((b * H + h) * S + i) * D + t]);
                    double kv = (double)bf16_value(k[(b * W + j) * D + t]);
                    logit = logit + qv * kv;
                }
                double relu = logit > 0.0 ? logit : 0.0;
                double wv = (double)bf16_value(w[(b * S + i) * H + h]);
                s = s + wv * relu;
            }
            *o = scale * s + 0.0;
        }
    }
}

/* Validity mask only: 1 where (row, j) is a candidate, else 0.  [n_rows, W]. */
void csa_oracle_valid(int64_t S, int64_t W, int64_t m, const int32_t *q_offset,
                      const int32_t *q_seg, const int32_t *k_seg, int64_t n_rows,
                      const int64_t *rows, uint8_t *out)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t row = rows ? rows[r] : r;
        int64_t b = row / S, i = row % S;
        for (int64_t j = 0; j < W; ++j)
            out[r * W + j] = (uint8_t)entry_is_valid(b, i, j, S, W, m, q_offset, q_seg, k_seg);
    }
}

typedef struct {
    float score;
    int32_t j;
} candidate;

/* Order: higher score first; equal scores -> lower entry index first. */
static int candidate_order(const void *pa, const void *pb)
{
    const candidate *a = (const candidate *)pa, *b = (const candidate *)pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    return (a->j > b->j) - (a->j < b->j);
}

/*
 * Top-k of each row of a dense [rows, W] fp32 score matrix.  An entry whose
 * score is -inf (masked) or NaN is never selected.  idx is [rows, top_k]:
 * the selected entry indices in the candidate order above, then -1s.
 */
void csa_oracle_topk(int64_t rows, int64_t W, int64_t top_k, const float *scores, int32_t *idx)
{
#pragma omp parallel
    {
        candidate *buf = (candidate *)malloc(sizeof(candidate) * (size_t)(W > 0 ? W : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < rows; ++r) {
            int64_t n = 0;
            for (int64_t j = 0; j < W; ++j) {
                float s = scores[r * W + j];
                if (s == -INFINITY || s != s)
                    continue;
                buf[n].score = s;
                buf[n].j = (int32_t)j;
                ++n;
            }
            qsort(buf, (size_t)n, sizeof(candidate), candidate_order);
            for (int64_t t = 0; t < top_k; ++t)
                idx[r * top_k + t] = t < n ? buf[t].j : -1;
        }
        free(buf);
    }
}

/* Probabilistic bound factor of float32 summation of n terms (Higham and
 * Mary 2019): the computed sum lies within
 * (exp(lambda sqrt(n) u + n u^2 / (1-u)) - 1) sum|x| of the exact one with
 * probability at least 1 - 2 n exp(-lambda^2 (1-u)^2 / 2), u = 2^-24.  With
 * lambda = 8 and n <= 2^14 that is 1 - 4e-10. */
static double sum_bound_factor(int64_t n)
{
    const double u = ldexp(1.0, -24), lambda = 8.0;
    return expm1(lambda * sqrt((double)n) * u + (double)n * u * u / (1.0 - u));
}

/* One logit in float64, and eps_l, the bound above on how far a float32 dot
 * product of the same bf16 values (products exact, n = D additions) may lie
 * from it. */
static double logit_f64(const uint16_t *qr, const uint16_t *kr, int64_t D, double *eps_l)
{
    double logit = 0.0, mag = 0.0;
    for (int64_t t = 0; t < D; ++t) {
        double prod = (double)bf16_value(qr[t]) * (double)bf16_value(kr[t]);
        logit = logit + prod;
        mag = mag + fabs(prod);
    }
    *eps_l = sum_bound_factor(D) * mag;
    return logit;
}

/*
 * Backward of the score (the vector-Jacobian product the custom VJP of
 * MaxText PR #5079 "Add StreamIndex Kernel for CSA" returns, written out in
 * closed form instead of differentiating a materialised [B,H,S,W] tensor, as
 * the review of that backward asks).  For an upstream gradient g[b,i,j] of
 * the scores, with l = sum_t q[b,h,i,t] k[b,j,t] and only unmasked (i, j)
 * taking part (a masked score is a constant):
 *
 *   dw[b,i,h]   = scale * sum_j g[b,i,j] * ReLU(l)
 *   dq[b,h,i,t] = scale * sum_j g[b,i,j] * w[b,i,h] * [l > 0] * k[b,j,t]
 *   dk[b,j,t]   = scale * sum_i sum_h g[b,i,j] * w[b,i,h] * [l > 0] * q[b,h,i,t]
 *
 * ReLU's derivative at 0 is taken as 0, matching ReLU(l) = (l > 0 ? l : 0).
 * Everything is accumulated in float64 in the order written.
 *
 * When the statistics arrays are non-NULL the same loops also record, per
 * output element, three sums over the element's terms from which a caller
 * bounds how far a float32 implementation may lie from the float64 value
 * (the terms are the summands above, e.g. scale g w k_t for dq):
 *   [0] sum of |term| over the terms whose [l > 0] is decided,
 *   [1] sum of term^2 over the same terms,
 *   [2] for dq and dk the sum of |term| over the undecided terms, those whose
 *       |l| <= eps_l, so that a float32 logit may have either sign; for dw
 *       the sum over all terms of |scale g| eps_l, the most that float32
 *       logits can move ReLU(l) by.
 * dq/sq are [B,H,S,D] (sq with 3 doubles per element), dk/sk [B,W,D],
 * dw/sw [B,S,H]; g is [B,S,W] float32.  sq, sk and sw are all NULL or all set.
 */
/* dq [H][D] and dw [H] of query row (b, i), with statistics when sq != NULL. */
static void backward_row(int64_t b, int64_t i, int64_t S, int64_t H, int64_t D, int64_t W, int64_t m,
                         double scale, const uint16_t *q, const uint16_t *k, const uint16_t *w,
                         const int32_t *q_offset, const int32_t *q_seg, const int32_t *k_seg, const float *g,
                         double *dq, double *dw, double *sq, double *sw)
{
    for (int64_t h = 0; h < H; ++h) {
        const uint16_t *qr = &q[((b * H + h) * S + i) * D];
        double wv = (double)bf16_value(w[(b * S + i) * H + h]);
        double *dqr = &dq[h * D];
        double *sqr = sq ? &sq[h * D * 3] : NULL;
        double dwv = 0.0, sw_abs = 0.0, sw_sq = 0.0, sw_lg = 0.0;
        for (int64_t t = 0; t < D; ++t) {
            dqr[t] = 0.0;
            if (sqr)
                sqr[3 * t] = sqr[3 * t + 1] = sqr[3 * t + 2] = 0.0;
        }
        for (int64_t j = 0; j < W; ++j) {
            if (!entry_is_valid(b, i, j, S, W, m, q_offset, q_seg, k_seg))
                continue;
            const uint16_t *kr = &k[(b * W + j) * D];
            double gv = (double)g[(b * S + i) * W + j];
            double eps_l;
            double logit = logit_f64(qr, kr, D, &eps_l);
            double relu = logit > 0.0 ? logit : 0.0;
            double tw = scale * gv * relu;
            dwv += tw;
            sw_abs += fabs(tw);
            sw_sq += tw * tw;
            sw_lg += fabs(scale * gv) * eps_l;
            int undecided = fabs(logit) <= eps_l;
            double c = scale * gv * wv;
            for (int64_t t = 0; t < D; ++t) {
                double term = c * (double)bf16_value(kr[t]);
                if (logit > 0.0)
                    dqr[t] += term;
                if (sqr) {
                    if (undecided) {
                        sqr[3 * t + 2] += fabs(term);
                    } else if (logit > 0.0) {
                        sqr[3 * t] += fabs(term);
                        sqr[3 * t + 1] += term * term;
                    }
                }
            }
        }
        dw[h] = dwv;
        if (sw) {
            sw[3 * h] = sw_abs;
            sw[3 * h + 1] = sw_sq;
            sw[3 * h + 2] = sw_lg;
        }
    }
}

/* dk [D] of entry (b, j): rows i in order, heads h in order. */
static void backward_entry(int64_t b, int64_t j, int64_t S, int64_t H, int64_t D, int64_t W, int64_t m,
                           double scale, const uint16_t *q, const uint16_t *k, const uint16_t *w,
                           const int32_t *q_offset, const int32_t *q_seg, const int32_t *k_seg, const float *g,
                           double *dk, double *sk)
{
    const uint16_t *kr = &k[(b * W + j) * D];
    for (int64_t t = 0; t < D; ++t) {
        dk[t] = 0.0;
        if (sk)
            sk[3 * t] = sk[3 * t + 1] = sk[3 * t + 2] = 0.0;
    }
    for (int64_t i = 0; i < S; ++i) {
        if (!entry_is_valid(b, i, j, S, W, m, q_offset, q_seg, k_seg))
            continue;
        double gv = (double)g[(b * S + i) * W + j];
        for (int64_t h = 0; h < H; ++h) {
            const uint16_t *qr = &q[((b * H + h) * S + i) * D];
            double eps_l;
            double logit = logit_f64(qr, kr, D, &eps_l);
            int undecided = fabs(logit) <= eps_l;
            if (!(logit > 0.0) && !(sk && undecided))
                continue;
            double c = scale * gv * (double)bf16_value(w[(b * S + i) * H + h]);
            for (int64_t t = 0; t < D; ++t) {
                double term = c * (double)bf16_value(qr[t]);
                if (logit > 0.0)
                    dk[t] += term;
                if (sk) {
                    if (undecided) {
                        sk[3 * t + 2] += fabs(term);
                    } else {
                        sk[3 * t] += fabs(term);
                        sk[3 * t + 1] += term * term;
                    }
                }
            }
        }
    }
}

void csa_oracle_backward_f64(int64_t B, int64_t S, int64_t H, int64_t D, int64_t W, int64_t m,
                             double scale, const uint16_t *q, const uint16_t *k, const uint16_t *w,
                             const int32_t *q_offset, const int32_t *q_seg, const int32_t *k_seg,
                             const float *g, double *dq, double *dk, double *dw,
                             double *sq, double *sk, double *sw)
{
#pragma omp parallel
    {
        double *rq = (double *)malloc(sizeof(double) * (size_t)(H * D));
        double *rs = (double *)malloc(sizeof(double) * (size_t)(H * D * 3));
#pragma omp for schedule(dynamic, 1)
        for (int64_t row = 0; row < B * S; ++row) {
            int64_t b = row / S, i = row % S;
            backward_row(b, i, S, H, D, W, m, scale, q, k, w, q_offset, q_seg, k_seg, g, rq, &dw[row * H],
                         sq ? rs : NULL, sw ? &sw[row * H * 3] : NULL);
            for (int64_t h = 0; h < H; ++h)
                for (int64_t t = 0; t < D; ++t) {
                    int64_t o = ((b * H + h) * S + i) * D + t;
                    dq[o] = rq[h * D + t];
                    if (sq) {
                        sq[3 * o] = rs[3 * (h * D + t)];
                        sq[3 * o + 1] = rs[3 * (h * D + t) + 1];
                        sq[3 * o + 2] = rs[3 * (h * D + t) + 2];
                    }
                }
        }
        free(rq);
        free(rs);
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t e = 0; e < B * W; ++e)
        backward_entry(e / W, e % W, S, H, D, W, m, scale, q, k, w, q_offset, q_seg, k_seg, g, &dk[e * D],
                       sk ? &sk[e * D * 3] : NULL);
}

/*
 * The same gradients for chosen query rows and entries only: dq [n_rows,H,D]
 * and dw [n_rows,H] of rows[r] = b*S + i, dk [n_entries,D] of entries[e] =
 * b*W + j, with statistics as above (3 doubles per element; all NULL or all
 * set).
 */
void csa_oracle_backward_sample_f64(int64_t B, int64_t S, int64_t H, int64_t D, int64_t W, int64_t m,
                                    double scale, const uint16_t *q, const uint16_t *k, const uint16_t *w,
                                    const int32_t *q_offset, const int32_t *q_seg, const int32_t *k_seg,
                                    const float *g, int64_t n_rows, const int64_t *rows, int64_t n_entries,
                                    const int64_t *entries, double *dq, double *dw, double *dk, double *sq,
                                    double *sw, double *sk)
{
    (void)B;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r)
        backward_row(rows[r] / S, rows[r] % S, S, H, D, W, m, scale, q, k, w, q_offset, q_seg, k_seg, g,
                     &dq[r * H * D], &dw[r * H], sq ? &sq[r * H * D * 3] : NULL, sw ? &sw[r * H * 3] : NULL);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t e = 0; e < n_entries; ++e)
        backward_entry(entries[e] / W, entries[e] % W, S, H, D, W, m, scale, q, k, w, q_offset, q_seg, k_seg,
                       g, &dk[e * D], sk ? &sk[e * D * 3] : NULL);
}

/*
 * Indexer loss: the KL divergence between a target distribution over a
 * row's entries and the softmax of the row's indexer scores (the loss that
 * MaxText PR #4564 "Implement QK attention head chunking in MLA" computes in
 * calculate_indexer_loss and chunks over heads).  The pages give no formula;
 * the reading taken is
 *
 *   p_j   = a_j / A,  A = sum over visible j of a_j   (a = caller's target, >= 0)
 *   lse   = log sum over visible j of exp(s_j)
 *   KL_i  = sum over visible j with p_j > 0 of p_j (log p_j - (s_j - lse))
 *   dKL_i/ds_j = exp(s_j - lse) - p_j   (visible j), 0 (masked j)
 *
 * over the entries j the row can see (the causal and segment masks of the
 * score).  Rows with no visible entry or zero target mass have KL = 0 and a
 * zero gradient.  Target values at masked positions are never read into a
 * result.
 *
 * csa_oracle_kl_from_scores works on given float64 scores [rows, W] (-inf =
 * masked) and float32 targets [rows, W]; kl [rows] and grad [rows, W] (NULL =
 * not computed) are float64.  mag [rows, 3] (NULL = not computed) receives
 * the magnitudes a float32 evaluation rounds against: sum p |log p|,
 * sum p |s|, |lse|.
 */
void csa_oracle_kl_from_scores(int64_t rows, int64_t W, const double *scores, const float *target, double *kl,
                               double *grad, double *mag)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
        const double *s = &scores[r * W];
        const float *a = &target[r * W];
        double smax = -INFINITY, A = 0.0;
        int64_t nvis = 0;
        for (int64_t j = 0; j < W; ++j) {
            if (s[j] == -INFINITY)
                continue;
            ++nvis;
            if (s[j] > smax)
                smax = s[j];
            A += (double)a[j];
        }
        double *gr = grad ? &grad[r * W] : NULL;
        if (nvis == 0 || !(A > 0.0)) {
            kl[r] = 0.0;
            if (gr)
                for (int64_t j = 0; j < W; ++j)
                    gr[j] = 0.0;
            if (mag)
                mag[3 * r] = mag[3 * r + 1] = mag[3 * r + 2] = 0.0;
            continue;
        }
        double sumexp = 0.0;
        for (int64_t j = 0; j < W; ++j)
            if (s[j] != -INFINITY)
                sumexp += exp(s[j] - smax);
        double lse = smax + log(sumexp);
        double acc = 0.0, m_plogp = 0.0, m_ps = 0.0;
        for (int64_t j = 0; j < W; ++j) {
            if (s[j] == -INFINITY)
                continue;
            double pj = (double)a[j] / A;
            if (pj > 0.0) {
                acc += pj * (log(pj) - (s[j] - lse));
                m_plogp += pj * fabs(log(pj));
                m_ps += pj * fabs(s[j]);
            }
        }
        kl[r] = acc;
        if (mag) {
            mag[3 * r] = m_plogp;
            mag[3 * r + 1] = m_ps;
            mag[3 * r + 2] = fabs(lse);
        }
        if (gr)
            for (int64_t j = 0; j < W; ++j)
                gr[j] = s[j] == -INFINITY ? 0.0 : exp(s[j] - lse) - (double)a[j] / A;
    }
}

int csa_oracle_version(void) { return 3; }

/* OpenMP threads the oracle's parallel loops use. */
int csa_oracle_threads(void) { return omp_get_max_threads(); }
