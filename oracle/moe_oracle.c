/*
 * moe_oracle.c -- CPU oracle for the local MoE expert layer (TEST INFRASTRUCTURE ONLY).
 *
 * Plain C11, fp64 arithmetic, libm exp. Loops are written in the order of the
 * definitions; OpenMP only splits independent outputs between threads, and each
 * output is summed by one thread in the order stated next to it.
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg use this file.
 * See moe_oracle.h for the pages this follows.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- typed element loads ------------------------------------------------ */

static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double ld(const void *p, int dt, int64_t i) {
    if (dt == ORACLE_BF16) return bf16_bits_to_double(((const uint16_t *)p)[i]);
    if (dt == ORACLE_F32) return (double)((const float *)p)[i];
    return ((const double *)p)[i];
}

/* ---- SwiGLU (Hysen Labs page, "The MoE class..." and "Interleaved by default") --
 * silu applied to the gate half times the up half; sigma(g) = 1/(1+exp(-g)). */
static double sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }
static double swiglu(double g, double u) { return g * sigmoid(g) * u; }
/* d a / d g and d a / d u for a = g*sigma(g)*u. */
static double dswiglu_dgate(double g, double u) {
    double s = sigmoid(g);
    return u * s * (1.0 + g * (1.0 - s));
}
static double dswiglu_dup(double g) { return g * sigmoid(g); }

/* ---- Metadata ----------------------------------------------------------------
 * GitHub issue #68 (metadata list; question 3): the pair list is token-major
 * with token_indices ascending. Reading: within a token, ascending slot k.
 * A slot is valid iff 0 <= topk_idx[t,k] < E; -1 marks an invalid slot (issue,
 * non-expand outputs). Ids outside [-1,E) are flagged and skipped.
 * Sort (serving-script notes, step 2 "sort by expert ID"): reading: a stable
 * counting sort, so ties keep ascending pair index q.
 * Directions (reading): x_gather_idx[s] = token of sorted position s;
 * s_scatter_idx[s] = pair index q of sorted position s; s_reverse_scatter_idx[q]
 * = sorted position of pair q; offsets are exclusive scans with E+1 / N+1 entries.
 */
int64_t oracle_build_metadata(int64_t N, int64_t K, int64_t E,
                              const int32_t *topk_idx, const float *topk_weights,
                              int32_t *expert_frequency, int32_t *expert_frequency_offset,
                              int32_t *x_gather_idx, int32_t *s_scatter_idx,
                              int32_t *s_reverse_scatter_idx,
                              int32_t *num_activated_expert_per_token_offset,
                              float *router_scores,
                              int32_t *pair_token, int32_t *pair_slot, int32_t *pair_expert,
                              uint32_t *flags) {
    uint32_t fl = 0;
    int32_t *pt = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N * K + 1));
    int32_t *pe = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N * K + 1));
    int32_t *cur = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));

    /* O1: enumerate valid pairs token-major, ascending k. */
    int64_t q = 0;
    for (int64_t t = 0; t < N; t++) {
        num_activated_expert_per_token_offset[t] = (int32_t)q;
        for (int64_t k = 0; k < K; k++) {
            int32_t e = topk_idx[t * K + k];
            if (e >= 0 && e < E) {
                pt[q] = (int32_t)t;
                pe[q] = e;
                if (pair_token) pair_token[q] = (int32_t)t;
                if (pair_slot) pair_slot[q] = (int32_t)k;
                if (pair_expert) pair_expert[q] = e;
                router_scores[q] = topk_weights[t * K + k];
                q++;
            } else if (e != -1) {
                fl |= ORACLE_FLAG_BAD_EXPERT;
            }
        }
    }
    int64_t P = q;
    num_activated_expert_per_token_offset[N] = (int32_t)P;

    /* O2: histogram and its exclusive scan. */
    for (int64_t e = 0; e < E; e++) expert_frequency[e] = 0;
    for (int64_t i = 0; i < P; i++) expert_frequency[pe[i]]++;
    expert_frequency_offset[0] = 0;
    for (int64_t e = 0; e < E; e++)
        expert_frequency_offset[e + 1] = expert_frequency_offset[e] + expert_frequency[e];

    /* O3: stable counting sort by expert, pairs visited in ascending q. */
    for (int64_t e = 0; e < E; e++) cur[e] = expert_frequency_offset[e];
    for (int64_t i = 0; i < P; i++) {
        int32_t s = cur[pe[i]]++;
        x_gather_idx[s] = pt[i];
        s_scatter_idx[s] = (int32_t)i;
        s_reverse_scatter_idx[i] = s;
    }
    free(pt);
    free(pe);
    free(cur);
    if (flags) *flags = fl;
    return P;
}

/* expert of every sorted position, from the segment offsets */
static int32_t *expert_of_positions(int64_t E, const int32_t *foff) {
    int64_t P = foff[E];
    int32_t *es = (int32_t *)malloc(sizeof(int32_t) * (size_t)(P + 1));
    for (int64_t e = 0; e < E; e++)
        for (int64_t s = foff[e]; s < foff[e + 1]; s++) es[s] = (int32_t)e;
    return es;
}

/* ---- Full forward --------------------------------------------------------- */
void oracle_forward(int64_t N, int64_t H, int64_t I, int64_t E,
                    const double *x, const double *w_up, const double *w_down,
                    const int32_t *foff, const int32_t *x_gather_idx,
                    const int32_t *s_rev, const int32_t *tok_off,
                    const float *router_scores,
                    double *h, double *a, double *y, double *out) {
    int64_t P = foff[E];
    int64_t I2 = 2 * I;
    int32_t *es = expert_of_positions(E, foff);

    /* O4 (grouped GEMM, issue #68 "grouped GEMM path"; x row gathered by
     * x_gather_idx): h[s,j] = sum_{i<H} x[t(s),i] * W_up[e(s),i,j], i ascending.
     * O5 (SwiGLU, interleaved columns 2j = gate_j, 2j+1 = up_j).
     * O6 (down projection): y[s,c] = sum_{j<I} a[s,j] * W_down[e(s),j,c]. */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t s = 0; s < P; s++) {
        const int64_t e = es[s];
        const double *xr = x + (int64_t)x_gather_idx[s] * H;
        const double *wu = w_up + e * H * I2;
        const double *wd = w_down + e * I * H;
        double *hr = h + s * I2;
        for (int64_t j = 0; j < I2; j++) {
            double acc = 0.0;
            for (int64_t i = 0; i < H; i++) acc += xr[i] * wu[i * I2 + j];
            hr[j] = acc;
        }
        double *ar = a + s * I;
        for (int64_t j = 0; j < I; j++) ar[j] = swiglu(hr[2 * j], hr[2 * j + 1]);
        double *yr = y + s * H;
        for (int64_t c = 0; c < H; c++) {
            double acc = 0.0;
            for (int64_t j = 0; j < I; j++) acc += ar[j] * wd[j * H + c];
            yr[c] = acc;
        }
    }

    /* O7 (combine; serving-script step 5 scatter-add, NKI unpermute scatter-add
     * accumulating over top-k): out[t,c] = sum over the token's pairs q in
     * ascending order of router_scores[q] * y[s_rev[q], c]. Empty rows are 0. */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < N; t++) {
        double *o = out + t * H;
        for (int64_t c = 0; c < H; c++) o[c] = 0.0;
        for (int64_t q = tok_off[t]; q < tok_off[t + 1]; q++) {
            const double w = (double)router_scores[q];
            const double *yr = y + (int64_t)s_rev[q] * H;
            for (int64_t c = 0; c < H; c++) o[c] += w * yr[c];
        }
    }
    free(es);
}

/* ---- Full backward (chain rule through O4..O7; issue #68 question 4 for the
 * router-score gradient returned in [N,K] layout) ---------------------------- */
void oracle_backward(int64_t N, int64_t K, int64_t H, int64_t I, int64_t E,
                     const double *x, const double *w_up, const double *w_down,
                     const double *dout,
                     const int32_t *foff, const int32_t *x_gather_idx,
                     const int32_t *s_scatter_idx, const int32_t *s_rev,
                     const int32_t *tok_off, const float *router_scores,
                     const int32_t *pair_token, const int32_t *pair_slot,
                     const double *h, const double *a, const double *y,
                     double *dx, double *dw_up, double *dw_down, double *d_topk_weights) {
    int64_t P = foff[E];
    int64_t I2 = 2 * I;
    int32_t *es = expert_of_positions(E, foff);
    double *dy = (double *)malloc(sizeof(double) * (size_t)(P * H + 1));
    double *dscore = (double *)malloc(sizeof(double) * (size_t)(P + 1));
    double *dh = (double *)malloc(sizeof(double) * (size_t)(P * I2 + 1));
    double *dxg = (double *)malloc(sizeof(double) * (size_t)(P * H + 1));

    /* O8: dy[s,c] = w_{q(s)} * dout[t(s),c]; dscore[q] = <dout[t(q)], y[s_rev[q]]>. */
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < P; s++) {
        const double w = (double)router_scores[s_scatter_idx[s]];
        const double *dr = dout + (int64_t)x_gather_idx[s] * H;
        for (int64_t c = 0; c < H; c++) dy[s * H + c] = w * dr[c];
    }
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < P; q++) {
        const double *dr = dout + (int64_t)pair_token[q] * H;
        const double *yr = y + (int64_t)s_rev[q] * H;
        double acc = 0.0;
        for (int64_t c = 0; c < H; c++) acc += dr[c] * yr[c];
        dscore[q] = acc;
    }

    /* O9: da[s,j] = sum_c dy[s,c] W_down[e,j,c]; O10: dh from da through SwiGLU. */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t s = 0; s < P; s++) {
        const int64_t e = es[s];
        const double *wd = w_down + e * I * H;
        for (int64_t j = 0; j < I; j++) {
            double acc = 0.0;
            for (int64_t c = 0; c < H; c++) acc += dy[s * H + c] * wd[j * H + c];
            const double g = h[s * I2 + 2 * j], u = h[s * I2 + 2 * j + 1];
            dh[s * I2 + 2 * j] = acc * dswiglu_dgate(g, u);
            dh[s * I2 + 2 * j + 1] = acc * dswiglu_dup(g);
        }
    }
    /* O9: dW_down[e,j,c] = sum over s in e's segment (ascending) of a[s,j]*dy[s,c]. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ej = 0; ej < E * I; ej++) {
        const int64_t e = ej / I, j = ej % I;
        double *row = dw_down + (e * I + j) * H;
        for (int64_t c = 0; c < H; c++) row[c] = 0.0;
        for (int64_t s = foff[e]; s < foff[e + 1]; s++) {
            const double av = a[s * I + j];
            for (int64_t c = 0; c < H; c++) row[c] += av * dy[s * H + c];
        }
    }
    /* O11: dxg[s,i] = sum_j dh[s,j] W_up[e,i,j];
     *      dW_up[e,i,j] = sum over s in e's segment (ascending) of x[t(s),i]*dh[s,j]. */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t s = 0; s < P; s++) {
        const int64_t e = es[s];
        const double *wu = w_up + e * H * I2;
        for (int64_t i = 0; i < H; i++) {
            double acc = 0.0;
            for (int64_t j = 0; j < I2; j++) acc += dh[s * I2 + j] * wu[i * I2 + j];
            dxg[s * H + i] = acc;
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ei = 0; ei < E * H; ei++) {
        const int64_t e = ei / H, i = ei % H;
        double *row = dw_up + (e * H + i) * I2;
        for (int64_t j = 0; j < I2; j++) row[j] = 0.0;
        for (int64_t s = foff[e]; s < foff[e + 1]; s++) {
            const double xv = x[(int64_t)x_gather_idx[s] * H + i];
            for (int64_t j = 0; j < I2; j++) row[j] += xv * dh[s * I2 + j];
        }
    }
    /* O12: dx[t,i] = sum over the token's pairs q ascending of dxg[s_rev[q],i];
     *      d_topk_weights[t,k] = dscore[q] at the pair's slot, 0 elsewhere. */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < N; t++) {
        double *r = dx + t * H;
        for (int64_t i = 0; i < H; i++) r[i] = 0.0;
        for (int64_t q = tok_off[t]; q < tok_off[t + 1]; q++) {
            const double *g = dxg + (int64_t)s_rev[q] * H;
            for (int64_t i = 0; i < H; i++) r[i] += g[i];
        }
        for (int64_t k = 0; k < K; k++) d_topk_weights[t * K + k] = 0.0;
        for (int64_t q = tok_off[t]; q < tok_off[t + 1]; q++)
            d_topk_weights[t * K + pair_slot[q]] = dscore[q];
    }
    free(es);
    free(dy);
    free(dscore);
    free(dh);
    free(dxg);
}

/* ---- Brute force: per token, per valid slot, the expert MLP applied directly. */
void oracle_bruteforce_forward(int64_t N, int64_t K, int64_t H, int64_t I, int64_t E,
                               const double *x, const int32_t *topk_idx,
                               const float *topk_weights,
                               const double *w_up, const double *w_down, double *out) {
    int64_t I2 = 2 * I;
#pragma omp parallel
    {
        double *hv = (double *)malloc(sizeof(double) * (size_t)I2);
        double *av = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < N; t++) {
            double *o = out + t * H;
            for (int64_t c = 0; c < H; c++) o[c] = 0.0;
            for (int64_t k = 0; k < K; k++) {
                const int32_t e = topk_idx[t * K + k];
                if (e < 0 || e >= E) continue;
                const double w = (double)topk_weights[t * K + k];
                const double *wu = w_up + (int64_t)e * H * I2;
                const double *wd = w_down + (int64_t)e * I * H;
                for (int64_t j = 0; j < I2; j++) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < H; i++) acc += x[t * H + i] * wu[i * I2 + j];
                    hv[j] = acc;
                }
                for (int64_t j = 0; j < I; j++) av[j] = swiglu(hv[2 * j], hv[2 * j + 1]);
                for (int64_t c = 0; c < H; c++) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < I; j++) acc += av[j] * wd[j * H + c];
                    o[c] += w * acc;
                }
            }
        }
        free(hv);
        free(av);
    }
}

/* ---- Sampled entry points ---------------------------------------------------
 * The same steps as above, restricted to the outputs asked for, reading typed
 * inputs element by element. */

/* h row of one pair: h[j] = sum_i x[t,i] W_up[e,i,j] (O4). */
static void up_row(int64_t H, int64_t I2, const void *x, int x_dt, int64_t t,
                   const void *w_up, int w_dt, int64_t e, double *hv, double *xrow) {
    for (int64_t i = 0; i < H; i++) xrow[i] = ld(x, x_dt, t * H + i);
    const int64_t base = e * H * I2;
    for (int64_t j = 0; j < I2; j++) hv[j] = 0.0;
    for (int64_t i = 0; i < H; i++) {
        const double xi = xrow[i];
        for (int64_t j = 0; j < I2; j++) hv[j] += xi * ld(w_up, w_dt, base + i * I2 + j);
    }
}

void oracle_sample_tokens(int64_t N, int64_t K, int64_t H, int64_t I, int64_t E,
                          const void *x, int x_dt, const void *w_up, int w_dt,
                          const void *w_down, const void *dout, int dout_dt,
                          const int32_t *topk_idx, const float *topk_weights,
                          int64_t n_tok, const int64_t *tokens,
                          double *out_rows, double *dx_rows, double *dtw_rows) {
    (void)N;
    const int64_t I2 = 2 * I;
#pragma omp parallel
    {
        double *xrow = (double *)malloc(sizeof(double) * (size_t)H);
        double *drow = (double *)malloc(sizeof(double) * (size_t)H);
        double *hv = (double *)malloc(sizeof(double) * (size_t)I2);
        double *av = (double *)malloc(sizeof(double) * (size_t)I);
        double *yv = (double *)malloc(sizeof(double) * (size_t)H);
        double *dhv = (double *)malloc(sizeof(double) * (size_t)I2);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_tok; n++) {
            const int64_t t = tokens[n];
            double *o = out_rows + n * H;
            double *dxr = dx_rows ? dx_rows + n * H : NULL;
            for (int64_t c = 0; c < H; c++) o[c] = 0.0;
            if (dout) {
                for (int64_t c = 0; c < H; c++) dxr[c] = 0.0;
                for (int64_t k = 0; k < K; k++) dtw_rows[n * K + k] = 0.0;
                for (int64_t c = 0; c < H; c++) drow[c] = ld(dout, dout_dt, t * H + c);
            }
            /* valid slots in ascending k = the token's pairs in ascending q */
            for (int64_t k = 0; k < K; k++) {
                const int32_t e = topk_idx[t * K + k];
                if (e < 0 || e >= E) continue;
                const double w = (double)topk_weights[t * K + k];
                up_row(H, I2, x, x_dt, t, w_up, w_dt, e, hv, xrow);
                for (int64_t j = 0; j < I; j++) av[j] = swiglu(hv[2 * j], hv[2 * j + 1]);
                const int64_t db = (int64_t)e * I * H;
                for (int64_t c = 0; c < H; c++) yv[c] = 0.0;
                for (int64_t j = 0; j < I; j++) {
                    const double aj = av[j];
                    for (int64_t c = 0; c < H; c++) yv[c] += aj * ld(w_down, w_dt, db + j * H + c);
                }
                for (int64_t c = 0; c < H; c++) o[c] += w * yv[c];
                if (!dout) continue;
                /* O8: dscore = <dout[t], y>; O9/O10: da, dh; O11: dxg; O12. */
                double ds = 0.0;
                for (int64_t c = 0; c < H; c++) ds += drow[c] * yv[c];
                dtw_rows[n * K + k] = ds;
                for (int64_t j = 0; j < I; j++) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < H; c++) acc += w * drow[c] * ld(w_down, w_dt, db + j * H + c);
                    const double g = hv[2 * j], u = hv[2 * j + 1];
                    dhv[2 * j] = acc * dswiglu_dgate(g, u);
                    dhv[2 * j + 1] = acc * dswiglu_dup(g);
                }
                const int64_t ub = (int64_t)e * H * I2;
                for (int64_t i = 0; i < H; i++) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < I2; j++) acc += dhv[j] * ld(w_up, w_dt, ub + i * I2 + j);
                    dxr[i] += acc;
                }
            }
        }
        free(xrow);
        free(drow);
        free(hv);
        free(av);
        free(yv);
        free(dhv);
    }
}

static int64_t expert_of(int64_t E, const int32_t *foff, int64_t s) {
    for (int64_t e = 0; e < E; e++)
        if (s >= foff[e] && s < foff[e + 1]) return e;
    return -1;
}

void oracle_sample_h_rows(int64_t H, int64_t I, int64_t E,
                          const void *x, int x_dt, const void *w_up, int w_dt,
                          const int32_t *foff, const int32_t *x_gather_idx,
                          int64_t n_rows, const int64_t *rows, double *h_rows) {
    const int64_t I2 = 2 * I;
#pragma omp parallel
    {
        double *xrow = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_rows; n++) {
            const int64_t s = rows[n];
            const int64_t e = expert_of(E, foff, s);
            up_row(H, I2, x, x_dt, x_gather_idx[s], w_up, w_dt, e, h_rows + n * I2, xrow);
        }
        free(xrow);
    }
}

/* g = h[s,2j], u = h[s,2j+1] of one pair, by direct dot products (O4). */
static void gate_up(int64_t H, int64_t I2, const double *xrow, const void *w_up, int w_dt,
                    int64_t e, int64_t j, double *g, double *u) {
    const int64_t base = e * H * I2;
    double ag = 0.0, au = 0.0;
    for (int64_t i = 0; i < H; i++) {
        ag += xrow[i] * ld(w_up, w_dt, base + i * I2 + 2 * j);
        au += xrow[i] * ld(w_up, w_dt, base + i * I2 + 2 * j + 1);
    }
    *g = ag;
    *u = au;
}

void oracle_sample_dw_down_rows(int64_t H, int64_t I, int64_t E,
                                const void *x, int x_dt, const void *w_up, int w_dt,
                                const void *dout, int dout_dt,
                                const int32_t *foff, const int32_t *x_gather_idx,
                                const int32_t *s_scatter_idx, const float *router_scores,
                                int64_t n, const int64_t *e_list, const int64_t *j_list,
                                double *rows) {
    const int64_t I2 = 2 * I;
    (void)E;
#pragma omp parallel
    {
        double *xrow = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; r++) {
            const int64_t e = e_list[r], j = j_list[r];
            double *row = rows + r * H;
            for (int64_t c = 0; c < H; c++) row[c] = 0.0;
            /* O9: sum over s in e's segment, ascending, of a[s,j] * dy[s,c]. */
            for (int64_t s = foff[e]; s < foff[e + 1]; s++) {
                const int64_t t = x_gather_idx[s];
                for (int64_t i = 0; i < H; i++) xrow[i] = ld(x, x_dt, t * H + i);
                double g, u;
                gate_up(H, I2, xrow, w_up, w_dt, e, j, &g, &u);
                const double av = swiglu(g, u);
                const double w = (double)router_scores[s_scatter_idx[s]];
                for (int64_t c = 0; c < H; c++) row[c] += av * (w * ld(dout, dout_dt, t * H + c));
            }
        }
        free(xrow);
    }
}

void oracle_sample_dw_up_cols(int64_t H, int64_t I, int64_t E,
                              const void *x, int x_dt, const void *w_up, int w_dt,
                              const void *w_down, const void *dout, int dout_dt,
                              const int32_t *foff, const int32_t *x_gather_idx,
                              const int32_t *s_scatter_idx, const float *router_scores,
                              int64_t n, const int64_t *e_list, const int64_t *jj_list,
                              double *cols) {
    const int64_t I2 = 2 * I;
    (void)E;
#pragma omp parallel
    {
        double *xrow = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; r++) {
            const int64_t e = e_list[r], jj = jj_list[r];
            double *cg = cols + (r * 2 + 0) * H;
            double *cu = cols + (r * 2 + 1) * H;
            for (int64_t i = 0; i < H; i++) cg[i] = cu[i] = 0.0;
            const int64_t db = e * I * H;
            for (int64_t s = foff[e]; s < foff[e + 1]; s++) {
                const int64_t t = x_gather_idx[s];
                for (int64_t i = 0; i < H; i++) xrow[i] = ld(x, x_dt, t * H + i);
                double g, u;
                gate_up(H, I2, xrow, w_up, w_dt, e, jj, &g, &u);
                /* O9: da[s,jj] = sum_c w * dout[t,c] * W_down[e,jj,c]; O10: dh. */
                const double w = (double)router_scores[s_scatter_idx[s]];
                double da = 0.0;
                for (int64_t c = 0; c < H; c++)
                    da += w * ld(dout, dout_dt, t * H + c) * ld(w_down, w_dt, db + jj * H + c);
                const double dg = da * dswiglu_dgate(g, u);
                const double du = da * dswiglu_dup(g);
                /* O11: dW_up[e,i,j] accumulates x[t,i] * dh[s,j], s ascending. */
                for (int64_t i = 0; i < H; i++) {
                    cg[i] += xrow[i] * dg;
                    cu[i] += xrow[i] * du;
                }
            }
        }
        free(xrow);
    }
}

/* Router: see the header. One token at a time; selection by repeated strict maxima
 * over the experts not yet taken, scanning e upward (so equal logits go to the lower
 * id); probabilities and the aux sums in fp64. */
void oracle_route(int64_t N, int64_t E, int64_t K, const void *logits, int logits_dt, int mode,
                  int renormalize, int32_t *topk_idx, double *topk_weights, double *aux) {
    double *l = (double *)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
    char *taken = (char *)malloc((size_t)(E > 0 ? E : 1));
    double *count = (double *)calloc((size_t)(E > 0 ? E : 1), sizeof(double));
    double *psum = (double *)calloc((size_t)(E > 0 ? E : 1), sizeof(double));
    for (int64_t t = 0; t < N; t++) {
        for (int64_t e = 0; e < E; e++) {
            l[e] = ld(logits, logits_dt, t * E + e);
            taken[e] = 0;
        }
        for (int64_t k = 0; k < K; k++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            topk_idx[t * K + k] = (int32_t)best;
            count[best] += 1.0;
        }
        const double mx = l[topk_idx[t * K]];
        double z_all = 0.0;
        for (int64_t e = 0; e < E; e++) z_all += exp(l[e] - mx);
        for (int64_t e = 0; e < E; e++) psum[e] += exp(l[e] - mx) / z_all;
        double z_sel = 0.0;
        for (int64_t k = 0; k < K; k++) z_sel += exp(l[topk_idx[t * K + k]] - mx);
        for (int64_t k = 0; k < K; k++) {
            const double v = exp(l[topk_idx[t * K + k]] - mx);
            double wk;
            if (mode == 0)
                wk = v / z_sel;
            else
                wk = renormalize ? (v / z_all) / (z_sel / z_all) : v / z_all;
            topk_weights[t * K + k] = wk;
        }
    }
    double a = 0.0;
    if (N > 0 && K > 0)
        for (int64_t e = 0; e < E; e++) a += (count[e] / (double)(N * K)) * (psum[e] / (double)N);
    *aux = (double)E * a;
    free(l);
    free(taken);
    free(count);
    free(psum);
}
