/*
 * Sanitizer driver for the oracle (test infrastructure; built and run by
 * tests/test_oracle_sanitize.py with gcc -fsanitize=address,undefined).
 *
 * Calls every entry point of oracle/moe_oracle.c on small seeded inputs, the edge
 * cases included (no rows, every slot invalid, ids outside [-1,E), repeated experts
 * in a row, K = 1 and E = 1), with every buffer allocated to exactly the size the
 * header states, so an out-of-bounds access, a use after free, a leak or undefined
 * behaviour stops the run. Along the way it checks what must hold between the entry
 * points: the metadata invariants, the brute-force forward against the metadata
 * forward, the sampled entry points against the full forward and backward, and the
 * router's selection and weight sums. Prints "ok" and exits 0 when everything held.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static uint64_t rng_state;
static uint64_t next_u64(void) { /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double uniform(void) { return (double)(next_u64() >> 11) * 0x1.0p-53; }

/* a value in [-scale, scale), truncated to a bf16 bit pattern */
static uint16_t rand_bf16(double scale) {
    const float f = (float)((2.0 * uniform() - 1.0) * scale);
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}
static double bf16_to_double(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* exactly n elements (one when n is 0, so that the pointer is valid) */
static void *xalloc(int64_t n, size_t size) {
    void *p = malloc((size_t)(n > 0 ? n : 1) * size);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int failures = 0;
static void fail(const char *what, int64_t at) {
    fprintf(stderr, "FAIL %s (at %lld)\n", what, (long long)at);
    failures++;
}
/* max |a - ref| <= 1e-12 max |ref|: the same sums, possibly in another grouping */
static void check_close(const char *what, const double *a, const double *ref, int64_t n) {
    double mx = 0.0, err = 0.0;
    for (int64_t i = 0; i < n; i++) {
        if (fabs(ref[i]) > mx) mx = fabs(ref[i]);
        if (!(fabs(a[i] - ref[i]) <= err)) err = fabs(a[i] - ref[i]);
    }
    if (!(err <= 1e-12 * (mx > 0.0 ? mx : 1.0))) {
        fprintf(stderr, "FAIL %s: max err %g, max ref %g\n", what, err, mx);
        failures++;
    }
}

static void run_route(int64_t N, int64_t E, int64_t K) {
    float *lf = xalloc(N * E, sizeof(float));
    uint16_t *lb = xalloc(N * E, sizeof(uint16_t));
    for (int64_t i = 0; i < N * E; i++) {
        lb[i] = rand_bf16(2.0);
        /* every fourth logit repeats its neighbour: ties between experts */
        if (i % 4 == 3) lb[i] = lb[i - 1];
        lf[i] = (float)bf16_to_double(lb[i]);
    }
    int32_t *idx = xalloc(N * K, sizeof(int32_t));
    double *w = xalloc(N * K, sizeof(double));
    for (int dt = 0; dt < 2; dt++)
        for (int mode = 0; mode < 2; mode++)
            for (int renorm = 0; renorm < 2; renorm++) {
                double aux = -1.0;
                oracle_route(N, E, K, dt ? (const void *)lf : (const void *)lb,
                             dt ? ORACLE_F32 : ORACLE_BF16, mode, renorm, idx, w, &aux);
                if (!(aux >= 0.0) || (N == 0 && aux != 0.0)) fail("route aux", N);
                for (int64_t t = 0; t < N; t++) {
                    double sum = 0.0;
                    for (int64_t k = 0; k < K; k++) {
                        const int32_t e = idx[t * K + k];
                        if (e < 0 || e >= E) fail("route id range", t);
                        for (int64_t j = 0; j < k; j++)
                            if (idx[t * K + j] == e) fail("route ids distinct", t);
                        if (!(w[t * K + k] > 0.0)) fail("route weight > 0", t);
                        sum += w[t * K + k];
                    }
                    const int to_one = mode == 0 || renorm || K == E;
                    if (to_one && fabs(sum - 1.0) > 1e-12) fail("route weights sum to 1", t);
                    if (!to_one && !(sum <= 1.0 + 1e-12)) fail("route weights sum <= 1", t);
                }
            }
    free(lf);
    free(lb);
    free(idx);
    free(w);
}

static void run_case(int64_t N, int64_t K, int64_t E, int64_t H, int64_t I, double p_invalid,
                     int bad_ids, uint64_t seed) {
    rng_state = seed;
    const int64_t NK = N * K, I2 = 2 * I;
    int32_t *topk = xalloc(NK, sizeof(int32_t));
    float *tw = xalloc(NK, sizeof(float));
    int64_t n_bad = 0;
    for (int64_t q = 0; q < NK; q++) {
        topk[q] = uniform() < p_invalid ? -1 : (int32_t)(next_u64() % (uint64_t)E);
        if (bad_ids && uniform() < 0.15) {
            topk[q] = uniform() < 0.5 ? (int32_t)(E + (int64_t)(next_u64() % 3))
                                      : (int32_t)(-2 - (int64_t)(next_u64() % 3));
            n_bad++;
        }
        tw[q] = (float)uniform();
    }

    /* ---- metadata */
    int32_t *freq = xalloc(E, sizeof(int32_t)), *foff = xalloc(E + 1, sizeof(int32_t));
    int32_t *xg = xalloc(NK, sizeof(int32_t)), *ss = xalloc(NK, sizeof(int32_t));
    int32_t *sr = xalloc(NK, sizeof(int32_t)), *off = xalloc(N + 1, sizeof(int32_t));
    int32_t *pt = xalloc(NK, sizeof(int32_t)), *pk = xalloc(NK, sizeof(int32_t));
    int32_t *pe = xalloc(NK, sizeof(int32_t));
    float *rs = xalloc(NK, sizeof(float));
    uint32_t flags = 0;
    const int64_t P = oracle_build_metadata(N, K, E, topk, tw, freq, foff, xg, ss, sr, off, rs,
                                            pt, pk, pe, &flags);
    if (P < 0 || P > NK || foff[0] != 0 || foff[E] != P || off[0] != 0 || off[N] != P)
        fail("metadata totals", P);
    if ((n_bad > 0) != (flags != 0)) fail("bad-id flag", n_bad);
    int64_t fsum = 0;
    for (int64_t e = 0; e < E; e++) {
        fsum += freq[e];
        if (foff[e + 1] - foff[e] != freq[e]) fail("offsets are the scan of the counts", e);
        for (int64_t s = foff[e]; s < foff[e + 1]; s++) {
            if (pe[ss[s]] != e) fail("segment holds its expert", s);
            if (s > foff[e] && ss[s] <= ss[s - 1]) fail("stable within a segment", s);
        }
    }
    if (fsum != P) fail("counts sum to P", fsum);
    for (int64_t s = 0; s < P; s++) {
        if (ss[s] < 0 || ss[s] >= P || sr[ss[s]] != s) fail("inverse permutations", s);
        else if (xg[s] != pt[ss[s]]) fail("gather index is the pair's token", s);
    }
    for (int64_t q = 0; q < P; q++)
        if (rs[q] != tw[pt[q] * K + pk[q]]) fail("router score copied", q);

    /* ---- inputs: bf16 bit patterns, and the same values in fp64 */
    uint16_t *xb = xalloc(N * H, 2), *wub = xalloc(E * H * I2, 2), *wdb = xalloc(E * I * H, 2);
    uint16_t *db = xalloc(N * H, 2);
    double *x = xalloc(N * H, 8), *wu = xalloc(E * H * I2, 8), *wd = xalloc(E * I * H, 8);
    double *dout = xalloc(N * H, 8);
    for (int64_t i = 0; i < N * H; i++) x[i] = bf16_to_double(xb[i] = rand_bf16(1.0));
    for (int64_t i = 0; i < E * H * I2; i++) wu[i] = bf16_to_double(wub[i] = rand_bf16(0.1));
    for (int64_t i = 0; i < E * I * H; i++) wd[i] = bf16_to_double(wdb[i] = rand_bf16(0.1));
    for (int64_t i = 0; i < N * H; i++) dout[i] = bf16_to_double(db[i] = rand_bf16(1.0));

    /* ---- forward, brute force, backward */
    double *h = xalloc(P * I2, 8), *a = xalloc(P * I, 8), *y = xalloc(P * H, 8);
    double *out = xalloc(N * H, 8), *out_bf = xalloc(N * H, 8);
    oracle_forward(N, H, I, E, x, wu, wd, foff, xg, sr, off, rs, h, a, y, out);
    oracle_bruteforce_forward(N, K, H, I, E, x, topk, tw, wu, wd, out_bf);
    check_close("brute force vs forward", out_bf, out, N * H);
    double *dx = xalloc(N * H, 8), *dwu = xalloc(E * H * I2, 8), *dwd = xalloc(E * I * H, 8);
    double *dtw = xalloc(NK, 8);
    oracle_backward(N, K, H, I, E, x, wu, wd, dout, foff, xg, ss, sr, off, rs, pt, pk, h, a, y,
                    dx, dwu, dwd, dtw);

    /* ---- sampled entry points (bf16 inputs) against the full ones */
    int64_t *toks = xalloc(N, sizeof(int64_t));
    for (int64_t t = 0; t < N; t++) toks[t] = t;
    double *out_s = xalloc(N * H, 8), *dx_s = xalloc(N * H, 8), *dtw_s = xalloc(NK, 8);
    oracle_sample_tokens(N, K, H, I, E, xb, ORACLE_BF16, wub, ORACLE_BF16, wdb, db, ORACLE_BF16,
                         topk, tw, N, toks, out_s, dx_s, dtw_s);
    check_close("sampled out", out_s, out, N * H);
    check_close("sampled dx", dx_s, dx, N * H);
    check_close("sampled d_topk_weights", dtw_s, dtw, NK);
    oracle_sample_tokens(N, K, H, I, E, xb, ORACLE_BF16, wub, ORACLE_BF16, wdb, NULL, ORACLE_BF16,
                         topk, tw, N, toks, out_s, NULL, NULL);
    check_close("sampled out, forward only", out_s, out, N * H);

    int64_t *rows = xalloc(P, sizeof(int64_t));
    for (int64_t s = 0; s < P; s++) rows[s] = s;
    double *h_s = xalloc(P * I2, 8);
    oracle_sample_h_rows(H, I, E, xb, ORACLE_BF16, wub, ORACLE_BF16, foff, xg, P, rows, h_s);
    check_close("sampled h rows", h_s, h, P * I2);

    const int64_t n = E * I;
    int64_t *el = xalloc(n, sizeof(int64_t)), *jl = xalloc(n, sizeof(int64_t));
    for (int64_t r = 0; r < n; r++) {
        el[r] = r / I;
        jl[r] = r % I;
    }
    double *dwd_s = xalloc(n * H, 8);
    oracle_sample_dw_down_rows(H, I, E, xb, ORACLE_BF16, wub, ORACLE_BF16, db, ORACLE_BF16, foff,
                               xg, ss, rs, n, el, jl, dwd_s);
    check_close("sampled dW_down rows", dwd_s, dwd, n * H); /* row (e,j) is dW_down[e,j,:] */
    double *cols = xalloc(n * 2 * H, 8), *cols_ref = xalloc(n * 2 * H, 8);
    oracle_sample_dw_up_cols(H, I, E, xb, ORACLE_BF16, wub, ORACLE_BF16, wdb, db, ORACLE_BF16,
                             foff, xg, ss, rs, n, el, jl, cols);
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < H; i++) {
            cols_ref[(r * 2 + 0) * H + i] = dwu[(el[r] * H + i) * I2 + 2 * jl[r]];
            cols_ref[(r * 2 + 1) * H + i] = dwu[(el[r] * H + i) * I2 + 2 * jl[r] + 1];
        }
    check_close("sampled dW_up columns", cols, cols_ref, n * 2 * H);

    if (K <= E) run_route(N, E, K);

    void *bufs[] = {topk, tw,  freq, foff, xg,    ss,     sr,    off,   pt,  pk,   pe,   rs,
                    xb,   wub, wdb,  db,   x,     wu,     wd,    dout,  h,   a,    y,    out,
                    out_bf, dx, dwu, dwd,  dtw,   toks,   out_s, dx_s,  dtw_s, rows, h_s, el,
                    jl,   dwd_s, cols, cols_ref};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; i++) free(bufs[i]);
}

int main(void) {
    /* N, K, E, H, I, share of invalid slots, ids outside [-1,E), seed */
    run_case(0, 2, 3, 8, 4, 0.0, 0, 1);    /* no rows */
    run_case(5, 2, 3, 8, 4, 1.0, 0, 2);    /* every slot invalid */
    run_case(9, 3, 4, 8, 4, 0.3, 1, 3);    /* ids outside [-1,E) */
    run_case(16, 1, 1, 16, 8, 0.0, 0, 4);  /* K = 1, E = 1 */
    run_case(23, 4, 6, 16, 8, 0.2, 0, 5);  /* repeated experts in a row, ragged segments */
    run_case(40, 8, 8, 8, 4, 0.5, 1, 6);   /* K = E */
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
