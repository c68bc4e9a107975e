/*
 * oracle_driver.c -- exercises every function of the fp64 oracle
 * (oracle/kda_oracle.c) on small exact-size heap buffers, for a host build
 * under AddressSanitizer and UndefinedBehaviorSanitizer: ragged and empty
 * packed sequences, conv widths 1..4, conv history in / out (also in place),
 * bias, with and without initial states, the correction dropped, head dims
 * that differ, special values for the bf16 rounding, and rejected arguments.
 * Exits 0 and prints "ok" when every call returns what it should; any memory
 * error or undefined behaviour aborts the run under the sanitizers.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_short_conv(const double *x, int64_t total_tokens, int64_t C, const double *w, int W,
                          const double *bias, const int32_t *cu_seqlens, int N,
                          const double *state_in, double *state_out, int silu, double *y);
void kda_oracle_bounded_gate(const double *z, int64_t T, int H, int D, const double *a_log,
                             const double *dt_bias, double lower_bound, double *g);
void kda_oracle_output_norm_gate(const double *o, const double *gate, int64_t T, int H, int D,
                                 const double *w, double eps, double *y);
void kda_oracle_l2norm(double *x, int64_t rows, int64_t D, double eps);
void kda_oracle_round_bf16(double *x, int64_t n);
int kda_oracle_recurrent(const double *q, const double *k, const double *v, const double *g,
                         const double *beta, const int32_t *cu_seqlens, int N,
                         int64_t total_tokens, int H, int DK, int DV, double scale,
                         const double *h0, double *o, double *hT, int delta_rule);
int kda_oracle_num_threads(void);

static uint64_t g_seed = 0x9E3779B97F4A7C15ull;
static double rnd(void) {   /* xorshift64*, uniform in [-1, 1) */
    g_seed ^= g_seed >> 12;
    g_seed ^= g_seed << 25;
    g_seed ^= g_seed >> 27;
    return (double)((g_seed * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}
static double *alloc(int64_t n) {   /* exact size; at least one element so malloc(0) is avoided */
    double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}
static int failures = 0;
static void expect(int cond, const char *what) {
    if (!cond) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}
static int all_finite(const double *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

int main(void) {
    const int32_t cu[] = {0, 0, 1, 4, 21, 21, 26};   /* lengths 0, 1, 3, 17, 0, 5 */
    const int N = 6;
    const int64_t T = 26;
    const int H = 2, D = 8, C = H * D;

    /* O1a: every width, with and without bias, history, SiLU; history in place */
    for (int W = 1; W <= 4; ++W) {
        for (int variant = 0; variant < 4; ++variant) {
            double *x = alloc(T * C), *w = alloc((int64_t)C * W), *b = alloc(C);
            double *y = alloc(T * C);
            double *st = alloc((int64_t)N * (W - 1) * C), *so = alloc((int64_t)N * (W - 1) * C);
            const int use_state = variant & 1, in_place = variant & 2;
            const int rc = kda_oracle_short_conv(x, T, C, w, W, variant ? b : NULL, cu, N,
                                                 use_state ? st : NULL, in_place ? st : so,
                                                 variant != 3, y);
            expect(rc == 0 && all_finite(y, T * C), "short_conv");
            free(x); free(w); free(b); free(y); free(st); free(so);
        }
    }
    {   /* rejected: NULL input, bad offsets, W = 0 */
        double *x = alloc(T * C), *w = alloc((int64_t)C * 4), *y = alloc(T * C);
        const int32_t bad[] = {0, 5, 3, 26, 26, 26, 26};
        expect(kda_oracle_short_conv(NULL, T, C, w, 4, NULL, cu, N, NULL, NULL, 1, y) != 0,
               "short_conv NULL x");
        expect(kda_oracle_short_conv(x, T, C, w, 4, NULL, bad, N, NULL, NULL, 1, y) != 0,
               "short_conv decreasing offsets");
        expect(kda_oracle_short_conv(x, T, C, w, 0, NULL, cu, N, NULL, NULL, 1, y) != 0,
               "short_conv width 0");
        expect(kda_oracle_short_conv(x, T, C, w, 4, NULL, cu, N, NULL, NULL, 1, y) == 0 &&
                   kda_oracle_short_conv(x, 0, C, w, 4, NULL, (const int32_t[]){0, 0}, 1, NULL,
                                         NULL, 1, y) == 0,
               "short_conv empty batch");
        free(x); free(w); free(y);
    }

    /* O1b, O1c */
    {
        double *x = alloc(T * C);
        kda_oracle_l2norm(x, T * H, D, 1e-6);
        expect(all_finite(x, T * C), "l2norm");
        kda_oracle_l2norm(x, 0, D, 1e-6);
        double sp[] = {0.0, -0.0, INFINITY, -INFINITY, NAN, 1.0, 1.00390625, 1.005859375,
                       -3.0e38, 1.2e-38, 65504.0, 0.1};
        kda_oracle_round_bf16(sp, (int64_t)(sizeof(sp) / sizeof(sp[0])));
        expect(sp[0] == 0.0 && isinf(sp[2]) && isnan(sp[4]) && sp[5] == 1.0 && sp[6] == 1.0 &&
                   sp[7] == 1.0078125,
               "round_bf16 special values and ties to even");
        kda_oracle_round_bf16(x, T * C);
        free(x);
    }

    /* O0, O3 */
    {
        double *z = alloc(T * C), *al = alloc(H), *dt = alloc(C), *g = alloc(T * C);
        kda_oracle_bounded_gate(z, T, H, D, al, dt, -5.0, g);
        int ok = 1;
        for (int64_t i = 0; i < T * C; ++i) ok &= g[i] <= 0.0 && g[i] >= -5.0;
        kda_oracle_bounded_gate(z, T, H, D, NULL, NULL, -8.0, g);
        for (int64_t i = 0; i < T * C; ++i) ok &= g[i] <= 0.0 && g[i] >= -8.0;
        expect(ok, "bounded_gate range");
        double *o = alloc(T * C), *gate = alloc(T * C), *w = alloc(D), *y = alloc(T * C);
        kda_oracle_output_norm_gate(o, gate, T, H, D, w, 1e-6, y);
        expect(all_finite(y, T * C), "output_norm_gate");
        memset(o, 0, sizeof(double) * (size_t)(T * C));
        kda_oracle_output_norm_gate(o, gate, T, H, D, NULL, 0.0, y);   /* 0 / sqrt(0): NaN */
        kda_oracle_output_norm_gate(o, gate, 0, H, D, NULL, 1e-6, y);
        free(z); free(al); free(dt); free(g); free(o); free(gate); free(w); free(y);
    }

    /* O2: key and value dims differ, with and without h0 / hT, correction on and off */
    for (int variant = 0; variant < 4; ++variant) {
        const int DK = 8, DV = 4;
        double *q = alloc(T * H * DK), *k = alloc(T * H * DK), *v = alloc(T * H * DV);
        double *g = alloc(T * H * DK), *beta = alloc(T * H), *h0 = alloc((int64_t)N * H * DK * DV);
        double *o = alloc(T * H * DV), *hT = alloc((int64_t)N * H * DK * DV);
        for (int64_t i = 0; i < T * H * DK; ++i) g[i] = -fabs(g[i]);
        for (int64_t i = 0; i < T * H; ++i) beta[i] = 0.5 * (beta[i] + 1.0);
        const int rc = kda_oracle_recurrent(q, k, v, g, beta, cu, N, T, H, DK, DV, 0.35,
                                            (variant & 1) ? h0 : NULL, o,
                                            (variant & 2) ? hT : NULL, variant != 2);
        expect(rc == 0 && all_finite(o, T * H * DV), "recurrent");
        expect(kda_oracle_recurrent(q, k, v, g, beta, cu, N, T, H, 0, DV, 1.0, NULL, o, NULL, 1) != 0,
               "recurrent DK = 0");
        expect(kda_oracle_recurrent(q, k, v, g, beta, NULL, N, T, H, DK, DV, 1.0, NULL, o, NULL,
                                    1) != 0,
               "recurrent NULL offsets");
        free(q); free(k); free(v); free(g); free(beta); free(h0); free(o); free(hT);
    }
    expect(kda_oracle_num_threads() >= 1, "num_threads");

    if (failures) return 1;
    printf("ok\n");
    return 0;
}
