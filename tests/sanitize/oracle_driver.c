/* Runs the float64 oracle's entry points on a small packed batch (three sequences, one
 * of them empty, GVA groups of two, every gate form, chunk-start states) built with
 * AddressSanitizer and UndefinedBehaviorSanitizer, and checks two exact facts the
 * recurrence implies: beta = 0 and g = 0 leave the state unchanged, and an empty
 * sequence's final state is its initial state.  Prints "oracle driver ok". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kda_oracle_fwd(int, const int64_t *, int, int, int, int, const double *, const double *, const double *,
                   const double *, const double *, const double *, const double *, int, double, int, int, double,
                   const double *, double *, double *, const unsigned char *, int);
int kda_oracle_fwd_states(int, const int64_t *, int, int, int, int, const double *, const double *,
                          const double *, const double *, const double *, const double *, const double *, int,
                          double, int, int, double, const double *, double *, double *, int, const int64_t *,
                          double *, int);
int kda_oracle_gate_cumsum(int, const int64_t *, int, int, int, const double *, const double *, const double *, int,
                           double, double *, double *);

static double rnd(unsigned *s) { *s = *s * 1103515245u + 12345u; return ((*s >> 8) & 0xffff) / 32768.0 - 1.0; }

int main(void) {
    enum { N = 3, H = 2, HV = 4, K = 8, V = 6, T = 37, C = 8 };
    const int64_t starts[N + 1] = {0, 21, 21, T};
    const int64_t chunk_first[N] = {0, 3, 3};   /* ceil(21/8) = 3, 0, ceil(16/8) = 2 -> 5 chunks */
    unsigned s = 7;
    double *q = malloc(sizeof(double) * T * H * K), *k = malloc(sizeof(double) * T * H * K);
    double *v = malloc(sizeof(double) * T * HV * V), *g = malloc(sizeof(double) * T * HV * K);
    double *beta = malloc(sizeof(double) * T * HV), *o = malloc(sizeof(double) * T * HV * V);
    double *h0 = malloc(sizeof(double) * N * HV * K * V), *ht = malloc(sizeof(double) * N * HV * K * V);
    double *st = malloc(sizeof(double) * 5 * HV * K * V);
    double *ga = malloc(sizeof(double) * T * HV * K), *gc = malloc(sizeof(double) * T * HV * K);
    double A_log[HV], dt[HV * K];
    for (int i = 0; i < T * H * K; ++i) { q[i] = rnd(&s); k[i] = rnd(&s); }
    for (int i = 0; i < T * HV * V; ++i) v[i] = rnd(&s);
    for (int i = 0; i < T * HV * K; ++i) g[i] = rnd(&s);
    for (int i = 0; i < T * HV; ++i) beta[i] = rnd(&s);
    for (int i = 0; i < N * HV * K * V; ++i) h0[i] = rnd(&s);
    for (int i = 0; i < HV; ++i) A_log[i] = 0.3 * rnd(&s);
    for (int i = 0; i < HV * K; ++i) dt[i] = 0.5 * rnd(&s);
    int bad = 0;
    for (int mode = 0; mode < 3; ++mode) {
        double *gg = g;
        double *neg = NULL;
        if (mode == 0) { /* pre-gated: must be a decay */
            neg = malloc(sizeof(double) * T * HV * K);
            for (int i = 0; i < T * HV * K; ++i) neg[i] = -fabs(g[i]);
            gg = neg;
        }
        if (kda_oracle_fwd(N, starts, H, HV, K, V, q, k, v, gg, beta, A_log, dt, mode, -3.0, 1, 2, 0.35, h0, o, ht,
                           NULL, 2) < 1) bad++;
        if (kda_oracle_fwd_states(N, starts, H, HV, K, V, q, k, v, gg, beta, A_log, dt, mode, -3.0, 1, 1, 0.35, h0,
                                  o, ht, C, chunk_first, st, 2) < 1) bad++;
        if (kda_oracle_gate_cumsum(N, starts, HV, K, C, gg, A_log, dt, mode, -3.0, ga, gc) != 0) bad++;
        for (int i = 0; i < HV * K * V; ++i) /* the empty sequence keeps its state */
            if (ht[1 * HV * K * V + i] != h0[1 * HV * K * V + i]) { bad++; break; }
        free(neg);
    }
    /* beta = 0, g = 0: the state never changes */
    for (int i = 0; i < T * HV; ++i) beta[i] = 0.0;
    for (int i = 0; i < T * HV * K; ++i) g[i] = 0.0;
    kda_oracle_fwd(N, starts, H, HV, K, V, q, k, v, g, beta, NULL, NULL, 0, 0.0, 0, 0, 1.0, h0, o, ht, NULL, 1);
    for (int i = 0; i < N * HV * K * V; ++i)
        if (ht[i] != h0[i]) { bad++; break; }
    free(q); free(k); free(v); free(g); free(beta); free(o); free(h0); free(ht); free(st); free(ga); free(gc);
    if (bad == 0) printf("oracle driver ok\n");
    return bad == 0 ? 0 : 1;
}
