/*
 * The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Built by tests/test_sanitizers.py together with oracle/msel_oracle.c (gcc, no GPU): runs
 * the forward (with chunk states), the chunk-state formula and the backward on a small
 * problem with every optional input, a ragged last chunk and several threads, then on one
 * without any optional input, and checks that the two ways of forming chunk states agree and
 * that every result is finite.  The sanitizers abort on the first error they find.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "msel_oracle.h"

static unsigned long long state = 88172645463325252ull;

/* xorshift64*, mapped to (-1, 1): deterministic inputs without any library generator */
static double rnd(void) {
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    unsigned long long r = state * 2685821657736338717ull;
    return (double)(r >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double *fill(long n, double scale, double shift) {
    double *p = (double *)malloc((size_t)n * sizeof(double));
    for (long i = 0; i < n; ++i) p[i] = shift + scale * rnd();
    return p;
}

static int all_finite(const double *p, long n) {
    for (long i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static int run(long bsz, long dim, long N, long L, long T, int optional, int threads) {
    long tc = bsz * dim * L, bnl = bsz * N * L, nch = (L + T - 1) / T;
    oracle_in in;
    in.batch = bsz;
    in.dim = dim;
    in.dstate = N;
    in.seqlen = L;
    in.softplus = optional;
    double *u = fill(tc, 1.0, 0.0), *delta = fill(tc, 0.5, 0.0), *B = fill(bnl, 1.0, 0.0);
    double *C = fill(bnl, 1.0, 0.0), *A = fill(dim * N, 0.5, -1.5);
    double *D = optional ? fill(dim, 1.0, 0.0) : NULL, *z = optional ? fill(tc, 1.0, 0.0) : NULL;
    double *bias = optional ? fill(dim, 1.0, -4.0) : NULL;
    double *h0 = optional ? fill(bsz * dim * N, 1.0, 0.0) : NULL;
    if (!optional)
        for (long i = 0; i < tc; ++i) delta[i] = fabs(delta[i]) * 0.2;  /* a positive step */
    in.u = u;
    in.delta = delta;
    in.A = A;
    in.B = B;
    in.C = C;
    in.D = D;
    in.z = z;
    in.bias = bias;
    in.h0 = h0;
    double *out = malloc(tc * sizeof(double)), *fin = malloc(bsz * dim * N * sizeof(double));
    double *cs = malloc(bsz * dim * nch * N * sizeof(double));
    double *cs2 = malloc(bsz * dim * nch * N * sizeof(double));
    double *fin2 = malloc(bsz * dim * N * sizeof(double));
    int bad = 0;
    bad |= oracle_fwd(&in, out, fin, T, cs, threads) != 0;
    bad |= oracle_chunk_states_formula(&in, T, cs2, fin2, threads) != 0;
    double *dout = fill(tc, 1.0, 0.0);
    double *du = malloc(tc * sizeof(double)), *ddelta = malloc(tc * sizeof(double));
    double *dz = optional ? malloc(tc * sizeof(double)) : NULL;
    double *dA = malloc(dim * N * sizeof(double)), *dB = malloc(bnl * sizeof(double));
    double *dC = malloc(bnl * sizeof(double)), *dD = malloc(dim * sizeof(double));
    double *dbias = malloc(dim * sizeof(double)), *dh0 = malloc(bsz * dim * N * sizeof(double));
    bad |= oracle_bwd(&in, dout, du, ddelta, dz, dA, dB, dC, dD, dbias, dh0, threads) != 0;
    double worst = 0.0, scale = 0.0;
    for (long i = 0; i < bsz * dim * nch * N; ++i) {
        double e = fabs(cs[i] - cs2[i]);
        if (e > worst) worst = e;
        if (fabs(cs[i]) > scale) scale = fabs(cs[i]);
    }
    bad |= worst > 1e-12 * (scale > 1.0 ? scale : 1.0);
    bad |= !all_finite(out, tc) || !all_finite(du, tc) || !all_finite(ddelta, tc) ||
           !all_finite(dA, dim * N) || !all_finite(dB, bnl) || !all_finite(dC, bnl);
    if (bad) fprintf(stderr, "oracle run %ldx%ldx%ldx%ld failed (chunk-state gap %g)\n", bsz,
                     dim, N, L, worst);
    free(u); free(delta); free(B); free(C); free(A); free(D); free(z); free(bias); free(h0);
    free(out); free(fin); free(cs); free(cs2); free(fin2); free(dout); free(du); free(ddelta);
    free(dz); free(dA); free(dB); free(dC); free(dD); free(dbias); free(dh0);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= run(2, 5, 7, 1100, 512, 1, 3);  /* every optional input, ragged last chunk */
    bad |= run(1, 3, 16, 64, 7, 0, 2);     /* none of them, chunks of 7 steps */
    bad |= run(1, 1, 1, 1, 1, 1, 1);       /* one step, one channel, one state */
    if (bad) return 1;
    printf("oracle_driver: all runs passed\n");
    return 0;
}
