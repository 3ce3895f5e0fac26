/*
 * msel_oracle.c -- plain, slow, sequential fp64 CPU oracle of the selective SSM scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link, load or call
 * this file: only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code, header, table or constant with the HIP kernels.
 *
 * What it computes (sources are the five web pages collected on "mamba paper"):
 *  - Selection: the step size Delta and the matrices B and C are functions of the input, one
 *    value per token, so the model can keep or forget state depending on the current token
 *    (page 1 abstract paragraph on letting the SSM parameters be functions of the input;
 *    page 2 and page 3 repeat it).
 *  - Discretization: the continuous system is discretized with a combination of zero-order
 *    hold and Euler (page 5, Mamba-3 post, bullet on the new discretization scheme).  Reading:
 *    zero-order hold for the transition, dA = exp(Delta*A); Euler for the input,
 *    dB*x = Delta*B*x.
 *  - Recurrent mode: inputs are consumed one time step at a time (page 3, "recurrent mode"
 *    sentence; page 1 "scan: recurrent operation").  h_t = dA_t*h_{t-1} + dB_t*x_t and the
 *    readout y_t = C_t.h_t + D*x_t, then the gate y*silu(z).
 *  - Chunking: a sequence too long for on-chip memory is split into chunks and the scan
 *    continues from the intermediate state of the previous chunk (page 4, Appendix D
 *    "Hardware-aware Algorithm For Selective SSMs", Speed paragraph).
 *  - Backward with recomputation: the intermediate states are not stored but recomputed in
 *    the backward pass (page 1; page 4 Appendix D, Memory paragraph).  The gradient formulas
 *    below are derived by hand from the forward recurrence with the chain rule.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - Delta = softplus(delta + bias[d]) when the softplus flag is set, else delta + bias[d];
 *    softplus(x) = max(x,0) + log1p(exp(-|x|)).
 *  - out = (sum_n C*h + D*u) * silu(z), silu(z) = z/(1+exp(-z)); without z, out = y.
 *  - B and C are shared by all channels d of a batch row and laid out [batch, dstate, seqlen].
 *  - u, delta, z, out are [batch, dim, seqlen]; A is [dim, dstate]; D, bias are [dim].
 *  - The initial state is h0 when given, else 0.  No gradient flows into the final state.
 *  - The chunk state H_c is the state before time step c*T (H_0 = h0).
 *
 * Everything is double precision, with libm exp/log1p and no fast-math; the build passes
 * -ffp-contract=off so that no multiply-add is fused.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#include "msel_oracle.h"

static double softplus_d(double x) {
    double ax = x < 0 ? -x : x;
    return (x > 0 ? x : 0.0) + log1p(exp(-ax));
}

static double sigmoid_d(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Delta for (b, d, t) before and after the optional softplus. */
static double delta_of(const oracle_in *in, long b, long d, long t, double *pre) {
    long L = in->seqlen;
    double x = in->delta[(b * in->dim + d) * L + t] + (in->bias ? in->bias[d] : 0.0);
    if (pre) *pre = x;
    return in->softplus ? softplus_d(x) : x;
}

/* ---------------------------------------------------------------------------------------- */
/* A tiny static thread pool: work units 0..n_units-1 are split into contiguous ranges.      */

typedef void (*unit_fn)(void *ctx, long unit, int tid);

typedef struct {
    unit_fn fn;
    void *ctx;
    long begin, end;
    int tid;
} range_job;

static void *run_range(void *p) {
    range_job *j = (range_job *)p;
    for (long u = j->begin; u < j->end; ++u) j->fn(j->ctx, u, j->tid);
    return NULL;
}

static int parallel_for(long n_units, int nthreads, unit_fn fn, void *ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n_units) nthreads = (int)(n_units > 0 ? n_units : 1);
    pthread_t th[256];
    range_job jobs[256];
    if (nthreads > 256) nthreads = 256;
    long per = n_units / nthreads, rem = n_units % nthreads, at = 0;
    for (int i = 0; i < nthreads; ++i) {
        long cnt = per + (i < rem ? 1 : 0);
        jobs[i].fn = fn;
        jobs[i].ctx = ctx;
        jobs[i].begin = at;
        jobs[i].end = at + cnt;
        jobs[i].tid = i;
        at += cnt;
    }
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, run_range, &jobs[i]) != 0) return -1;
    run_range(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    return nthreads;
}

/* ---------------------------------------------------------------------------------------- */
/* Forward: the recurrent mode, one time step at a time, per (b, d).                         */

typedef struct {
    const oracle_in *in;
    double *out, *final_state, *chunk_states;
    long chunk_len;
} fwd_ctx;

static void fwd_unit(void *p, long unit, int tid) {
    (void)tid;
    fwd_ctx *c = (fwd_ctx *)p;
    const oracle_in *in = c->in;
    long Dm = in->dim, N = in->dstate, L = in->seqlen;
    long b = unit / Dm, d = unit % Dm;
    long n_chunks = c->chunk_states ? (L + c->chunk_len - 1) / c->chunk_len : 0;
    double *h = (double *)malloc(sizeof(double) * (size_t)N);
    for (long n = 0; n < N; ++n) h[n] = in->h0 ? in->h0[(b * Dm + d) * N + n] : 0.0;
    const double *A = in->A + d * N;
    for (long t = 0; t < L; ++t) {
        if (c->chunk_states && t % c->chunk_len == 0) {
            double *dst = c->chunk_states + ((b * Dm + d) * n_chunks + t / c->chunk_len) * N;
            for (long n = 0; n < N; ++n) dst[n] = h[n];
        }
        double dt = delta_of(in, b, d, t, NULL);
        double x = in->u[(b * Dm + d) * L + t];
        double y = 0.0;
        for (long n = 0; n < N; ++n) {
            double Bv = in->B[(b * N + n) * L + t];
            double Cv = in->C[(b * N + n) * L + t];
            double dA = exp(dt * A[n]);           /* zero-order hold for the transition */
            double dBx = dt * Bv * x;             /* Euler for the input                */
            h[n] = dA * h[n] + dBx;
            y += Cv * h[n];
        }
        if (in->D) y += in->D[d] * x;
        if (in->z) {
            double zz = in->z[(b * Dm + d) * L + t];
            y = y * (zz * sigmoid_d(zz));
        }
        c->out[(b * Dm + d) * L + t] = y;
    }
    if (c->final_state)
        for (long n = 0; n < N; ++n) c->final_state[(b * Dm + d) * N + n] = h[n];
    free(h);
}

int oracle_fwd(const oracle_in *in, double *out, double *final_state, long chunk_len,
               double *chunk_states, int nthreads) {
    if (!in || !out || !in->u || !in->delta || !in->A || !in->B || !in->C) return -1;
    if (in->batch <= 0 || in->dim <= 0 || in->dstate <= 0 || in->seqlen <= 0) return -2;
    if (chunk_states && chunk_len <= 0) return -2;
    fwd_ctx c = {in, out, final_state, chunk_states, chunk_len};
    return parallel_for(in->batch * in->dim, nthreads, fwd_unit, &c) > 0 ? 0 : -3;
}

/* ---------------------------------------------------------------------------------------- */
/* Chunk states by the chunk formula (page 4 Appendix D, Speed): for every chunk c the local */
/* scan from a zero state gives S_c, the transition over the chunk is                         */
/* P_c = exp(A * sum of Delta over the chunk), and the chunks are linked by                   */
/* H_{c+1} = P_c * H_c + S_c with H_0 = h0.                                                  */

typedef struct {
    const oracle_in *in;
    long chunk_len;
    double *chunk_states, *final_state;
} cc_ctx;

static void cc_unit(void *p, long unit, int tid) {
    (void)tid;
    cc_ctx *c = (cc_ctx *)p;
    const oracle_in *in = c->in;
    long Dm = in->dim, N = in->dstate, L = in->seqlen, T = c->chunk_len;
    long b = unit / Dm, d = unit % Dm;
    long n_chunks = (L + T - 1) / T;
    const double *A = in->A + d * N;
    double *S = (double *)malloc(sizeof(double) * (size_t)N);
    double *H = (double *)malloc(sizeof(double) * (size_t)N);
    for (long n = 0; n < N; ++n) H[n] = in->h0 ? in->h0[(b * Dm + d) * N + n] : 0.0;
    for (long ck = 0; ck < n_chunks; ++ck) {
        if (c->chunk_states) {
            double *dst = c->chunk_states + ((b * Dm + d) * n_chunks + ck) * N;
            for (long n = 0; n < N; ++n) dst[n] = H[n];
        }
        long t0 = ck * T, t1 = t0 + T < L ? t0 + T : L;
        double sum_dt = 0.0;
        for (long n = 0; n < N; ++n) S[n] = 0.0;
        for (long t = t0; t < t1; ++t) {
            double dt = delta_of(in, b, d, t, NULL);
            double x = in->u[(b * Dm + d) * L + t];
            sum_dt += dt;
            for (long n = 0; n < N; ++n) {
                double Bv = in->B[(b * N + n) * L + t];
                S[n] = exp(dt * A[n]) * S[n] + dt * Bv * x;
            }
        }
        for (long n = 0; n < N; ++n) H[n] = exp(A[n] * sum_dt) * H[n] + S[n];
    }
    if (c->final_state)
        for (long n = 0; n < N; ++n) c->final_state[(b * Dm + d) * N + n] = H[n];
    free(S);
    free(H);
}

int oracle_chunk_states_formula(const oracle_in *in, long chunk_len, double *chunk_states,
                                double *final_state, int nthreads) {
    if (!in || !in->u || !in->delta || !in->A || !in->B) return -1;
    if (in->batch <= 0 || in->dim <= 0 || in->dstate <= 0 || in->seqlen <= 0) return -2;
    if (chunk_len <= 0) return -2;
    cc_ctx c = {in, chunk_len, chunk_states, final_state};
    return parallel_for(in->batch * in->dim, nthreads, cc_unit, &c) > 0 ? 0 : -3;
}

/* ---------------------------------------------------------------------------------------- */
/* Backward.  With a_t = exp(Delta_t A_n), p_t = Delta_t B_t u_t, y the pre-gate readout:    */
/*   dy_t  = dout_t * silu(z_t)                 (dout_t without z)                          */
/*   dz_t  = dout_t * y_t * s (1 + z (1 - s)),  s = sigmoid(z_t)                             */
/*   lam_t = C_t dy_t + a_{t+1} lam_{t+1},      lam beyond the last step is 0                */
/*   dC_t += dy_t h_t ;  dB_t += lam_t Delta_t u_t ;  du_t += lam_t Delta_t B_t + dy_t D     */
/*   g_t   = lam_t h_{t-1} a_t ;  dA += g_t Delta_t ;  dDelta_t += g_t A + lam_t B_t u_t      */
/*   ddelta_t = dDelta_t * sigmoid(delta_t + bias) (softplus) or dDelta_t ; dbias += ddelta */
/*   dD += dy_t u_t ;  dh0 = a_0 lam_0                                                       */
/* The intermediate states are recomputed here from the inputs, as the backward pass on the  */
/* pages does.                                                                               */

typedef struct {
    const oracle_in *in;
    const double *dout;
    double *du, *ddelta, *dz;
    double *dA_part, *dD_part, *dbias_part; /* [batch, dim, (dstate)] partials */
    double *dB_thr, *dC_thr;                /* [nthreads, batch, dstate, seqlen] */
    double *dh0;
} bwd_ctx;

static void bwd_unit(void *p, long unit, int tid) {
    bwd_ctx *c = (bwd_ctx *)p;
    const oracle_in *in = c->in;
    long Bt = in->batch, Dm = in->dim, N = in->dstate, L = in->seqlen;
    long b = unit / Dm, d = unit % Dm;
    const double *A = in->A + d * N;
    size_t bnl = (size_t)(Bt * N * L);
    double *dB = c->dB_thr ? c->dB_thr + (size_t)tid * bnl : NULL;
    double *dC = c->dC_thr ? c->dC_thr + (size_t)tid * bnl : NULL;

    /* recompute the forward pass, keeping every state h_t (row t+1; row 0 is h0) */
    double *hs = (double *)malloc(sizeof(double) * (size_t)((L + 1) * N));
    double *dts = (double *)malloc(sizeof(double) * (size_t)L);
    double *pres = (double *)malloc(sizeof(double) * (size_t)L);
    double *ys = (double *)malloc(sizeof(double) * (size_t)L);
    double *lam_next = (double *)malloc(sizeof(double) * (size_t)N); /* a_{t+1} lam_{t+1} */
    for (long n = 0; n < N; ++n) hs[n] = in->h0 ? in->h0[(b * Dm + d) * N + n] : 0.0;
    for (long t = 0; t < L; ++t) {
        double dt = delta_of(in, b, d, t, &pres[t]);
        double x = in->u[(b * Dm + d) * L + t];
        double y = 0.0;
        dts[t] = dt;
        for (long n = 0; n < N; ++n) {
            double hprev = hs[t * N + n];
            double hn = exp(dt * A[n]) * hprev + dt * in->B[(b * N + n) * L + t] * x;
            hs[(t + 1) * N + n] = hn;
            y += in->C[(b * N + n) * L + t] * hn;
        }
        if (in->D) y += in->D[d] * x;
        ys[t] = y;
    }

    for (long n = 0; n < N; ++n) lam_next[n] = 0.0;
    double dA_acc[4096];
    double *dAp = N <= 4096 ? dA_acc : (double *)malloc(sizeof(double) * (size_t)N);
    for (long n = 0; n < N; ++n) dAp[n] = 0.0;
    double dD_acc = 0.0, dbias_acc = 0.0;
    for (long t = L - 1; t >= 0; --t) {
        long it = (b * Dm + d) * L + t;
        double g_out = c->dout[it];
        double x = in->u[it];
        double dt = dts[t];
        double dy;
        if (in->z) {
            double zz = in->z[it];
            double s = sigmoid_d(zz);
            dy = g_out * zz * s;
            if (c->dz) c->dz[it] = g_out * ys[t] * s * (1.0 + zz * (1.0 - s));
        } else {
            dy = g_out;
        }
        double du = in->D ? dy * in->D[d] : 0.0;
        dD_acc += dy * x;
        double dDelta = 0.0;
        for (long n = 0; n < N; ++n) {
            long ib = (b * N + n) * L + t;
            double Bv = in->B[ib], Cv = in->C[ib];
            double lam = Cv * dy + lam_next[n];
            double h = hs[(t + 1) * N + n];
            double hprev = hs[t * N + n];
            double a = exp(dt * A[n]);
            double g = lam * hprev * a;
            if (dC) dC[ib] += dy * h;
            if (dB) dB[ib] += lam * dt * x;
            dAp[n] += g * dt;
            dDelta += g * A[n] + lam * Bv * x;
            du += lam * dt * Bv;
            lam_next[n] = a * lam;
        }
        double dd = in->softplus ? dDelta * sigmoid_d(pres[t]) : dDelta;
        if (c->du) c->du[it] = du;
        if (c->ddelta) c->ddelta[it] = dd;
        dbias_acc += dd;
    }
    if (c->dh0)
        for (long n = 0; n < N; ++n) c->dh0[(b * Dm + d) * N + n] = lam_next[n];
    for (long n = 0; n < N; ++n) c->dA_part[(b * Dm + d) * N + n] = dAp[n];
    c->dD_part[b * Dm + d] = dD_acc;
    c->dbias_part[b * Dm + d] = dbias_acc;
    if (dAp != dA_acc) free(dAp);
    free(hs);
    free(dts);
    free(pres);
    free(ys);
    free(lam_next);
}

int oracle_bwd(const oracle_in *in, const double *dout, double *du, double *ddelta, double *dz,
               double *dA, double *dB, double *dC, double *dD, double *dbias, double *dh0,
               int nthreads) {
    if (!in || !dout || !in->u || !in->delta || !in->A || !in->B || !in->C) return -1;
    if (in->batch <= 0 || in->dim <= 0 || in->dstate <= 0 || in->seqlen <= 0) return -2;
    long Bt = in->batch, Dm = in->dim, N = in->dstate, L = in->seqlen;
    long units = Bt * Dm;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)units;
    if (nthreads > 256) nthreads = 256;
    size_t bnl = (size_t)(Bt * N * L);
    bwd_ctx c;
    memset(&c, 0, sizeof c);
    c.in = in;
    c.dout = dout;
    c.du = du;
    c.ddelta = ddelta;
    c.dz = in->z ? dz : NULL;
    c.dh0 = dh0;
    c.dA_part = (double *)calloc((size_t)(units * N), sizeof(double));
    c.dD_part = (double *)calloc((size_t)units, sizeof(double));
    c.dbias_part = (double *)calloc((size_t)units, sizeof(double));
    c.dB_thr = dB ? (double *)calloc(bnl * (size_t)nthreads, sizeof(double)) : NULL;
    c.dC_thr = dC ? (double *)calloc(bnl * (size_t)nthreads, sizeof(double)) : NULL;
    if (!c.dA_part || !c.dD_part || !c.dbias_part || (dB && !c.dB_thr) || (dC && !c.dC_thr))
        return -4;
    int used = parallel_for(units, nthreads, bwd_unit, &c);
    int rc = used > 0 ? 0 : -3;
    /* fixed-order reductions: over threads for dB/dC, over batch for dA/dD/dbias */
    if (rc == 0 && dB)
        for (size_t i = 0; i < bnl; ++i) {
            double s = 0.0;
            for (int k = 0; k < used; ++k) s += c.dB_thr[(size_t)k * bnl + i];
            dB[i] = s;
        }
    if (rc == 0 && dC)
        for (size_t i = 0; i < bnl; ++i) {
            double s = 0.0;
            for (int k = 0; k < used; ++k) s += c.dC_thr[(size_t)k * bnl + i];
            dC[i] = s;
        }
    if (rc == 0) {
        for (long d = 0; d < Dm; ++d) {
            double sD = 0.0, sb = 0.0;
            for (long b = 0; b < Bt; ++b) {
                sD += c.dD_part[b * Dm + d];
                sb += c.dbias_part[b * Dm + d];
            }
            if (dD) dD[d] = sD;
            if (dbias) dbias[d] = sb;
            for (long n = 0; n < N; ++n) {
                double s = 0.0;
                for (long b = 0; b < Bt; ++b) s += c.dA_part[(b * Dm + d) * N + n];
                if (dA) dA[d * N + n] = s;
            }
        }
    }
    free(c.dA_part);
    free(c.dD_part);
    free(c.dbias_part);
    free(c.dB_thr);
    free(c.dC_thr);
    return rc;
}
