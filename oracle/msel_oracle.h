/*
 * msel_oracle.h -- declarations of the fp64 CPU oracle (TEST INFRASTRUCTURE ONLY).
 *
 * Used only by the tests, the smoke check and the benchmark's CPU-baseline leg, through
 * ctypes.  Shares nothing with the library headers under include/.
 *
 * Layouts (all double, row-major, contiguous):
 *   u, delta, z, out, dout, du, ddelta, dz : [batch, dim, seqlen]
 *   B, C, dB, dC                           : [batch, dstate, seqlen]
 *   A, dA                                  : [dim, dstate]
 *   D, bias, dD, dbias                     : [dim]
 *   h0, final_state, dh0                   : [batch, dim, dstate]
 *   chunk_states                           : [batch, dim, ceil(seqlen/chunk_len), dstate]
 * Nullable inputs: D, z, bias, h0 (treated as absent / zero).
 * Return value: 0 on success, negative on bad arguments or allocation failure.
 */
#ifndef MSEL_ORACLE_H
#define MSEL_ORACLE_H

typedef struct {
    long batch, dim, dstate, seqlen;
    int softplus;
    const double *u, *delta, *A, *B, *C, *D, *z, *bias, *h0;
} oracle_in;

int oracle_fwd(const oracle_in *in, double *out, double *final_state, long chunk_len,
               double *chunk_states, int nthreads);

int oracle_chunk_states_formula(const oracle_in *in, long chunk_len, double *chunk_states,
                                double *final_state, int nthreads);

int oracle_bwd(const oracle_in *in, const double *dout, double *du, double *ddelta, double *dz,
               double *dA, double *dB, double *dC, double *dD, double *dbias, double *dh0,
               int nthreads);

#endif
