/*
 * Host-side argument checks of libmsel under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Built by tests/test_sanitizers.py against a host-only, sanitizer-instrumented build of the
 * library's sources (no GPU code, no GPU needed): every msel_validate_* check is run on valid
 * arguments and on each kind of invalid one, and the entry points are called with invalid
 * arguments, on which they return before any HIP call.  Device pointers are fake addresses
 * that nothing dereferences.  Exit status 0 when every expectation holds; the sanitizers abort
 * on the first error they find.
 */
#include <stdio.h>
#include <string.h>

#include "msel.h"

static int failures = 0;
static uintptr_t next_addr = 0x10000000u;

static void *fake(void) {
    void *p = (void *)next_addr;
    next_addr += 0x100000u;
    return p;
}

#define EXPECT(expr, want)                                                               \
    do {                                                                                 \
        int got_ = (int)(expr);                                                          \
        if (got_ != (int)(want)) {                                                       \
            fprintf(stderr, "%s:%d: %s = %d, expected %d\n", __FILE__, __LINE__, #expr,   \
                    got_, (int)(want));                                                  \
            ++failures;                                                                  \
        }                                                                                \
    } while (0)

static msel_scan_args good_args(int batch, int dim, int N, int L) {
    msel_scan_args a;
    memset(&a, 0, sizeof a);
    a.abi_version = MSEL_ABI_VERSION;
    a.batch = batch;
    a.dim = dim;
    a.dstate = N;
    a.seqlen = L;
    a.dtype = MSEL_F32;
    a.delta_softplus = 1;
    a.u = fake();
    a.delta = fake();
    a.B = fake();
    a.C = fake();
    a.z = fake();
    a.A = fake();
    a.D = fake();
    a.delta_bias = fake();
    a.out = fake();
    a.final_state = fake();
    return a;
}

static msel_scan_grads good_grads(void) {
    msel_scan_grads g;
    g.dout = fake();
    g.du = fake();
    g.ddelta = fake();
    g.dz = fake();
    g.dA = fake();
    g.dB = fake();
    g.dC = fake();
    g.dD = fake();
    g.ddelta_bias = fake();
    g.dh0 = fake();
    return g;
}

static void scan_checks(void) {
    msel_scan_args a = good_args(2, 3, 16, 1000);
    EXPECT(msel_validate_fwd(&a), MSEL_OK);
    EXPECT(msel_validate_fwd(NULL), MSEL_ERR_NULL);
    msel_scan_args b = a;
    b.abi_version = 2;
    EXPECT(msel_validate_fwd(&b), MSEL_ERR_VERSION);
    b = a;
    b.seqlen = 0;
    EXPECT(msel_validate_fwd(&b), MSEL_ERR_SHAPE);
    b = a;
    b.seqlen = MSEL_MAX_SEQLEN + 1;
    EXPECT(msel_validate_fwd(&b), MSEL_ERR_SHAPE);
    b = a;
    b.batch = 1 << 16;
    b.dim = 1 << 16;  /* batch * dim = 2^32: the product is formed in 64 bits */
    EXPECT(msel_validate_fwd(&b), MSEL_ERR_SHAPE);
    b = a;
    b.dstate = MSEL_MAX_DSTATE + 1;
    EXPECT(msel_validate_fwd(&b), MSEL_ERR_UNSUPPORTED);
    b = a;
    b.dtype = 7;
    EXPECT(msel_validate_fwd(&b), MSEL_ERR_DTYPE);
    b = a;
    b.u = (const char *)a.u + 8;
    EXPECT(msel_validate_fwd(&b), MSEL_ERR_ALIGN);
    b = a;
    b.out = (void *)a.u;
    EXPECT(msel_validate_fwd(&b), MSEL_ERR_ALIAS);
    b = a;
    b.h0 = fake();
    b.final_state = (float *)b.h0;  /* the state updated in place is allowed */
    EXPECT(msel_validate_fwd(&b), MSEL_OK);
    b = a;
    b.C = NULL;
    EXPECT(msel_scan_fwd(&b, NULL), MSEL_ERR_NULL);
    EXPECT(msel_scan_chunk_carry(&a, NULL), MSEL_ERR_NULL);  /* chunk_states required */

    a.chunk_states = NULL;
    msel_scan_grads g = good_grads();
    size_t need = msel_scan_bwd_workspace_bytes(&a);
    if (need == 0) {
        fprintf(stderr, "workspace bytes of a valid problem is 0\n");
        ++failures;
    }
    void *ws = fake();
    EXPECT(msel_validate_bwd(&a, &g, ws, need), MSEL_OK);
    EXPECT(msel_validate_bwd(&a, &g, ws, need - 1), MSEL_ERR_WORKSPACE);
    EXPECT(msel_validate_bwd(&a, &g, NULL, need), MSEL_ERR_WORKSPACE);
    EXPECT(msel_validate_bwd(&a, &g, (char *)ws + 16, need), MSEL_ERR_ALIGN);
    EXPECT(msel_scan_bwd(&a, &g, NULL, 0, NULL), MSEL_ERR_WORKSPACE);
    msel_scan_grads h = g;
    h.du = (void *)g.dout;
    EXPECT(msel_validate_bwd(&a, &h, ws, need), MSEL_ERR_ALIAS);
    h = g;
    h.dz = NULL;
    EXPECT(msel_validate_bwd(&a, &h, ws, need), MSEL_ERR_NULL);
    /* the backward without a workspace argument: too large a problem, bad arguments */
    msel_scan_args big = good_args(1, 4096, 16, 65536);
    EXPECT(msel_scan_bwd_noalloc(&big, &g, NULL), MSEL_ERR_TOO_LARGE);
    h = g;
    h.ddelta = NULL;
    EXPECT(msel_scan_bwd_noalloc(&a, &h, NULL), MSEL_ERR_NULL);

    msel_trap_args tr = {fake(), NULL, NULL};
    EXPECT(msel_validate_trap_fwd(&a, &tr), MSEL_OK);
    tr.lambda = a.u;
    EXPECT(msel_validate_trap_fwd(&a, &tr), MSEL_OK);  /* lambda may be any input buffer */
    tr.lambda = a.out;
    EXPECT(msel_validate_trap_fwd(&a, &tr), MSEL_ERR_ALIAS);
    msel_scan_args c = a;
    c.dstate = 7;
    EXPECT(msel_validate_complex_fwd(&c), MSEL_ERR_SHAPE);
    c.dstate = 8;
    EXPECT(msel_validate_complex_fwd(&c), MSEL_OK);
    /* chunk_states NULL: rebuilt into the front of a workspace sized for that */
    size_t need_c = msel_scan_bwd_workspace_bytes(&c);
    EXPECT(msel_validate_complex_bwd(&c, &g, ws, need_c), MSEL_OK);
    EXPECT(msel_validate_complex_bwd(&c, &g, ws, need_c - 1), MSEL_ERR_WORKSPACE);
    EXPECT(msel_scan_complex_bwd(&c, &g, ws, need_c - 1, NULL), MSEL_ERR_WORKSPACE);
}

static void conv_checks(void) {
    msel_conv_args a;
    memset(&a, 0, sizeof a);
    a.abi_version = MSEL_ABI_VERSION;
    a.batch = 2;
    a.dim = 5;
    a.seqlen = 300;
    a.width = 4;
    a.dtype = MSEL_BF16;
    a.activation = 1;
    a.x = fake();
    a.weight = fake();
    a.bias = fake();
    a.state_in = fake();
    a.out = fake();
    a.state_out = fake();
    EXPECT(msel_validate_conv_fwd(&a), MSEL_OK);
    msel_conv_args b = a;
    b.width = MSEL_MAX_CONV_WIDTH + 1;
    EXPECT(msel_validate_conv_fwd(&b), MSEL_ERR_UNSUPPORTED);
    b = a;
    b.out = (void *)a.x;
    EXPECT(msel_validate_conv_fwd(&b), MSEL_ERR_ALIAS);
    b = a;
    b.state_out = (void *)a.state_in;  /* the cache updated in place is allowed */
    EXPECT(msel_validate_conv_fwd(&b), MSEL_OK);
    msel_conv_grads g = {fake(), fake(), fake(), fake(), fake()};
    EXPECT(msel_validate_conv_bwd(&a, &g), MSEL_OK);
    g.dx = (void *)g.dout;
    EXPECT(msel_validate_conv_bwd(&a, &g), MSEL_ERR_ALIAS);
    EXPECT(msel_conv1d_bwd(&a, &g, NULL), MSEL_ERR_ALIAS);
}

int main(void) {
    EXPECT(msel_abi_version(), MSEL_ABI_VERSION);
    EXPECT(msel_num_chunks(0), 0);
    EXPECT(msel_num_chunks(1), 1);
    EXPECT(msel_num_chunks(MSEL_MAX_SEQLEN), MSEL_MAX_SEQLEN / msel_chunk_len());
    for (int s = 0; s <= 11; ++s)
        if (msel_status_string((msel_status)s) == NULL) ++failures;
    scan_checks();
    conv_checks();
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("validate_driver: all checks passed\n");
    return 0;
}
