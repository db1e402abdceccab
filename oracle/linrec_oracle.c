/*
 * linrec_oracle.c -- float64 CPU oracle for the channel-wise first-order
 * linear recurrence.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load or call this library.  It shares
 * no code, header, helper or constant with the HIP path, and the HIP path
 * never calls it.
 *
 * What it computes (the plain definition, written out):
 *
 *   for every batch row b in [0,B) and channel d in [0,D):
 *     h[b,0,d] = b_in[b,0,d]                                (zero initial state)
 *     h[b,0,d] = a[b,0,d] * h_init[b,d] + b_in[b,0,d]       (when h_init is given)
 *     h[b,t,d] = a[b,t,d] * h[b,t-1,d] + b_in[b,t,d]         for t = 1 .. L-1
 *
 * Source: POPCORNBENCH transcript "Kimi-K2.6 l1_p9" (the linear-recurrence
 * scan problem), opening problem statement of its first reasoning block, and
 * the same statement in the "FW-GLM-5-1 l1_p9" transcript.  The problem's
 * PyTorch reference model, quoted in the second reasoning block of the
 * Kimi-K2.6 l1_p9 transcript, runs exactly this loop over t starting from a
 * zero state, which fixes the reading that a[b,0,d] never contributes when
 * there is no initial state.  The optional h_init generalises that zero state
 * to a given one; the first reasoning block's running-carry passage ("only
 * the running h crosses a chunk boundary") is the same update with h_init as
 * the carried value.
 *
 * Reverse-time form (linrec_oracle_rev_f64): the same update run from the
 * last step back to the first,
 *
 *     h[b,L-1,d] = b_in[b,L-1,d]                            (zero final state)
 *     h[b,L-1,d] = a[b,L-1,d] * h_init[b,d] + b_in[b,L-1,d] (when h_init is given)
 *     h[b,t,d]   = a[b,t,d] * h[b,t+1,d] + b_in[b,t,d]       for t = L-2 .. 0
 *
 * The pages do not treat it.  It is the time reversal of the definition
 * above, and its use is the gradient of the scan: for h = scan(a, b) from a
 * zero state and an incoming gradient g = dLoss/dh, dLoss/db is this reverse
 * recurrence over g with a shifted one step (a[b,t+1,d] at position t).
 *
 * Layout: a, b_in and h are (B, L, D) row-major with D contiguous, element
 * (b,t,d) at offset (b*L + t)*D + d.  h_init is (B, D) row-major.
 *
 * Arithmetic: inputs are fp32 and widen exactly to float64; every product and
 * sum is a float64 operation, written as a separate multiply and add and
 * compiled with -ffp-contract=off, so the vectorised and scalar iterations
 * round identically.  Channels are independent, so the OpenMP split over
 * (b, block of channels) gives bit-identical output for any thread count.
 *
 * Parity pins: see tests/oracle_pins.py (closed forms, library routines,
 * exact rational brute force, the pages' symbolic worked values, invariants).
 */
#include <stddef.h>
#include <stdint.h>

#define ORACLE_CHANNEL_BLOCK 64

/* Returns 0 on success, 1 on an invalid argument (negative size, or a null
 * buffer while there is at least one element to compute). */
int linrec_oracle_f64(const float *a, const float *b_in, const double *h_init,
                      double *h, int64_t B, int64_t L, int64_t D, int threads)
{
    if (B < 0 || L < 0 || D < 0) return 1;
    if (B == 0 || L == 0 || D == 0) return 0;
    if (a == NULL || b_in == NULL || h == NULL) return 1;
    if (threads < 1) threads = 1;

#pragma omp parallel for collapse(2) schedule(static) num_threads(threads)
    for (int64_t bi = 0; bi < B; ++bi) {
        for (int64_t d0 = 0; d0 < D; d0 += ORACLE_CHANNEL_BLOCK) {
            int64_t d1 = d0 + ORACLE_CHANNEL_BLOCK < D ? d0 + ORACLE_CHANNEL_BLOCK : D;
            const float *ab = a + bi * L * D;
            const float *bb = b_in + bi * L * D;
            double *hb = h + bi * L * D;

            /* t = 0: the state before the sequence is zero (a[b,0,d] unused)
             * or the given h_init[b,d]. */
            for (int64_t d = d0; d < d1; ++d) {
                if (h_init != NULL)
                    hb[d] = (double)ab[d] * h_init[bi * D + d] + (double)bb[d];
                else
                    hb[d] = (double)bb[d];
            }

            /* t >= 1: one affine step per time position. */
            for (int64_t t = 1; t < L; ++t) {
                const float *at = ab + t * D;
                const float *bt = bb + t * D;
                const double *hprev = hb + (t - 1) * D;
                double *ht = hb + t * D;
                for (int64_t d = d0; d < d1; ++d)
                    ht[d] = (double)at[d] * hprev[d] + (double)bt[d];
            }
        }
    }
    return 0;
}

/* Reverse-time form; same arguments, errors and layout as linrec_oracle_f64. */
int linrec_oracle_rev_f64(const float *a, const float *b_in, const double *h_init,
                          double *h, int64_t B, int64_t L, int64_t D, int threads)
{
    if (B < 0 || L < 0 || D < 0) return 1;
    if (B == 0 || L == 0 || D == 0) return 0;
    if (a == NULL || b_in == NULL || h == NULL) return 1;
    if (threads < 1) threads = 1;

#pragma omp parallel for collapse(2) schedule(static) num_threads(threads)
    for (int64_t bi = 0; bi < B; ++bi) {
        for (int64_t d0 = 0; d0 < D; d0 += ORACLE_CHANNEL_BLOCK) {
            int64_t d1 = d0 + ORACLE_CHANNEL_BLOCK < D ? d0 + ORACLE_CHANNEL_BLOCK : D;
            const float *rab = a + bi * L * D;
            const float *rbb = b_in + bi * L * D;
            double *rhb = h + bi * L * D;
            const int64_t last = (L - 1) * D;

            /* t = L-1: the state after the sequence is zero (a[b,L-1,d] unused)
             * or the given h_init[b,d]. */
            for (int64_t d = d0; d < d1; ++d) {
                if (h_init != NULL)
                    rhb[last + d] = (double)rab[last + d] * h_init[bi * D + d] + (double)rbb[last + d];
                else
                    rhb[last + d] = (double)rbb[last + d];
            }

            /* t <= L-2, walking back: one affine step per time position. */
            for (int64_t t = L - 2; t >= 0; --t) {
                const float *rat = rab + t * D;
                const float *rbt = rbb + t * D;
                const double *hnext = rhb + (t + 1) * D;
                double *rht = rhb + t * D;
                for (int64_t d = d0; d < d1; ++d)
                    rht[d] = (double)rat[d] * hnext[d] + (double)rbt[d];
            }
        }
    }
    return 0;
}
