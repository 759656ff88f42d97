/*
 * ssd_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of the selective state-space layer
 * that the SSD kernels compute.  It exists so that tests and the benchmark's
 * CPU-baseline leg have something independent to compare the GPU path with;
 * no product code may link, load or call it.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * What it computes (the recurrence, evaluated token by token, no chunks):
 *   "Transformers are SSMs Review" (dimensionstp.github.io), section 3-2(4)
 *   says the chunked SSD algorithm only changes the evaluation order of the
 *   state-space recurrence, so the oracle is that recurrence itself:
 *     - "Mamba-2는 왜 Transformer와 닮았는가" (bdev.io), the problem section,
 *       states h_t = A_t h_{t-1} + B_t x_t and y_t = C_t^T h_t;
 *     - the SSM textbook chapter 20.1 (sungeuns.github.io), section 1, gives
 *       the discretisation Abar = exp(dt*A), Bbar ~= dt*B and the skip D*x;
 *       its section 3 restricts A to a scalar times identity (one scalar per
 *       head for SSD); its section 5 code updates the state first and reads
 *       the output from the updated state;
 *     - the Mamba-2 review, section 3-2(6), cuts the state at sequence
 *       boundaries when sequences are packed back to back (varlen).
 *
 * Per sequence s and head h, with group g = h / (H/G):
 *     S      = init_state[s,h]            (P x N, zero when absent)
 *     for t in the sequence, in order:
 *         abar = exp(dt[t,h] * A[h])
 *         S    = abar * S + dt[t,h] * x[t,h,:] (outer) B[t,g,:]
 *         y[t,h,p] = sum_n S[p,n] * C[t,g,n] + D[h] * x[t,h,p]
 *     final_state[s,h] = S
 *
 * Layouts (row-major, contiguous; token index t is the flat packed index):
 *     x, y   [T][H][P]      dt [T][H]      A, D [H]
 *     B, C   [T][G][N]      states [nseq][H][P][N]
 *
 * Every (sequence, head) pair is independent, so OpenMP runs them on the
 * host's cores; inside one pair the loop is strictly sequential.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Returns 0 on success, -1 on invalid arguments, -2 on allocation failure. */
int ssd_oracle_fwd(int64_t nseq, const int64_t *seq_start, const int64_t *seq_len,
                   int64_t H, int64_t P, int64_t N, int64_t G,
                   const double *x, const double *dt, const double *A,
                   const double *B, const double *C, const double *D,
                   const double *init_state, const uint8_t *unit_mask,
                   double *y, double *final_state, int nthreads)
{
    if (nseq < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0)
        return -1;
    if (!seq_start || !seq_len || !x || !dt || !A || !B || !C || !y)
        return -1;
    const int64_t heads_per_group = H / G;
    const int64_t units = nseq * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t s = u / H;
        const int64_t h = u % H;
        if (unit_mask && !unit_mask[u]) continue;
        const int64_t g = h / heads_per_group;
        double *S = (double *)malloc((size_t)(P * N) * sizeof(double));
        if (!S) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        if (init_state)
            memcpy(S, init_state + u * P * N, (size_t)(P * N) * sizeof(double));
        else
            memset(S, 0, (size_t)(P * N) * sizeof(double));

        const double Dh = D ? D[h] : 0.0;
        for (int64_t k = 0; k < seq_len[s]; ++k) {
            const int64_t t = seq_start[s] + k;
            const double d = dt[t * H + h];
            const double abar = exp(d * A[h]);
            const double *xt = x + (t * H + h) * P;
            const double *Bt = B + (t * G + g) * N;
            const double *Ct = C + (t * G + g) * N;
            double *yt = y + (t * H + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                double *row = S + p * N;
                const double dx = d * xt[p];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    row[n] = abar * row[n] + dx * Bt[n];
                    acc += row[n] * Ct[n];
                }
                yt[p] = acc + Dh * xt[p];
            }
        }
        if (final_state)
            memcpy(final_state + u * P * N, S, (size_t)(P * N) * sizeof(double));
        free(S);
    }
    return failed ? -2 : 0;
}

/*
 * One recurrent (decode) step: the same update and read-out applied once to
 * a given state, in place.  Constant-size state per generated token is the
 * inference mode the Mamba-2 review describes in its problem section.
 *     state [batch][H][P][N] (in/out), x [batch][H][P], dt [batch][H],
 *     B, C [batch][G][N], y [batch][H][P].
 */
int ssd_oracle_decode(int64_t batch, int64_t H, int64_t P, int64_t N, int64_t G,
                      double *state, const double *x, const double *dt,
                      const double *A, const double *B, const double *C,
                      const double *D, double *y, int nthreads)
{
    if (batch < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0)
        return -1;
    if (!state || !x || !dt || !A || !B || !C || !y) return -1;
    const int64_t heads_per_group = H / G;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t u = 0; u < batch * H; ++u) {
        const int64_t b = u / H;
        const int64_t h = u % H;
        const int64_t g = h / heads_per_group;
        const double d = dt[u];
        const double abar = exp(d * A[h]);
        const double *xt = x + u * P;
        const double *Bt = B + (b * G + g) * N;
        const double *Ct = C + (b * G + g) * N;
        double *S = state + u * P * N;
        const double Dh = D ? D[h] : 0.0;
        for (int64_t p = 0; p < P; ++p) {
            double *row = S + p * N;
            const double dx = d * xt[p];
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                row[n] = abar * row[n] + dx * Bt[n];
                acc += row[n] * Ct[n];
            }
            y[u * P + p] = acc + Dh * xt[p];
        }
    }
    return 0;
}
