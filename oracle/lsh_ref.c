/* Random-rotation LSH bucket ids in plain C: the reference loop.
 *
 * TEST INFRASTRUCTURE ONLY: part of the CPU oracle; never linked into the
 * GPU library.
 *
 * For each row x (length d) and rotation R (d x half, row-major, float32):
 *   p_c = sum_{k=0}^{d-1} x_k * R[k][c], accumulated in double in increasing k
 *   (every product of a float32 by a float32 is exact in double, so only the
 *   additions round, in this fixed order);
 *   bucket = first index of the maximum of [p_0..p_{half-1}, -p_0..-p_{half-1}].
 * This is the bucket function of the random-rotation LSH used by the
 * Hash-sparse workloads of the SCFA summary page ("2. Hash-Sparse").
 */
#include <stdint.h>
#include <stdlib.h>

void lsh_ref_buckets(const float *x, const float *R, long T, int d, int half,
                     int32_t *out, int threads)
{
#pragma omp parallel for schedule(static) num_threads(threads)
    for (long t = 0; t < T; ++t) {
        double *acc = (double *)malloc(sizeof(double) * (size_t)half);
        const float *row = x + (size_t)t * (size_t)d;
        for (int c = 0; c < half; ++c) acc[c] = 0.0;
        for (int k = 0; k < d; ++k) {
            const double xk = (double)row[k];
            const float *rk = R + (size_t)k * (size_t)half;
            for (int c = 0; c < half; ++c) acc[c] = acc[c] + xk * (double)rk[c];
        }
        int best = 0;
        double bestv = acc[0];
        for (int c = 1; c < half; ++c)
            if (acc[c] > bestv) { bestv = acc[c]; best = c; }
        for (int c = 0; c < half; ++c)
            if (-acc[c] > bestv) { bestv = -acc[c]; best = half + c; }
        out[t] = best;
        free(acc);
    }
}
