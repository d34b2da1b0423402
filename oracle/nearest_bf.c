/*
 * nearest_bf.c -- brute-force nearest codebook entry, the plain definition
 * of the stage-1 and residual searches ("glq 0.1.1", PyPI project page,
 * section "How it works", item 1: each 8-weight group is replaced by a
 * codebook entry; the nearest one in Euclidean distance, with the lowest
 * index winning an exact tie, is this oracle's reading).
 *
 * TEST INFRASTRUCTURE ONLY: part of the oracle. Only tests/, the smoke check
 * and the benchmark's CPU baseline load it; the library never does.
 *
 *   out[r] = argmin_i  sum_{c=0..7} (x[r][c] - cb[i][c])^2
 *
 * in float64, the eight squared differences summed in coordinate order,
 * the lowest i taken on an exact tie (strict < while scanning upward).
 * cb is the caller's table (the oracle's own codebook), [size][8] float64.
 */
#include <stdint.h>

void oracle_nearest_bf(const double *x, int64_t nx, const double *cb, int64_t size, int64_t *out)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < nx; ++r) {
        const double *p = x + 8 * r;
        double best = 0.0;
        int64_t arg = -1;
        for (int64_t i = 0; i < size; ++i) {
            const double *c = cb + 8 * i;
            double d = 0.0;
            for (int t = 0; t < 8; ++t) {
                const double e = p[t] - c[t];
                d += e * e;
            }
            if (arg < 0 || d < best) {
                best = d;
                arg = i;
            }
        }
        out[r] = arg;
    }
}
