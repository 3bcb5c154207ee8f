/* The float64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every code
 * path of oracle_attention (causal and not, decode offsets, local windows, the
 * probability output, several threads, rejected arguments) on small shapes, with the
 * worked example's value checked.  Exit status 0 when every expectation holds. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attention(const double *q, const double *k, const double *v, double *out, double *probs, int B,
                     int Hq, int Hkv, int Tq, int Tk, int d, double scale, int causal, long pos0, long window,
                     int nthreads);

static int fails = 0;

static double *filled(size_t n, unsigned seed) {
    double *x = (double *)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) {
        seed = seed * 1103515245u + 12345u;
        x[i] = ((seed >> 8) & 0xffff) / 32768.0 - 1.0;
    }
    return x;
}

static void run(int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, long pos0, long window, int threads,
                int want_rc) {
    double *q = filled((size_t)B * Hq * Tq * d + 1, 1u + Tq), *k = filled((size_t)B * Hkv * Tk * d + 1, 2u + Tk);
    double *v = filled((size_t)B * Hkv * Tk * d + 1, 3u + d);
    double *out = (double *)calloc((size_t)B * Hq * Tq * d + 1, sizeof(double));
    double *p = (double *)calloc((size_t)B * Hq * Tq * Tk + 1, sizeof(double));
    const int rc = oracle_attention(q, k, v, out, p, B, Hq, Hkv, Tq, Tk, d, 0.3, causal, pos0, window, threads);
    if (rc != want_rc) {
        printf("FAIL: B%d Hq%d Hkv%d Tq%d Tk%d d%d causal%d pos0 %ld window %ld -> %d, want %d\n", B, Hq, Hkv, Tq,
               Tk, d, causal, pos0, window, rc, want_rc);
        ++fails;
    }
    if (rc == 0) /* every row of P sums to one */
        for (long r = 0; r < (long)B * Hq * Tq; ++r) {
            double s = 0;
            for (int j = 0; j < Tk; ++j) s += p[r * Tk + j];
            if (fabs(s - 1.0) > 1e-12) {
                printf("FAIL: row %ld sums to %.17g\n", r, s);
                ++fails;
                break;
            }
        }
    free(q);
    free(k);
    free(v);
    free(out);
    free(p);
}

int main(void) {
    /* the multi-query primer's tiny example: q = (1, 0) over keys (1,0), (0,1), (1,1),
       values 1, 2, 3, unscaled -> (4e + 2) / (2e + 1) = 2 */
    double q[2] = {1, 0}, k[6] = {1, 0, 0, 1, 1, 1}, v[6] = {1, 0, 2, 0, 3, 0}, out[2];
    if (oracle_attention(q, k, v, out, NULL, 1, 1, 1, 1, 3, 2, 1.0, 0, 0, 0, 1) != 0 || fabs(out[0] - 2.0) > 1e-15) {
        printf("FAIL: worked example gave %.17g\n", out[0]);
        ++fails;
    }
    run(1, 1, 1, 16, 16, 8, 1, 0, 0, 1, 0);
    run(2, 4, 2, 9, 9, 3, 1, 0, 0, 3, 0);
    run(2, 6, 2, 7, 7, 5, 0, 0, 0, 4, 0);
    run(1, 4, 1, 3, 20, 8, 1, 17, 0, 2, 0);  /* decode: rows at positions 17..19 */
    run(1, 2, 2, 12, 12, 4, 1, 0, 5, 2, 0);  /* local window of 5 */
    run(1, 2, 1, 1, 1, 1, 1, 0, 0, 8, 0);    /* more threads than units */
    run(0, 2, 1, 4, 4, 8, 1, 0, 0, 1, 0);    /* empty batch */
    run(1, 3, 2, 4, 4, 8, 1, 0, 0, 1, -1);   /* Hq % Hkv != 0 */
    run(1, 2, 1, 4, 4, 8, 1, 2, 0, 1, -1);   /* rows past the keys */
    run(1, 2, 1, 4, 4, 8, 0, 0, 3, 1, -1);   /* a window without the causal mask */
    printf("oracle host checks: %d failures\n", fails);
    return fails ? 1 : 0;
}
