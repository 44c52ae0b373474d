/* Calls the float64 oracle on small seeded inputs, including its edge cases
 * (sequences with no new rows, R = 1, W = 1, row subsets, sink and gate, bad
 * arguments), for a build with AddressSanitizer and UndefinedBehaviorSanitizer.
 * Exit status 0 = every call behaved. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int rba_oracle_attend(int64_t batch, const int64_t* q_lens, const int64_t* seq_lens, int64_t Hq, int64_t Hkv,
                      int64_t dqk, int64_t dv, int64_t R, int64_t W, double scale, const double* q,
                      const double* k, const double* v, const double* rel, const double* sink,
                      const double* gate, const int64_t* rows, int64_t n_rows, double* out, double* lse);

static uint64_t st = 88172645463325252ull;
static double rnd(void) { /* xorshift64, uniform in [-1, 1) */
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return (double)(st >> 11) / 4503599627370496.0 - 1.0;
}

static double* arr(int64_t n) {
    double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) a[i] = rnd();
    return a;
}

static int run(int64_t batch, const int64_t* ql, const int64_t* sl, int64_t Hq, int64_t Hkv, int64_t R, int64_t W,
               int use_rows, int gated) {
    int64_t tq = 0, tk = 0;
    for (int64_t b = 0; b < batch; ++b) { tq += ql[b]; tk += sl[b]; }
    const int64_t dqk = 8, dv = 4;
    double *q = arr(tq * Hq * dqk), *k = arr(tk * Hkv * dqk), *v = arr(tk * Hkv * dv), *rel = arr(tq * Hq * R);
    double *sink = gated ? arr(tq * Hq) : NULL, *gate = gated ? arr(tq * Hq) : NULL;
    double *out = arr(tq * Hq * dv), *lse = arr(tq * Hq);
    int64_t rows[3] = {0, tq > 1 ? tq - 1 : 0, tq / 2};
    const int rc = rba_oracle_attend(batch, ql, sl, Hq, Hkv, dqk, dv, R, W, 0.35, q, k, v, rel, sink, gate,
                                     use_rows ? rows : NULL, use_rows ? 3 : 0, out, lse);
    int bad = rc != 0;
    for (int64_t i = 0; i < tq * Hq * dv && !use_rows; ++i) bad |= !isfinite(out[i]);
    free(q); free(k); free(v); free(rel); free(sink); free(gate); free(out); free(lse);
    return bad;
}

int main(void) {
    int fails = 0;
    const int64_t ql1[] = {5}, sl1[] = {9};
    const int64_t ql2[] = {0, 7, 3}, sl2[] = {4, 20, 3};
    const int64_t ql3[] = {1, 1}, sl3[] = {1, 33};
    for (int64_t R = 1; R <= 9; R += 4)
        for (int64_t W = 0; W <= 3; W += 3)
            for (int g = 0; g < 2; ++g)
                for (int u = 0; u < 2; ++u) {
                    fails += run(1, ql1, sl1, 4, 2, R, W, u, g);
                    fails += run(3, ql2, sl2, 6, 3, R, W, u, g);
                    fails += run(2, ql3, sl3, 2, 1, R, W, u, g);
                }
    /* bad arguments are rejected, not read */
    double x[8] = {0};
    const int64_t qb[] = {3}, sb[] = {2};
    fails += rba_oracle_attend(1, qb, sb, 2, 1, 2, 2, 1, 0, 1.0, x, x, x, x, NULL, NULL, NULL, 0, x, x) != -1;
    fails += rba_oracle_attend(1, ql1, sl1, 3, 2, 2, 2, 1, 0, 1.0, x, x, x, x, NULL, NULL, NULL, 0, x, x) != -1;
    fails += rba_oracle_attend(1, ql1, sl1, 2, 1, 2, 2, 0, 0, 1.0, x, x, x, x, NULL, NULL, NULL, 0, x, x) != -1;
    if (fails) {
        fprintf(stderr, "%d oracle call(s) misbehaved\n", fails);
        return 1;
    }
    printf("oracle driver: all calls behaved\n");
    return 0;
}
