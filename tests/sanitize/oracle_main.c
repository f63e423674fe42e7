/* Host sanitizer driver for the fp64 oracle (test infrastructure): every
 * exported routine on small random inputs of each family, under AddressSanitizer
 * and UndefinedBehaviorSanitizer.  It checks that every output is finite and
 * that the request batch equals its own pieces composed by hand. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gate_dim(int family, int dk);
int oracle_run(int family, int dk, int dv, int64_t n, const double *q, const double *k, const double *v,
               const double *g, const double *beta, double gamma, double *S, double *O);
int oracle_pair(int family, int dk, int dv, int64_t n, const double *k, const double *v, const double *g,
                const double *beta, double gamma, double *T, double *S);
void oracle_compose(int dk, int dv, const double *T, const double *SC, const double *Sin, double *Sout);
void oracle_combine(int dk, int dv, const double *Tb, const double *Sb, const double *Ta, const double *Sa,
                    double *Tout, double *Sout);
int oracle_request_batch(int family, int dk, int dv, int n_chains, int64_t n_tok, int n_seg, const int64_t *bounds,
                         int w, const double *q, const double *k, const double *v, const double *g,
                         const double *beta, const double *gamma, double *T_out, double *S_out, double *state_out,
                         double *O_out, int nthreads);
void oracle_rope_matrix(int d, double p, double base, double *R);
void oracle_rerotate(int dk, int dv, const double *R, const double *T, const double *S, double *Tout, double *Sout);
void oracle_conv(int64_t n, int d, int K, const double *x, const double *w, int act, double *y);

static uint64_t st = 88172645463325252ull;
static double urand(void) { /* xorshift64 */
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return (double)(st >> 11) / 9007199254740992.0;
}
static double *arr(size_t n, double lo, double hi) {
    double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; i++) p[i] = lo + (hi - lo) * urand();
    return p;
}
static int finite_all(const double *p, size_t n) {
    for (size_t i = 0; i < n; i++)
        if (!isfinite(p[i])) return 0;
    return 1;
}
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void) {
    const int dk = 8, dv = 8, C = 2, w = 3;
    const int64_t n = 40;
    const int64_t bounds[4] = {0, 11, 25, 40};
    for (int fam = 0; fam <= 6; fam++) {
        const int gd = oracle_gate_dim(fam, dk);
        double *q = arr((size_t)C * n * dk, -0.5, 0.5), *k = arr((size_t)C * n * dk, -0.5, 0.5);
        double *v = arr((size_t)C * n * dv, -1, 1), *g = arr((size_t)C * n * (gd ? gd : 1), -0.3, 0.0);
        double *beta = arr((size_t)C * n, 0.1, 0.9), *gam = arr(C, 0.8, 0.99);
        double *T = arr((size_t)dk * dk, 0, 0), *S = arr((size_t)dk * dv, 0, 0), *O = arr((size_t)n * dv, 0, 0);
        memset(S, 0, sizeof(double) * dk * dv);
        CHECK(oracle_run(fam, dk, dv, n, q, k, v, gd ? g : NULL, beta, gam[0], S, O) == 0);
        CHECK(finite_all(S, (size_t)dk * dv) && finite_all(O, (size_t)n * dv));
        CHECK(oracle_pair(fam, dk, dv, n, k, v, gd ? g : NULL, beta, gam[0], T, S) == 0);
        CHECK(finite_all(T, (size_t)dk * dk) && finite_all(S, (size_t)dk * dv));
        /* the batch against its pieces: the last chain's state */
        double *Tb = arr((size_t)3 * C * dk * dk, 0, 0), *Sb = arr((size_t)3 * C * dk * dv, 0, 0);
        double *state = arr((size_t)C * dk * dv, 0, 0), *Ob = arr((size_t)3 * w * C * dv, 0, 0);
        memset(Ob, 0, sizeof(double) * 3 * w * C * dv);
        CHECK(oracle_request_batch(fam, dk, dv, C, n, 3, bounds, w, q, k, v, gd ? g : NULL, beta, gam, Tb, Sb,
                                   state, Ob, 1) == 0);
        CHECK(finite_all(Tb, (size_t)3 * C * dk * dk) && finite_all(state, (size_t)C * dk * dv));
        double *run_S = arr((size_t)dk * dv, 0, 0), *run_O = arr((size_t)n * dv, 0, 0);
        memset(run_S, 0, sizeof(double) * dk * dv);
        const int c = C - 1;
        CHECK(oracle_run(fam, dk, dv, n, q + (int64_t)c * n * dk, k + (int64_t)c * n * dk, v + (int64_t)c * n * dv,
                         gd ? g + (int64_t)c * n * gd : NULL, beta + (int64_t)c * n, gam[c], run_S, run_O) == 0);
        double err = 0, ref = 0;
        for (int i = 0; i < dk * dv; i++) {
            err += (state[(int64_t)c * dk * dv + i] - run_S[i]) * (state[(int64_t)c * dk * dv + i] - run_S[i]);
            ref += run_S[i] * run_S[i];
        }
        CHECK(sqrt(err) <= 1e-9 * sqrt(ref) + 1e-300);
        /* compose and combine on the batch's pairs */
        double *S1 = arr((size_t)dk * dv, 0, 0), *T2 = arr((size_t)dk * dk, 0, 0), *S2 = arr((size_t)dk * dv, 0, 0);
        oracle_compose(dk, dv, Tb + (int64_t)(1 * C + 0) * dk * dk, Sb + (int64_t)(1 * C + 0) * dk * dv,
                       Sb, S1);
        oracle_combine(dk, dv, Tb + (int64_t)(2 * C) * dk * dk, Sb + (int64_t)(2 * C) * dk * dv,
                       Tb + (int64_t)(1 * C) * dk * dk, Sb + (int64_t)(1 * C) * dk * dv, T2, S2);
        CHECK(finite_all(S1, (size_t)dk * dv) && finite_all(T2, (size_t)dk * dk) && finite_all(S2, (size_t)dk * dv));
        free(q); free(k); free(v); free(g); free(beta); free(gam); free(T); free(S); free(O);
        free(Tb); free(Sb); free(state); free(Ob); free(run_S); free(run_O); free(S1); free(T2); free(S2);
    }
    /* rotary re-rotation and the short convolution */
    {
        const int d = 8;
        double *R = arr((size_t)d * d, 0, 0), *T = arr((size_t)d * d, -1, 1), *S = arr((size_t)d * d, -1, 1);
        double *To = arr((size_t)d * d, 0, 0), *So = arr((size_t)d * d, 0, 0);
        oracle_rope_matrix(d, 123456.0, 10000.0, R);
        oracle_rerotate(d, d, R, T, S, To, So);
        CHECK(finite_all(To, (size_t)d * d) && finite_all(So, (size_t)d * d));
        double *x = arr((size_t)20 * d, -1, 1), *wt = arr((size_t)d * 4, -1, 1), *y = arr((size_t)20 * d, 0, 0);
        oracle_conv(20, d, 4, x, wt, 1, y);
        CHECK(finite_all(y, (size_t)20 * d));
        free(R); free(T); free(S); free(To); free(So); free(x); free(wt); free(y);
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
