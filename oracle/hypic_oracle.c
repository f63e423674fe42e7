/*
 * hypic_oracle.c -- plain, slow fp64 CPU oracle for segment state caching in
 * linear-attention layers (HYPIC).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header or constant with the HIP library, and the HIP library never
 * calls it.
 *
 * What it computes (HYPIC, codernav.top article, section "linear layers:
 * caching the segment-accumulated transition operator"; xix.ai article, the
 * paragraph on linear layers):
 *   - every token applies a transition matrix A_t to the recurrent state and
 *     writes beta_t k_t v_t^T:          S_t = A_t S_{t-1} + beta_t k_t v_t^T
 *     with the read-out                  o_t = S_t^T q_t   (post-update state);
 *   - a segment C caches the ordered product of its transitions,
 *     T_C = A_n ... A_1 (later tokens on the left), and its zero-initial final
 *     state S(C|0);
 *   - reuse composes with S(C1.C2) = T(C2) S(C1) + S(C2);
 *   - the seam window: the first w tokens of every internal segment are not
 *     cached; at reuse the running state is advanced through them token by
 *     token and their outputs are emitted (same article, section on full
 *     attention layers and seam windows).
 *
 * Transition per family (the pages list RetNet, Mamba2, GLA, DeltaNet, GDN
 * and KDA next to plain linear attention; the matrix forms are those
 * families' published recurrences, state S is dk x dv):
 *   LINEAR    A = I,                          beta = 1
 *   RETNET    A = gamma I  (gamma per head),  beta = 1
 *   MAMBA2    A = exp(g_t) I  (scalar g),      beta = 1
 *   GLA       A = diag(exp(g_t)) (g in R^dk),  beta = 1
 *   DELTANET  A = I - beta_t k_t k_t^T
 *   GDN       A = exp(g_t) (I - beta_t k_t k_t^T)
 *   KDA       A = (I - beta_t k_t k_t^T) diag(exp(g_t))   (decay, then erase)
 * Multiplying by A_t is done from these definitions (a rank-one correction
 * costs O(dk*cols) instead of forming A_t); T is always kept as a dense
 * dk x dk matrix, whatever the family.
 *
 * Arrays are fp64 and row-major.  Per chain, token tensors are token-major:
 * q, k [n][dk], v [n][dv], beta [n], g [n] (scalar gates) or [n][dk] (GLA/KDA).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { F_LINEAR = 0, F_RETNET = 1, F_MAMBA2 = 2, F_GLA = 3, F_DELTANET = 4, F_GDN = 5, F_KDA = 6 };

static int fam_has_beta(int f) { return f == F_DELTANET || f == F_GDN || f == F_KDA; }
static int fam_vec_gate(int f) { return f == F_GLA || f == F_KDA; }

int oracle_gate_dim(int family, int dk) {
    if (family == F_MAMBA2 || family == F_GDN) return 1;
    if (fam_vec_gate(family)) return dk;
    return 0;
}

/* X (dk x ncols, row stride ldx) <- A_t X for one token.  k: [dk]; g: the
 * token's gate (1 or dk values, may be NULL when unused); beta, gamma scalars. */
void oracle_apply_transition(int family, int dk, int ncols, int ldx, double *X,
                             const double *k, const double *g, double beta, double gamma) {
    int i, j;
    switch (family) {
    case F_LINEAR:
        return;
    case F_RETNET:
        for (i = 0; i < dk; i++)
            for (j = 0; j < ncols; j++) X[i * ldx + j] *= gamma;
        return;
    case F_MAMBA2: {
        double a = exp(g[0]);
        for (i = 0; i < dk; i++)
            for (j = 0; j < ncols; j++) X[i * ldx + j] *= a;
        return;
    }
    case F_GLA:
        for (i = 0; i < dk; i++) {
            double a = exp(g[i]);
            for (j = 0; j < ncols; j++) X[i * ldx + j] *= a;
        }
        return;
    case F_DELTANET:
    case F_GDN:
    case F_KDA: {
        /* KDA decays first (diag(exp g) X) ... */
        if (family == F_KDA) {
            for (i = 0; i < dk; i++) {
                double a = exp(g[i]);
                for (j = 0; j < ncols; j++) X[i * ldx + j] *= a;
            }
        }
        /* ... then every family with erasure applies (I - beta k k^T): X -= beta k (k^T X) */
        for (j = 0; j < ncols; j++) {
            double kx = 0.0;
            for (i = 0; i < dk; i++) kx += k[i] * X[i * ldx + j];
            for (i = 0; i < dk; i++) X[i * ldx + j] -= beta * k[i] * kx;
        }
        /* GDN's scalar decay multiplies the whole transition */
        if (family == F_GDN) {
            double a = exp(g[0]);
            for (i = 0; i < dk; i++)
                for (j = 0; j < ncols; j++) X[i * ldx + j] *= a;
        }
        return;
    }
    default:
        return;
    }
}

/* One recurrence step on S (dk x dv): S <- A_t S + beta_t k_t v_t^T. */
static void token_step(int family, int dk, int dv, double *S, const double *k, const double *v,
                       const double *g, double beta, double gamma) {
    int i, j;
    double b = fam_has_beta(family) ? beta : 1.0;
    oracle_apply_transition(family, dk, dv, dv, S, k, g, b, gamma);
    for (i = 0; i < dk; i++)
        for (j = 0; j < dv; j++) S[i * dv + j] += b * k[i] * v[j];
}

/* Run the recurrence over n tokens from the state in S (in/out, dk x dv).
 * If O is not NULL it receives o_t = S_t^T q_t, [n][dv]. */
int oracle_run(int family, int dk, int dv, int64_t n, const double *q, const double *k,
               const double *v, const double *g, const double *beta, double gamma, double *S,
               double *O) {
    int gd = oracle_gate_dim(family, dk);
    int64_t t;
    int i, j;
    for (t = 0; t < n; t++) {
        token_step(family, dk, dv, S, k + t * dk, v + t * dv, gd ? g + t * gd : NULL,
                   beta ? beta[t] : 1.0, gamma);
        if (O) {
            for (j = 0; j < dv; j++) {
                double acc = 0.0;
                for (i = 0; i < dk; i++) acc += S[i * dv + j] * q[t * dk + i];
                O[t * dv + j] = acc;
            }
        }
    }
    return 0;
}

/* The cached pair of a segment of n tokens: T = A_n ... A_1 (dk x dk),
 * S = S(C|0) (dk x dv). */
int oracle_pair(int family, int dk, int dv, int64_t n, const double *k, const double *v,
                const double *g, const double *beta, double gamma, double *T, double *S) {
    int gd = oracle_gate_dim(family, dk);
    int64_t t;
    int i;
    memset(T, 0, sizeof(double) * dk * dk);
    for (i = 0; i < dk; i++) T[i * dk + i] = 1.0;
    memset(S, 0, sizeof(double) * dk * dv);
    for (t = 0; t < n; t++) {
        const double *gt = gd ? g + t * gd : NULL;
        double b = fam_has_beta(family) ? beta[t] : 1.0;
        oracle_apply_transition(family, dk, dk, dk, T, k + t * dk, gt, b, gamma);
        token_step(family, dk, dv, S, k + t * dk, v + t * dv, gt, b, gamma);
    }
    return 0;
}

/* Composition law: Sout = T Sin + SC  (dk x dk times dk x dv). */
void oracle_compose(int dk, int dv, const double *T, const double *SC, const double *Sin, double *Sout) {
    int i, j, l;
    for (i = 0; i < dk; i++)
        for (j = 0; j < dv; j++) {
            double acc = SC[i * dv + j];
            for (l = 0; l < dk; l++) acc += T[i * dk + l] * Sin[l * dv + j];
            Sout[i * dv + j] = acc;
        }
}

/* Associative combine of two adjacent pairs, a first then b:
 * (Tb, Sb) o (Ta, Sa) = (Tb Ta, Tb Sa + Sb). */
void oracle_combine(int dk, int dv, const double *Tb, const double *Sb, const double *Ta,
                    const double *Sa, double *Tout, double *Sout) {
    int i, j, l;
    for (i = 0; i < dk; i++)
        for (j = 0; j < dk; j++) {
            double acc = 0.0;
            for (l = 0; l < dk; l++) acc += Tb[i * dk + l] * Ta[l * dk + j];
            Tout[i * dk + j] = acc;
        }
    oracle_compose(dk, dv, Tb, Sb, Sa, Sout);
}

/*
 * The reuse path of one request over many chains.
 *
 * Segments are [bounds[j], bounds[j+1]), j = 0..n_seg-1, on the chain's own
 * token axis.  The first segment is cached whole; every later (internal)
 * segment keeps its first w tokens out of the cache (the seam window) and
 * caches only its body [bounds[j] + w, bounds[j+1]).  The running state
 * starts from zero (the first segment's pair gives S = S(C_1|0)), then for
 * j >= 1: advance through the w seam tokens emitting o_t, then
 * S <- T_body S + S_body.
 *
 * Inputs per chain c: q + c*n_tok*dk (and likewise for k, v, g, beta);
 * gamma[c] for RetNet.  Outputs (any may be NULL):
 *   T_out [n_seg][n_chains][dk][dk], S_out [n_seg][n_chains][dk][dv]  the pairs
 *   state_out [n_chains][dk][dv]                                      final state
 *   O_out [n_seg][w][n_chains][dv]   seam outputs (rows of segment 0 untouched)
 * Chains run in parallel over nthreads OpenMP threads (<= 0: library default).
 * Returns 0, or -1 when a segment is not longer than w.
 */
int oracle_request_batch(int family, int dk, int dv, int n_chains, int64_t n_tok, int n_seg,
                         const int64_t *bounds, int w, const double *q, const double *k,
                         const double *v, const double *g, const double *beta,
                         const double *gamma, double *T_out, double *S_out, double *state_out,
                         double *O_out, int nthreads) {
    int gd = oracle_gate_dim(family, dk);
    int j, bad = 0;
    for (j = 1; j < n_seg; j++)
        if (bounds[j + 1] - bounds[j] <= w) bad = 1;
    if (bad) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    {
        int c;
#pragma omp parallel for schedule(dynamic, 1)
        for (c = 0; c < n_chains; c++) {
            const double *qc = q ? q + (int64_t)c * n_tok * dk : NULL;
            const double *kc = k + (int64_t)c * n_tok * dk;
            const double *vc = v + (int64_t)c * n_tok * dv;
            const double *gc = gd ? g + (int64_t)c * n_tok * gd : NULL;
            const double *bc = beta ? beta + (int64_t)c * n_tok : NULL;
            double gm = gamma ? gamma[c] : 1.0;
            double *T = (double *)malloc(sizeof(double) * dk * dk);
            double *Sc = (double *)malloc(sizeof(double) * dk * dv);
            double *S = (double *)calloc((size_t)dk * dv, sizeof(double));
            double *Sn = (double *)malloc(sizeof(double) * dk * dv);
            double *O = (double *)malloc(sizeof(double) * (w > 0 ? w : 1) * dv);
            int jj, i;
            for (jj = 0; jj < n_seg; jj++) {
                int64_t b = bounds[jj], e = bounds[jj + 1];
                if (jj > 0 && w > 0) {
                    oracle_run(family, dk, dv, w, qc + b * dk, kc + b * dk, vc + b * dv,
                               gd ? gc + b * gd : NULL, bc ? bc + b : NULL, gm, S, O);
                    if (O_out)
                        for (i = 0; i < w; i++)
                            memcpy(O_out + (((int64_t)jj * w + i) * n_chains + c) * dv, O + i * dv,
                                   sizeof(double) * dv);
                    b += w;
                }
                oracle_pair(family, dk, dv, e - b, kc + b * dk, vc + b * dv,
                            gd ? gc + b * gd : NULL, bc ? bc + b : NULL, gm, T, Sc);
                if (T_out) memcpy(T_out + ((int64_t)jj * n_chains + c) * dk * dk, T, sizeof(double) * dk * dk);
                if (S_out) memcpy(S_out + ((int64_t)jj * n_chains + c) * dk * dv, Sc, sizeof(double) * dk * dv);
                oracle_compose(dk, dv, T, Sc, S, Sn);
                memcpy(S, Sn, sizeof(double) * dk * dv);
            }
            if (state_out) memcpy(state_out + (int64_t)c * dk * dv, S, sizeof(double) * dk * dv);
            free(T); free(Sc); free(S); free(Sn); free(O);
        }
    }
    return 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Variant patches (codernav.top article, section on linear layers, its last
 * paragraph; xix.ai article, the end of the paragraph on linear layers): two
 * model variants need a patch around the cached pair at reuse.
 *
 * Short causal convolution before the recurrence.  A depthwise convolution
 * of K taps over a channel's raw inputs x (zero before the first token):
 *     y_t = act( sum_{j=0}^{K-1} w[j] x_{t-K+1+j} )
 * (act: identity, or SiLU z / (1 + e^-z)).  A seam token's taps reach back
 * into the previous segment; the warm-up feeds them that segment's last K-1
 * raw inputs, which is the whole-sequence convolution at those positions.
 *
 * Rotary position embeddings on the keys.  R(p) rotates each pair of
 * channels (i, i + d/2), i < d/2, by the angle p * theta_i with
 * theta_i = base^(-2i/d):
 *     (R x)_i       = cos x_i - sin x_{i+d/2}
 *     (R x)_{i+d/2} = sin x_i + cos x_{i+d/2}
 * A segment cached with keys at local positions 0 .. n-1 and reused at offset
 * P has keys R(P) R(local) k; the transitions that keys enter through become
 * R(P) A_t R(P)^T when the decay commutes with R(P), so the re-rotated pair is
 *     T' = R(P) T R(P)^T,   S' = R(P) S.
 * These are plain matrix products here, with R(P) formed explicitly.
 */

/* R(p) as an explicit d x d matrix (d even), angles in fp64. */
void oracle_rope_matrix(int d, double p, double base, double *R) {
    int h = d / 2, i;
    memset(R, 0, sizeof(double) * d * d);
    for (i = 0; i < h; i++) {
        double th = pow(base, -2.0 * i / d), a = p * th;
        double c = cos(a), s = sin(a);
        R[i * d + i] = c;
        R[i * d + i + h] = -s;
        R[(i + h) * d + i] = s;
        R[(i + h) * d + i + h] = c;
    }
}

/* T' = R T R^T (T dense dk x dk), S' = R S (dk x dv). */
void oracle_rerotate(int dk, int dv, const double *R, const double *T, const double *S, double *Tout,
                     double *Sout) {
    int i, j, l;
    double *A = (double *)malloc(sizeof(double) * dk * dk);
    for (i = 0; i < dk; i++)
        for (j = 0; j < dk; j++) {
            double acc = 0.0;
            for (l = 0; l < dk; l++) acc += R[i * dk + l] * T[l * dk + j];
            A[i * dk + j] = acc;
        }
    for (i = 0; i < dk; i++)
        for (j = 0; j < dk; j++) {
            double acc = 0.0;
            for (l = 0; l < dk; l++) acc += A[i * dk + l] * R[j * dk + l];
            Tout[i * dk + j] = acc;
        }
    for (i = 0; i < dk; i++)
        for (j = 0; j < dv; j++) {
            double acc = 0.0;
            for (l = 0; l < dk; l++) acc += R[i * dk + l] * S[l * dv + j];
            Sout[i * dv + j] = acc;
        }
    free(A);
}

/* Causal depthwise convolution of one chain's raw inputs x [n][d] with
 * taps w [d][K] (zero before token 0), act 0: none, 1: SiLU; y [n][d]. */
void oracle_conv(int64_t n, int d, int K, const double *x, const double *w, int act, double *y) {
    int64_t t;
    int c, j;
    for (t = 0; t < n; t++)
        for (c = 0; c < d; c++) {
            double z = 0.0;
            for (j = 0; j < K; j++) {
                int64_t u = t - K + 1 + j;
                if (u >= 0) z += w[c * K + j] * x[u * d + c];
            }
            y[t * d + c] = act == 1 ? z / (1.0 + exp(-z)) : z;
        }
}
