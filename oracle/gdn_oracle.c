/*
 * gdn_oracle.c -- fp64 CPU oracle of the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library; neither includes the other.
 *
 * What it computes.  The GDN layer mixer named by the lithos-metal README
 * ("How it works", region table, "GDN mixer" row) keeps an fp32 recurrent
 * state with a key side and a value side (devdoido audit, "How does
 * lithos-metal fuse layer mixers on Metal?").  The pages never print the
 * update, so this file follows the gated delta rule as published for Gated
 * DeltaNet (Yang, Kautz & Hatamizadeh, ICLR 2025):
 *
 *     S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
 *
 * with S in R^{dv x dk}, a_t = exp(g_t) (g is the log-decay), b_t = beta_t.
 * Expanding the product gives the row-wise form used below, one value row i at
 * a time (row i of S needs only row i of S, v_i and the shared k, q, a, b):
 *
 *     u_i   = sum_j S_ij k_j                  (the old state's read of k_t)
 *     d_i   = b_t (v_i - a_t u_i)             (delta-rule correction)
 *     S_ij <- a_t S_ij + d_i k_j              (decay, then rank-1 write)
 *     o_i   = sum_j S_ij q_j                  (read of the UPDATED state)
 *
 * Layouts (row-major, C order):
 *     S     [B][H][dv][dk]
 *     q, k  [B][L][H][dk]
 *     v     [B][L][H][dv]
 *     g, b  [B][L][H]
 *     o     [B][L][H][dv]
 *
 * Every entry point works independently on each (instance, head) pair, which
 * is what makes the OpenMP loop over pairs legal: no pair reads another's data.
 *
 * Pins (the oracle is checked against something other than itself in the
 * test suite): a=1,b=0 keeps S and gives o=S0 q; a=1,b=1,|k|=1 maps k to v;
 * b=0 gives S_t = exp(G_t) S0; basis keys overwrite columns; an exact rational
 * recurrence at dk=2..4; a hand-worked example; superposition, homogeneity and
 * row-permutation invariants; chunked == sequential.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of OpenMP threads the oracle will use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Sequential recurrence over L tokens for every (instance, head).
 *
 *   S0     initial state, [B][H][dv][dk]; never modified.
 *   keep   per-instance count of steps whose state is returned in S_out
 *          (0..L; 0 returns S0 unchanged, byte for byte).  NULL means L.
 *          This is the commit of the accepted prefix: S_out = S_{keep[b]}.
 *   o      outputs for all L tokens, or NULL.
 *   S_out  state after keep[b] steps, or NULL.  May not alias S0.
 *
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_gdn_seq(int B, int H, int dk, int dv, int L,
                   const double *S0, const double *q, const double *k,
                   const double *v, const double *g, const double *beta,
                   const int *keep, double *o, double *S_out) {
    if (B < 0 || H < 0 || dk < 1 || dv < 1 || L < 0) return -1;
    if (keep) {
        for (int b = 0; b < B; ++b)
            if (keep[b] < 0 || keep[b] > L) return -1;
    }
    const size_t state_sz = (size_t)dv * dk;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long pair = 0; pair < (long)B * H; ++pair) {
        const int b = (int)(pair / H), h = (int)(pair % H);
        const double *s0 = S0 + (size_t)pair * state_sz;
        double *S = (double *)malloc(state_sz * sizeof(double));
        if (!S) { failed = 1; continue; }
        memcpy(S, s0, state_sz * sizeof(double));
        const int n_keep = keep ? keep[b] : L;
        if (S_out && n_keep == 0)
            memcpy(S_out + (size_t)pair * state_sz, s0, state_sz * sizeof(double));
        /* Tokens past the kept prefix are only needed for outputs. */
        const int steps = o ? L : n_keep;
        for (int t = 0; t < steps; ++t) {
            const size_t row = (size_t)b * L + t;              /* (b, t) */
            const double *kt = k + (row * H + h) * dk;
            const double *qt = q + (row * H + h) * dk;
            const double *vt = v + (row * H + h) * dv;
            const double a = exp(g[row * H + h]);
            const double bt = beta[row * H + h];
            double *ot = o ? o + (row * H + h) * dv : NULL;
            for (int i = 0; i < dv; ++i) {
                double *Si = S + (size_t)i * dk;
                double u = 0.0;
                for (int j = 0; j < dk; ++j) u += Si[j] * kt[j];
                const double d = bt * (vt[i] - a * u);
                for (int j = 0; j < dk; ++j) Si[j] = a * Si[j] + d * kt[j];
                if (ot) {
                    double acc = 0.0;
                    for (int j = 0; j < dk; ++j) acc += Si[j] * qt[j];
                    ot[i] = acc;
                }
            }
            if (S_out && t + 1 == n_keep)
                memcpy(S_out + (size_t)pair * state_sz, S, state_sz * sizeof(double));
        }
        free(S);
    }
    return failed ? -1 : 0;
}

/*
 * Chunked (UT / WY) form of the same recurrence, in fp64.  It exists to check
 * the chunk algebra that a blocked implementation relies on against the plain
 * sequential definition above; it is not the reference the GPU is judged by.
 *
 * Per chunk of C tokens (the last one may be shorter), with the log-decay
 * prefix G_t = sum of g over the chunk up to t (restarted at every chunk),
 * gamma_t = exp(G_t) and Gamma_tj = exp(G_t - G_j):
 *
 *   A   = strictly-lower( b_t Gamma_tj k_t.k_j )
 *   Tm  = (I + A)^{-1} diag(b)                   (forward substitution)
 *   U   = Tm V,      W = Tm diag(gamma) K
 *   D   = U - W S^T                               (the chunk's delta rows)
 *   O   = diag(gamma) Q S^T + lower-incl( Gamma o Q K^T ) D
 *   S  <- gamma_last S + D^T diag(exp(G_last - G)) K
 *
 * Decays appear only as exp of a difference of prefix sums (never 1/gamma).
 * S is updated in place: on entry the initial state, on exit the final one.
 */
int oracle_gdn_chunked(int B, int H, int dk, int dv, int L, int C,
                       double *S, const double *q, const double *k,
                       const double *v, const double *g, const double *beta,
                       double *o) {
    if (B < 0 || H < 0 || dk < 1 || dv < 1 || L < 0 || C < 1) return -1;
    const size_t state_sz = (size_t)dv * dk;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long pair = 0; pair < (long)B * H; ++pair) {
        const int b = (int)(pair / H), h = (int)(pair % H);
        double *Sh = S + (size_t)pair * state_sz;
        double *G = (double *)malloc((size_t)C * sizeof(double));
        double *Tm = (double *)malloc((size_t)C * C * sizeof(double));
        double *W = (double *)malloc((size_t)C * dk * sizeof(double));
        double *D = (double *)malloc((size_t)C * dv * sizeof(double));
        double *Sn = (double *)malloc(state_sz * sizeof(double));
        if (!G || !Tm || !W || !D || !Sn) {
            failed = 1;
            free(G); free(Tm); free(W); free(D); free(Sn);
            continue;
        }
#define IDX(t) (((size_t)b * L + (size_t)(t)) * H + h)
        for (int c0 = 0; c0 < L; c0 += C) {
            const int n = (L - c0 < C) ? (L - c0) : C;
            /* Log-decay prefix sums within the chunk. */
            double acc = 0.0;
            for (int t = 0; t < n; ++t) { acc += g[IDX(c0 + t)]; G[t] = acc; }
            /* Tm = (I + A)^{-1} diag(b): solve (I + A) Tm = diag(b) row by
               row, since I + A is unit lower triangular. */
            for (int t = 0; t < n; ++t) {
                const double bt = beta[IDX(c0 + t)];
                const double *kt = k + IDX(c0 + t) * dk;
                for (int col = 0; col < n; ++col) Tm[(size_t)t * C + col] = (col == t) ? bt : 0.0;
                for (int j = 0; j < t; ++j) {
                    const double *kj = k + IDX(c0 + j) * dk;
                    double kk = 0.0;
                    for (int m = 0; m < dk; ++m) kk += kt[m] * kj[m];
                    const double A_tj = bt * exp(G[t] - G[j]) * kk;
                    for (int col = 0; col <= j; ++col)
                        Tm[(size_t)t * C + col] -= A_tj * Tm[(size_t)j * C + col];
                }
            }
            /* W = Tm diag(gamma) K. */
            for (int t = 0; t < n; ++t)
                for (int m = 0; m < dk; ++m) {
                    double s = 0.0;
                    for (int j = 0; j <= t; ++j)
                        s += Tm[(size_t)t * C + j] * exp(G[j]) * k[IDX(c0 + j) * dk + m];
                    W[(size_t)t * dk + m] = s;
                }
            /* D = Tm V - W S^T. */
            for (int t = 0; t < n; ++t)
                for (int i = 0; i < dv; ++i) {
                    double u = 0.0;
                    for (int j = 0; j <= t; ++j)
                        u += Tm[(size_t)t * C + j] * v[IDX(c0 + j) * dv + i];
                    double ws = 0.0;
                    for (int m = 0; m < dk; ++m) ws += W[(size_t)t * dk + m] * Sh[(size_t)i * dk + m];
                    D[(size_t)t * dv + i] = u - ws;
                }
            /* O = diag(gamma) Q S^T + lower-incl(Gamma o Q K^T) D. */
            if (o) {
                for (int t = 0; t < n; ++t) {
                    const double *qt = q + IDX(c0 + t) * dk;
                    double *ot = o + IDX(c0 + t) * dv;
                    const double gam = exp(G[t]);
                    for (int i = 0; i < dv; ++i) {
                        double qs = 0.0;
                        for (int m = 0; m < dk; ++m) qs += qt[m] * Sh[(size_t)i * dk + m];
                        ot[i] = gam * qs;
                    }
                    for (int j = 0; j <= t; ++j) {
                        const double *kj = k + IDX(c0 + j) * dk;
                        double qk = 0.0;
                        for (int m = 0; m < dk; ++m) qk += qt[m] * kj[m];
                        const double P_tj = exp(G[t] - G[j]) * qk;
                        for (int i = 0; i < dv; ++i) ot[i] += P_tj * D[(size_t)j * dv + i];
                    }
                }
            }
            /* S <- gamma_last S + D^T diag(exp(G_last - G)) K. */
            const double glast = G[n - 1];
            for (int i = 0; i < dv; ++i)
                for (int m = 0; m < dk; ++m) {
                    double s = exp(glast) * Sh[(size_t)i * dk + m];
                    for (int j = 0; j < n; ++j)
                        s += D[(size_t)j * dv + i] * exp(glast - G[j]) * k[IDX(c0 + j) * dk + m];
                    Sn[(size_t)i * dk + m] = s;
                }
            memcpy(Sh, Sn, state_sz * sizeof(double));
        }
#undef IDX
        free(G); free(Tm); free(W); free(D); free(Sn);
    }
    return failed ? -1 : 0;
}
