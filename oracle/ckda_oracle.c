/*
 * ckda_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, float64 CPU reference for the Complex KDA (CKDA) recurrence.
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg may load it; the GPU library never links or calls it, and the two share
 * no source.  Built with -O2 -ffp-contract=off so that every product and sum
 * is rounded exactly where it is written.
 *
 * What is computed (one head, one sequence; "chain" below), token by token:
 *
 *   alpha_t = s_t * exp(g_t)                 signed per-channel gate, s = +-1
 *   S      <- Diag(alpha_t) S                gate first ...
 *   p       = S^T k_t
 *   u       = beta_t (v_t - p)
 *   S      <- S + k_t u^T                    ... then the delta-rule correction,
 *                                            i.e. S_t = (I - beta k k^T) Diag(alpha) S_{t-1}
 *                                                       + beta k v^T
 *   o_t     = scale * S^T q_t                output read after the update
 *
 * with S in R^{DK x DV}.  Sources: the Complex KDA paper page, section 3
 * ("CKDA." paragraph: KDA with gates in [-1,1] and beta in [0,2]) and section 2
 * ("Linear RNNs": DeltaNet's I - beta k k^T acting on the columns of the state,
 * KDA's channel-wise gate); section 4 (a CKDA transform is the element-wise
 * scaling followed by the Householder-type part, which fixes the order above);
 * the model card "complex-kda-1.3B-100B" (gate carried as log-magnitude plus a
 * sign).  The formulas themselves are missing from the extracted page text;
 * the order "gate, then correction, then output" is the reading adopted here.
 *
 * ckda_ref_fwd_folded() runs the same recurrence the way the model card says
 * the kernels do: the running +-1 product P_t of the signs is pushed onto q and
 * k, the state is kept in the folded frame Diag(P_t) S_t and only exp(g) ever
 * multiplies it.  It exists to pin that the fold is exact.
 *
 * ckda_ref_bwd() is reverse-mode differentiation of L = <do, o> + <dST, S_T>
 * through the token recurrence above, with per-token states recomputed from
 * checkpoints taken every `every` tokens.  The sign s gets no gradient; the
 * gradient w.r.t. g = log|alpha| is alpha * dL/dalpha.
 *
 * Layouts: every chain is contiguous.  q,k,g,s: [n][T][DK]; v,o,do,dv: [n][T][DV];
 * beta: [n][T]; states: [n][DK][DV] (row c = key channel, column j = value channel).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the signed recurrence on one chain.  S is updated in place.
 * p, u: scratch of length DV.  If o != NULL, writes o[0..DV). */
static void token_step(int DK, int DV, const double* q, const double* k, const double* v,
                       const double* g, const double* s, double beta, double scale,
                       double* S, double* p, double* u, double* o)
{
    for (int c = 0; c < DK; ++c) {
        const double a = s[c] * exp(g[c]);
        double* row = S + (size_t)c * DV;
        for (int j = 0; j < DV; ++j) row[j] = a * row[j];
    }
    for (int j = 0; j < DV; ++j) p[j] = 0.0;
    for (int c = 0; c < DK; ++c) {
        const double* row = S + (size_t)c * DV;
        for (int j = 0; j < DV; ++j) p[j] += row[j] * k[c];
    }
    for (int j = 0; j < DV; ++j) u[j] = beta * (v[j] - p[j]);
    for (int c = 0; c < DK; ++c) {
        double* row = S + (size_t)c * DV;
        for (int j = 0; j < DV; ++j) row[j] += k[c] * u[j];
    }
    if (o) {
        for (int j = 0; j < DV; ++j) o[j] = 0.0;
        for (int c = 0; c < DK; ++c) {
            const double* row = S + (size_t)c * DV;
            for (int j = 0; j < DV; ++j) o[j] += row[j] * q[c];
        }
        for (int j = 0; j < DV; ++j) o[j] *= scale;
    }
}

int ckda_ref_fwd(int n, int T, int DK, int DV,
                 const double* q, const double* k, const double* v,
                 const double* g, const double* s, const double* beta, double scale,
                 const double* S0, double* o, double* ST)
{
    if (n < 0 || T < 0 || DK <= 0 || DV <= 0) return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ch = 0; ch < n; ++ch) {
        const size_t sk = (size_t)T * DK, sv = (size_t)T * DV, ss = (size_t)DK * DV;
        double* S = (double*)malloc(ss * sizeof(double));
        double* p = (double*)malloc(DV * sizeof(double));
        double* u = (double*)malloc(DV * sizeof(double));
        if (!S || !p || !u) {
            err = -2;
        } else {
            if (S0) memcpy(S, S0 + ch * ss, ss * sizeof(double));
            else memset(S, 0, ss * sizeof(double));
            for (int t = 0; t < T; ++t) {
                token_step(DK, DV, q + ch * sk + (size_t)t * DK, k + ch * sk + (size_t)t * DK,
                           v + ch * sv + (size_t)t * DV, g + ch * sk + (size_t)t * DK,
                           s + ch * sk + (size_t)t * DK, beta[(size_t)ch * T + t], scale, S, p, u,
                           o ? o + ch * sv + (size_t)t * DV : NULL);
            }
            if (ST) memcpy(ST + ch * ss, S, ss * sizeof(double));
        }
        free(S); free(p); free(u);
    }
    return err;
}

/* Folded frame: St = Diag(P_t) S_t with P_t = prod_{tau<=t} s_tau (P_{-1} = +1
 * unless P0 is given).  The true state enters as Diag(P0) S0; on return ST holds
 * the TRUE final state Diag(P_T) St and PT the final sign product. */
int ckda_ref_fwd_folded(int n, int T, int DK, int DV,
                        const double* q, const double* k, const double* v,
                        const double* g, const double* s, const double* beta, double scale,
                        const double* S0, const double* P0, double* o, double* ST, double* PT)
{
    if (n < 0 || T < 0 || DK <= 0 || DV <= 0) return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ch = 0; ch < n; ++ch) {
        const size_t sk = (size_t)T * DK, sv = (size_t)T * DV, ss = (size_t)DK * DV;
        double* S = (double*)malloc(ss * sizeof(double));
        double* P = (double*)malloc(DK * sizeof(double));
        double* qt = (double*)malloc(DK * sizeof(double));
        double* kt = (double*)malloc(DK * sizeof(double));
        double* one = (double*)malloc(DK * sizeof(double));
        double* p = (double*)malloc(DV * sizeof(double));
        double* u = (double*)malloc(DV * sizeof(double));
        if (!S || !P || !qt || !kt || !one || !p || !u) {
            err = -2;
        } else {
            for (int c = 0; c < DK; ++c) { P[c] = P0 ? P0[(size_t)ch * DK + c] : 1.0; one[c] = 1.0; }
            /* folded state = Diag(P) * true state */
            for (int c = 0; c < DK; ++c)
                for (int j = 0; j < DV; ++j)
                    S[(size_t)c * DV + j] = S0 ? P[c] * S0[ch * ss + (size_t)c * DV + j] : 0.0;
            for (int t = 0; t < T; ++t) {
                const double* st = s + ch * sk + (size_t)t * DK;
                for (int c = 0; c < DK; ++c) {
                    P[c] = P[c] * st[c];
                    qt[c] = P[c] * q[ch * sk + (size_t)t * DK + c];
                    kt[c] = P[c] * k[ch * sk + (size_t)t * DK + c];
                }
                /* unsigned recurrence: gate magnitude only (sign +1 everywhere) */
                token_step(DK, DV, qt, kt, v + ch * sv + (size_t)t * DV, g + ch * sk + (size_t)t * DK,
                           one, beta[(size_t)ch * T + t], scale, S, p, u,
                           o ? o + ch * sv + (size_t)t * DV : NULL);
            }
            if (ST)
                for (int c = 0; c < DK; ++c)
                    for (int j = 0; j < DV; ++j)
                        ST[ch * ss + (size_t)c * DV + j] = P[c] * S[(size_t)c * DV + j];
            if (PT) memcpy(PT + (size_t)ch * DK, P, DK * sizeof(double));
        }
        free(S); free(P); free(qt); free(kt); free(one); free(p); free(u);
    }
    return err;
}

/* Reverse mode through one token.  Spre = S_{t-1} (state before the token).
 * dS holds dL/dS_t on entry and dL/dS_{t-1} on return.  Work arrays:
 * Sa, St: DK*DV; p, u, du: DV. */
static void token_bwd(int DK, int DV, const double* q, const double* k, const double* v,
                      const double* g, const double* s, double beta, double scale,
                      const double* Spre, const double* dot, double* dS,
                      double* dq, double* dk, double* dv, double* dg, double* dbeta,
                      double* Sa, double* St, double* p, double* u, double* du)
{
    const size_t ss = (size_t)DK * DV;
    /* recompute the forward token */
    for (int c = 0; c < DK; ++c) {
        const double a = s[c] * exp(g[c]);
        for (int j = 0; j < DV; ++j) Sa[(size_t)c * DV + j] = a * Spre[(size_t)c * DV + j];
    }
    for (int j = 0; j < DV; ++j) p[j] = 0.0;
    for (int c = 0; c < DK; ++c)
        for (int j = 0; j < DV; ++j) p[j] += Sa[(size_t)c * DV + j] * k[c];
    for (int j = 0; j < DV; ++j) u[j] = beta * (v[j] - p[j]);
    for (size_t e = 0; e < ss; ++e) St[e] = Sa[e];
    for (int c = 0; c < DK; ++c)
        for (int j = 0; j < DV; ++j) St[(size_t)c * DV + j] += k[c] * u[j];

    /* o = scale * St^T q */
    for (int c = 0; c < DK; ++c) {
        double acc = 0.0;
        for (int j = 0; j < DV; ++j) acc += St[(size_t)c * DV + j] * dot[j];
        dq[c] = scale * acc;
    }
    for (int c = 0; c < DK; ++c)
        for (int j = 0; j < DV; ++j) dS[(size_t)c * DV + j] += scale * q[c] * dot[j];
    /* St = Sa + k u^T */
    for (int c = 0; c < DK; ++c) {
        double acc = 0.0;
        for (int j = 0; j < DV; ++j) acc += dS[(size_t)c * DV + j] * u[j];
        dk[c] = acc;
    }
    for (int j = 0; j < DV; ++j) du[j] = 0.0;
    for (int c = 0; c < DK; ++c)
        for (int j = 0; j < DV; ++j) du[j] += dS[(size_t)c * DV + j] * k[c];
    /* u = beta (v - p) */
    double db = 0.0;
    for (int j = 0; j < DV; ++j) db += du[j] * (v[j] - p[j]);
    *dbeta = db;
    for (int j = 0; j < DV; ++j) dv[j] = beta * du[j];
    /* dp = -beta du ; p = Sa^T k  => dSa = dS + k dp^T, dk += Sa dp */
    for (int j = 0; j < DV; ++j) du[j] = -beta * du[j]; /* du now holds dp */
    for (int c = 0; c < DK; ++c) {
        double acc = 0.0;
        for (int j = 0; j < DV; ++j) acc += Sa[(size_t)c * DV + j] * du[j];
        dk[c] += acc;
    }
    for (int c = 0; c < DK; ++c)
        for (int j = 0; j < DV; ++j) dS[(size_t)c * DV + j] += k[c] * du[j];
    /* Sa = Diag(alpha) Spre, alpha = s exp(g):
     * dL/dg_c = alpha_c * sum_j dSa[c][j] Spre[c][j] = sum_j dSa[c][j] Sa[c][j] */
    for (int c = 0; c < DK; ++c) {
        double acc = 0.0;
        for (int j = 0; j < DV; ++j) acc += dS[(size_t)c * DV + j] * Sa[(size_t)c * DV + j];
        dg[c] = acc;
        const double a = s[c] * exp(g[c]);
        for (int j = 0; j < DV; ++j) dS[(size_t)c * DV + j] = a * dS[(size_t)c * DV + j];
    }
}

int ckda_ref_bwd(int n, int T, int DK, int DV,
                 const double* q, const double* k, const double* v,
                 const double* g, const double* s, const double* beta, double scale,
                 const double* S0, const double* dO, const double* dST, int every,
                 double* dq, double* dk, double* dv, double* dg, double* dbeta, double* dS0)
{
    if (n < 0 || T < 0 || DK <= 0 || DV <= 0 || every <= 0) return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ch = 0; ch < n; ++ch) {
        const size_t sk = (size_t)T * DK, sv = (size_t)T * DV, ss = (size_t)DK * DV;
        const int nseg = (T + every - 1) / every;
        double* ck = (double*)malloc(((size_t)nseg + 1) * ss * sizeof(double));
        double* seg = (double*)malloc((size_t)every * ss * sizeof(double));
        double* S = (double*)malloc(ss * sizeof(double));
        double* dS = (double*)malloc(ss * sizeof(double));
        double* Sa = (double*)malloc(ss * sizeof(double));
        double* St = (double*)malloc(ss * sizeof(double));
        double* p = (double*)malloc(DV * sizeof(double));
        double* u = (double*)malloc(DV * sizeof(double));
        double* du = (double*)malloc(DV * sizeof(double));
        if (!ck || !seg || !S || !dS || !Sa || !St || !p || !u || !du) {
            err = -2;
        } else {
            /* forward: checkpoint the state before tokens 0, every, 2*every, ... */
            if (S0) memcpy(S, S0 + ch * ss, ss * sizeof(double));
            else memset(S, 0, ss * sizeof(double));
            for (int t = 0; t < T; ++t) {
                if (t % every == 0) memcpy(ck + (size_t)(t / every) * ss, S, ss * sizeof(double));
                token_step(DK, DV, q + ch * sk + (size_t)t * DK, k + ch * sk + (size_t)t * DK,
                           v + ch * sv + (size_t)t * DV, g + ch * sk + (size_t)t * DK,
                           s + ch * sk + (size_t)t * DK, beta[(size_t)ch * T + t], scale, S, p, u, NULL);
            }
            if (dST) memcpy(dS, dST + ch * ss, ss * sizeof(double));
            else memset(dS, 0, ss * sizeof(double));
            for (int sg = nseg - 1; sg >= 0; --sg) {
                const int t0 = sg * every;
                const int t1 = (t0 + every < T) ? t0 + every : T;
                /* recompute the states before each token of the segment */
                memcpy(S, ck + (size_t)sg * ss, ss * sizeof(double));
                for (int t = t0; t < t1; ++t) {
                    memcpy(seg + (size_t)(t - t0) * ss, S, ss * sizeof(double));
                    token_step(DK, DV, q + ch * sk + (size_t)t * DK, k + ch * sk + (size_t)t * DK,
                               v + ch * sv + (size_t)t * DV, g + ch * sk + (size_t)t * DK,
                               s + ch * sk + (size_t)t * DK, beta[(size_t)ch * T + t], scale, S, p, u, NULL);
                }
                for (int t = t1 - 1; t >= t0; --t) {
                    token_bwd(DK, DV, q + ch * sk + (size_t)t * DK, k + ch * sk + (size_t)t * DK,
                              v + ch * sv + (size_t)t * DV, g + ch * sk + (size_t)t * DK,
                              s + ch * sk + (size_t)t * DK, beta[(size_t)ch * T + t], scale,
                              seg + (size_t)(t - t0) * ss, dO + ch * sv + (size_t)t * DV, dS,
                              dq + ch * sk + (size_t)t * DK, dk + ch * sk + (size_t)t * DK,
                              dv + ch * sv + (size_t)t * DV, dg + ch * sk + (size_t)t * DK,
                              dbeta + (size_t)ch * T + t, Sa, St, p, u, du);
                }
            }
            if (dS0) memcpy(dS0 + ch * ss, dS, ss * sizeof(double));
        }
        free(ck); free(seg); free(S); free(dS); free(Sa); free(St); free(p); free(u); free(du);
    }
    return err;
}

void ckda_ref_set_threads(int nt)
{
#ifdef _OPENMP
    if (nt > 0) omp_set_num_threads(nt);
#else
    (void)nt;
#endif
}

int ckda_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
