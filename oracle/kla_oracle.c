/*
 * kla_oracle.c -- fp64 CPU oracle for the Kalman Linear Attention forward pass
 * (and its backward pass, kla_oracle_bwd, at the end of this file).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  The product
 * path (the HIP library under scan_amd/) never includes, links or calls it,
 * and this file includes nothing from there.
 *
 * Sources (cited by title and section):
 *  [KLA]  "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient
 *         Language Modelling and State Tracking", gist.science explainer,
 *         technical summary (技術要約) > method (手法) §1-§3.
 *  [KDN]  "Kalman Delta Networks: Uncertainty-aware Associative Memory",
 *         abstract (fugumt page): diagonal and isotropic variants.
 *
 * What is computed.  [KLA] method §1 models the memory as a linear-Gaussian
 * state-space model: an exactly discretised OU prior (decay a, process noise
 * qn), noisy observations through the key k with observation noise r (the
 * value precision is 1/r), and a readout of the posterior mean through the
 * query q.  The filter runs in information form (precision l, information
 * eta = l * mean), [KLA] method §2.  The pages give the Mobius form of the
 * precision map but not its coefficients, so this library fixes one concrete
 * recurrence; it is the exact Kalman filter of the independent scalar chains
 *     x_t[i,j] = a_t[i] x_{t-1}[i,j] + N(0, qn[i]),
 *     v_t[j]   = k_t[i] x_t[i,j]     + N(0, r_t),
 * i.e. the diagonal (mean-field) family of [KDN]:
 *
 *   predict:  lp          = l / (a^2 + qn*l)           (variance a^2/l + qn)
 *   gate:     g           = lp * a / l                  (information carried)
 *   update:   l_t         = lp + k^2 / r
 *             eta_t[i,:]  = g * eta_{t-1}[i,:] + k * v_t / r
 *   readout:  o_t         = sum_i q_t[i] * eta_t[i,:] / l_t[i]
 *
 * The readout uses the posterior at t (token t included).  Isotropic mode
 * ([KDN]: one uncertainty scalar per head) keeps a scalar l per head with
 * per-token a_t and qn_t, and takes the precision increment as the
 * trace-matched isotropic projection b_t = sum_i k_t[i]^2 / (d_k r_t); the
 * information rows are updated exactly as above with the scalar gate.
 *
 * No blocking, no reordering: a plain sequential loop over t per (b,h),
 * OpenMP only across independent (b,h) sequences.
 *
 * Layouts (dense, row-major):
 *   q,k [B,H,T,dk]  v,o [B,H,T,dv]  r [B,H,T]
 *   diag: a [B,H,T,dk]  qn [H,dk]   l0,lT [B,H,dk]
 *   iso:  a [B,H,T]     qn [B,H,T]  l0,lT [B,H]
 *   eta0,etaT [B,H,dk,dv]
 * l0 == NULL means l0 = 1, eta0 == NULL means eta0 = 0.  lT, etaT, l_all
 * (the precision after every token: [B,H,T,dk] or [B,H,T]) may be NULL.
 */
#include <stdlib.h>
#include <string.h>

#define KLA_ORACLE_DIAG 0
#define KLA_ORACLE_ISO 1

static void run_sequence(int T, int dk, int dv, int cov,
                         const double* q, const double* k, const double* v,
                         const double* a, const double* qn, const double* r,
                         double* l, double* eta, double* o, double* l_all,
                         double* lnew)
{
    for (int t = 0; t < T; ++t) {
        const double* qt = q + (size_t)t * dk;
        const double* kt = k + (size_t)t * dk;
        const double* vt = v + (size_t)t * dv;
        const double rt = r[t];
        if (cov == KLA_ORACLE_DIAG) {
            const double* at = a + (size_t)t * dk;
            for (int i = 0; i < dk; ++i) {
                const double lprev = l[i];
                const double lp = lprev / (at[i] * at[i] + qn[i] * lprev);
                const double g = lp * at[i] / lprev;
                lnew[i] = lp + kt[i] * kt[i] / rt;
                double* row = eta + (size_t)i * dv;
                for (int j = 0; j < dv; ++j)
                    row[j] = g * row[j] + kt[i] * vt[j] / rt;
            }
            for (int i = 0; i < dk; ++i) l[i] = lnew[i];
            if (l_all)
                for (int i = 0; i < dk; ++i) l_all[(size_t)t * dk + i] = l[i];
        } else {
            const double at = a[t];
            const double qt_noise = qn[t];
            double ksq = 0.0;
            for (int i = 0; i < dk; ++i) ksq += kt[i] * kt[i];
            const double lprev = l[0];
            const double lp = lprev / (at * at + qt_noise * lprev);
            const double g = lp * at / lprev;
            l[0] = lp + ksq / ((double)dk * rt);
            for (int i = 0; i < dk; ++i) {
                double* row = eta + (size_t)i * dv;
                for (int j = 0; j < dv; ++j)
                    row[j] = g * row[j] + kt[i] * vt[j] / rt;
            }
            if (l_all) l_all[t] = l[0];
        }
        double* ot = o + (size_t)t * dv;
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double li = (cov == KLA_ORACLE_DIAG) ? l[i] : l[0];
            const double* row = eta + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) ot[j] += qt[i] * row[j] / li;
        }
    }
}

/* Returns 0 on success, nonzero on bad arguments or allocation failure. */
int kla_oracle_fwd(int B, int H, int T, int dk, int dv, int cov,
                   const double* q, const double* k, const double* v,
                   const double* a, const double* qn, const double* r,
                   const double* l0, const double* eta0,
                   double* o, double* lT, double* etaT, double* l_all,
                   int nthreads)
{
    if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return 1;
    if (cov != KLA_ORACLE_DIAG && cov != KLA_ORACLE_ISO) return 1;
    if (!q || !k || !v || !a || !qn || !r || !o) return 1;
    const int nl = (cov == KLA_ORACLE_DIAG) ? dk : 1;
    const long long nseq = (long long)B * H;
    int failed = 0;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
    for (long long s = 0; s < nseq; ++s) {
        const int h = (int)(s % H);
        double* l = (double*)malloc(sizeof(double) * (size_t)nl);
        double* lnew = (double*)malloc(sizeof(double) * (size_t)nl);
        double* eta = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        if (!l || !lnew || !eta) {
            free(l); free(lnew); free(eta);
            failed |= 1;
            continue;
        }
        for (int i = 0; i < nl; ++i) l[i] = l0 ? l0[s * nl + i] : 1.0;
        for (size_t e = 0; e < (size_t)dk * dv; ++e)
            eta[e] = eta0 ? eta0[(size_t)s * dk * dv + e] : 0.0;

        const size_t tk = (size_t)s * T * dk, tv = (size_t)s * T * dv;
        const double* as;
        const double* qns;
        if (cov == KLA_ORACLE_DIAG) {
            as = a + tk;
            qns = qn + (size_t)h * dk;
        } else {
            as = a + (size_t)s * T;
            qns = qn + (size_t)s * T;
        }
        run_sequence(T, dk, dv, cov, q + tk, k + tk, v + tv, as, qns,
                     r + (size_t)s * T, l, eta, o + tv,
                     l_all ? l_all + (size_t)s * T * nl : NULL, lnew);
        if (lT)
            for (int i = 0; i < nl; ++i) lT[s * nl + i] = l[i];
        if (etaT)
            memcpy(etaT + (size_t)s * dk * dv, eta, sizeof(double) * (size_t)dk * dv);
        free(l); free(lnew); free(eta);
    }
    return failed;
}

/*
 * One decode step for every (b,h): the same recurrence with T = 1, state
 * updated in place.  q,k [B,H,dk]; v,o [B,H,dv]; r [B,H]; diag: a [B,H,dk],
 * qn [H,dk], l [B,H,dk]; iso: a, qn, l [B,H]; eta [B,H,dk,dv].
 */
int kla_oracle_step(int B, int H, int dk, int dv, int cov,
                    const double* q, const double* k, const double* v,
                    const double* a, const double* qn, const double* r,
                    double* l, double* eta, double* o, int nthreads)
{
    if (!l || !eta) return 1;
    /* With T = 1 the per-sequence layouts of fwd coincide with step's. */
    return kla_oracle_fwd(B, H, 1, dk, dv, cov, q, k, v, a, qn, r, l, eta,
                          o, l, eta, NULL, nthreads);
}

/*
 * Residual-write forward (the Kalman-gain-weighted residual write of [KDN]).
 *
 * The memory x_t (dk x dv) is observed through the full key contraction,
 *     v_t[j] = sum_i k_t[i] x_t[i,j] + N(0, r_t),
 * with the same OU transition per row as above.  Each one-step posterior is
 * projected onto the diagonal (or isotropic) Gaussian family by mean-field
 * variational inference, which keeps the exact posterior mean and takes the
 * diagonal of the posterior precision (its trace average for the isotropic
 * family).  The state is (l, m) with m the posterior mean (mean form, not
 * information form):
 *
 *   predict:  lp   = l / (a^2 + qn*l),   m_pred = a (.) m   (row i scaled by a_i)
 *   gain:     g_i  = (k_i / lp_i) / (sum_j k_j^2 / lp_j + r)
 *   residual: u    = v - m_pred^T k
 *   update:   m_t  = m_pred + g u^T,      l_t = lp + k^2 / r
 *   readout:  o_t  = m_t^T q_t
 *
 * Isotropic mode: one lp per head, g = k / (|k|^2 + r lp), and
 * l_t = lp + |k|^2 / (d_k r).  Same layouts and conventions as
 * kla_oracle_fwd, with m0/mT (the mean) in place of eta0/etaT.
 */
static void run_sequence_residual(int T, int dk, int dv, int cov,
                                  const double* q, const double* k, const double* v,
                                  const double* a, const double* qn, const double* r,
                                  double* l, double* m, double* o, double* lp, double* g,
                                  double* u)
{
    for (int t = 0; t < T; ++t) {
        const double* qt = q + (size_t)t * dk;
        const double* kt = k + (size_t)t * dk;
        const double* vt = v + (size_t)t * dv;
        const double rt = r[t];
        /* predict: precision and mean */
        if (cov == KLA_ORACLE_DIAG) {
            const double* at = a + (size_t)t * dk;
            for (int i = 0; i < dk; ++i) {
                lp[i] = l[i] / (at[i] * at[i] + qn[i] * l[i]);
                for (int j = 0; j < dv; ++j) m[(size_t)i * dv + j] *= at[i];
            }
        } else {
            lp[0] = l[0] / (a[t] * a[t] + qn[t] * l[0]);
            for (size_t e = 0; e < (size_t)dk * dv; ++e) m[e] *= a[t];
        }
        /* gain */
        double s = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double lpi = (cov == KLA_ORACLE_DIAG) ? lp[i] : lp[0];
            s += kt[i] * kt[i] / lpi;
        }
        for (int i = 0; i < dk; ++i) {
            const double lpi = (cov == KLA_ORACLE_DIAG) ? lp[i] : lp[0];
            g[i] = (kt[i] / lpi) / (s + rt);
        }
        /* residual against the predicted mean, then the write */
        for (int j = 0; j < dv; ++j) {
            double pred = 0.0;
            for (int i = 0; i < dk; ++i) pred += m[(size_t)i * dv + j] * kt[i];
            u[j] = vt[j] - pred;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) m[(size_t)i * dv + j] += g[i] * u[j];
        /* precision update */
        if (cov == KLA_ORACLE_DIAG) {
            for (int i = 0; i < dk; ++i) l[i] = lp[i] + kt[i] * kt[i] / rt;
        } else {
            double ksq = 0.0;
            for (int i = 0; i < dk; ++i) ksq += kt[i] * kt[i];
            l[0] = lp[0] + ksq / ((double)dk * rt);
        }
        /* readout of the posterior mean */
        double* ot = o + (size_t)t * dv;
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += qt[i] * m[(size_t)i * dv + j];
            ot[j] = acc;
        }
    }
}

/* Returns 0 on success, nonzero on bad arguments or allocation failure. */
int kla_oracle_fwd_residual(int B, int H, int T, int dk, int dv, int cov,
                            const double* q, const double* k, const double* v,
                            const double* a, const double* qn, const double* r,
                            const double* l0, const double* m0,
                            double* o, double* lT, double* mT, int nthreads)
{
    if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return 1;
    if (cov != KLA_ORACLE_DIAG && cov != KLA_ORACLE_ISO) return 1;
    if (!q || !k || !v || !a || !qn || !r || !o) return 1;
    const int nl = (cov == KLA_ORACLE_DIAG) ? dk : 1;
    const long long nseq = (long long)B * H;
    int failed = 0;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
    for (long long s = 0; s < nseq; ++s) {
        const int h = (int)(s % H);
        double* l = (double*)malloc(sizeof(double) * (size_t)nl);
        double* lp = (double*)malloc(sizeof(double) * (size_t)nl);
        double* g = (double*)malloc(sizeof(double) * (size_t)dk);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        double* m = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        if (!l || !lp || !g || !u || !m) {
            free(l); free(lp); free(g); free(u); free(m);
            failed |= 1;
            continue;
        }
        for (int i = 0; i < nl; ++i) l[i] = l0 ? l0[s * nl + i] : 1.0;
        for (size_t e = 0; e < (size_t)dk * dv; ++e)
            m[e] = m0 ? m0[(size_t)s * dk * dv + e] : 0.0;

        const size_t tk = (size_t)s * T * dk, tv = (size_t)s * T * dv;
        const double* as;
        const double* qns;
        if (cov == KLA_ORACLE_DIAG) {
            as = a + tk;
            qns = qn + (size_t)h * dk;
        } else {
            as = a + (size_t)s * T;
            qns = qn + (size_t)s * T;
        }
        run_sequence_residual(T, dk, dv, cov, q + tk, k + tk, v + tv, as, qns,
                              r + (size_t)s * T, l, m, o + tv, lp, g, u);
        if (lT)
            for (int i = 0; i < nl; ++i) lT[s * nl + i] = l[i];
        if (mT)
            memcpy(mT + (size_t)s * dk * dv, m, sizeof(double) * (size_t)dk * dv);
        free(l); free(lp); free(g); free(u); free(m);
    }
    return failed;
}

/*
 * Backward pass of kla_oracle_fwd: reverse-mode adjoint of the sequential
 * recurrence above ("Kalman Linear Attention ...", fugumt abstract page: the
 * information-form filter is a primitive for parallel training, so its
 * gradients are part of the method).
 *
 * Given the upstream gradients dO = dL/do [B,H,T,dv], dlT = dL/dlT and
 * detaT = dL/detaT (either may be NULL = 0), it returns dL/dq, dL/dk, dL/dv,
 * dL/da, dL/dqn, dL/dr, dL/dl0, dL/deta0 of the scalar L.  Per (b,h) the
 * forward trajectory (l_t and eta_t for every t) is recomputed and kept, then
 * one reverse sweep applies the chain rule to each step of the forward, last
 * token first:
 *
 *   readout  o_t = sum_i q_t[i] eta_t[i,:] / l_t[i]
 *     dq_t[i]     = sum_j dO_t[j] eta_t[i,j] / l_t[i]
 *     ebar_t[i,:] += q_t[i] dO_t / l_t[i]
 *     lbar_t[i]   -= q_t[i] dq_t[i] / l_t[i]
 *   update   eta_t = g_t eta_{t-1} + k_t v_t^T / r_t,   g_t = a_t / D_t
 *     gbar_t[i]   = sum_j ebar_t[i,j] eta_{t-1}[i,j]
 *     dk_t[i]    += sum_j ebar_t[i,j] v_t[j] / r_t
 *     dv_t[j]     = sum_i ebar_t[i,j] k_t[i] / r_t
 *     dr_t       -= sum_ij ebar_t[i,j] k_t[i] v_t[j] / r_t^2
 *     ebar_{t-1}  = g_t ebar_t
 *   precision l_t = lp_t + k_t^2 / r_t,  lp_t = l_{t-1} / D_t,
 *             D_t = a_t^2 + qn l_{t-1}
 *     dk_t += lbar_t 2 k_t / r_t,  dr_t -= lbar_t k_t^2 / r_t^2
 *     lbar_{t-1} = lbar_t a_t^2 / D_t^2 - gbar_t a_t qn / D_t^2
 *     da_t       = -lbar_t 2 a_t l_{t-1} / D_t^2 + gbar_t (qn l_{t-1} - a_t^2) / D_t^2
 *     dqn       += -lbar_t l_{t-1}^2 / D_t^2 - gbar_t a_t l_{t-1} / D_t^2
 *
 * dl0 = lbar_{-1}, deta0 = ebar_{-1}.  Isotropic mode: the same with the
 * scalar l, g, D per head; the precision increment sum_i k_i^2 / (d_k r) gives
 * dk_t[i] += lbar_t 2 k_t[i] / (d_k r_t) and dr_t -= lbar_t sum_i k_t[i]^2 /
 * (d_k r_t^2), and gbar_t sums over every (i,j).  The diagonal qn [H,dk] is
 * shared by the batch, so its gradient is summed over b (in order of b);
 * the isotropic qn is per token.  Shapes as kla_oracle_fwd; da [B,H,T,dk]
 * (iso [B,H,T]); dqn [H,dk] (iso [B,H,T]); dl0 [B,H,dk] (iso [B,H]).
 * dl0 and deta0 may be NULL.  Returns 0 on success.
 */
static void adjoint_sequence(int T, int dk, int dv, int cov,
                             const double* q, const double* k, const double* v,
                             const double* a, const double* qn, const double* r,
                             const double* lstart, const double* etastart,
                             const double* dO, const double* dlT, const double* detaT,
                             double* dq, double* dkk, double* dvv, double* da, double* dqn_acc,
                             double* dr, double* dl0, double* deta0,
                             double* ltraj, double* etraj, double* lbar, double* ebar)
{
    const int nl = (cov == KLA_ORACLE_DIAG) ? dk : 1;
    const size_t ne = (size_t)dk * dv;
    /* forward trajectory: slot 0 holds the state before token 0, slot t+1
       the state after token t */
    for (int i = 0; i < nl; ++i) ltraj[i] = lstart ? lstart[i] : 1.0;
    for (size_t e = 0; e < ne; ++e) etraj[e] = etastart ? etastart[e] : 0.0;
    for (int t = 0; t < T; ++t) {
        const double* lo = ltraj + (size_t)t * nl;
        double* ln = ltraj + (size_t)(t + 1) * nl;
        const double* eo = etraj + (size_t)t * ne;
        double* en = etraj + (size_t)(t + 1) * ne;
        const double* kt = k + (size_t)t * dk;
        const double* vt = v + (size_t)t * dv;
        const double rt = r[t];
        if (cov == KLA_ORACLE_DIAG) {
            for (int i = 0; i < dk; ++i) {
                const double ai = a[(size_t)t * dk + i];
                const double den = ai * ai + qn[i] * lo[i];
                ln[i] = lo[i] / den + kt[i] * kt[i] / rt;
                for (int j = 0; j < dv; ++j)
                    en[(size_t)i * dv + j] = (ai / den) * eo[(size_t)i * dv + j] + kt[i] * vt[j] / rt;
            }
        } else {
            const double at = a[t];
            const double den = at * at + qn[t] * lo[0];
            double ksq = 0.0;
            for (int i = 0; i < dk; ++i) ksq += kt[i] * kt[i];
            ln[0] = lo[0] / den + ksq / ((double)dk * rt);
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    en[(size_t)i * dv + j] = (at / den) * eo[(size_t)i * dv + j] + kt[i] * vt[j] / rt;
        }
    }
    /* adjoints of the final state */
    for (int i = 0; i < nl; ++i) lbar[i] = dlT ? dlT[i] : 0.0;
    for (size_t e = 0; e < ne; ++e) ebar[e] = detaT ? detaT[e] : 0.0;
    for (int t = T - 1; t >= 0; --t) {
        const double* lt_ = ltraj + (size_t)(t + 1) * nl;   /* l_t     */
        const double* lp_ = ltraj + (size_t)t * nl;         /* l_{t-1} */
        const double* et_ = etraj + (size_t)(t + 1) * ne;   /* eta_t   */
        const double* ep_ = etraj + (size_t)t * ne;         /* eta_{t-1} */
        const double* qt = q + (size_t)t * dk;
        const double* kt = k + (size_t)t * dk;
        const double* vt = v + (size_t)t * dv;
        const double* dOt = dO + (size_t)t * dv;
        const double rt = r[t];
        /* readout */
        for (int i = 0; i < dk; ++i) {
            const double li = (cov == KLA_ORACLE_DIAG) ? lt_[i] : lt_[0];
            double s = 0.0;
            for (int j = 0; j < dv; ++j) s += dOt[j] * et_[(size_t)i * dv + j];
            dq[(size_t)t * dk + i] = s / li;
            for (int j = 0; j < dv; ++j) ebar[(size_t)i * dv + j] += qt[i] * dOt[j] / li;
            lbar[(cov == KLA_ORACLE_DIAG) ? i : 0] -= qt[i] * (s / li) / li;
        }
        /* information update */
        double gb_iso = 0.0, drt = 0.0;
        for (int j = 0; j < dv; ++j) dvv[(size_t)t * dv + j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            double gb = 0.0, u = 0.0;
            for (int j = 0; j < dv; ++j) {
                gb += ebar[(size_t)i * dv + j] * ep_[(size_t)i * dv + j];
                u += ebar[(size_t)i * dv + j] * vt[j];
                dvv[(size_t)t * dv + j] += ebar[(size_t)i * dv + j] * kt[i] / rt;
            }
            dkk[(size_t)t * dk + i] = u / rt;
            drt -= kt[i] * u / (rt * rt);
            if (cov == KLA_ORACLE_DIAG) {
                /* precision of key dim i, then carry the adjoints back */
                const double ai = a[(size_t)t * dk + i], lprev = lp_[i], qni = qn[i];
                const double den = ai * ai + qni * lprev, den2 = den * den;
                const double lb = lbar[i];
                dkk[(size_t)t * dk + i] += lb * 2.0 * kt[i] / rt;
                drt -= lb * kt[i] * kt[i] / (rt * rt);
                da[(size_t)t * dk + i] = -lb * 2.0 * ai * lprev / den2 + gb * (qni * lprev - ai * ai) / den2;
                dqn_acc[i] += -lb * lprev * lprev / den2 - gb * ai * lprev / den2;
                lbar[i] = lb * ai * ai / den2 - gb * ai * qni / den2;
                for (int j = 0; j < dv; ++j) ebar[(size_t)i * dv + j] *= ai / den;
            } else {
                gb_iso += gb;
            }
        }
        if (cov == KLA_ORACLE_ISO) {
            const double at = a[t], lprev = lp_[0], qnt = qn[t];
            const double den = at * at + qnt * lprev, den2 = den * den;
            const double lb = lbar[0];
            double ksq = 0.0;
            for (int i = 0; i < dk; ++i) {
                dkk[(size_t)t * dk + i] += lb * 2.0 * kt[i] / ((double)dk * rt);
                ksq += kt[i] * kt[i];
            }
            drt -= lb * ksq / ((double)dk * rt * rt);
            da[t] = -lb * 2.0 * at * lprev / den2 + gb_iso * (qnt * lprev - at * at) / den2;
            dqn_acc[t] = -lb * lprev * lprev / den2 - gb_iso * at * lprev / den2;
            lbar[0] = lb * at * at / den2 - gb_iso * at * qnt / den2;
            for (size_t e = 0; e < ne; ++e) ebar[e] *= at / den;
        }
        dr[t] = drt;
    }
    if (dl0)
        for (int i = 0; i < nl; ++i) dl0[i] = lbar[i];
    if (deta0) memcpy(deta0, ebar, sizeof(double) * ne);
}

int kla_oracle_bwd(int B, int H, int T, int dk, int dv, int cov,
                   const double* q, const double* k, const double* v,
                   const double* a, const double* qn, const double* r,
                   const double* l0, const double* eta0,
                   const double* dO, const double* dlT, const double* detaT,
                   double* dq, double* dk_out, double* dv_out, double* da, double* dqn,
                   double* dr, double* dl0, double* deta0, int nthreads)
{
    if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return 1;
    if (cov != KLA_ORACLE_DIAG && cov != KLA_ORACLE_ISO) return 1;
    if (T > 0 && (!q || !k || !v || !a || !qn || !r || !dO || !dq || !dk_out || !dv_out || !da || !dr))
        return 1;
    if (!dqn) return 1;
    const int nl = (cov == KLA_ORACLE_DIAG) ? dk : 1;
    const long long nseq = (long long)B * H;
    const size_t ne = (size_t)dk * dv;
    /* per-sequence partial of the diagonal qn gradient, summed over b below */
    double* dqn_part = NULL;
    if (cov == KLA_ORACLE_DIAG) {
        dqn_part = (double*)calloc((size_t)nseq * dk, sizeof(double));
        if (!dqn_part) return 1;
    }
    int failed = 0;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
    for (long long s = 0; s < nseq; ++s) {
        const int h = (int)(s % H);
        double* ltraj = (double*)malloc(sizeof(double) * (size_t)(T + 1) * nl);
        double* etraj = (double*)malloc(sizeof(double) * (size_t)(T + 1) * ne);
        double* lbar = (double*)malloc(sizeof(double) * (size_t)nl);
        double* ebar = (double*)malloc(sizeof(double) * ne);
        if (!ltraj || !etraj || !lbar || !ebar) {
            free(ltraj); free(etraj); free(lbar); free(ebar);
            failed |= 1;
            continue;
        }
        const size_t tk = (size_t)s * T * dk, tv = (size_t)s * T * dv;
        const double* as = (cov == KLA_ORACLE_DIAG) ? a + tk : a + (size_t)s * T;
        const double* qns = (cov == KLA_ORACLE_DIAG) ? qn + (size_t)h * dk : qn + (size_t)s * T;
        double* dqn_s = (cov == KLA_ORACLE_DIAG) ? dqn_part + (size_t)s * dk : dqn + (size_t)s * T;
        double* da_s = (cov == KLA_ORACLE_DIAG) ? da + tk : da + (size_t)s * T;
        adjoint_sequence(T, dk, dv, cov, q + tk, k + tk, v + tv, as, qns, r + (size_t)s * T,
                         l0 ? l0 + (size_t)s * nl : NULL, eta0 ? eta0 + (size_t)s * ne : NULL,
                         dO + tv, dlT ? dlT + (size_t)s * nl : NULL, detaT ? detaT + (size_t)s * ne : NULL,
                         dq + tk, dk_out + tk, dv_out + tv, da_s, dqn_s, dr + (size_t)s * T,
                         dl0 ? dl0 + (size_t)s * nl : NULL, deta0 ? deta0 + (size_t)s * ne : NULL,
                         ltraj, etraj, lbar, ebar);
        free(ltraj); free(etraj); free(lbar); free(ebar);
    }
    if (cov == KLA_ORACLE_DIAG) {
        for (int hh = 0; hh < H; ++hh)
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int b = 0; b < B; ++b) acc += dqn_part[((size_t)b * H + hh) * dk + i];
                dqn[(size_t)hh * dk + i] = acc;
            }
        free(dqn_part);
    }
    return failed;
}
