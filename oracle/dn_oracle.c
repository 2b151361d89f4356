/*
 * dn_oracle.c -- plain, slow fp64 CPU reference of the (gated) delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header or table with
 * the HIP library, and it is never a fallback for it.
 *
 * What it computes, token by token, for every (sequence, value head) pair:
 *
 *   The state S is a map from keys to values (S k = v), so it is d_v x d_k.
 *   Frankenstein "DeltaNet Attention" page, module docstring (the update equation):
 *       S_t = S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T .
 *   Mutichung garden "DeltaNet" page, section "The Delta Rule" (the same update in
 *   error-correction form, which is what is coded here):
 *       S_t = S_{t-1} - beta_t (S_{t-1} k_t - v_t) k_t^T .
 *   nnterp "linear_attention" page, LinearAttention class text: for each token the
 *   state first decays by the gate, then takes up the beta-scaled key/value pair,
 *   then the query reads against it.  The gate ("decays") is the log of the
 *   fraction of the state kept, so the decay factor is exp(g_t):
 *       S'_t = exp(g_t) S_{t-1},   S_t = S'_t - beta_t (S'_t k_t - v_t) k_t^T,
 *       o_t  = scale * S_t q_t      (read after the write; scale = 1 on the pages).
 *   A missing gate (g == NULL) is the plain rule (exp(0) = 1).
 *   Channel gates (gdim == Dk): the nnterp page types a gate per key channel,
 *   [batch, seq, heads, key_dim] ("ChannelGates", the KDA variant).  Read as the same
 *   gate taken per key channel: S'_t = S_{t-1} diag(exp(g_t)), i.e. column i of S (the
 *   state's weights on key channel i) keeps the fraction exp(g_t[i]).
 *   Optional in-rule normalisation (qk_l2norm != 0): the frankenstein class text
 *   L2-normalises queries and keys before the rule, and the mutichung DeltaNet block
 *   flowchart puts an "L2 Norm" on q and k right before the "Delta Rule" box; the
 *   nnterp queries/keys accessors list the conv, the activation and the head repeat
 *   but no normalisation, so the rule itself may be handed raw q and k.  Each q_t
 *   and k_t (per query/key head) is then replaced by x / sqrt(sum_i x_i^2 + eps)
 *   before it is used (eps keeps a zero vector at zero; the pages give no value).
 *   The nnterp page's state_input: None on a fresh prompt (zero state here), else
 *   the state the call starts from.  A decode step is the same loop run for one
 *   token from the cached state.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   q, k   [Ttot, Hqk, Dk]      token-major; a batch of B rows of T tokens is the
 *   v      [Ttot, Hv,  Dv]      same memory as Ttot = B*T packed tokens with
 *   beta   [Ttot, Hv]           cu = {0, T, 2T, ...}
 *   g      [Ttot, Hv, gdim] or NULL; gdim = 1 (one gate per head) or Dk (per key channel)
 *   cu     [N + 1] token offsets of the N sequences (cu[0] = 0, non-decreasing)
 *   init   [N, Hv, Dk, Dv] or NULL.  Stored key-major: init[n,h,i,j] = S[j][i]
 *          (the nnterp page's "key_dim by value_dim matrix per head").
 *   o      [Ttot, Hv, Dv]       written
 *   final  [N, Hv, Dk, Dv] or NULL, key-major like init; written
 * Value head h reads query/key head h / (Hv / Hqk): the query/key heads are
 * repeated to the value heads, each one serving Hv/Hqk consecutive value heads.
 *
 * Returns 0, or -1 on a bad argument (nothing written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int dn_oracle_fwd(int64_t N, const int64_t *cu,
                  int64_t Hqk, int64_t Hv, int64_t Dk, int64_t Dv,
                  const double *q, const double *k, const double *v,
                  const double *beta, const double *g, int64_t gdim, const double *init,
                  double scale, int qk_l2norm, double eps,
                  double *o, double *final_state, int nthreads)
{
    if (N < 0 || Hqk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0 || Hv % Hqk != 0)
        return -1;
    if (qk_l2norm && !(eps >= 0.0))
        return -1;
    if (g && gdim != 1 && gdim != Dk)
        return -1;
    if (!cu || (N > 0 && (!q || !k || !v || !beta || !o)))
        return -1;
    if (cu[0] != 0)
        return -1;
    for (int64_t n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n])
            return -1;
    const int64_t group = Hv / Hqk;
    int64_t units = N * Hv;
    int err = 0;

#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : err)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t n = u / Hv, h = u % Hv, hq = h / group;
        /* S[j * Dk + i]: value row j, key column i -- the pages' S, d_v x d_k. */
        double *S = (double *)malloc(sizeof(double) * (size_t)(Dv * Dk));
        double *pred = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *kq_n = (double *)malloc(sizeof(double) * (size_t)(2 * Dk));
        if (!S || !pred || !kq_n) {
            free(S);
            free(pred);
            free(kq_n);
            err |= 1;
            continue;
        }
        if (init) {
            const double *m0 = init + u * Dk * Dv;
            for (int64_t i = 0; i < Dk; ++i)
                for (int64_t j = 0; j < Dv; ++j)
                    S[j * Dk + i] = m0[i * Dv + j];
        } else {
            memset(S, 0, sizeof(double) * (size_t)(Dv * Dk));
        }
        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const double *kt = k + (t * Hqk + hq) * Dk;
            const double *qt = q + (t * Hqk + hq) * Dk;
            const double *vt = v + (t * Hv + h) * Dv;
            if (qk_l2norm) {
                /* k_t / sqrt(|k_t|^2 + eps), q_t / sqrt(|q_t|^2 + eps) */
                double sk = 0.0, sq = 0.0;
                for (int64_t i = 0; i < Dk; ++i) {
                    sk += kt[i] * kt[i];
                    sq += qt[i] * qt[i];
                }
                const double ik = 1.0 / sqrt(sk + eps), iq = 1.0 / sqrt(sq + eps);
                for (int64_t i = 0; i < Dk; ++i) {
                    kq_n[i] = kt[i] * ik;
                    kq_n[Dk + i] = qt[i] * iq;
                }
                kt = kq_n;
                qt = kq_n + Dk;
            }
            const double bt = beta[t * Hv + h];
            /* decay first: S <- exp(g_t) S */
            if (g && gdim == 1) {
                const double a = exp(g[t * Hv + h]);
                for (int64_t e = 0; e < Dv * Dk; ++e)
                    S[e] *= a;
            }
            /* channel gates: S <- S diag(exp(g_t)), key channel i keeps exp(g_t[i]) */
            if (g && gdim != 1) {
                for (int64_t i = 0; i < Dk; ++i) {
                    const double a = exp(g[(t * Hv + h) * Dk + i]);
                    for (int64_t j = 0; j < Dv; ++j)
                        S[j * Dk + i] *= a;
                }
            }
            /* prediction error S k_t - v_t */
            for (int64_t j = 0; j < Dv; ++j) {
                double s = 0.0;
                for (int64_t i = 0; i < Dk; ++i)
                    s += S[j * Dk + i] * kt[i];
                pred[j] = s - vt[j];
            }
            /* S <- S - beta_t (S k_t - v_t) k_t^T */
            for (int64_t j = 0; j < Dv; ++j)
                for (int64_t i = 0; i < Dk; ++i)
                    S[j * Dk + i] -= bt * pred[j] * kt[i];
            /* o_t = scale * S_t q_t */
            double *ot = o + (t * Hv + h) * Dv;
            for (int64_t j = 0; j < Dv; ++j) {
                double s = 0.0;
                for (int64_t i = 0; i < Dk; ++i)
                    s += S[j * Dk + i] * qt[i];
                ot[j] = scale * s;
            }
        }
        if (final_state) {
            double *m1 = final_state + u * Dk * Dv;
            for (int64_t i = 0; i < Dk; ++i)
                for (int64_t j = 0; j < Dv; ++j)
                    m1[i * Dv + j] = S[j * Dk + i];
        }
        free(S);
        free(pred);
        free(kq_n);
    }
    return err ? -2 : 0;
}

/* Threads an OpenMP region would use by default (the core count the oracle is timed on). */
int dn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
