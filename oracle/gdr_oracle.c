/*
 * gdr_oracle.c -- fp64 CPU oracle for the (gated) delta-rule memory.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark have an obviously correct reference.  It
 * shares no code, header or constant with the HIP library.
 *
 * What it computes, one token at a time in double precision, for every
 * (batch, head) chain independently (state S is d_v x d_k, row i = value
 * channel i, so a read is o = S q):
 *
 *   a      = exp(log_alpha_t)        scalar (Gated DeltaNet), per key channel
 *                                    (Kimi Delta Attention) or 1 (DeltaNet)
 *   Sbar   = S Diag(a)               decay along the key dimension
 *   pred   = Sbar k_t                prediction from the *decayed* memory
 *   u      = beta_t (v_t - pred)     delta-rule residual, scaled by beta
 *   S      = Sbar + u k_t^T          erase-then-write
 *   o_t    = S q_t                   read after the write
 *
 * Sources (cited by title and section):
 *  - "Linear Attention Architectures: Mechanisms, Trade-offs, and Cross-Layer
 *    Routing", Sec. 3: shared read rule Eq. (8) (output is read after the
 *    memory has been updated), prediction and residual Eqs. (9)-(10), the
 *    DeltaNet update, the Gated DeltaNet decay-adjusted prediction, and the
 *    Kimi Delta Attention channel-wise decay acting on the key dimension
 *    (diagonal matrix multiplying the memory on the right).
 *  - "linear attention and its gated descendants" (blog), sections
 *    "DeltaNet" (S_t = S_{t-1} + beta (v - S_{t-1} k) k^T), "Gated DeltaNet"
 *    (prediction from the decayed memory alpha S_{t-1} k) and "Kimi Delta
 *    Attention" (decay old memory first, then apply the delta-rule update;
 *    written there in the transposed d_k x d_v orientation).
 *  - "Linear Attention & DeltaNet" (wiki), "How it works" items 3-4 and the
 *    recurrent reference pseudocode, which the page calls the semantic
 *    reference.  Its gated line predicts from the undecayed memory; the
 *    three other statements above (including the same page's own update
 *    formula) predict from the decayed one, and this file follows them.
 *
 * no_delta = 1 replaces the residual by u = beta_t v_t (plain gated linear
 * attention with write strength beta).  It exists only so that tests can
 * check the loop against the masked parallel form of linear attention
 * ("Chunkwise Parallel Form" section of the blog post).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_ALPHA_NONE 0
#define ORC_ALPHA_SCALAR 1
#define ORC_ALPHA_CHANNEL 2

/* One chain: L tokens, state S (dv x dk, row-major) updated in place. */
static void orc_chain(int L, int dk, int dv, int mode, int no_delta,
                      const double *q, const double *k, const double *v,
                      const double *beta, const double *log_alpha,
                      double *S, double *o, double *a, double *u)
{
    for (int t = 0; t < L; ++t) {
        const double *qt = q + (size_t)t * dk;
        const double *kt = k + (size_t)t * dk;
        const double *vt = v + (size_t)t * dv;

        /* decay factors along the key dimension */
        if (mode == ORC_ALPHA_NONE) {
            for (int j = 0; j < dk; ++j) a[j] = 1.0;
        } else if (mode == ORC_ALPHA_SCALAR) {
            double s = exp(log_alpha[t]);
            for (int j = 0; j < dk; ++j) a[j] = s;
        } else {
            const double *lt = log_alpha + (size_t)t * dk;
            for (int j = 0; j < dk; ++j) a[j] = exp(lt[j]);
        }

        for (int i = 0; i < dv; ++i) {
            double *row = S + (size_t)i * dk;
            /* Sbar = S Diag(a) */
            for (int j = 0; j < dk; ++j) row[j] *= a[j];
            /* residual against the decayed prediction */
            double pred = 0.0;
            for (int j = 0; j < dk; ++j) pred += row[j] * kt[j];
            u[i] = no_delta ? beta[t] * vt[i] : beta[t] * (vt[i] - pred);
            /* write u k^T, then read with q */
            double out = 0.0;
            for (int j = 0; j < dk; ++j) {
                row[j] += u[i] * kt[j];
                out += row[j] * qt[j];
            }
            o[(size_t)t * dv + i] = out;
        }
    }
}

/*
 * Run the recurrence over BH independent chains.
 *   q, k       [BH][L][dk]      v [BH][L][dv]      beta [BH][L]
 *   log_alpha  NULL (mode 0) | [BH][L] (mode 1) | [BH][L][dk] (mode 2)
 *   S0         NULL => zero state | [BH][dv][dk]
 *   o          [BH][L][dv]      S_final NULL | [BH][dv][dk]
 *   nthreads   <= 0 => OpenMP default
 * Returns 0 on success, -1 on a bad argument or allocation failure.
 */
int gdr_oracle_run(int BH, int L, int dk, int dv, int mode, int no_delta,
                   const double *q, const double *k, const double *v,
                   const double *beta, const double *log_alpha, const double *S0,
                   double *o, double *S_final, int nthreads)
{
    if (BH < 0 || L < 0 || dk <= 0 || dv <= 0) return -1;
    if (mode < ORC_ALPHA_NONE || mode > ORC_ALPHA_CHANNEL) return -1;
    if (mode != ORC_ALPHA_NONE && log_alpha == NULL) return -1;
    if (BH > 0 && L > 0 && (!q || !k || !v || !beta || !o)) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(|| : failed)
#endif
    for (int c = 0; c < BH; ++c) {
        size_t sz = (size_t)dv * dk;
        double *S = (double *)malloc(sizeof(double) * (sz + (size_t)dk + (size_t)dv));
        if (!S) { failed = 1; continue; }
        double *a = S + sz, *u = a + dk;
        if (S0) memcpy(S, S0 + (size_t)c * sz, sizeof(double) * sz);
        else memset(S, 0, sizeof(double) * sz);
        const double *la = NULL;
        if (mode == ORC_ALPHA_SCALAR) la = log_alpha + (size_t)c * L;
        if (mode == ORC_ALPHA_CHANNEL) la = log_alpha + (size_t)c * L * dk;
        orc_chain(L, dk, dv, mode, no_delta,
                  q + (size_t)c * L * dk, k + (size_t)c * L * dk, v + (size_t)c * L * dv,
                  beta + (size_t)c * L, la, S, o + (size_t)c * L * dv, a, u);
        if (S_final) memcpy(S_final + (size_t)c * sz, S, sizeof(double) * sz);
        free(S);
    }
    (void)nthreads;
    return failed ? -1 : 0;
}

/* Number of OpenMP threads a run with nthreads <= 0 would use. */
int gdr_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
