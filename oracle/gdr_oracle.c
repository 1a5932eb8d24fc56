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

/*
 * Reverse mode (gradients) of the same recurrence, for training.  The
 * derivative of one token step, written out by the chain rule in the order
 * opposite to the forward step (dS is the gradient of the loss with respect
 * to S_t, carried from later tokens; "+=" accumulates):
 *
 *   forward                      backward
 *   Sbar = S_{t-1} Diag(a)       dS      += do_t q_t^T        (o_t = S_t q_t)
 *   pred = Sbar k_t              dq_t     = S_t^T do_t
 *   u    = beta (v - pred)       du       = dS k_t            (S_t = Sbar + u k^T)
 *   S_t  = Sbar + u k_t^T        dk_t     = dS^T u
 *   o_t  = S_t q_t               dv_t     = beta du           (u = beta (v - pred))
 *                                dbeta_t  = du . (v - pred)
 *                                dpred    = -beta du
 *                                dSbar    = dS + dpred k_t^T  (pred = Sbar k)
 *                                dk_t    += Sbar^T dpred
 *                                dlog a_j = sum_i dSbar_ij Sbar_ij  (a_j = e^{log a_j})
 *                                dS_{t-1} = dSbar Diag(a)
 *
 * Scalar alpha sums dlog a_j over j; alpha = 1 has no gate gradient.  The
 * step needs S_{t-1}: the forward states are kept every ORC_CKPT tokens and
 * each block of ORC_CKPT states is recomputed forward before its tokens are
 * walked backward (no division by alpha, which may be tiny).
 */
#define ORC_CKPT 64

static void orc_decay(int mode, int dk, const double *la_t, double *a)
{
    if (mode == ORC_ALPHA_NONE) {
        for (int j = 0; j < dk; ++j) a[j] = 1.0;
    } else if (mode == ORC_ALPHA_SCALAR) {
        double s = exp(la_t[0]);
        for (int j = 0; j < dk; ++j) a[j] = s;
    } else {
        for (int j = 0; j < dk; ++j) a[j] = exp(la_t[j]);
    }
}

/* One token forward from S (= S_{t-1}) into Sn (= S_t). */
static void orc_step(int dk, int dv, const double *a, const double *qt, const double *kt,
                     const double *vt, double bt, const double *S, double *Sn)
{
    (void)qt;
    for (int i = 0; i < dv; ++i) {
        const double *row = S + (size_t)i * dk;
        double *nrow = Sn + (size_t)i * dk;
        double pred = 0.0;
        for (int j = 0; j < dk; ++j) pred += row[j] * a[j] * kt[j];
        const double u = bt * (vt[i] - pred);
        for (int j = 0; j < dk; ++j) nrow[j] = row[j] * a[j] + u * kt[j];
    }
}

static int orc_chain_backward(int L, int dk, int dv, int mode,
                              const double *q, const double *k, const double *v,
                              const double *beta, const double *log_alpha, const double *S0,
                              const double *dout, const double *dS_final,
                              double *dq, double *dkk, double *dvv, double *dbeta,
                              double *dla, double *dS0)
{
    const size_t sz = (size_t)dv * dk;
    const int nblk = (L + ORC_CKPT - 1) / ORC_CKPT;
    const int lstride = mode == ORC_ALPHA_CHANNEL ? dk : 1;
    /* ckpt[b] = state before block b's first token; blk[i] = S_{t0 + i - 1}, i = 0..ORC_CKPT */
    double *ckpt = (double *)malloc(sizeof(double) * sz * (size_t)(nblk > 0 ? nblk : 1));
    double *blk = (double *)malloc(sizeof(double) * sz * (ORC_CKPT + 1));
    double *dS = (double *)malloc(sizeof(double) * (sz + (size_t)dk + 3 * (size_t)dv));
    if (!ckpt || !blk || !dS) { free(ckpt); free(blk); free(dS); return -1; }
    double *a = dS + sz, *du = a + dk, *dpred = du + dv, *r = dpred + dv;

    /* forward: the checkpoints */
    if (S0) memcpy(blk, S0, sizeof(double) * sz);
    else memset(blk, 0, sizeof(double) * sz);
    for (int b = 0; b < nblk; ++b) {
        memcpy(ckpt + (size_t)b * sz, blk, sizeof(double) * sz);
        const int t0 = b * ORC_CKPT, t1 = t0 + ORC_CKPT < L ? t0 + ORC_CKPT : L;
        for (int t = t0; t < t1; ++t) {
            orc_decay(mode, dk, log_alpha ? log_alpha + (size_t)t * lstride : NULL, a);
            orc_step(dk, dv, a, q + (size_t)t * dk, k + (size_t)t * dk, v + (size_t)t * dv, beta[t],
                     blk, blk + sz);
            memcpy(blk, blk + sz, sizeof(double) * sz);
        }
    }

    /* backward */
    if (dS_final) memcpy(dS, dS_final, sizeof(double) * sz);
    else memset(dS, 0, sizeof(double) * sz);
    for (int b = nblk - 1; b >= 0; --b) {
        const int t0 = b * ORC_CKPT, t1 = t0 + ORC_CKPT < L ? t0 + ORC_CKPT : L;
        memcpy(blk, ckpt + (size_t)b * sz, sizeof(double) * sz);
        for (int t = t0; t < t1; ++t) {
            orc_decay(mode, dk, log_alpha ? log_alpha + (size_t)t * lstride : NULL, a);
            orc_step(dk, dv, a, q + (size_t)t * dk, k + (size_t)t * dk, v + (size_t)t * dv, beta[t],
                     blk + (size_t)(t - t0) * sz, blk + (size_t)(t - t0 + 1) * sz);
        }
        for (int t = t1 - 1; t >= t0; --t) {
            const double *qt = q + (size_t)t * dk, *kt = k + (size_t)t * dk, *vt = v + (size_t)t * dv;
            const double *do_t = dout + (size_t)t * dv;
            const double *Sp = blk + (size_t)(t - t0) * sz;       /* S_{t-1} */
            const double *St = blk + (size_t)(t - t0 + 1) * sz;   /* S_t */
            const double bt = beta[t];
            orc_decay(mode, dk, log_alpha ? log_alpha + (size_t)t * lstride : NULL, a);
            double *dqt = dq + (size_t)t * dk, *dkt = dkk + (size_t)t * dk;
            for (int j = 0; j < dk; ++j) { dqt[j] = 0.0; dkt[j] = 0.0; }
            double dbt = 0.0;
            /* dS += do q^T; dq = S_t^T do; du = dS k; residual r = v - pred */
            for (int i = 0; i < dv; ++i) {
                double *drow = dS + (size_t)i * dk;
                const double *srow = St + (size_t)i * dk, *prow = Sp + (size_t)i * dk;
                double acc = 0.0, pred = 0.0;
                for (int j = 0; j < dk; ++j) {
                    drow[j] += do_t[i] * qt[j];
                    dqt[j] += srow[j] * do_t[i];
                    acc += drow[j] * kt[j];
                    pred += prow[j] * a[j] * kt[j];
                }
                du[i] = acc;
                r[i] = vt[i] - pred;
                dbt += acc * r[i];
                dpred[i] = -bt * acc;
                dvv[(size_t)t * dv + i] = bt * acc;
            }
            dbeta[t] = dbt;
            /* dk = dS^T u + Sbar^T dpred; dSbar = dS + dpred k^T; gate; dS_{t-1} */
            double dls = 0.0;
            double *dlt = NULL;
            if (mode == ORC_ALPHA_CHANNEL) { dlt = dla + (size_t)t * dk; for (int j = 0; j < dk; ++j) dlt[j] = 0.0; }
            for (int i = 0; i < dv; ++i) {
                const double u = bt * r[i];
                double *drow = dS + (size_t)i * dk;
                const double *prow = Sp + (size_t)i * dk;
                for (int j = 0; j < dk; ++j) {
                    const double sbar = prow[j] * a[j];
                    dkt[j] += drow[j] * u + sbar * dpred[i];
                    const double dsb = drow[j] + dpred[i] * kt[j];
                    if (mode == ORC_ALPHA_CHANNEL) dlt[j] += dsb * sbar;
                    else dls += dsb * sbar;
                    drow[j] = dsb * a[j];
                }
            }
            if (mode == ORC_ALPHA_SCALAR) dla[t] = dls;
        }
    }
    if (dS0) memcpy(dS0, dS, sizeof(double) * sz);
    free(ckpt); free(blk); free(dS);
    return 0;
}

/*
 * Gradients over BH independent chains (layouts as gdr_oracle_run):
 *   dout [BH][L][dv] (gradient of the outputs), dS_final NULL | [BH][dv][dk]
 *   -> dq, dk [BH][L][dk], dv [BH][L][dv], dbeta [BH][L],
 *      dlog_alpha NULL (mode 0) | [BH][L] | [BH][L][dk], dS0 NULL | [BH][dv][dk]
 */
int gdr_oracle_backward(int BH, int L, int dk, int dv, int mode,
                        const double *q, const double *k, const double *v,
                        const double *beta, const double *log_alpha, const double *S0,
                        const double *dout, const double *dS_final,
                        double *dq, double *dkk, double *dvv, double *dbeta,
                        double *dlog_alpha, double *dS0, int nthreads)
{
    if (BH < 0 || L < 0 || dk <= 0 || dv <= 0) return -1;
    if (mode < ORC_ALPHA_NONE || mode > ORC_ALPHA_CHANNEL) return -1;
    if (mode != ORC_ALPHA_NONE && (log_alpha == NULL || dlog_alpha == NULL)) return -1;
    if (BH > 0 && L > 0 && (!q || !k || !v || !beta || !dout || !dq || !dkk || !dvv || !dbeta))
        return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(|| : failed)
#endif
    for (int c = 0; c < BH; ++c) {
        const size_t sz = (size_t)dv * dk;
        const int ls = mode == ORC_ALPHA_CHANNEL ? dk : 1;
        const size_t lo = (size_t)c * L;
        if (orc_chain_backward(L, dk, dv, mode, q + lo * dk, k + lo * dk, v + lo * dv, beta + lo,
                               mode == ORC_ALPHA_NONE ? NULL : log_alpha + lo * ls,
                               S0 ? S0 + (size_t)c * sz : NULL, dout + lo * dv,
                               dS_final ? dS_final + (size_t)c * sz : NULL,
                               dq + lo * dk, dkk + lo * dk, dvv + lo * dv, dbeta + lo,
                               mode == ORC_ALPHA_NONE ? NULL : dlog_alpha + lo * ls,
                               dS0 ? dS0 + (size_t)c * sz : NULL) != 0)
            failed = 1;
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
