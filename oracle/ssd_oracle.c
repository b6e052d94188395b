/*
 * ssd_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU evaluation of the Mamba-2 selective
 * state-space recurrence in fp64.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may call it; the product path (the HIP library)
 * never does, and the two share no code.
 *
 * What it computes ("Accelerating Mamba-2 with High-Performance Forward Pass
 * Kernels in NVIDIA CUDA Tile", section "Mamba-2 architecture"):
 *
 *   the core recurrence      h_t = exp(A dt_t) h_{t-1} + dt_t B_t x_t^T
 *   renamed with a_t = A dt_t and b_t = dt_t B_t (same section, the
 *   second displayed equation),
 *   and the readout of the no-decay expansion in the same section,
 *                            y_t = c_t^T h_t + D x_t .
 *
 * Reading of the pages fixed here (the pages write the readout both with
 * h_{t-1} and with h_t): the readout uses the state AFTER the update at t.
 * This is the only reading under which the chunked output formula with the
 * causal mask that keeps the diagonal, and an inclusive cumulative sum G,
 * equals the recurrence.
 *
 * Layouts (all dense, row-major, fp64):
 *   x  (batch, seqlen, nheads, headdim)      dt (batch, seqlen, nheads)
 *   A  (nheads)   D (nheads) or NULL => 0
 *   Bm (batch, seqlen, ngroups, dstate)      Cm (batch, seqlen, ngroups, dstate)
 *   h0 (batch, nheads, headdim, dstate) or NULL => zero initial state
 *   y  (batch, seqlen, nheads, headdim)      (output)
 *   hT (batch, nheads, headdim, dstate) or NULL  (output: state after the
 *      last token, which the fwd_pass_state section also returns)
 *   ckpt (batch, nheads, ceil(seqlen/ckpt_stride), headdim, dstate) or NULL
 *      (output: the state before token k*ckpt_stride is consumed, i.e. the
 *      state at the start of each chunk, the quantity the fwd_pass_state
 *      section stores for every chunk).
 *
 * The state h is the S x H matrix of the pages (dstate x headdim); it is stored
 * transposed, row p = one headdim index with the dstate index contiguous, the
 * [head, state] tile orientation of the fwd_pass_state section.
 *
 * Heads map to B/C groups contiguously: group = head / (nheads / ngroups)
 * (fwd_pass_state prologue).
 *
 * Every (batch, head, headdim-row) unit is independent; OpenMP runs over them.
 * Returns 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

int ssd_oracle_scan(int64_t batch, int64_t seqlen, int64_t nheads,
                    int64_t headdim, int64_t dstate, int64_t ngroups,
                    const double *x, const double *dt, const double *A,
                    const double *Bm, const double *Cm, const double *D,
                    const double *h0, double *y, double *hT,
                    int64_t ckpt_stride, double *ckpt)
{
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 ||
        ngroups <= 0 || nheads % ngroups != 0)
        return -1;
    if (ckpt != NULL && ckpt_stride <= 0)
        return -1;
    if (!x || !dt || !A || !Bm || !Cm || !y)
        return -1;

    const int64_t heads_per_group = nheads / ngroups;
    const int64_t nckpt = (ckpt != NULL) ? (seqlen + ckpt_stride - 1) / ckpt_stride : 0;
    const int64_t units = batch * nheads * headdim;
    int failed = 0;

#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)dstate * sizeof(double));
        if (s == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t u = 0; u < units; ++u) {
            if (s == NULL)
                continue;
            const int64_t b = u / (nheads * headdim);
            const int64_t h = (u / headdim) % nheads;
            const int64_t p = u % headdim;
            const int64_t g = h / heads_per_group;
            const double d_skip = (D != NULL) ? D[h] : 0.0;

            /* state row p of h_0 */
            for (int64_t n = 0; n < dstate; ++n)
                s[n] = (h0 != NULL) ? h0[((b * nheads + h) * headdim + p) * dstate + n] : 0.0;

            for (int64_t t = 0; t < seqlen; ++t) {
                if (ckpt != NULL && t % ckpt_stride == 0) {
                    double *dst = ckpt + (((b * nheads + h) * nckpt + t / ckpt_stride) * headdim + p) * dstate;
                    for (int64_t n = 0; n < dstate; ++n)
                        dst[n] = s[n];
                }
                const double dt_t = dt[(b * seqlen + t) * nheads + h];
                const double decay = exp(A[h] * dt_t);          /* exp(a_t), a_t = A dt_t */
                const double x_tp = x[((b * seqlen + t) * nheads + h) * headdim + p];
                const double *B_t = Bm + ((b * seqlen + t) * ngroups + g) * dstate;
                const double *C_t = Cm + ((b * seqlen + t) * ngroups + g) * dstate;
                double acc = 0.0;
                for (int64_t n = 0; n < dstate; ++n) {
                    /* h_t = exp(a_t) h_{t-1} + b_t x_t^T with b_t = dt_t B_t */
                    s[n] = decay * s[n] + (dt_t * B_t[n]) * x_tp;
                    /* y_t = c_t^T h_t  (post-update state) */
                    acc += C_t[n] * s[n];
                }
                y[((b * seqlen + t) * nheads + h) * headdim + p] = acc + d_skip * x_tp;
            }
            if (hT != NULL)
                for (int64_t n = 0; n < dstate; ++n)
                    hT[((b * nheads + h) * headdim + p) * dstate + n] = s[n];
        }
        free(s);
    }
    return failed ? -1 : 0;
}

/*
 * ssd_oracle_scan_bwd -- TEST INFRASTRUCTURE ONLY.
 *
 * Gradients of the scalar L = sum_{b,t,h,p} dy[b,t,h,p] y[b,t,h,p]
 *                           + sum_{b,h,p,n} dhT[b,h,p,n] hT[b,h,p,n]
 * with respect to every input of ssd_oracle_scan (the recurrence of section
 * "Mamba-2 architecture", readout after the update), by the adjoint of the
 * same recurrence in fp64 -- the chain rule applied to each step in reverse:
 *
 *   forward   h_t = alpha_t h_{t-1} + dt_t x_t B_t^T   (rows p, columns n)
 *             y_t = h_t C_t + D x_t,   alpha_t = exp(A dt_t)
 *   adjoint   Lam_t = dy_t C_t^T + alpha_{t+1} Lam_{t+1}   (Lam after the last
 *             token = dhT), the total derivative of L by h_t;
 *   then      dx_t    = dt_t Lam_t B_t + D dy_t
 *             dB_t   += dt_t Lam_t^T x_t          (summed over the group's heads)
 *             dC_t   += h_t^T dy_t                (summed over the group's heads)
 *             ddt_t   = x_t . (Lam_t B_t) + A alpha_t <Lam_t, h_{t-1}>
 *             dA     += dt_t alpha_t <Lam_t, h_{t-1}>
 *             dD     += dy_t . x_t
 *             dh0     = alpha_0 Lam_0 .
 *
 * Layouts as ssd_oracle_scan; dy like y, dhT like hT (NULL => 0).  Outputs
 * (all fp64, written, not accumulated): dx like x, ddt like dt, dA (nheads),
 * dB like Bm, dC like Cm, dD (nheads), dh0 like h0 (may be NULL).
 * Units are (batch, head) pairs; each keeps all seqlen + 1 states of its
 * head (headdim x dstate doubles each), so it is meant for test sizes.  The
 * group sums of dB and dC run serially after the parallel part.
 * Returns 0 on success, -1 on an invalid argument or allocation failure.
 */
int ssd_oracle_scan_bwd(int64_t batch, int64_t seqlen, int64_t nheads,
                        int64_t headdim, int64_t dstate, int64_t ngroups,
                        const double *x, const double *dt, const double *A,
                        const double *Bm, const double *Cm, const double *D,
                        const double *h0, const double *dy, const double *dhT,
                        double *dx, double *ddt, double *dA, double *dB,
                        double *dC, double *dD, double *dh0)
{
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 ||
        ngroups <= 0 || nheads % ngroups != 0)
        return -1;
    if (!x || !dt || !A || !Bm || !Cm || !dy || !dx || !ddt || !dA || !dB || !dC || !dD)
        return -1;

    const int64_t hpg = nheads / ngroups;
    const int64_t P = headdim, N = dstate, PN = headdim * dstate;
    /* per-head partial sums of dB and dC: (batch, seqlen, nheads, dstate) */
    double *dBh = (double *)calloc((size_t)(batch * seqlen * nheads * N > 0 ? batch * seqlen * nheads * N : 1), sizeof(double));
    double *dCh = (double *)calloc((size_t)(batch * seqlen * nheads * N > 0 ? batch * seqlen * nheads * N : 1), sizeof(double));
    double *dAp = (double *)calloc((size_t)(batch * nheads), sizeof(double));
    double *dDp = (double *)calloc((size_t)(batch * nheads), sizeof(double));
    if (!dBh || !dCh || (batch > 0 && (!dAp || !dDp))) {
        free(dBh); free(dCh); free(dAp); free(dDp);
        return -1;
    }
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < batch * nheads; ++u) {
        const int64_t b = u / nheads, h = u % nheads, g = h / hpg;
        const double d_skip = (D != NULL) ? D[h] : 0.0;
        /* states: hs[(t + 1) * PN + p * N + n] = h_t, t = -1 .. seqlen - 1 */
        double *hs = (double *)malloc((size_t)(seqlen + 1) * PN * sizeof(double));
        double *lam = (double *)malloc((size_t)PN * sizeof(double));
        if (hs == NULL || lam == NULL) {
#pragma omp atomic write
            failed = 1;
            free(hs); free(lam);
            continue;
        }
        for (int64_t k = 0; k < PN; ++k)
            hs[k] = (h0 != NULL) ? h0[(b * nheads + h) * PN + k] : 0.0;
        /* forward: every state */
        for (int64_t t = 0; t < seqlen; ++t) {
            const double dtv = dt[(b * seqlen + t) * nheads + h];
            const double alpha = exp(A[h] * dtv);
            const double *xt = x + ((b * seqlen + t) * nheads + h) * P;
            const double *Bt = Bm + ((b * seqlen + t) * ngroups + g) * N;
            const double *prev = hs + t * PN;
            double *cur = hs + (t + 1) * PN;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n)
                    cur[p * N + n] = alpha * prev[p * N + n] + dtv * xt[p] * Bt[n];
        }
        /* reverse: the adjoint, carried as alpha_{t+1} Lam_{t+1} (dhT at the end) */
        for (int64_t k = 0; k < PN; ++k)
            lam[k] = (dhT != NULL) ? dhT[(b * nheads + h) * PN + k] : 0.0;
        double dA_acc = 0.0, dD_acc = 0.0;
        for (int64_t t = seqlen - 1; t >= 0; --t) {
            const double dtv = dt[(b * seqlen + t) * nheads + h];
            const double alpha = exp(A[h] * dtv);
            const double *xt = x + ((b * seqlen + t) * nheads + h) * P;
            const double *Bt = Bm + ((b * seqlen + t) * ngroups + g) * N;
            const double *Ct = Cm + ((b * seqlen + t) * ngroups + g) * N;
            const double *dyt = dy + ((b * seqlen + t) * nheads + h) * P;
            const double *ht = hs + (t + 1) * PN, *hprev = hs + t * PN;
            double *dxt = dx + ((b * seqlen + t) * nheads + h) * P;
            double *dBt = dBh + ((b * seqlen + t) * nheads + h) * N;
            double *dCt = dCh + ((b * seqlen + t) * nheads + h) * N;
            /* Lam_t = dy_t C_t^T + (carried) */
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n)
                    lam[p * N + n] += dyt[p] * Ct[n];
            double xLB = 0.0, inner = 0.0, dyx = 0.0;
            for (int64_t p = 0; p < P; ++p) {
                double lb = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    lb += lam[p * N + n] * Bt[n];
                    inner += lam[p * N + n] * hprev[p * N + n];
                }
                dxt[p] = dtv * lb + d_skip * dyt[p];
                xLB += xt[p] * lb;
                dyx += dyt[p] * xt[p];
            }
            for (int64_t n = 0; n < N; ++n) {
                double sb = 0.0, sc = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    sb += lam[p * N + n] * xt[p];
                    sc += ht[p * N + n] * dyt[p];
                }
                dBt[n] = dtv * sb;
                dCt[n] = sc;
            }
            ddt[(b * seqlen + t) * nheads + h] = xLB + A[h] * alpha * inner;
            dA_acc += dtv * alpha * inner;
            dD_acc += dyx;
            for (int64_t k = 0; k < PN; ++k)
                lam[k] *= alpha;
        }
        if (dh0 != NULL)
            for (int64_t k = 0; k < PN; ++k)
                dh0[(b * nheads + h) * PN + k] = lam[k];
        dAp[u] = dA_acc;
        dDp[u] = dD_acc;
        free(hs);
        free(lam);
    }
    if (!failed) {
        for (int64_t h = 0; h < nheads; ++h) {
            double sa = 0.0, sd = 0.0;
            for (int64_t b = 0; b < batch; ++b) {
                sa += dAp[b * nheads + h];
                sd += dDp[b * nheads + h];
            }
            dA[h] = sa;
            dD[h] = sd;
        }
        for (int64_t b = 0; b < batch; ++b)
            for (int64_t t = 0; t < seqlen; ++t)
                for (int64_t g = 0; g < ngroups; ++g)
                    for (int64_t n = 0; n < N; ++n) {
                        double sb = 0.0, sc = 0.0;
                        for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
                            sb += dBh[((b * seqlen + t) * nheads + h) * N + n];
                            sc += dCh[((b * seqlen + t) * nheads + h) * N + n];
                        }
                        dB[((b * seqlen + t) * ngroups + g) * N + n] = sb;
                        dC[((b * seqlen + t) * ngroups + g) * N + n] = sc;
                    }
    }
    free(dBh); free(dCh); free(dAp); free(dDp);
    return failed ? -1 : 0;
}
