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
