/*
 * Plain CPU oracle for the backward pass of the Mamba selective-scan forward.
 *
 * TEST INFRASTRUCTURE ONLY, like ssm_ref.c: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no code with the GPU library.
 *
 * The forward (ssm_ref.c) is, per batch row b and channel d, with s_t the step size:
 *   x_t = delta_t + bias_d,  s_t = softplus(x_t) (or x_t),  a_t[n] = exp(s_t A[d,n])
 *   h_t[n] = a_t[n] h_{t-1}[n] + s_t B_t[n] u_t,            h_{-1} = h0 (or 0)
 *   y_t = sum_n C_t[n] h_t[n] + D_d u_t,   out_t = y_t z_t sigmoid(z_t) (or y_t)
 *   final[n] = h_{L-1}[n]
 * The pages define only this forward (ybb.press, "Mamba state-space model: from theory to
 * production CUDA kernel optimisation", sections 1.2, 2.3 and 7.1; p1, mhpq.cn/news/
 * 1077344, section 3.3, names recomputation of the scan in the backward pass without
 * spelling it out). This file is its reverse-mode derivative, written out by the chain
 * rule and nothing else, for a loss L = sum_t dout_t out_t + sum_n dfinal[n] final[n]:
 *
 *   gate:   dy_t = dout_t z sig(z),  dz_t = dout_t y_t sig(z) (1 + z (1 - sig(z)))
 *   state adjoint, backwards in t (g_t = dL/dh_t):
 *           g_{L-1} = C_{L-1} dy_{L-1} + dfinal,   g_t = C_t dy_t + a_{t+1} g_{t+1}
 *   then, for every t and n:
 *           dC_t[n] += dy_t h_t[n]            (summed over channels d)
 *           dB_t[n] += g_t[n] s_t u_t         (summed over channels d)
 *           du_t    += g_t[n] s_t B_t[n]      (plus D_d dy_t once)
 *           ds_t    += g_t[n] (A[d,n] a_t[n] h_{t-1}[n] + B_t[n] u_t)
 *           dA[d,n] += g_t[n] a_t[n] s_t h_{t-1}[n]   (summed over batch rows)
 *           dD_d    += dy_t u_t                        (summed over batch rows)
 *   step size: ddelta_t = ds_t sig(x_t) with softplus (1 above the threshold 20, where the
 *           forward returns x itself), ds_t without; dbias_d += ddelta_t.
 *   initial state: dh0[n] = a_0[n] g_0[n].
 * A padding position (mask 0; mhpq.cn/news/1057127 section 4) keeps the state, h_t =
 * h_{t-1}: there a_t acts as 1, nothing flows into dB, du, dA or ddelta through the state,
 * and dC and the D and gate terms are as at any other step.
 *
 * The forward states h_t of a row are kept in a per-row buffer (the recomputation the
 * pages mention, done in the plainest way). Channel-summed outputs dB and dC are
 * accumulated per thread and added in thread order; per-channel sums (dA, dD, dbias) are
 * owned by the thread that owns the channel.
 *
 * Pinned by tests/test_oracle_bwd_pins.py: central finite differences of the forward
 * oracle for every input, and adjoint (dot-product) identities for the inputs the output
 * depends on linearly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#include "ssm_ref.h"

static double softplus_ref(double x) { return x > 20.0 ? x : log1p(exp(x)); }
static double sigmoid_ref(double x) { return 1.0 / (1.0 + exp(-x)); }

int ssm_ref_scan_bwd_f64(const double* u, const double* delta, const double* A,
                         const double* B, const double* C, const double* D, const double* z,
                         const double* delta_bias, int delta_softplus, const double* h0,
                         const unsigned char* mask, const double* dout,
                         const double* dfinal, double* du,
                         double* ddelta, double* dA, double* dB, double* dC, double* dD,
                         double* dz, double* dbias, double* dh0, int64_t batch, int64_t dim,
                         int64_t dstate, int64_t seqlen, int nthreads)
{
    if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA || !dB || !dC)
        return -1;
    if (z && !dz) return -1;
    if (batch < 0 || dim < 0 || dstate < 1 || seqlen < 0) return -1;
    const int64_t N = dstate, L = seqlen;
    const int64_t bc = batch * N * L;
    const int nt = nthreads > 0 ? nthreads : 1;

    memset(dA, 0, (size_t)(dim * N) * sizeof(double));
    memset(dB, 0, (size_t)bc * sizeof(double));
    memset(dC, 0, (size_t)bc * sizeof(double));
    if (dD) memset(dD, 0, (size_t)dim * sizeof(double));
    if (dbias) memset(dbias, 0, (size_t)dim * sizeof(double));

    /* per-thread partial sums of dB and dC (they sum over channels) */
    double* part = (double*)calloc((size_t)nt * 2 * (size_t)(bc > 0 ? bc : 1), sizeof(double));
    if (!part) return -2;
    int bad_alloc = 0;

#pragma omp parallel num_threads(nt)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double* pB = part + (size_t)tid * 2 * (size_t)(bc > 0 ? bc : 1);
        double* pC = pB + (bc > 0 ? bc : 1);
        double* hist = (double*)malloc((size_t)(L + 1) * (size_t)N * sizeof(double));
        double* g = (double*)malloc((size_t)N * sizeof(double));
        double* sv = (double*)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
        if (!hist || !g || !sv) {
#pragma omp atomic write
            bad_alloc = 1;
        }
        /* channels are split statically, so a channel's sums have one owner */
#pragma omp for schedule(static)
        for (int64_t d = 0; d < dim; ++d) {
            if (!hist || !g || !sv) continue;
            const double* A_d = A + d * N;
            const double bias = delta_bias ? delta_bias[d] : 0.0;
            for (int64_t b = 0; b < batch; ++b) {
                const int64_t r = b * dim + d;
                const double* u_r = u + r * L;
                const double* dl_r = delta + r * L;
                const double* z_r = z ? z + r * L : NULL;
                const double* do_r = dout + r * L;
                const double* B_b = B + b * N * L;
                const double* C_b = C + b * N * L;
                double* pB_b = pB + b * N * L;
                double* pC_b = pC + b * N * L;

                /* forward, keeping every state: hist[(t + 1) N + n] = h_t[n] */
                for (int64_t n = 0; n < N; ++n) hist[n] = h0 ? h0[r * N + n] : 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    const double x = dl_r[t] + bias;
                    const double s = delta_softplus ? softplus_ref(x) : x;
                    const int live = !mask || mask[b * L + t];
                    sv[t] = s;
                    for (int64_t n = 0; n < N; ++n)
                        hist[(t + 1) * N + n] = live ? exp(s * A_d[n]) * hist[t * N + n] +
                                                           s * B_b[n * L + t] * u_r[t]
                                                     : hist[t * N + n];
                }

                /* backward */
                for (int64_t n = 0; n < N; ++n) g[n] = dfinal ? dfinal[r * N + n] : 0.0;
                for (int64_t t = L - 1; t >= 0; --t) {
                    const double s = sv[t], ut = u_r[t];
                    const int live = !mask || mask[b * L + t];
                    const double* h_t = hist + (t + 1) * N;
                    const double* h_p = hist + t * N;
                    double dy = do_r[t];
                    if (z_r) {
                        double y = D ? D[d] * ut : 0.0;
                        for (int64_t n = 0; n < N; ++n) y += C_b[n * L + t] * h_t[n];
                        const double zz = z_r[t], sg = sigmoid_ref(zz);
                        dz[r * L + t] = do_r[t] * y * sg * (1.0 + zz * (1.0 - sg));
                        dy = do_r[t] * zz * sg;
                    }
                    double du_t = D ? D[d] * dy : 0.0;
                    if (dD) dD[d] += dy * ut;
                    double ds = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        const double Bt = B_b[n * L + t], Ct = C_b[n * L + t];
                        g[n] += Ct * dy;                      /* g_t = C_t dy_t + a_{t+1} g_{t+1} */
                        pC_b[n * L + t] += dy * h_t[n];
                        if (!live) continue;                  /* h_t = h_{t-1}: g passes on */
                        const double a = exp(s * A_d[n]);
                        pB_b[n * L + t] += g[n] * s * ut;
                        du_t += g[n] * s * Bt;
                        ds += g[n] * (A_d[n] * a * h_p[n] + Bt * ut);
                        dA[d * N + n] += g[n] * a * s * h_p[n];
                        g[n] *= a;                            /* a_t g_t, carried to t - 1 */
                    }
                    du[r * L + t] = du_t;
                    double dx = ds;
                    if (delta_softplus) {
                        const double x = dl_r[t] + bias;
                        dx = x > 20.0 ? ds : ds * sigmoid_ref(x);
                    }
                    ddelta[r * L + t] = dx;
                    if (dbias) dbias[d] += dx;
                }
                if (dh0)
                    for (int64_t n = 0; n < N; ++n) dh0[r * N + n] = g[n];
            }
        }
        free(hist);
        free(g);
        free(sv);
    }
    if (!bad_alloc) {
        for (int t = 0; t < nt; ++t) {
            const double* pB = part + (size_t)t * 2 * (size_t)(bc > 0 ? bc : 1);
            const double* pC = pB + (bc > 0 ? bc : 1);
            for (int64_t i = 0; i < bc; ++i) {
                dB[i] += pB[i];
                dC[i] += pC[i];
            }
        }
    }
    free(part);
    return bad_alloc ? -2 : 0;
}
