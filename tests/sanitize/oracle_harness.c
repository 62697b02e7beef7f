/* Host-only harness for the oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built and run by tests/test_host_sanitizers.py). Calls every oracle entry point on small
 * problems with every optional input present and absent, ragged sizes, a padding mask and
 * the empty shapes, and checks one exact result (the prefix sum 1,2,3,4 -> 1,3,6,10).
 * Exit status 0 and "oracle harness ok" on success. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ssm_ref.h"

static double* vec(size_t n, unsigned* seed, double scale) {
  double* p = (double*)malloc((n ? n : 1) * sizeof(double));
  for (size_t i = 0; i < n; ++i) {
    *seed = *seed * 1103515245u + 12345u;
    p[i] = scale * ((double)((*seed >> 8) & 0xffff) / 32768.0 - 1.0);
  }
  return p;
}

static int run_case(int64_t b, int64_t d, int64_t n, int64_t L, int opt, unsigned seed) {
  const size_t e = (size_t)(b * d * L), bc = (size_t)(b * n * L), st = (size_t)(b * d * n);
  double *u = vec(e, &seed, 1), *dl = vec(e, &seed, 0.5), *A = vec((size_t)(d * n), &seed, 1);
  double *B = vec(bc, &seed, 1), *C = vec(bc, &seed, 1), *D = vec((size_t)d, &seed, 1);
  double *z = vec(e, &seed, 1), *bias = vec((size_t)d, &seed, 0.1), *h0 = vec(st, &seed, 1);
  double *out = vec(e, &seed, 0), *fin = vec(st, &seed, 0), *dout = vec(e, &seed, 1);
  double *dfin = vec(st, &seed, 1);
  double *du = vec(e, &seed, 0), *dd = vec(e, &seed, 0), *dA = vec((size_t)(d * n), &seed, 0);
  double *dB = vec(bc, &seed, 0), *dC = vec(bc, &seed, 0), *dD = vec((size_t)d, &seed, 0);
  double *dz = vec(e, &seed, 0), *dbias = vec((size_t)d, &seed, 0), *dh0 = vec(st, &seed, 0);
  float* f = (float*)malloc((e ? e : 1) * sizeof(float) * 4 + (bc ? bc : 1) * sizeof(float) * 2 +
                            (size_t)(d * n + 1) * sizeof(float) + (st + 1) * sizeof(float) * 2);
  unsigned char* mask = (unsigned char*)malloc((size_t)(b * L) + 1);
  for (int64_t i = 0; i < b * L; ++i) mask[i] = (unsigned char)((i * 7) % 5 != 0);
  for (size_t i = 0; i < (size_t)(d * n); ++i) A[i] = -fabs(A[i]) - 0.1;
  const int sp = opt & 1, use_opt = (opt & 2) != 0, use_mask = (opt & 4) != 0;
  int rc = ssm_ref_scan_f64(u, dl, A, B, C, use_opt ? D : NULL, use_opt ? z : NULL,
                            use_opt ? bias : NULL, sp, use_opt ? h0 : NULL,
                            use_mask ? mask : NULL, out, fin, b, d, n, L, 3);
  if (rc != 0) return 1;
  /* the float32 instantiation on the same values */
  float *fu = f, *fdl = fu + e, *fz = fdl + e, *fo = fz + e, *fB = fo + e, *fC = fB + bc;
  float *fA = fC + bc, *ffin = fA + d * n, *fh0 = ffin + st;
  for (size_t i = 0; i < e; ++i) { fu[i] = (float)u[i]; fdl[i] = (float)dl[i]; fz[i] = (float)z[i]; }
  for (size_t i = 0; i < bc; ++i) { fB[i] = (float)B[i]; fC[i] = (float)C[i]; }
  for (size_t i = 0; i < (size_t)(d * n); ++i) fA[i] = (float)A[i];
  for (size_t i = 0; i < st; ++i) fh0[i] = (float)h0[i];
  rc = ssm_ref_scan_f32(fu, fdl, fA, fB, fC, NULL, use_opt ? fz : NULL, NULL, sp,
                        use_opt ? fh0 : NULL, use_mask ? mask : NULL, fo, ffin, b, d, n, L, 2);
  if (rc != 0) return 2;
  rc = ssm_ref_scan_bwd_f64(u, dl, A, B, C, use_opt ? D : NULL, use_opt ? z : NULL,
                            use_opt ? bias : NULL, sp, use_opt ? h0 : NULL,
                            use_mask ? mask : NULL, dout, use_opt ? dfin : NULL, du, dd, dA, dB,
                            dC, use_opt ? dD : NULL, use_opt ? dz : NULL,
                            use_opt ? dbias : NULL, dh0, b, d, n, L, 3);
  if (rc != 0) return 3;
  double* all[] = {u, dl, A, B, C, D, z, bias, h0, out, fin, dout, dfin, du, dd, dA, dB, dC,
                   dD, dz, dbias, dh0};
  for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
  free(f);
  free(mask);
  return 0;
}

int main(void) {
  /* the worked example: A = 0, delta = 1, B = C = e_0, u = 1 2 3 4 */
  double u[4] = {1, 2, 3, 4}, dl[4] = {1, 1, 1, 1}, A[2] = {0, 0};
  double B[8] = {1, 1, 1, 1, 0, 0, 0, 0}, out[4], fin[2];
  if (ssm_ref_scan_f64(u, dl, A, B, B, NULL, NULL, NULL, 0, NULL, NULL, out, fin, 1, 1, 2, 4,
                       1) != 0 ||
      out[0] != 1 || out[1] != 3 || out[2] != 6 || out[3] != 10) {
    printf("prefix sum wrong\n");
    return 1;
  }
  /* argument errors are reported, not dereferenced */
  if (ssm_ref_scan_f64(NULL, dl, A, B, B, NULL, NULL, NULL, 0, NULL, NULL, out, fin, 1, 1, 2, 4,
                       1) != -1)
    return 1;
  const int64_t shapes[][4] = {{1, 1, 1, 1}, {2, 3, 5, 7}, {1, 4, 17, 37}, {3, 2, 64, 9},
                               {2, 5, 3, 130}, {0, 3, 4, 5}, {2, 0, 4, 5}, {2, 3, 4, 0}};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
    for (int opt = 0; opt < 8; ++opt) {
      const int rc = run_case(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], opt,
                              (unsigned)(17 * s + opt));
      if (rc) {
        printf("case %zu opt %d failed (%d)\n", s, opt, rc);
        return 1;
      }
    }
  printf("oracle harness ok\n");
  return 0;
}
