/*
 * Oracle ABI (TEST INFRASTRUCTURE ONLY). Host pointers, C-contiguous:
 *   u, delta, z, out : [batch, dim, seqlen]
 *   B, C             : [batch, dstate, seqlen]
 *   A                : [dim, dstate]
 *   D, delta_bias    : [dim]
 *   h0, final_state  : [batch, dim, dstate]
 *   mask             : [batch, seqlen] bytes, 0 = padding position
 * D, z, delta_bias, h0, mask and final_state may be NULL (no skip, no gate, zero bias, zero
 * initial state, no padding, state not returned). nthreads <= 0 means one thread.
 * Returns 0, -1 for a bad argument, -2 if a row's scratch could not be allocated.
 */
#ifndef SSM_REF_H
#define SSM_REF_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

int ssm_ref_scan_f64(const double* u, const double* delta, const double* A, const double* B,
                     const double* C, const double* D, const double* z,
                     const double* delta_bias, int delta_softplus, const double* h0,
                     const unsigned char* mask, double* out, double* final_state,
                     int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int nthreads);

int ssm_ref_scan_f32(const float* u, const float* delta, const float* A, const float* B,
                     const float* C, const float* D, const float* z,
                     const float* delta_bias, int delta_softplus, const float* h0,
                     const unsigned char* mask, float* out, float* final_state,
                     int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int nthreads);

/* Reverse-mode derivative of ssm_ref_scan_f64 for the loss
 * sum(dout * out) + sum(dfinal * final_state) (ssm_ref_bwd.c).
 *   dout [batch, dim, seqlen] required; dfinal [batch, dim, dstate] may be NULL (zero).
 *   du, ddelta [batch, dim, seqlen], dA [dim, dstate], dB, dC [batch, dstate, seqlen]
 *   required; dz required when z is given; dD, dbias, dh0 may be NULL (not returned). */
int ssm_ref_scan_bwd_f64(const double* u, const double* delta, const double* A,
                         const double* B, const double* C, const double* D, const double* z,
                         const double* delta_bias, int delta_softplus, const double* h0,
                         const unsigned char* mask, const double* dout,
                         const double* dfinal, double* du,
                         double* ddelta, double* dA, double* dB, double* dC, double* dD,
                         double* dz, double* dbias, double* dh0, int64_t batch, int64_t dim,
                         int64_t dstate, int64_t seqlen, int nthreads);

int ssm_ref_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
