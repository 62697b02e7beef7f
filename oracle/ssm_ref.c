/*
 * Plain CPU oracle for the Mamba selective-scan forward.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline
 * leg are the only code that may load this library. It shares no source, header, table
 * or helper with the GPU library, and the GPU library never calls it.
 *
 * It is the sequential definition written out, a straight loop per (batch, channel):
 *
 *   h[n] = h0[b,d,n]  (or 0)                                   initial state
 *   for t in 0 .. L-1:
 *       dt   = softplus(delta[b,d,t] + bias[d])                 step size
 *       h[n] = exp(dt * A[d,n]) * h[n] + dt * B[b,n,t] * u[b,d,t]   for each n
 *       (a padding position, mask[b,t] == 0, keeps h[n] unchanged instead)
 *       y    = sum_n C[b,n,t] * h[n] + D[d] * u[b,d,t]
 *       out[b,d,t] = y * z * sigmoid(z)   (gate present)   or   y
 *   final_state[b,d,n] = h[n]
 *
 * Sources on the pages (all four are web articles on Mamba's selective scan):
 *  - ybb.press, "Mamba state-space model: from theory to production CUDA kernel
 *    optimisation": section 1.2 (discretisation, h_t = A_bar h_{t-1} + B_bar x_t,
 *    y_t = C h_t), section 2.3 (causal selective scan: per step exp(delta*A), delta*B,
 *    state update, output, then the D residual), section 7.1 (PyTorch version with
 *    softplus on delta, an optional initial state and the returned final state).
 *  - jsqmd.com, "From matrix summation to state updates: Blelloch parallel scan as the
 *    engine of Mamba.py", section 3.2 (deltaA = exp(delta*A), deltaB = delta*B,
 *    BX = deltaB*x, y = hs @ C + D*x).
 *  - mhpq.cn/news/1057127, "The hardware truth of Mamba's parallel scan", section 1
 *    (diagonal A: the N state chains are independent), section 4 (a padding mask: at a
 *    masked position the state is inherited from the previous step, not updated).
 *
 * Readings where the pages are silent or garbled (each is listed with its reason in the
 * design notes): B_bar = delta * B (not the ZOH form); bias is added before softplus;
 * softplus(x) = log1p(exp(x)), returning x above 20; y uses the state after the update;
 * the gate multiplies (C.h + D u) by silu(z) and leaves the state alone; A is [dim, N];
 * B and C are [batch, N, seqlen]; a masked position still produces an output from the
 * (unchanged) state, and the mask is per (batch, step), shared by every channel.
 *
 * Parity pins (tests/test_oracle_pins.py) tie this code to the pages' worked examples,
 * closed forms and brute-force expansions. Every function here is pinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "ssm_ref.h"

#define REAL double
#define EXP exp
#define LOG1P log1p
#define FN ssm_ref_scan_f64
#include "ssm_ref_body.inc"
#undef REAL
#undef EXP
#undef LOG1P
#undef FN

/* The same loop in float32: used only to measure the rounding floor of a float32
 * implementation against the float64 one, never as a reference. */
#define REAL float
#define EXP expf
#define LOG1P log1pf
#define FN ssm_ref_scan_f32
#include "ssm_ref_body.inc"
#undef REAL
#undef EXP
#undef LOG1P
#undef FN

int ssm_ref_abi_version(void) { return 1; }
