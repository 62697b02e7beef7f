/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective-scan forward library.
 *
 * The operation (Mamba's selective scan, forward pass) is defined on these pages:
 *   - ybb.press, "Mamba state-space model: from theory to production CUDA kernel
 *     optimisation": section 1.2 (discretisation and recurrence h_t = A_bar h_{t-1} +
 *     B_bar x_t, y_t = C h_t), section 2.3 (causal selective scan with delta-dependent
 *     exp(delta*A) and delta*B, then the D skip), section 3.2 (the associative combine
 *     (A1,B1) o (A2,B2) = (A2*A1, A2*B1 + B2)), section 4.2 (kernel arguments u, delta, A,
 *     B, C, D, out, final_state with u/delta/out laid out [batch, dim, seq_len]),
 *     section 7.1 (softplus on delta, initial state, returned final state);
 *   - jsqmd.com, "From matrix summation to state updates: Blelloch parallel scan as the
 *     engine of Mamba.py", section 3.2 (deltaA = exp(delta*A), deltaB = delta*B, y = hs@C
 *     + D*x);
 *   - mhpq.cn/news/1057127, "The hardware truth of Mamba's parallel scan", section 1
 *     (diagonal A, independent state chains) and section 2 (one fused kernel including a
 *     sigmoid-type gate).
 *
 * For every batch row b < batch, channel d < dim and state n < dstate:
 *
 *   dt_t     = delta[b,d,t] + delta_bias[d]         (bias optional, 0 if NULL)
 *   dt_t     = softplus(dt_t)                       (if SSM_DELTA_SOFTPLUS)
 *   h_t[n]   = exp(dt_t * A[d,n]) * h_{t-1}[n] + dt_t * B[b,n,t] * u[b,d,t]
 *   y_t      = sum_n C[b,n,t] * h_t[n] + D[d] * u[b,d,t]     (D optional)
 *   out[b,d,t] = y_t * z * sigmoid(z), z = z[b,d,t]          (gate optional: y_t if NULL)
 *   final_state[b,d,n] = h_{L-1}[n]                          (ungated state after the last step)
 *
 * with h_{-1} = 0, or h_{-1} = final_state[b,d,:] on entry when SSM_INITIAL_STATE is set.
 * softplus(x) = log(1 + exp(x)), taken as x itself above 20.
 *
 * Memory: every pointer is a DEVICE pointer owned by the caller; arrays are C-contiguous:
 *   u, delta, z, out : [batch, dim, seqlen]   storage type from the flags (fp32 or bf16)
 *   B, C             : [batch, dstate, seqlen] same storage type, shared by all channels
 *   A                : [dim, dstate]   fp32
 *   D, delta_bias    : [dim]           fp32
 *   final_state      : [batch, dim, dstate] fp32
 * Arithmetic is fp32 throughout (state, exp, accumulation); bf16 outputs are rounded to
 * nearest-even once at the store.
 *
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream) and return
 * once the work is queued. The library allocates nothing, keeps no per-call state, uses no
 * atomics (results are bitwise reproducible run to run) and is safe to call from several
 * host threads. A fault inside the kernel surfaces at the caller's next synchronisation.
 *
 * Every argument check happens before any HIP call, so an invalid call returns its error
 * code without touching the device.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported from libssmscan.so (built with hidden visibility for everything else). */
#if defined(__GNUC__) || defined(__clang__)
#define SSM_API __attribute__((visibility("default")))
#else
#define SSM_API
#endif

/* flags: bits 0-1 storage type of u, delta, B, C, z and out */
#define SSM_IO_F32 0u
#define SSM_IO_BF16 1u
#define SSM_IO_MASK 3u
/* delta <- softplus(delta + delta_bias) before use */
#define SSM_DELTA_SOFTPLUS (1u << 4)
/* final_state is in/out: read as h_{-1}, overwritten with h_{L-1} */
#define SSM_INITIAL_STATE (1u << 5)
/* Launch-shape hints for the chunked scan (seqlen > 32), forward entry points only: how many
 * wavefronts share one channel's states. With neither bit the library chooses: fp32 launches
 * whose workgroups all fit on the device at once take two waves per channel, every other
 * launch one. Two waves per channel exist for fp32 storage only (SSM_ERR_UNSUPPORTED with
 * bf16); setting both bits is SSM_ERR_INVALID_ARG. The two forms compute every state in the
 * same order (final and saved states bitwise equal) and sum y over the states in a different
 * order (outputs equal to fp32 rounding). Sequences of at most 32 steps ignore the hint. */
#define SSM_WAVES_PER_CHANNEL_1 (1u << 8)
#define SSM_WAVES_PER_CHANNEL_2 (1u << 9)
/* Backward (ssm_scan_bwd and ssm_scan_bwd_workspace_bytes) only: keep every channel's whole
 * sequence in one workgroup. Without it, a backward with a workspace on a problem whose
 * channels alone do not fill the device cuts each sequence into segments of whole saved-state
 * intervals, scanned by different workgroups from the state adjoint carried into them (a
 * first launch finds each segment's adjoint from a zero start; the carries are then combined
 * right to left, which p1 section 3.3's chunked backward implies). The two forms agree to fp32
 * rounding; each is bitwise reproducible. */
#define SSM_BWD_UNSPLIT (1u << 10)

/* status codes */
#define SSM_OK 0
#define SSM_ERR_INVALID_ARG (-1) /* NULL required pointer, negative size, unknown flag bit,
                                    SSM_INITIAL_STATE without final_state, out overlapping
                                    an input */
#define SSM_ERR_UNSUPPORTED (-2) /* dstate outside [1, 64], storage type not fp32/bf16,
                                    sizes whose products overflow 64-bit offsets, batch*dim
                                    or seqlen above 2^31 - 1, or one row (seqlen elements)
                                    or one batch row of B (dstate*seqlen elements) above
                                    2 GiB */
#define SSM_ERR_MISALIGNED (-3)  /* a pointer not aligned to its element size */
#define SSM_ERR_HIP (-4)         /* the HIP runtime refused the launch (no gfx950 device,
                                    bad stream, ...) */
#define SSM_ERR_SCRATCH_TOO_SMALL (-5) /* an allocation-free entry point: the problem needs
                                    more workspace than its static device buffer holds */

/*
 * ssm_scan_fwd -- the selective-scan forward described above.
 *
 * Required: u, delta, A, B, C, out (each may be NULL only when its array is empty).
 * Optional (NULL): D (no skip), z (no gate), delta_bias (zero bias), final_state (state not
 * returned; required with SSM_INITIAL_STATE unless batch*dim == 0).
 * Sizes: batch, dim, seqlen >= 0; 1 <= dstate <= 64. batch*dim == 0 is a no-op; seqlen == 0
 * leaves out untouched and sets final_state to the initial state (zeros unless
 * SSM_INITIAL_STATE). Any seqlen >= 1 is supported (no multiple-of constraint). Up to 32
 * steps run a per-step kernel (decode, state passing), longer sequences the chunked scan;
 * the two agree to fp32 rounding, not bitwise. Pointers
 * need only element alignment (16-byte aligned rows take the vector path).
 * out must not overlap u, delta, z, B, C, A, D, delta_bias or final_state.
 * Returns SSM_OK or one of the SSM_ERR_* codes above.
 */
SSM_API int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* z, const float* delta_bias,
                 uint32_t flags, void* out, float* final_state, int64_t batch, int64_t dim,
                 int64_t dstate, int64_t seqlen, void* stream);

/*
 * Training: the forward that also saves states, and the backward pass.
 *
 * The backward recomputes the scan from states the forward saved at regular intervals,
 * instead of keeping every h_t: mhpq.cn/news/1077344 (section 3.3) describes the fused
 * scan's backward this way (only chunk-boundary states are stored; the scan is run again
 * from them inside the kernel before the gradients are formed).
 */

/* Saved states sit every SSM_CKPT_INTERVAL steps: entry k is the state entering step
 * k * SSM_CKPT_INTERVAL (entry 0 is the initial state). */
#define SSM_CKPT_INTERVAL 256

/* Number of saved states per (batch row, channel): ceil(seqlen / SSM_CKPT_INTERVAL), 0 for
 * seqlen <= 0. */
SSM_API int64_t ssm_scan_ckpt_count(int64_t seqlen);

/*
 * ssm_scan_fwd_ckpt -- ssm_scan_fwd that also writes the saved states.
 * chunk_states: fp32 [batch, dim, ssm_scan_ckpt_count(seqlen), dstate], device, written
 * (required unless empty; must not overlap out). Every other argument and error code is
 * that of ssm_scan_fwd, whose outputs it produces bit for bit.
 */
SSM_API int ssm_scan_fwd_ckpt(const void* u, const void* delta, const float* A, const void* B,
                              const void* C, const float* D, const void* z,
                              const float* delta_bias, uint32_t flags, void* out,
                              float* final_state, float* chunk_states, int64_t batch,
                              int64_t dim, int64_t dstate, int64_t seqlen, void* stream);

/*
 * ssm_scan_fwd_masked -- the forward with a padding mask, and optionally the saved states.
 * mask: [batch, seqlen] bytes on the device (nullable: no padding). At a step whose byte is
 * 0 the state is inherited from the previous step instead of updated, as the padding mask
 * of mhpq.cn/news/1057127 (section 4) does; the output there is still sum_n C h + D u
 * (gated) of that state, and the step size is not used. The mask is shared by all
 * channels of a batch row; a per-row length is the mask t < len. chunk_states: as for
 * ssm_scan_fwd_ckpt, or NULL. Otherwise as ssm_scan_fwd.
 */
SSM_API int ssm_scan_fwd_masked(const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D, const void* z,
                                const float* delta_bias, const uint8_t* mask, uint32_t flags,
                                void* out, float* final_state, float* chunk_states,
                                int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                void* stream);

/*
 * ssm_scan_bwd -- gradients of L = sum(dout * out) + sum(dfinal * final_state) with
 * respect to every input of ssm_scan_fwd.
 *
 * Inputs: the forward's u, delta, A, B, C, D, z, delta_bias, mask and flags (SSM_INITIAL_STATE
 * is accepted and has no further effect: the initial state is entry 0 of chunk_states),
 * chunk_states from ssm_scan_fwd_ckpt on the same inputs, dout [batch, dim, seqlen] in the
 * storage type, dfinal fp32 [batch, dim, dstate] (NULL: zero).
 * Outputs (device, written; the "summed" ones are overwritten, not accumulated into):
 *   du, ddelta   [batch, dim, seqlen]  storage type (ddelta is the gradient of the raw
 *                delta, through softplus when SSM_DELTA_SOFTPLUS is set)
 *   dz           [batch, dim, seqlen]  storage type; required when z is given, else unused
 *   dA           [dim, dstate]         fp32, summed over batch rows
 *   dB, dC       [batch, dstate, seqlen] fp32, summed over channels
 *   dD, dbias    [dim]                 fp32, summed over batch rows and steps; NULL = not
 *                wanted (ignored when D or delta_bias is NULL)
 *   dh0          [batch, dim, dstate]  fp32, gradient of the initial state; NULL = not
 *                wanted
 * workspace: NULL, or ssm_scan_bwd_workspace_bytes(batch, dim, dstate, seqlen, flags) bytes
 * (workspace_bytes, at least that), 256-byte aligned, device scratch owned by the caller,
 * overlapping no other argument; its contents are overwritten and need not be kept between
 * calls, and calls that share it must not overlap in time.
 * The summed gradients (dA, dB, dC, dD, dbias) add up contributions of many channels or
 * batch rows. With a workspace, each workgroup stores its partial sums there and a second
 * launch adds them in a fixed order: every output is bitwise reproducible. Without one they
 * are accumulated with floating-point atomics (after a zero fill), which needs no scratch but
 * is slower and not reproducible from run to run (within fp32 rounding of one another); du,
 * ddelta, dz and dh0 are reproducible either way. Errors as for ssm_scan_fwd, plus
 * SSM_ERR_INVALID_ARG for a workspace that is too small or overlaps an argument,
 * SSM_ERR_MISALIGNED for one not 256-byte aligned, and SSM_ERR_UNSUPPORTED for a row of
 * seqlen elements above 1 GiB (two channel rows are addressed as one 2 GiB block).
 */
SSM_API int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B,
                         const void* C, const float* D, const void* z,
                         const float* delta_bias, const uint8_t* mask, uint32_t flags,
                         const float* chunk_states,
                         const void* dout, const float* dfinal, void* du, void* ddelta,
                         float* dA, float* dB, float* dC, float* dD, void* dz, float* dbias,
                         float* dh0, void* workspace, int64_t workspace_bytes, int64_t batch,
                         int64_t dim, int64_t dstate, int64_t seqlen, void* stream);

/*
 * Bytes of workspace ssm_scan_bwd needs for reproducible sums: each workgroup's sums of dB
 * and dC over its channels (32 channels per workgroup, whatever the storage type in flags
 * bits 0-1), 2 x dstate x seqlen fp32 per workgroup, and dA, dD and dbias per batch row and
 * segment, plus each segment's carried adjoint when the current device's rule cuts the
 * sequences into segments (see SSM_BWD_UNSPLIT; the size then depends on the device's
 * compute-unit count). ssm_scan_bwd uses as many segments as the workspace it is given holds,
 * down to none: a workspace of the size queried with SSM_BWD_UNSPLIT always works. 0 for
 * empty problems; -1 for negative sizes, an unknown storage type or a size past int64.
 */
SSM_API int64_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t dstate,
                                             int64_t seqlen, uint32_t flags);

/* Static, human-readable text for a status code (never NULL). */
SSM_API const char* ssm_scan_strerror(int status);

/* Version of this ABI (bumped on any incompatible change): 6. */
SSM_API int ssm_scan_abi_version(void);

/*
 * ssm_scan_debug_wave_combine -- runs only the wave-level inclusive scan of the pages'
 * combine, (a1,b1) o (a2,b2) = (a2*a1, a2*b1 + b2) (ybb.press section 3.2; mhpq.cn/news/
 * 1077344 section 2.2), over groups of 64 consecutive pairs, one 64-lane wavefront per
 * group. a, b, a_out, b_out are device arrays of 64*groups floats; a_out[i], b_out[i]
 * receive the combine of pairs 64*g .. i in order. It uses the same device routine as the
 * forward kernel and exists so that tests can check that routine's lane wiring exactly.
 */
SSM_API int ssm_scan_debug_wave_combine(const float* a, const float* b, float* a_out, float* b_out,
                                int64_t groups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
