/*
 * ssm_ssd.h -- C ABI of the Mamba-2 (SSD) forward in libssmscan.so (gfx950).
 *
 * The operation is the selective recurrence of ssm_scan.h with A constrained to one scalar
 * per head, as ybb.press/ai-applications/14118.html ("Mamba state-space model: from theory
 * to production CUDA kernel optimisation", section 2.2) states for Mamba-2: nheads heads of
 * headdim channels; channel d = h * headdim + p belongs to head h and shares that head's A
 * and step size. For batch row b, step t and state n:
 *
 *   dt_t      = dt[b,h,t] + dt_bias[h]                  (bias optional, 0 if NULL)
 *   dt_t      = softplus(dt_t)                          (if SSM_DELTA_SOFTPLUS; 0 at padding)
 *   h_t[d,n]  = exp(dt_t * A[h]) * h_{t-1}[d,n] + dt_t * B[b,n,t] * x[b,d,t]
 *   y_t[d]    = sum_n C[b,n,t] * h_t[d,n] + D[d] * x[b,d,t]        (D optional)
 *   out[b,d,t] = y_t[d] * z * sigmoid(z), z = z[b,d,t]             (gate optional)
 *   final_state[b,d,n] = h_{L-1}[d,n]
 *
 * How it is computed: the semiseparable-matrix (state-space duality) form and its block
 * decomposition of mhpq.cn/news/1077344 (section 5.1, the recurrence unrolled into one
 * lower-triangular matrix per head; section 5.2, blocks handled by matrix products and a
 * scan between blocks) and ybb.press section 4.4 / section 8.1 (matrix units for the
 * large-state case). In 64-step blocks the kernels form G = C^T B once per (batch row,
 * block) and, per head, the block-diagonal part, the block-end state and the carried
 * state's contribution as bf16 MFMA products with fp32 accumulation (the decay between
 * two steps of a block factored through the block's midpoint where its range allows, the
 * decayed block matrix otherwise); the state itself is carried in fp32 (every fp32 value
 * that enters a product is split into two bf16 terms, so it keeps fp32-level accuracy).
 *
 * Memory: device pointers owned by the caller; C-contiguous arrays:
 *   x, z, out   : [batch, nheads*headdim, seqlen]   bf16
 *   dt          : [batch, nheads, seqlen]           bf16 (raw, before bias and softplus)
 *   B, C        : [batch, dstate, seqlen]           bf16, shared by all heads
 *   A, dt_bias  : [nheads]                          fp32
 *   D           : [nheads*headdim]                  fp32
 *   mask        : [batch, seqlen] bytes, 0 = padding step (the state is kept), as the
 *                 padding mask of mhpq.cn/news/1057127 (section 4)
 *   final_state : [batch, nheads*headdim, dstate]   fp32 (in/out with SSM_INITIAL_STATE)
 *   workspace   : ssm_ssd_workspace_bytes(batch, nheads, dstate, seqlen) bytes, 256-byte aligned,
 *                 scratch owned by the caller; its contents are overwritten and need not be
 *                 kept between calls. Calls that share a workspace must not overlap.
 *
 * Flags and status codes are those of ssm_scan.h (SSM_IO_BF16 is the only storage type
 * here; SSM_DELTA_SOFTPLUS, SSM_INITIAL_STATE). Calls are asynchronous on `stream`, use no
 * atomics (bitwise reproducible) and allocate nothing; every check happens before any HIP
 * call.
 */
#ifndef SSM_SSD_H
#define SSM_SSD_H

#include <stddef.h>
#include <stdint.h>

#include "ssm_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of workspace ssm_ssd_fwd needs: per (batch row, 64-step block) 64x64 bf16 for G
 * and 64 x dstate bf16 for C^T, and per (batch row, head, block) 1 KB of per-step factors
 * (4 x 64 fp32). 0 for empty problems; -1 for negative sizes or a size past int64. */
SSM_API int64_t ssm_ssd_workspace_bytes(int64_t batch, int64_t nheads, int64_t dstate,
                                        int64_t seqlen);

/*
 * ssm_ssd_fwd -- the Mamba-2 forward described above.
 *
 * Required: x, dt, A, B, C, out, workspace (each may be NULL only when its array is empty).
 * Optional (NULL): D, z, dt_bias, mask, final_state (required with SSM_INITIAL_STATE).
 * Sizes: batch, nheads, seqlen >= 0; headdim a positive multiple of 16; dstate one of 64,
 * 128, 256. seqlen == 0 leaves out untouched and sets final_state to the initial state.
 * Any seqlen >= 1; rows whose length is a multiple of 8 elements (with 16-byte aligned
 * x, z, out, B, C) take the vector path.
 * out must not overlap x, dt, z, B, C, A, D, dt_bias, mask, final_state or workspace.
 * Returns SSM_OK, SSM_ERR_INVALID_ARG, SSM_ERR_UNSUPPORTED (storage type not bf16, dstate or
 * headdim outside the above, sizes too large for 32-bit element offsets within one
 * batch row), SSM_ERR_MISALIGNED (an element-misaligned pointer, a workspace not 256-byte
 * aligned, final_state not 16-byte aligned) or SSM_ERR_HIP.
 */
SSM_API int ssm_ssd_fwd(const void* x, const void* dt, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* dt_bias,
                        const uint8_t* mask, uint32_t flags, void* out, float* final_state,
                        void* workspace, int64_t workspace_bytes, int64_t batch,
                        int64_t nheads, int64_t headdim, int64_t dstate, int64_t seqlen,
                        void* stream);

/*
 * ssm_ssd_fwd_noalloc -- ssm_ssd_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.
 *
 * The workspace is a static device buffer of SSM_SSD_NOALLOC_SCRATCH_BYTES (32 MiB) inside
 * the library; each device the library runs on holds its own copy until the process ends.
 * Arguments, layouts, results and status codes are those of ssm_ssd_fwd, bit for bit; a
 * problem whose ssm_ssd_workspace_bytes exceeds the buffer returns
 * SSM_ERR_SCRATCH_TOO_SMALL before any HIP call (the ssd workload of b4, 32 heads of 64
 * channels, 128 states, 2048 steps needs 7.3 MB). The call allocates nothing: no
 * hipMalloc, no hipFree, no library routine that allocates. The buffer's device address is
 * looked up once per device (hipGetSymbolAddress), on the first call on that device.
 *
 * Every call on one device shares that device's buffer, and a call leaves its contents
 * behind (nothing in it needs clearing: each call writes every part it reads). Calls that
 * may run at the same time on one device -- on different streams, or from different host
 * threads without ordering -- race on the buffer and must not be issued.
 */
#define SSM_SSD_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)

SSM_API int ssm_ssd_fwd_noalloc(const void* x, const void* dt, const float* A, const void* B,
                                const void* C, const float* D, const void* z,
                                const float* dt_bias, const uint8_t* mask, uint32_t flags,
                                void* out, float* final_state, int64_t batch, int64_t nheads,
                                int64_t headdim, int64_t dstate, int64_t seqlen, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SSD_H */
