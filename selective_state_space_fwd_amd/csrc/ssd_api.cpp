// C-ABI entry points of the Mamba-2 (SSD) forward (declared in include/ssm_ssd.h).
// Argument checking happens here, before any HIP call; the launches are in ssd_kernels.hip.
#include <stdint.h>

#include "api_util.h"
#include "scan_launch.h"
#include "ssm_ssd.h"

using ssm_api::aligned;
using ssm_api::kInt32Max;
using ssm_api::mul_ok;
using ssm_api::overlaps;
using ssm_api::Range;
using ssm_api::span;

namespace {

// ceil(seqlen / block), without forming seqlen + block - 1 (overflows near INT64_MAX)
int64_t nblocks_of(int64_t seqlen) {
  return seqlen / ssm::kSsdBlock + (seqlen % ssm::kSsdBlock != 0);
}

}  // namespace

extern "C" {

int64_t ssm_ssd_workspace_bytes(int64_t batch, int64_t nheads, int64_t dstate,
                                int64_t seqlen) {
  if (batch < 0 || nheads < 0 || dstate < 0 || seqlen < 0) return -1;
  int64_t per_block, blocks, shared, head_blocks, steps, total;
  const int64_t q = ssm::kSsdBlock;
  // per (batch row, block): G (q x q bf16) and C^T (q x dstate bf16); per (batch row, head,
  // block): the step record, 4 x q fp32
  if (!mul_ok(dstate, 2 * q, &per_block) || per_block > INT64_MAX - q * q * 2 ||
      !mul_ok(batch, nblocks_of(seqlen), &blocks) ||
      !mul_ok(blocks, q * q * 2 + per_block, &shared) ||
      !mul_ok(blocks, nheads, &head_blocks) || !mul_ok(head_blocks, 4 * q * 4, &steps) ||
      shared > INT64_MAX - steps)
    return -1;
  total = shared + steps;
  return total;
}

}  // extern "C"

namespace ssm {

int ssd_fwd_impl(const void* x, const void* dt, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* dt_bias, const uint8_t* mask,
                 uint32_t flags, void* out, float* final_state, void* workspace,
                 int64_t workspace_bytes, int64_t batch, int64_t nheads, int64_t headdim,
                 int64_t dstate, int64_t seqlen, void* stream, const SsdScratch* scratch) {
  const uint32_t known = SSM_IO_MASK | SSM_DELTA_SOFTPLUS | SSM_INITIAL_STATE;
  if (flags & ~known) return SSM_ERR_INVALID_ARG;
  if (batch < 0 || nheads < 0 || headdim < 0 || dstate < 0 || seqlen < 0)
    return SSM_ERR_INVALID_ARG;
  if ((flags & SSM_IO_MASK) != SSM_IO_BF16) return SSM_ERR_UNSUPPORTED;
  if (dstate != 64 && dstate != 128 && dstate != 256) return SSM_ERR_UNSUPPORTED;
  if (headdim < 16 || headdim % 16 != 0) return SSM_ERR_UNSUPPORTED;
  const bool initial_state = (flags & SSM_INITIAL_STATE) != 0;

  int64_t dim, row_elems, elems, bc_row, bc, rows, state, head_steps, hl, need;
  if (!mul_ok(nheads, headdim, &dim) || !mul_ok(dim, seqlen, &row_elems) ||
      !mul_ok(batch, row_elems, &elems) || !mul_ok(dstate, seqlen, &bc_row) ||
      !mul_ok(batch, bc_row, &bc) || !mul_ok(batch, dim, &rows) ||
      !mul_ok(rows, dstate, &state) || !mul_ok(nheads, seqlen, &head_steps) ||
      !mul_ok(batch, head_steps, &hl))
    return SSM_ERR_UNSUPPORTED;
  // One batch row of x/z/out and of B/C is addressed with 32-bit byte offsets.
  if (row_elems * 2 >= (int64_t(1) << 31) || bc_row * 2 >= (int64_t(1) << 31) ||
      batch > 65535 || nheads > 65535 || seqlen > kInt32Max)
    return SSM_ERR_UNSUPPORTED;
  need = ssm_ssd_workspace_bytes(batch, nheads, dstate, seqlen);
  if (need < 0) return SSM_ERR_UNSUPPORTED;
  // The kernels run one-dimensional grids: batch x blocks plus (batch x heads x blocks) / 4
  // workgroups, and batch x heads x groups of 32 channels.
  if (batch * nblocks_of(seqlen) + (batch * nheads * nblocks_of(seqlen) + 3) / 4 > kInt32Max ||
      batch * nheads * ((headdim + 31) / 32) > kInt32Max)
    return SSM_ERR_UNSUPPORTED;

  const bool any = elems > 0;
  if ((any && (!x || !dt || !out || (!workspace && !scratch))) || (bc > 0 && (!B || !C)) ||
      (nheads > 0 && !A))
    return SSM_ERR_INVALID_ARG;
  if (scratch) {
    if (need > scratch->max_bytes) return SSM_ERR_SCRATCH_TOO_SMALL;
  } else if (any && workspace_bytes < need) {
    return SSM_ERR_INVALID_ARG;
  }
  if (initial_state && state > 0 && !final_state) return SSM_ERR_INVALID_ARG;

  if (!aligned(x, 2) || !aligned(dt, 2) || !aligned(B, 2) || !aligned(C, 2) ||
      !aligned(out, 2) || (z && !aligned(z, 2)) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
      (dt_bias && !aligned(dt_bias, 4)) || (final_state && !aligned(final_state, 16)) ||
      (!scratch && !aligned(workspace, 256)))
    return SSM_ERR_MISALIGNED;

  if (any) {
    const Range o = span(out, elems * 2);
    if (overlaps(o, span(x, elems * 2)) || overlaps(o, span(dt, hl * 2)) ||
        (z && overlaps(o, span(z, elems * 2))) || overlaps(o, span(B, bc * 2)) ||
        overlaps(o, span(C, bc * 2)) || overlaps(o, span(A, nheads * 4)) ||
        (D && overlaps(o, span(D, dim * 4))) ||
        (dt_bias && overlaps(o, span(dt_bias, nheads * 4))) ||
        (mask && overlaps(o, span(mask, batch * seqlen))) ||
        (final_state && overlaps(o, span(final_state, state * 4))) ||
        (!scratch && overlaps(o, span(workspace, need))))
      return SSM_ERR_INVALID_ARG;
  }

  if (batch == 0 || dim == 0) return SSM_OK;
  if (seqlen == 0) {
    // An empty scan leaves the state where it started.
    if (final_state && !initial_state)
      return ssm::launch_fill_zero(final_state, state, stream) == 0 ? SSM_OK : SSM_ERR_HIP;
    return SSM_OK;
  }

  // Every check has passed: only now may the workspace come from the static scratch
  // buffer (its address is looked up with a HIP call on first use on a device).
  if (scratch) {
    workspace = scratch->get();
    if (!workspace) return SSM_ERR_HIP;
  }

  ssm::SsdArgs a;
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.z = z;
  a.dt_bias = dt_bias;
  a.mask = mask;
  a.out = out;
  a.final_state = final_state;
  a.workspace = workspace;
  a.batch = batch;
  a.nheads = nheads;
  a.headdim = headdim;
  a.dstate = dstate;
  a.seqlen = seqlen;
  a.softplus = (flags & SSM_DELTA_SOFTPLUS) != 0;
  a.initial_state = initial_state;
  a.vec_ok = seqlen % 8 == 0 && aligned(x, 16) && aligned(out, 16) && aligned(B, 16) &&
             aligned(C, 16) && (!z || aligned(z, 16));
  return ssm::launch_ssd_fwd(a, stream) == 0 ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace ssm

extern "C" {

int ssm_ssd_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* dt_bias, const uint8_t* mask,
                uint32_t flags, void* out, float* final_state, void* workspace,
                int64_t workspace_bytes, int64_t batch, int64_t nheads, int64_t headdim,
                int64_t dstate, int64_t seqlen, void* stream) {
  return ssm::ssd_fwd_impl(x, dt, A, B, C, D, z, dt_bias, mask, flags, out, final_state,
                           workspace, workspace_bytes, batch, nheads, headdim, dstate, seqlen,
                           stream, nullptr);
}

}  // extern "C"
