// C-ABI entry points of libssmscan.so (declared in include/ssm_scan.h).
// Argument checking happens here, before any HIP call; the launches are in
// scan_kernels.hip.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include "api_util.h"
#include "scan_launch.h"
#include "ssm_scan.h"

namespace {

using ssm_api::aligned;
using ssm_api::kInt32Max;
using ssm_api::mul_ok;
using ssm_api::overlaps;
using ssm_api::Range;
using ssm_api::span;

}  // namespace

extern "C" {

int ssm_scan_abi_version(void) { return 6; }

const char* ssm_scan_strerror(int status) {
  switch (status) {
    case SSM_OK:
      return "ok";
    case SSM_ERR_INVALID_ARG:
      return "invalid argument (NULL required pointer, negative size, unknown flag, "
             "SSM_INITIAL_STATE without final_state, or out overlapping an input)";
    case SSM_ERR_UNSUPPORTED:
      return "unsupported (dstate outside [1, 64], storage type other than fp32/bf16, or "
             "sizes beyond the supported range)";
    case SSM_ERR_MISALIGNED:
      return "a pointer is not aligned to its element size";
    case SSM_ERR_HIP:
      return "the HIP runtime refused the launch";
    case SSM_ERR_SCRATCH_TOO_SMALL:
      return "the problem needs more workspace than the allocation-free entry point's static "
             "device buffer holds (use the entry point that takes a workspace)";
    default:
      return "unknown status";
  }
}

}  // extern "C"

namespace {

static_assert(ssm::kCkptInterval == SSM_CKPT_INTERVAL, "one saved-state spacing");

int64_t ckpt_count(int64_t seqlen) {
  // ceil(seqlen / interval), without forming seqlen + interval - 1 (overflows near INT64_MAX)
  return seqlen <= 0 ? 0 : seqlen / SSM_CKPT_INTERVAL + (seqlen % SSM_CKPT_INTERVAL != 0);
}

int fwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
             const float* D, const void* z, const float* delta_bias, const uint8_t* mask,
             uint32_t flags, void* out, float* final_state, float* ckpt, bool want_ckpt,
             int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, void* stream) {
  const uint32_t hints = SSM_WAVES_PER_CHANNEL_1 | SSM_WAVES_PER_CHANNEL_2;
  const uint32_t known = SSM_IO_MASK | SSM_DELTA_SOFTPLUS | SSM_INITIAL_STATE | hints;
  if (flags & ~known) return SSM_ERR_INVALID_ARG;
  if ((flags & hints) == hints) return SSM_ERR_INVALID_ARG;
  if (batch < 0 || dim < 0 || dstate < 0 || seqlen < 0) return SSM_ERR_INVALID_ARG;
  const bool initial_state = (flags & SSM_INITIAL_STATE) != 0;

  const uint32_t io = flags & SSM_IO_MASK;
  if (io != SSM_IO_F32 && io != SSM_IO_BF16) return SSM_ERR_UNSUPPORTED;
  if (dstate < 1 || dstate > 64) return SSM_ERR_UNSUPPORTED;
  if (io == SSM_IO_BF16 && (flags & SSM_WAVES_PER_CHANNEL_2)) return SSM_ERR_UNSUPPORTED;
  const int64_t esz = (io == SSM_IO_BF16) ? 2 : 4;

  int64_t rows, elems, elems_bytes, bc, bc_bytes, state, state_bytes, a_elems;
  if (!mul_ok(batch, dim, &rows) || !mul_ok(rows, seqlen, &elems) ||
      !mul_ok(elems, esz, &elems_bytes) || !mul_ok(batch, dstate, &bc) ||
      !mul_ok(bc, seqlen, &bc) || !mul_ok(bc, esz, &bc_bytes) ||
      !mul_ok(rows, dstate, &state) || !mul_ok(state, 4, &state_bytes) ||
      !mul_ok(dim, dstate, &a_elems))
    return SSM_ERR_UNSUPPORTED;
  if (rows > kInt32Max || seqlen > kInt32Max || dim > kInt32Max ||
      rows / 64 + 1 > kInt32Max)
    return SSM_ERR_UNSUPPORTED;
  // Rows of u/delta/z/out and each batch row's B/C block are addressed with 32-bit byte
  // offsets (with one chunk of slack past the end).
  if (seqlen * esz > (int64_t(1) << 31) || dstate * seqlen * esz > (int64_t(1) << 31))
    return SSM_ERR_UNSUPPORTED;

  // A required array may be NULL only when it holds no element.
  if ((elems > 0 && (!u || !delta || !out)) || (bc > 0 && (!B || !C)) || (a_elems > 0 && !A))
    return SSM_ERR_INVALID_ARG;
  if (initial_state && state > 0 && !final_state) return SSM_ERR_INVALID_ARG;
  int64_t ckpt_elems = 0, ckpt_bytes = 0;
  if (want_ckpt) {
    if (!mul_ok(state, ckpt_count(seqlen), &ckpt_elems) || !mul_ok(ckpt_elems, 4, &ckpt_bytes))
      return SSM_ERR_UNSUPPORTED;
    if (ckpt_elems > 0 && !ckpt) return SSM_ERR_INVALID_ARG;
    if (!aligned(ckpt, 4)) return SSM_ERR_MISALIGNED;
  }

  const uintptr_t ea = static_cast<uintptr_t>(esz);
  if (!aligned(u, ea) || !aligned(delta, ea) || !aligned(B, ea) || !aligned(C, ea) ||
      !aligned(out, ea) || (z && !aligned(z, ea)) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
      (delta_bias && !aligned(delta_bias, 4)) || (final_state && !aligned(final_state, 4)))
    return SSM_ERR_MISALIGNED;

  // out is written while the inputs are still being read: it must not overlap any of them.
  if (elems_bytes > 0) {
    const Range o = span(out, elems_bytes);
    if (overlaps(o, span(u, elems_bytes)) || overlaps(o, span(delta, elems_bytes)) ||
        (z && overlaps(o, span(z, elems_bytes))) || overlaps(o, span(B, bc_bytes)) ||
        overlaps(o, span(C, bc_bytes)) || overlaps(o, span(A, a_elems * 4)) ||
        (D && overlaps(o, span(D, dim * 4))) ||
        (delta_bias && overlaps(o, span(delta_bias, dim * 4))) ||
        (final_state && overlaps(o, span(final_state, state_bytes))) ||
        (ckpt_bytes > 0 && overlaps(o, span(ckpt, ckpt_bytes))) ||
        (mask && overlaps(o, span(mask, batch * seqlen))))
      return SSM_ERR_INVALID_ARG;
  }

  if (rows == 0) return SSM_OK;
  if (seqlen == 0) {
    // An empty scan leaves the state where it started.
    if (final_state && !initial_state)
      return ssm::launch_fill_zero(final_state, state, stream) == 0 ? SSM_OK : SSM_ERR_HIP;
    return SSM_OK;
  }

  ssm::FwdArgs a;
  a.u = u;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.z = z;
  a.bias = delta_bias;
  a.out = out;
  a.final_state = final_state;
  a.batch = batch;
  a.dim = dim;
  a.dstate = dstate;
  a.seqlen = seqlen;
  a.io = (io == SSM_IO_BF16) ? ssm::Io::BF16 : ssm::Io::F32;
  a.softplus = (flags & SSM_DELTA_SOFTPLUS) != 0;
  a.initial_state = initial_state;
  a.vec_ok = ((seqlen * esz) % 16 == 0) && aligned(u, 16) && aligned(delta, 16) &&
             aligned(B, 16) && aligned(C, 16) && aligned(out, 16) && (!z || aligned(z, 16));
  a.ckpt = want_ckpt ? ckpt : nullptr;
  a.mask = mask;
  a.waves_per_channel = (flags & SSM_WAVES_PER_CHANNEL_1) ? 1
                        : (flags & SSM_WAVES_PER_CHANNEL_2) ? 2 : 0;
  return ssm::launch_scan_fwd(a, stream) == 0 ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* z, const float* delta_bias,
                 uint32_t flags, void* out, float* final_state, int64_t batch, int64_t dim,
                 int64_t dstate, int64_t seqlen, void* stream) {
  return fwd_impl(u, delta, A, B, C, D, z, delta_bias, nullptr, flags, out, final_state,
                  nullptr, false, batch, dim, dstate, seqlen, stream);
}

int ssm_scan_fwd_masked(const void* u, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* delta_bias,
                        const uint8_t* mask, uint32_t flags, void* out, float* final_state,
                        float* chunk_states, int64_t batch, int64_t dim, int64_t dstate,
                        int64_t seqlen, void* stream) {
  return fwd_impl(u, delta, A, B, C, D, z, delta_bias, mask, flags, out, final_state,
                  chunk_states, chunk_states != nullptr, batch, dim, dstate, seqlen, stream);
}

int ssm_scan_fwd_ckpt(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias,
                      uint32_t flags, void* out, float* final_state, float* chunk_states,
                      int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                      void* stream) {
  return fwd_impl(u, delta, A, B, C, D, z, delta_bias, nullptr, flags, out, final_state,
                  chunk_states, true, batch, dim, dstate, seqlen, stream);
}

int64_t ssm_scan_ckpt_count(int64_t seqlen) { return ckpt_count(seqlen); }

namespace {

// Bytes of a backward workspace laid out for `segments` segments (-1 on overflow).
int64_t bwd_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm::Io io,
                  int64_t segments) {
  ssm::BwdWorkspace w;
  if (!ssm::bwd_workspace(batch, dim, dstate, seqlen, io, segments, &w)) return -1;
  return w.floats * 4;
}

// The segments a backward on the current device would cut each sequence into.
int64_t bwd_segments_here(int64_t batch, int64_t dim, int64_t seqlen, ssm::Io io,
                          uint32_t flags) {
  if (flags & SSM_BWD_UNSPLIT) return 1;
  return ssm::bwd_segments(batch, dim, seqlen, io, ssm::device_cus());
}

}  // namespace

int64_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                     uint32_t flags) {
  if (batch < 0 || dim < 0 || dstate < 0 || seqlen < 0) return -1;
  const uint32_t io = flags & SSM_IO_MASK;
  if (io != SSM_IO_F32 && io != SSM_IO_BF16) return -1;
  const ssm::Io t = io == SSM_IO_BF16 ? ssm::Io::BF16 : ssm::Io::F32;
  return bwd_bytes(batch, dim, dstate, seqlen, t, bwd_segments_here(batch, dim, seqlen, t, flags));
}

int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* z, const float* delta_bias,
                 const uint8_t* mask, uint32_t flags, const float* chunk_states, const void* dout,
                 const float* dfinal, void* du, void* ddelta, float* dA, float* dB, float* dC,
                 float* dD, void* dz, float* dbias, float* dh0, void* workspace,
                 int64_t workspace_bytes, int64_t batch, int64_t dim, int64_t dstate,
                 int64_t seqlen, void* stream) {
  const uint32_t known = SSM_IO_MASK | SSM_DELTA_SOFTPLUS | SSM_INITIAL_STATE | SSM_BWD_UNSPLIT;
  if (flags & ~known) return SSM_ERR_INVALID_ARG;
  if (batch < 0 || dim < 0 || dstate < 0 || seqlen < 0) return SSM_ERR_INVALID_ARG;
  const uint32_t io = flags & SSM_IO_MASK;
  if (io != SSM_IO_F32 && io != SSM_IO_BF16) return SSM_ERR_UNSUPPORTED;
  if (dstate < 1 || dstate > 64) return SSM_ERR_UNSUPPORTED;
  const int64_t esz = (io == SSM_IO_BF16) ? 2 : 4;

  int64_t rows, elems, bc, state, a_elems, ck;
  if (!mul_ok(batch, dim, &rows) || !mul_ok(rows, seqlen, &elems) || !mul_ok(elems, esz, &ck) ||
      !mul_ok(batch, dstate, &bc) || !mul_ok(bc, seqlen, &bc) || !mul_ok(bc, 4, &ck) ||
      !mul_ok(rows, dstate, &state) || !mul_ok(state, 4, &ck) || !mul_ok(dim, dstate, &a_elems) ||
      !mul_ok(state, ckpt_count(seqlen), &ck) || !mul_ok(ck, 4, &ck))
    return SSM_ERR_UNSUPPORTED;
  if (rows > kInt32Max || seqlen > kInt32Max || dim > kInt32Max || rows / 64 + 1 > kInt32Max)
    return SSM_ERR_UNSUPPORTED;
  // A wave addresses its two channels' rows as one buffer with 32-bit byte offsets.
  if (2 * seqlen * esz > (int64_t(1) << 31) || dstate * seqlen * esz > (int64_t(1) << 31))
    return SSM_ERR_UNSUPPORTED;

  // required arrays (NULL only when empty)
  if (elems > 0 && (!u || !delta || !dout || !du || !ddelta)) return SSM_ERR_INVALID_ARG;
  if (bc > 0 && (!B || !C || !dB || !dC)) return SSM_ERR_INVALID_ARG;
  if (a_elems > 0 && (!A || !dA)) return SSM_ERR_INVALID_ARG;
  if (elems > 0 && !chunk_states) return SSM_ERR_INVALID_ARG;
  if (z && elems > 0 && !dz) return SSM_ERR_INVALID_ARG;

  const uintptr_t ea = static_cast<uintptr_t>(esz);
  if (!aligned(u, ea) || !aligned(delta, ea) || !aligned(B, ea) || !aligned(C, ea) ||
      !aligned(dout, ea) || !aligned(du, ea) || !aligned(ddelta, ea) || (z && !aligned(z, ea)) ||
      (dz && !aligned(dz, ea)) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
      (delta_bias && !aligned(delta_bias, 4)) || !aligned(chunk_states, 4) ||
      (dfinal && !aligned(dfinal, 4)) || !aligned(dA, 4) || !aligned(dB, 4) ||
      !aligned(dC, 4) || (dD && !aligned(dD, 4)) || (dbias && !aligned(dbias, 4)) ||
      (dh0 && !aligned(dh0, 4)) || (workspace && !aligned(workspace, 256)))
    return SSM_ERR_MISALIGNED;
  // With a workspace: as many segments as this device's rule asks for and the workspace
  // holds (a workspace of the unsegmented size always works: one segment).
  const ssm::Io iot = io == SSM_IO_BF16 ? ssm::Io::BF16 : ssm::Io::F32;
  int64_t segments = 1;
  if (workspace) {
    if (bwd_bytes(batch, dim, dstate, seqlen, iot, 1) < 0) return SSM_ERR_UNSUPPORTED;
    for (int64_t s = bwd_segments_here(batch, dim, seqlen, iot, flags); s > 1; --s) {
      const int64_t b = bwd_bytes(batch, dim, dstate, seqlen, iot, s);
      if (b >= 0 && b <= workspace_bytes) {
        segments = s;
        break;
      }
    }
    // the segment count takes whole intervals per segment, none empty
    const int64_t n = ssm::bwd_intervals(seqlen), per = (n + segments - 1) / segments;
    segments = per > 0 ? (n + per - 1) / per : 1;
    const int64_t need = bwd_bytes(batch, dim, dstate, seqlen, iot, segments);
    if (need < 0) return SSM_ERR_UNSUPPORTED;
    if (workspace_bytes < need) return SSM_ERR_INVALID_ARG;
    // The partial sums are written while the inputs are read and read while the summed
    // gradients are written: the workspace must overlap no other array.
    const int64_t eb = elems * esz, bcb = bc * 4, sb = state * 4, ab = a_elems * 4;
    const Range w = span(workspace, need);
    // an array that is absent or empty occupies nothing
    auto sp = [](const void* p, int64_t n) { return (p && n > 0) ? span(p, n) : Range{0, 0}; };
    const Range others[] = {
        sp(u, eb), sp(delta, eb), sp(dout, eb), sp(du, eb), sp(ddelta, eb),
        sp(z, z ? eb : 0), sp(dz, z ? eb : 0), sp(B, bc * esz),
        sp(C, bc * esz), sp(dB, bcb), sp(dC, bcb), sp(A, ab), sp(dA, ab),
        sp(D, D ? dim * 4 : 0), sp(dD, (D && dD) ? dim * 4 : 0),
        sp(delta_bias, delta_bias ? dim * 4 : 0),
        sp(dbias, (delta_bias && dbias) ? dim * 4 : 0), sp(dfinal, dfinal ? sb : 0),
        sp(dh0, dh0 ? sb : 0), sp(mask, mask ? batch * seqlen : 0),
        sp(chunk_states, sb * ssm_scan_ckpt_count(seqlen))};
    for (const Range& r : others)
      if (overlaps(w, r)) return SSM_ERR_INVALID_ARG;
  }

  if (rows == 0 && bc == 0 && a_elems == 0) return SSM_OK;
  if (seqlen == 0) {
    // Nothing to differentiate through: the state gradient passes straight back.
    int st = 0;
    if (a_elems > 0) st = ssm::launch_fill_zero(dA, a_elems, stream);
    if (st == 0 && D && dD && dim > 0) st = ssm::launch_fill_zero(dD, dim, stream);
    if (st == 0 && delta_bias && dbias && dim > 0) st = ssm::launch_fill_zero(dbias, dim, stream);
    if (st == 0 && dh0 && state > 0) {
      if (dfinal)
        st = int(hipMemcpyAsync(dh0, dfinal, size_t(state) * 4, hipMemcpyDeviceToDevice,
                                static_cast<hipStream_t>(stream)));
      else
        st = ssm::launch_fill_zero(dh0, state, stream);
    }
    return st == 0 ? SSM_OK : SSM_ERR_HIP;
  }
  if (rows == 0) {  // no channel: every summed gradient is zero
    int st = 0;
    if (bc > 0) st = ssm::launch_fill_zero(dB, bc, stream);
    if (st == 0 && bc > 0) st = ssm::launch_fill_zero(dC, bc, stream);
    if (st == 0 && a_elems > 0) st = ssm::launch_fill_zero(dA, a_elems, stream);
    return st == 0 ? SSM_OK : SSM_ERR_HIP;
  }

  ssm::BwdArgs a;
  a.u = u;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.z = z;
  a.bias = delta_bias;
  a.ckpt = chunk_states;
  a.dout = dout;
  a.dfinal = dfinal;
  a.du = du;
  a.ddelta = ddelta;
  a.dA = dA;
  a.dB = dB;
  a.dC = dC;
  a.dD = D ? dD : nullptr;
  a.dz = dz;
  a.dbias = delta_bias ? dbias : nullptr;
  a.dh0 = dh0;
  a.mask = mask;
  a.workspace = static_cast<float*>(workspace);
  a.segments = workspace ? segments : 1;
  a.batch = batch;
  a.dim = dim;
  a.dstate = dstate;
  a.seqlen = seqlen;
  a.io = (io == SSM_IO_BF16) ? ssm::Io::BF16 : ssm::Io::F32;
  a.softplus = (flags & SSM_DELTA_SOFTPLUS) != 0;
  a.vec_ok = ((seqlen * esz) % 16 == 0) && aligned(u, 16) && aligned(delta, 16) &&
             aligned(dout, 16) && aligned(du, 16) && aligned(ddelta, 16) && aligned(B, 16) &&
             aligned(C, 16) && (!z || (aligned(z, 16) && aligned(dz, 16)));
  return ssm::launch_scan_bwd(a, stream) == 0 ? SSM_OK : SSM_ERR_HIP;
}

int ssm_scan_debug_wave_combine(const float* a, const float* b, float* a_out, float* b_out,
                                int64_t groups, void* stream) {
  if (!a || !b || !a_out || !b_out || groups < 0) return SSM_ERR_INVALID_ARG;
  if (groups > kInt32Max) return SSM_ERR_UNSUPPORTED;
  if (!aligned(a, 4) || !aligned(b, 4) || !aligned(a_out, 4) || !aligned(b_out, 4))
    return SSM_ERR_MISALIGNED;
  if (groups == 0) return SSM_OK;
  return ssm::launch_debug_wave_combine(a, b, a_out, b_out, groups, stream) == 0 ? SSM_OK
                                                                                  : SSM_ERR_HIP;
}

}  // extern "C"
