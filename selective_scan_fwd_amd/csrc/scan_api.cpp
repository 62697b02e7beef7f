// C-ABI entry points of libssmscan.so (declared in include/ssm_scan.h).
// Argument checking happens here, before any HIP call; the launches are in
// scan_kernels.hip.
#include <stdint.h>
#include <string.h>

#include "scan_launch.h"
#include "ssm_scan.h"

namespace {

constexpr int64_t kInt32Max = 2147483647;

// a * b with overflow detection for non-negative operands.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range x, Range y) { return x.lo < y.hi && y.lo < x.hi; }

Range span(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

int ssm_scan_abi_version(void) { return 1; }

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
    default:
      return "unknown status";
  }
}

int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* z, const float* delta_bias,
                 uint32_t flags, void* out, float* final_state, int64_t batch, int64_t dim,
                 int64_t dstate, int64_t seqlen, void* stream) {
  const uint32_t known = SSM_IO_MASK | SSM_DELTA_SOFTPLUS | SSM_INITIAL_STATE;
  if (flags & ~known) return SSM_ERR_INVALID_ARG;
  if (batch < 0 || dim < 0 || dstate < 0 || seqlen < 0) return SSM_ERR_INVALID_ARG;
  const bool initial_state = (flags & SSM_INITIAL_STATE) != 0;

  const uint32_t io = flags & SSM_IO_MASK;
  if (io != SSM_IO_F32 && io != SSM_IO_BF16) return SSM_ERR_UNSUPPORTED;
  if (dstate < 1 || dstate > 64) return SSM_ERR_UNSUPPORTED;
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
        (final_state && overlaps(o, span(final_state, state_bytes))))
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
  return ssm::launch_scan_fwd(a, stream) == 0 ? SSM_OK : SSM_ERR_HIP;
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
