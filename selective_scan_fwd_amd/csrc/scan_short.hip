// Selective-scan forward for short sequences (decode and state passing) on gfx950.
//
// Same operation as the chunked kernel (include/ssm_scan.h): per batch row b, channel d and
// state n, h_t = exp(dt_t A[d,n]) h_{t-1} + dt_t B[b,n,t] u_t, y_t = sum_n C[b,n,t] h_t + D u_t,
// out = y_t silu(z_t). Here it is laid out for a handful of steps, where the chunked
// kernel's 64*T-step chunks would leave almost every lane idle: the decode step that
// advances a cached state by one token, and short continuations of it (ybb.press, "Mamba
// state-space model: from theory to production CUDA kernel optimisation", section 5.1: the
// per-layer state cache replaces a growing KV cache; one decode step reads and rewrites it).
//
// Mapping: one lane per (channel, state). A channel's states occupy N2 consecutive lanes
// (N2 = dstate rounded up to a power of two, so a channel never straddles two wavefronts);
// lanes n >= dstate carry zeros. Each lane walks t = 0..L-1 sequentially with its own state
// in a register (the recurrence itself, no scan), and y_t is the sum over the channel's
// lanes of C h (butterfly over N2 lanes). The state is read once (initial state) and
// written once (final state), both coalesced over n.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "scan_launch.h"

namespace ssm {
namespace {

struct ShortParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  void* out;
  float* final_state;
  float* ckpt;   // nullable: [rows, 1, dstate], the state entering step 0
  const uint8_t* mask;  // nullable: [batch, seqlen], 0 = padding step (state kept)
  int64_t rows;  // batch * dim
  int dim, dstate, seqlen;
  int n2_log2;
  int softplus, initial_state;
};

template <typename Elem>
__device__ __forceinline__ float load_elem(const void* base, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const void* base, int64_t i) {
  return static_cast<const float*>(base)[i];
}
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const void* base, int64_t i) {
  return bf16_lo(static_cast<const uint16_t*>(base)[i]);
}

template <typename Elem>
__device__ __forceinline__ void store_elem(void* base, int64_t i, float v);
template <>
__device__ __forceinline__ void store_elem<float>(void* base, int64_t i, float v) {
  static_cast<float*>(base)[i] = v;
}
template <>
__device__ __forceinline__ void store_elem<uint16_t>(void* base, int64_t i, float v) {
  static_cast<uint16_t*>(base)[i] = uint16_t(pack_bf16x2(v, 0.0f));
}

constexpr int kThreads = 256;

template <typename Elem>
__global__ __launch_bounds__(kThreads) void scan_short_kernel(ShortParams p) {
  const int n2 = 1 << p.n2_log2;
  const int64_t gid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t row = gid >> p.n2_log2;  // b * dim + d
  const int n = int(gid & (n2 - 1));
  const bool row_ok = row < p.rows;
  const bool lane_ok = row_ok && n < p.dstate;
  const int N = p.dstate, L = p.seqlen;
  const int64_t rr = row_ok ? row : 0;
  const int d = int(rr % p.dim);
  const int64_t b = rr / p.dim;

  const float a2 = lane_ok ? p.A[int64_t(d) * N + n] * kLog2e : 0.0f;
  const float Dd = (row_ok && p.D) ? p.D[d] : 0.0f;
  const float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
  float h = (lane_ok && p.initial_state) ? p.final_state[rr * N + n] : 0.0f;
  if (lane_ok && p.ckpt) p.ckpt[rr * N + n] = h;  // seqlen <= 32: one saved state
  const int64_t bc0 = (b * N + (lane_ok ? n : 0)) * L;  // B[b, n, 0], C[b, n, 0]
  const int64_t x0 = rr * L;                           // u, delta, z, out [b, d, 0]

  for (int t = 0; t < L; ++t) {
    float u = 0.0f, x = 0.0f, bv = 0.0f, cv = 0.0f;
    if (row_ok) {
      u = load_elem<Elem>(p.u, x0 + t);
      x = load_elem<Elem>(p.delta, x0 + t) + bias;
    }
    if (lane_ok) {
      bv = load_elem<Elem>(p.B, bc0 + t);
      cv = load_elem<Elem>(p.C, bc0 + t);
    }
    float dt = p.softplus ? softplus_f(x) : x;
    if (p.mask && p.mask[b * L + t] == 0) dt = 0.0f;  // padding: the state is kept
    h = __builtin_fmaf(exp2_hw(dt * a2), h, (dt * u) * bv);
    float y = cv * h;
    for (int m = n2 >> 1; m > 0; m >>= 1) y += __shfl_xor(y, m, 64);
    y = __builtin_fmaf(Dd, u, y);
    if (row_ok && n == 0) {
      if (p.z) y = gate_f(y, load_elem<Elem>(p.z, x0 + t));
      store_elem<Elem>(p.out, x0 + t, y);
    }
  }
  if (lane_ok && p.final_state) p.final_state[rr * N + n] = h;
}

}  // namespace

int launch_scan_short(const FwdArgs& a, void* stream) {
  ShortParams p;
  p.u = a.u;
  p.delta = a.delta;
  p.A = a.A;
  p.B = a.B;
  p.C = a.C;
  p.D = a.D;
  p.z = a.z;
  p.bias = a.bias;
  p.out = a.out;
  p.final_state = a.final_state;
  p.ckpt = a.ckpt;
  p.mask = a.mask;
  p.rows = a.batch * a.dim;
  p.dim = int(a.dim);
  p.dstate = int(a.dstate);
  p.seqlen = int(a.seqlen);
  int lg = 0;
  while ((1 << lg) < a.dstate) ++lg;  // dstate <= 64, so lg <= 6
  p.n2_log2 = lg;
  p.softplus = a.softplus ? 1 : 0;
  p.initial_state = a.initial_state ? 1 : 0;
  const int64_t lanes = p.rows << lg;
  const int64_t blocks = (lanes + kThreads - 1) / kThreads;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.io == Io::BF16)
    hipLaunchKernelGGL(scan_short_kernel<uint16_t>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(scan_short_kernel<float>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, p);
  return int(hipGetLastError());
}

}  // namespace ssm
