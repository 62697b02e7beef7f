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
// Mapping: one lane per (channel, four consecutive states), or per (channel, state) when
// dstate is not a multiple of four or a state pointer is not 16-byte aligned. A channel's
// lanes are consecutive and a power of two in number, so a channel never straddles two
// wavefronts; lanes past dstate carry zeros. Each lane walks t = 0..L-1 sequentially with
// its states in registers (the recurrence itself, no scan), and y_t is the sum over the
// channel's lanes of C h (butterfly). The state is read once (initial state) and written
// once (final state), both coalesced over n.
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

// S consecutive states per lane (S = 1 or 4). With S = 4 the state, A and the saved state
// move as one 16-byte access per lane, so a decode step needs a quarter of the waves and
// every wave has four times the bytes in flight.
template <int S>
struct Quad {
  float v[S];
};

template <int S>
__device__ __forceinline__ Quad<S> load_states(const float* base, int64_t i) {
  Quad<S> q;
  if constexpr (S == 4) {
    const float4 w = *reinterpret_cast<const float4*>(base + i);
    q.v[0] = w.x; q.v[1] = w.y; q.v[2] = w.z; q.v[3] = w.w;
  } else {
    q.v[0] = base[i];
  }
  return q;
}

template <int S>
__device__ __forceinline__ void store_states(float* base, int64_t i, const Quad<S>& q) {
  if constexpr (S == 4) {
    *reinterpret_cast<float4*>(base + i) = make_float4(q.v[0], q.v[1], q.v[2], q.v[3]);
  } else {
    base[i] = q.v[0];
  }
}

// Lanes per channel: ceil(dstate / S) rounded up to a power of two (2^lanes_log2 <= 64),
// so a channel never straddles two wavefronts. Lane j of a channel holds states
// S*j .. S*j+S-1; with S = 4 the launcher only picks this form when dstate % 4 == 0.
template <typename Elem, int S>
__global__ __launch_bounds__(kThreads) void scan_short_kernel(ShortParams p) {
  const int lanes = 1 << p.n2_log2;
  const int64_t gid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t row = gid >> p.n2_log2;  // b * dim + d
  const int j = int(gid & (lanes - 1));
  const int n0 = j * S;
  const bool row_ok = row < p.rows;
  const bool lane_ok = row_ok && n0 < p.dstate;
  const int N = p.dstate, L = p.seqlen;
  const int64_t rr = row_ok ? row : 0;
  const int d = int(rr % p.dim);
  const int64_t b = rr / p.dim;
  const int64_t si = rr * N + (lane_ok ? n0 : 0);  // final_state / ckpt [b, d, n0]

  Quad<S> a2, h;
  if (lane_ok) {
    a2 = load_states<S>(p.A, int64_t(d) * N + n0);
    for (int k = 0; k < S; ++k) a2.v[k] *= kLog2e;
  } else {
    for (int k = 0; k < S; ++k) a2.v[k] = 0.0f;
  }
  if (lane_ok && p.initial_state) {
    h = load_states<S>(p.final_state, si);
  } else {
    for (int k = 0; k < S; ++k) h.v[k] = 0.0f;
  }
  const float Dd = (row_ok && p.D) ? p.D[d] : 0.0f;
  const float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
  if (lane_ok && p.ckpt) store_states<S>(p.ckpt, si, h);  // seqlen <= 32: one saved state
  const int64_t bc0 = (b * N + (lane_ok ? n0 : 0)) * L;  // B[b, n0, 0], C[b, n0, 0]
  const int64_t x0 = rr * L;                            // u, delta, z, out [b, d, 0]

  for (int t = 0; t < L; ++t) {
    // Every load of the step is issued before any arithmetic, the gate's z included.
    float u = 0.0f, x = 0.0f, zv = 0.0f, bv[S], cv[S];
    if (row_ok) {
      u = load_elem<Elem>(p.u, x0 + t);
      x = load_elem<Elem>(p.delta, x0 + t) + bias;
      if (p.z) zv = load_elem<Elem>(p.z, x0 + t);
    }
    for (int k = 0; k < S; ++k) {
      bv[k] = lane_ok ? load_elem<Elem>(p.B, bc0 + int64_t(k) * L + t) : 0.0f;
      cv[k] = lane_ok ? load_elem<Elem>(p.C, bc0 + int64_t(k) * L + t) : 0.0f;
    }
    float dt = p.softplus ? softplus_f(x) : x;
    if (p.mask && p.mask[b * L + t] == 0) dt = 0.0f;  // padding: the state is kept
    const float du = dt * u;
    float y = 0.0f;
    for (int k = 0; k < S; ++k) {
      h.v[k] = __builtin_fmaf(exp2_hw(dt * a2.v[k]), h.v[k], du * bv[k]);
      y = __builtin_fmaf(cv[k], h.v[k], y);
    }
    for (int m = lanes >> 1; m > 0; m >>= 1) y += __shfl_xor(y, m, 64);
    y = __builtin_fmaf(Dd, u, y);
    if (row_ok && j == 0) {
      if (p.z) y = gate_f(y, zv);
      store_elem<Elem>(p.out, x0 + t, y);
    }
  }
  if (lane_ok && p.final_state) store_states<S>(p.final_state, si, h);
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
  // Four states per lane when the state rows split into aligned 16-byte quads.
  const bool quad = a.dstate % 4 == 0 && reinterpret_cast<uintptr_t>(a.A) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(a.final_state) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(a.ckpt) % 16 == 0;
  const int64_t per_lane = quad ? 4 : 1;
  int lg = 0;
  while ((int64_t(1) << lg) * per_lane < a.dstate) ++lg;  // dstate <= 64, so lg <= 6
  p.n2_log2 = lg;
  p.softplus = a.softplus ? 1 : 0;
  p.initial_state = a.initial_state ? 1 : 0;
  const int64_t lanes = p.rows << lg;
  const int64_t blocks = (lanes + kThreads - 1) / kThreads;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid{unsigned(blocks)}, block{unsigned(kThreads)};
  if (a.io == Io::BF16) {
    if (quad)
      hipLaunchKernelGGL((scan_short_kernel<uint16_t, 4>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((scan_short_kernel<uint16_t, 1>), grid, block, 0, s, p);
  } else {
    if (quad)
      hipLaunchKernelGGL((scan_short_kernel<float, 4>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((scan_short_kernel<float, 1>), grid, block, 0, s, p);
  }
  return int(hipGetLastError());
}

}  // namespace ssm
