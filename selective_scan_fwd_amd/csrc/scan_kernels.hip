// Selective-scan forward for gfx950 (CDNA4, wave64).
//
// What is computed (per batch row b, channel d, state n; see include/ssm_scan.h):
//   dA_t = exp(dt_t * A[d,n]), dBu_t = dt_t * B[b,n,t] * u_t, h_t = dA_t h_{t-1} + dBu_t,
//   y_t = sum_n C[b,n,t] h_t[n] + D[d] u_t, out = y_t * silu(z_t)
// (ybb.press, "Mamba state-space model: from theory to production CUDA kernel
// optimisation", sections 1.2, 2.3, 7.1; jsqmd.com, "Blelloch parallel scan as the engine
// of Mamba.py", section 3.2).
//
// How (one fused kernel, every streamed byte read once and written once, h never leaves
// the chip -- the fusion argument of mhpq.cn/news/1077344 section 3.2):
//   * one 64-lane wavefront owns one (b, d) row; waves are independent (no LDS, no
//     barriers); a workgroup packs K rows of the same batch so they share B and C in L1;
//   * the time axis is cut into chunks of 64*T steps; lane i owns the T consecutive steps
//     [t0 + i*T, t0 + i*T + T) of the chunk (the lane-holds-consecutive-steps mapping of
//     mhpq.cn/news/1057127 section 1);
//   * per state n (diagonal A: the N chains are independent, same page section 1):
//       1. discretise the lane's T steps (exp2 with A pre-scaled by log2 e);
//       2. fold them sequentially into the lane's segment operator (a, b), where
//          a = prod dA = exp(A * sum dt) and b is the segment's state from a zero start
//          (lane 0 starts from the chunk's carry-in instead);
//       3. inclusive wave64 Hillis-Steele scan of (a, b) under the combine
//          (a1,b1) o (a2,b2) = (a2 a1, a2 b1 + b2) (ybb.press section 3.2; mhpq.cn/news/
//          1077344 sections 2.2-2.3) over DPP: row_shr 1,2,4,8 then row_bcast 15/31;
//       4. lane i's carry-in is lane i-1's inclusive result (DPP wave_shr:1), lane 63's
//          result is the carry into the next chunk (chunked scan with a serial carry,
//          mhpq.cn/news/1077344 section 2.4; mhpq.cn/news/1057127 section 3);
//       5. replay the T steps from the carry-in, accumulating y += C h.
//   * after the n loop: D skip, silu gate, rounding to the storage type, store.
// No MFMA: nothing here is a dense contraction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_launch.h"

namespace ssm {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float readlane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// softplus(x) = log(1 + e^x); above 20 it returns x (the omitted log1p(e^-x) is < 2.1e-9
// relative). log1p(e) is taken as log(w) * e / (w - 1) with w = 1 + e, which cancels the
// rounding of 1 + e (Goldberg, "What every computer scientist should know about
// floating-point arithmetic", 1991, theorem 4); when w rounds to 1, log1p(e) = e.
__device__ __forceinline__ float softplus_f(float x) {
  const float e = exp2_hw(x * kLog2e);
  const float w = 1.0f + e;
  const float r = (w == 1.0f) ? e : (log2_hw(w) * kLn2) * e * rcp_hw(w - 1.0f);
  return (x > 20.0f) ? x : r;
}

// y * silu(z) = y * z / (1 + e^-z)
__device__ __forceinline__ float gate_f(float y, float z) {
  return y * z * rcp_hw(1.0f + exp2_hw(-z * kLog2e));
}

// ---------------------------------------------------------------- storage types

template <typename IoT>
struct Stream;

template <>
struct Stream<float> {
  using Elem = float;
  static constexpr int kVec = 4;  // elements per 16-byte access
  __device__ static float widen(float v) { return v; }
};

template <>
struct Stream<uint16_t> {  // bf16 bit patterns
  using Elem = uint16_t;
  static constexpr int kVec = 8;
  __device__ static float widen(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }
};

// Load the T values row[tb .. tb+T) as fp32, zero past `len`. `vec` says that row starts
// 16-byte aligned; T is a multiple of the vector width, so a whole in-range block is a
// run of aligned 16-byte loads.
template <int T>
__device__ __forceinline__ void load_block(const float* row, int tb, int len, bool vec,
                                           float (&v)[T]) {
  if (vec && tb + T <= len) {
    const float4* p = reinterpret_cast<const float4*>(row + tb);
#pragma unroll
    for (int q = 0; q < T / 4; ++q) {
      const float4 x = p[q];
      v[4 * q + 0] = x.x;
      v[4 * q + 1] = x.y;
      v[4 * q + 2] = x.z;
      v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < T; ++j) v[j] = (tb + j < len) ? row[tb + j] : 0.0f;
  }
}

template <int T>
__device__ __forceinline__ void load_block(const uint16_t* row, int tb, int len, bool vec,
                                           float (&v)[T]) {
  if (vec && tb + T <= len) {
    const uint4* p = reinterpret_cast<const uint4*>(row + tb);
#pragma unroll
    for (int q = 0; q < T / 8; ++q) {
      const uint4 w = p[q];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * q + 2 * k + 0] = __uint_as_float(ws[k] << 16);
        v[8 * q + 2 * k + 1] = __uint_as_float(ws[k] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < T; ++j)
      v[j] = (tb + j < len) ? __uint_as_float(uint32_t(row[tb + j]) << 16) : 0.0f;
  }
}

template <int T>
__device__ __forceinline__ void store_block(float* row, int tb, int len, bool vec,
                                            const float (&v)[T]) {
  if (vec && tb + T <= len) {
    float4* p = reinterpret_cast<float4*>(row + tb);
#pragma unroll
    for (int q = 0; q < T / 4; ++q)
      p[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  } else {
#pragma unroll
    for (int j = 0; j < T; ++j)
      if (tb + j < len) row[tb + j] = v[j];
  }
}

// Round to bf16, nearest-even (v_cvt_pk_bf16_f32 on gfx950), two values per dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 l = (__bf16)lo, h = (__bf16)hi;
  return uint32_t(__builtin_bit_cast(uint16_t, l)) |
         (uint32_t(__builtin_bit_cast(uint16_t, h)) << 16);
}

template <int T>
__device__ __forceinline__ void store_block(uint16_t* row, int tb, int len, bool vec,
                                            const float (&v)[T]) {
  if (vec && tb + T <= len) {
    uint4* p = reinterpret_cast<uint4*>(row + tb);
#pragma unroll
    for (int q = 0; q < T / 8; ++q)
      p[q] = make_uint4(pack_bf16x2(v[8 * q + 0], v[8 * q + 1]),
                        pack_bf16x2(v[8 * q + 2], v[8 * q + 3]),
                        pack_bf16x2(v[8 * q + 4], v[8 * q + 5]),
                        pack_bf16x2(v[8 * q + 6], v[8 * q + 7]));
  } else {
#pragma unroll
    for (int j = 0; j < T; ++j)
      if (tb + j < len) row[tb + j] = __builtin_bit_cast(uint16_t, (__bf16)v[j]);
  }
}

// ---------------------------------------------------------------- wave64 combine scan

// One Hillis-Steele step: lane i combines the operator of the lane CTRL names (earlier in
// time) on its left. Lanes whose source is out of range, or whose row ROW_MASK disables,
// keep their value: update_dpp returns `old`, the identity (1, 0), for them.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void combine_step(float& a, float& b) {
  const float aj = __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(1.0f), __float_as_int(a), CTRL, ROW_MASK, 0xf, false));
  const float bj = __int_as_float(__builtin_amdgcn_update_dpp(
      0, __float_as_int(b), CTRL, ROW_MASK, 0xf, false));
  b = __builtin_fmaf(a, bj, b);  // a_i * b_j + b_i   (uses a_i before it is updated)
  a = a * aj;                    // a_i * a_j
}

// Inclusive scan across the 64 lanes of a wavefront, lane 0 earliest.
// DPP controls: 0x111/0x112/0x114/0x118 = row_shr:1/2/4/8 (inside 16-lane rows);
// 0x142 = row_bcast:15 (lane 15 of a row to the next row; written to rows 1 and 3);
// 0x143 = row_bcast:31 (lane 31 to rows 2 and 3).
__device__ __forceinline__ void wave_scan_inclusive(float& a, float& b) {
  combine_step<0x111, 0xf>(a, b);
  combine_step<0x112, 0xf>(a, b);
  combine_step<0x114, 0xf>(a, b);
  combine_step<0x118, 0xf>(a, b);
  combine_step<0x142, 0xa>(a, b);
  combine_step<0x143, 0xc>(a, b);
}

// Lane i receives lane i-1's value; lane 0 receives `first` (DPP wave_shr:1).
__device__ __forceinline__ float shift_up_one(float v, float first) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(first), __float_as_int(v),
                                                    0x138, 0xf, 0xf, false));
}

// ---------------------------------------------------------------- forward kernel

struct KParams {
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
  int64_t rows;  // batch * dim
  int dim, dstate, seqlen;
  int softplus, initial_state, vec_ok;
};

template <typename Elem, int T, int K>
__global__ __launch_bounds__(64 * K) void scan_fwd_kernel(KParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = int64_t(blockIdx.x) * K + wave;
  if (row >= p.rows) return;  // whole wavefront leaves together
  const int N = p.dstate, L = p.seqlen;
  const int b = int(row / p.dim);
  const int d = int(row - int64_t(b) * p.dim);
  const bool vec = p.vec_ok != 0;

  const Elem* u_r = static_cast<const Elem*>(p.u) + row * L;
  const Elem* dl_r = static_cast<const Elem*>(p.delta) + row * L;
  const Elem* z_r = p.z ? static_cast<const Elem*>(p.z) + row * L : nullptr;
  Elem* out_r = static_cast<Elem*>(p.out) + row * L;
  const Elem* B_b = static_cast<const Elem*>(p.B) + int64_t(b) * N * L;
  const Elem* C_b = static_cast<const Elem*>(p.C) + int64_t(b) * N * L;

  const float Dd = p.D ? p.D[d] : 0.0f;
  const float bias_d = p.bias ? p.bias[d] : 0.0f;

  // Per-state values live one per lane: lane n holds A[d,n]*log2(e) and the carry h[n].
  float a2_lane = 0.0f, hc_lane = 0.0f;
  if (lane < N) {
    a2_lane = p.A[int64_t(d) * N + lane] * kLog2e;
    if (p.initial_state) hc_lane = p.final_state[row * N + lane];
  }

  for (int t0 = 0; t0 < L; t0 += 64 * T) {
    const int tb = t0 + lane * T;
    float dt[T], du[T], y[T];
    float sdt = 0.0f;
    {
      float uv[T], dr[T];
      load_block<T>(u_r, tb, L, vec, uv);
      load_block<T>(dl_r, tb, L, vec, dr);
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const float x = dr[j] + bias_d;
        const float s = p.softplus ? softplus_f(x) : x;
        dt[j] = (tb + j < L) ? s : 0.0f;  // steps past L: identity (dA = 1, dBu = 0)
        du[j] = dt[j] * uv[j];
        y[j] = Dd * uv[j];
        sdt += dt[j];
      }
    }

    for (int n = 0; n < N; ++n) {
      const float a2 = readlane(a2_lane, n);
      const float hc = readlane(hc_lane, n);
      float Bv[T], Cv[T], dA[T], dBu[T];
      load_block<T>(B_b + int64_t(n) * L, tb, L, vec, Bv);
      load_block<T>(C_b + int64_t(n) * L, tb, L, vec, Cv);

      float bseg = (lane == 0) ? hc : 0.0f;
#pragma unroll
      for (int j = 0; j < T; ++j) {
        dA[j] = exp2_hw(dt[j] * a2);
        dBu[j] = du[j] * Bv[j];
        bseg = __builtin_fmaf(dA[j], bseg, dBu[j]);
      }
      float aseg = exp2_hw(sdt * a2);

      wave_scan_inclusive(aseg, bseg);         // bseg: state at the end of this lane's steps
      const float carry_out = readlane(bseg, 63);
      float h = shift_up_one(bseg, hc);        // state entering this lane's steps
      hc_lane = (lane == n) ? carry_out : hc_lane;

#pragma unroll
      for (int j = 0; j < T; ++j) {
        h = __builtin_fmaf(dA[j], h, dBu[j]);
        y[j] = __builtin_fmaf(Cv[j], h, y[j]);
      }
    }

    if (z_r) {
      float zv[T];
      load_block<T>(z_r, tb, L, vec, zv);
#pragma unroll
      for (int j = 0; j < T; ++j) y[j] = gate_f(y[j], zv[j]);
    }
    store_block<T>(out_r, tb, L, vec, y);
  }

  if (p.final_state && lane < N) p.final_state[row * N + lane] = hc_lane;
}

__global__ void fill_zero_kernel(float* p, int64_t count) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0.0f;
}

__global__ __launch_bounds__(64) void debug_wave_combine_kernel(const float* a, const float* b,
                                                                float* a_out, float* b_out) {
  const int64_t i = int64_t(blockIdx.x) * 64 + threadIdx.x;
  float av = a[i], bv = b[i];
  wave_scan_inclusive(av, bv);
  a_out[i] = av;
  b_out[i] = bv;
}

template <typename Elem, int T, int K>
int launch_typed(const FwdArgs& a, hipStream_t s) {
  KParams p;
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
  p.rows = a.batch * a.dim;
  p.dim = int(a.dim);
  p.dstate = int(a.dstate);
  p.seqlen = int(a.seqlen);
  p.softplus = a.softplus ? 1 : 0;
  p.initial_state = a.initial_state ? 1 : 0;
  p.vec_ok = a.vec_ok ? 1 : 0;
  const int64_t blocks = (p.rows + K - 1) / K;
  hipLaunchKernelGGL((scan_fwd_kernel<Elem, T, K>), dim3(unsigned(blocks)), dim3(64 * K), 0, s,
                     p);
  return int(hipGetLastError());
}

}  // namespace

int launch_scan_fwd(const FwdArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.io == Io::BF16) return launch_typed<uint16_t, 8, 4>(a, s);
  return launch_typed<float, 8, 4>(a, s);
}

int launch_fill_zero(float* p, int64_t count, void* stream) {
  const int64_t blocks = (count + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p, count);
  return int(hipGetLastError());
}

int launch_debug_wave_combine(const float* a, const float* b, float* a_out, float* b_out,
                              int64_t groups, void* stream) {
  hipLaunchKernelGGL(debug_wave_combine_kernel, dim3(unsigned(groups)), dim3(64), 0,
                     static_cast<hipStream_t>(stream), a, b, a_out, b_out);
  return int(hipGetLastError());
}

}  // namespace ssm
