// Device arithmetic shared by the forward kernels: hardware exp2/log2/rcp, softplus, the
// silu gate and bf16 conversion. fp32 throughout.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = max(x, 0) + log1p(e), e = exp(-|x|) in (0, 1]. With w = fl(1 + e), the
// rounding error d = (w - 1) - e is exact (w - 1 is exact for w in [1, 2], and the error of
// a rounded sum is representable), and log1p(e) = log(w) - d / w + O(d^2); replacing d / w
// by d changes the result by d * e / (1 + e), below 1e-7 relative since log1p(e) >= e ln 2.
// When w rounds to 1, the result is e exactly. Two transcendentals (exp2, log2).
// max(x, 0) is one v_max_f32: written as fmaxf, the compiler first canonicalises x, one
// more instruction per call. x is the result of an add here, never a signalling NaN; at
// x = -inf the result is 0 + log1p(0) = 0, and a NaN x propagates through e.
__device__ __forceinline__ float max0_f(float x) {
  float r;
  asm("v_max_f32 %0, 0, %1" : "=v"(r) : "v"(x));
  return r;
}

__device__ __forceinline__ float softplus_f(float x) {
  const float e = exp2_hw(-__builtin_fabsf(x) * kLog2e);
  const float w = 1.0f + e;
  const float err = (w - 1.0f) - e;
  return max0_f(x) + __builtin_fmaf(log2_hw(w), kLn2, -err);
}

// y * silu(z) = y * z / (1 + e^-z)
__device__ __forceinline__ float gate_f(float y, float z) {
  return y * z * rcp_hw(1.0f + exp2_hw(-z * kLog2e));
}

// ---------------------------------------------------------------- storage types

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to bf16, nearest-even, two values per dword. Converted as one two-element vector,
// this is a single v_cvt_pk_bf16_f32 on gfx950; two scalar conversions would cost two of
// them plus a shift and an or to merge the halves.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

}  // namespace ssm
