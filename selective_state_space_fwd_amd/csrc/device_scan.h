// Device building blocks shared by the chunked forward and backward kernels: the wave64
// combine scan over DPP, lane shifts, raw buffer resources with hardware range checks, and
// 16-byte word loads and stores of the storage types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"

namespace ssm {

__device__ __forceinline__ float readlane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// v_writelane_b32: the LLVM intrinsic, which this compiler exposes under no builtin name;
// declared through its symbol so that the compiler sees it (and inserts its hazard waits).
__device__ int ssm_llvm_writelane(int value, int lane, int old) __asm("llvm.amdgcn.writelane");

// `old` with lane `lane` (uniform) replaced by the uniform value `v`.
__device__ __forceinline__ float writelane(float old, float v, int lane) {
  return __int_as_float(ssm_llvm_writelane(__float_as_int(v), lane, __float_as_int(old)));
}

// Elements per 16-byte access.
template <typename Elem>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int kN = 4;
};
template <>
struct Vec<uint16_t> {
  static constexpr int kN = 8;
};

template <typename Elem>
__device__ __forceinline__ void widen_raw16(uint4 w, float* v);
template <>
__device__ __forceinline__ void widen_raw16<float>(uint4 w, float* v) {
  v[0] = __uint_as_float(w.x);
  v[1] = __uint_as_float(w.y);
  v[2] = __uint_as_float(w.z);
  v[3] = __uint_as_float(w.w);
}
template <>
__device__ __forceinline__ void widen_raw16<uint16_t>(uint4 w, float* v) {
  v[0] = bf16_lo(w.x);
  v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y);
  v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z);
  v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w);
  v[7] = bf16_hi(w.w);
}

// ---------------------------------------------------------------- wave64 combine scan

// Inclusive scan of the operators (a, b) across the 64 lanes of a wavefront, lane 0
// earliest, under (a1,b1) o (a2,b2) = (a2 a1, a2 b1 + b2).
//
// Each Hillis-Steele step is two DPP instructions reading the operator of the lane the
// control names (earlier in time):
//   v_fmac_f32_dpp b, b, a   ->  b_i = b_j * a_i + b_i      (uses a_i before its update)
//   v_mul_f32_dpp  a, a, a   ->  a_i = a_j * a_i
// Without bound_ctrl, a lane whose source is outside its row, or whose row the row_mask
// excludes, is not written: it keeps its operator, i.e. combines with the identity (1, 0).
// Controls: row_shr:1/2/4/8 inside 16-lane rows; row_bcast:15 (lane 15 of a row into the
// next row; written to rows 1 and 3 by row_mask 0xa); row_bcast:31 (lane 31 into rows 2
// and 3, row_mask 0xc). The final a is not needed by the caller, so the last step updates
// b only.
//
// gfx950 needs two wait states between a VALU write of a VGPR and a DPP read of it: the
// block starts with s_nop 1 (its inputs were just written) and every step is followed by
// s_nop 0, so each DPP read is at least two instructions after the write it depends on.
__device__ __forceinline__ void wave_scan_inclusive(float& a, float& b) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(a), "+v"(b));
}

// Lane i receives lane i-1's value; lane 0 receives `first` (DPP wave_shr:1).
__device__ __forceinline__ float shift_up_one(float v, float first) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(first), __float_as_int(v),
                                                    0x138, 0xf, 0xf, false));
}

// ---------------------------------------------------------------- buffer access

// Raw buffer resources (base, byte length): an access at or past the length reads 0 and a
// store there is dropped by the hardware range check, so tails, inactive waves and the
// "next chunk" past the end of the sequence need no branches. Branch-free loads also let
// the compiler count outstanding loads exactly (vmcnt completes in order), which is what
// keeps a prefetch in flight across later waits.
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) dword access

struct Buf {
  __amdgpu_buffer_rsrc_t r;
  __device__ Buf(const void* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                            kRsrcWord3)) {}
  __device__ uint4 load16(uint32_t off) const {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
  // With a uniform part of the offset in a scalar register (soff). Callers keep an access
  // that must miss the buffer out of range through `off` alone.
  __device__ uint4 load16(uint32_t off, uint32_t soff) const {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
  }
  // Non-temporal (streaming) load, cache policy bit 1: for a last use, so that the line is
  // the first to leave L2 and data still to be read again stays.
  __device__ uint4 load16_nt(uint32_t off) const {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
  }
  __device__ uint32_t load4(uint32_t off, uint32_t soff) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
  }
  __device__ uint2 load8(uint32_t off) const {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  }
  __device__ uint32_t load4(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ uint32_t load2(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
  __device__ uint32_t load1(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
  }
  __device__ void store16(uint4 v, uint32_t off) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, 0);
  }
  // Non-temporal (streaming) store: cache policy bit 1 (nt), for data nothing reads again
  // soon, so that it does not push out of L2 data that will be.
  __device__ void store16_nt(uint4 v, uint32_t off) const {
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, 2);
  }
  __device__ void store8(uint2 v, uint32_t off) const {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v), r, off, 0, 0);
  }
  __device__ void store4(uint32_t v, uint32_t off) const {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
  }
  __device__ void store4(uint32_t v, uint32_t off, uint32_t soff) const {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, soff, 0);
  }
  __device__ void store2(uint16_t v, uint32_t off) const {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
  }
};

// One 16-byte word of storage elements starting at element e (byte offset e*sizeof). With
// kVecRows every such word is 16-byte aligned and lies wholly inside or outside the row;
// otherwise it is gathered element by element.
template <typename Elem, bool kVecRows>
__device__ __forceinline__ uint4 load_word(const Buf& b, uint32_t e) {
  if constexpr (kVecRows) {
    return b.load16(e * uint32_t(sizeof(Elem)));
  } else if constexpr (sizeof(Elem) == 4) {
    return make_uint4(b.load4(4 * e), b.load4(4 * e + 4), b.load4(4 * e + 8), b.load4(4 * e + 12));
  } else {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = b.load2(2 * e + 4 * k) | (b.load2(2 * e + 4 * k + 2) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <typename Elem, bool kVecRows, int T>
__device__ __forceinline__ void store_lane_block(const Buf& b, uint32_t e0, const float (&v)[T]) {
  if constexpr (sizeof(Elem) == 4) {
#pragma unroll
    for (int q = 0; q < T / 4; ++q) {
      const uint4 w = make_uint4(__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                                 __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3]));
      if constexpr (kVecRows) {
        b.store16(w, 4 * (e0 + 4 * q));
      } else {
        b.store4(w.x, 4 * (e0 + 4 * q));
        b.store4(w.y, 4 * (e0 + 4 * q + 1));
        b.store4(w.z, 4 * (e0 + 4 * q + 2));
        b.store4(w.w, 4 * (e0 + 4 * q + 3));
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < T / 8; ++q) {
      const uint4 w = make_uint4(pack_bf16x2(v[8 * q + 0], v[8 * q + 1]),
                                 pack_bf16x2(v[8 * q + 2], v[8 * q + 3]),
                                 pack_bf16x2(v[8 * q + 4], v[8 * q + 5]),
                                 pack_bf16x2(v[8 * q + 6], v[8 * q + 7]));
      if constexpr (kVecRows) {
        b.store16(w, 2 * (e0 + 8 * q));
      } else {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          b.store2(uint16_t(ws[k]), 2 * (e0 + 8 * q + 2 * k));
          b.store2(uint16_t(ws[k] >> 16), 2 * (e0 + 8 * q + 2 * k + 1));
        }
      }
    }
  }
}

}  // namespace ssm
