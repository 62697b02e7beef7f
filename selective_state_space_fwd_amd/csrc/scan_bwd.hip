// Selective-scan backward for gfx950 (CDNA4, wave64).
//
// Gradients of L = sum(dout * out) + sum(dfinal * final_state) for the forward of
// include/ssm_scan.h. The forward saves the state every kCkptInterval steps; the backward
// restarts from those states and recomputes the scan inside each interval instead of
// keeping every h_t, which is how p1 (mhpq.cn/news/1077344, section 3.3) describes the
// backward of a fused scan: only chunk-boundary states are stored, the scan is run again
// from them, then the gradients are formed.
//
// With s_t the step size, a_t = exp(s_t A), c_t = C_t dy_t and g_t = dL/dh_t, the state
// adjoint runs backwards in time, g_t = c_t + a_{t+1} g_{t+1}. In the pre-multiplied form
// e_t = a_t g_t it is a linear recurrence read from the right, e_t = a_t e_{t+1} + a_t c_t,
// so it has the same combine as the forward, (a1,b1) o (a2,b2) = (a2 a1, a2 b1 + b2), with
// the later step first. A lane folds its steps from the right into one operator, the
// lanes of a channel scan those operators from the last lane down, and each lane replays
// its steps with the adjoint entering from its right, forming per step:
//   dC_t += dy_t h_t,  dB_t += g_t s_t u_t  (summed over channels: first the two of a wave
//   in registers, then the wave rows of a workgroup in LDS, then the workgroups: partial
//   sums in a workspace added up in a fixed order by a second launch, or float atomics
//   when there is no workspace), du_t += g_t s_t B_t,
//   ds_t += g_t (A a_t h_{t-1} + B_t u_t), dA += g_t a_t s_t h_{t-1}.
//
// Mapping: a wavefront owns two channels of one batch row, one per 32-lane half, and lane
// i of a half owns T = 8 consecutive steps of a kCkptInterval-step interval (32 x 8 = 256);
// the intervals are processed last to first, carrying the state adjoint between them. The
// two halves of a wave scan independently (DPP inside 16-lane rows, then the row pair), and
// their dB/dC rows are added with one cross-half swap (v_permlane32_swap) before they
// reach LDS. A workgroup of W waves owns 2 W channels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "device_scan.h"
#include "scan_launch.h"

namespace ssm {
namespace {

struct BParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  const float* ckpt;
  const void* dout;
  const float* dfinal;
  void* du;
  void* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;
  void* dz;
  float* dbias;
  float* dh0;
  const uint8_t* mask;
  int dim, dstate, seqlen, dblocks, softplus, n_ckpt;
  // 0: dA, dB, dC, dD and dbias are the outputs, summed into with float atomics. 1: they
  // point into a workspace, where the kernel stores partial sums with plain stores (dB at
  // [workgroup][dB, dC][state][step], dC unused; dA at [row][state]; dD and dbias at [row])
  // for bwd_reduce_kernel to add up.
  int partials;
  // Segments: each channel's sequence cut into nseg runs of seg_chunks intervals (the last
  // maybe shorter), each its own workgroup; workgroup blockIdx.x takes segment
  // blockIdx.x / wgs of group blockIdx.x % wgs (wgs = batch dblocks). rows = batch dim: the
  // stride of one segment's slots of dA, dD, dbias and the carries. cq, cp: each segment's
  // state adjoint from a zero start at its right end, [nseg][rows][dstate], and its sum of
  // step sizes, [nseg][rows] (written by the carry launch; bwd_carry_kernel then turns cq
  // into the adjoint entering each segment, which the main launch reads).
  int nseg, seg_chunks, wgs;
  int64_t rows;
  float* cq;
  float* cp;
};

constexpr int kT = 8;                      // steps per lane
constexpr int kHalfLanes = 32;             // lanes per channel
constexpr int kMaxStates = 64;             // the C-ABI layer rejects larger dstate
static_assert(kHalfLanes * kT == kCkptInterval, "one interval per pass of a channel's lanes");

// Inclusive scan inside each 32-lane half, lane 0 of the half earliest, under the forward's
// combine. Rows (16 lanes) first, by DPP row_shr:1/2/4/8 (a lane whose source lies outside
// its row is not written: it combines with the identity), then lane 15 of rows 0 and 2 into
// rows 1 and 3 (row_bcast:15, row_mask 0xa), which does not cross the halves. Only b is
// complete afterwards (the caller does not need a). Two wait states between a VALU write
// and a DPP read of the same VGPR, as in the wave64 scan.
__device__ __forceinline__ void half_scan_inclusive(float& a, float& b) {
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
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(a), "+v"(b));
}

// Inclusive scan from the right inside each 32-lane half: lane i ends with the composition
// of the operators of lanes i..31 of its half, the last lane applied first:
// (a, b) <- (a_i a_j, a_i b_j + b_i) for the lanes j to its right.
//   1. Inside each row, DPP row_shl:1/2/4/8 (a lane whose source is past the row's end is
//      not written: the identity).
//   2. The first lanes of rows 1 and 3 now hold those rows' whole operators; rows 0 and 2
//      compose them in (rows 1 and 3 have nothing to their right inside their half). A DPP
//      wave_shl:1 copy moves lane 16's operator to lane 15 and lane 48's to lane 47 (the
//      last lanes of rows 0 and 2); DPP row_newbcast:15 reads that lane in every lane of
//      its row, and row_mask 0x5 writes rows 0 and 2 only.
// Two wait states between a VALU write and a DPP read of the same VGPR.
__device__ __forceinline__ void half_scan_from_right(float& a, float& b) {
  float na, nb;
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_mov_b32_dpp %2, %0 wave_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32_dpp %3, %1 wave_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %3, %0 row_newbcast:15 row_mask:0x5 bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %2, %0 row_newbcast:15 row_mask:0x5 bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(a), "+v"(b), "=&v"(na), "=&v"(nb));
}

// Sum over each 32-lane half, complete in the half's last lane (31 or 63): DPP row_shr
// partial sums inside each row, then row 0's and row 2's totals into rows 1 and 3.
__device__ __forceinline__ float half_sum_to_last(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
  return v;
}

// Lane i receives lane i+1's (shift_down_any, DPP wave_shl:1) or lane i-1's (shift_up_any,
// wave_shr:1) value; what the last (first) lane of each half receives is another channel's
// value or 0, for callers that select there. Each shift is pinned by an empty asm, so that it
// is taken in every lane, before the caller's select: moved under the select, it would run
// with the selected-away lanes disabled, and a DPP read from a disabled lane returns nothing.
__device__ __forceinline__ float shift_down_any(float v) {
  float s = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x130, 0xf, 0xf, true));
  asm volatile("" : "+v"(s));
  return s;
}
__device__ __forceinline__ float shift_up_any(float v) {
  float s = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x138, 0xf, 0xf, true));
  asm volatile("" : "+v"(s));
  return s;
}

// For two values per lane, lo and hi: the first 32 lanes end with lo + (the same lane of
// the other half's lo), the last 32 with hi + (the other half's hi); either way the first
// half's value is added to the second's. v_permlane32_swap exchanges the upper 32 lanes of
// its first operand with the lower 32 lanes of its second.
__device__ __forceinline__ float sum_halves(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float sigmoid_f(float x) { return rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

// T steps of a lane from a buffer holding the wave's two channel rows back to back. e0:
// element offset of the lane's first step t0 inside that buffer; `end` the buffer's length
// in elements: a word (or, element-wise, an element) at or past step L of its row is read
// at `end`, i.e. as zero, so that it never reaches into the next row. kLastUse: the
// interval's second read of an input, after its state loop; streamed (non-temporal), so that
// its lines leave L2 first and other workgroups' inputs, still to be read again, stay (reads
// 184 -> 160 MB per call on the layer workload, same time).
template <typename Elem, bool kVecRows, bool kLastUse = false>
__device__ __forceinline__ void load_steps(const Buf& b, uint32_t e0, int t0, int L,
                                           uint32_t end, float (&v)[kT]) {
  constexpr int kVec = Vec<Elem>::kN;
  constexpr uint32_t kEsz = sizeof(Elem);
  if constexpr (kVecRows) {
#pragma unroll
    for (int q = 0; q < kT / kVec; ++q) {
      const uint32_t e = (t0 + q * kVec < L) ? e0 + q * kVec : end;
      widen_raw16<Elem>(kLastUse ? b.load16_nt(e * kEsz) : b.load16(e * kEsz), &v[q * kVec]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kT; ++j) {
      const uint32_t e = (t0 + j < L) ? e0 + j : end;
      v[j] = (kEsz == 4) ? __uint_as_float(b.load4(4 * e)) : bf16_lo(b.load2(2 * e));
    }
  }
}

// The store counterpart: steps at or past L are dropped (written at `end`). The stores are
// non-temporal: the gradients are not read again here, and the interval's inputs, read
// again after its state loop, stay in L2 in their place (reads 244 -> 185 MB per call on
// the layer workload, with the partial sums' stores non-temporal as well).
template <typename Elem, bool kVecRows>
__device__ __forceinline__ void store_steps(const Buf& b, uint32_t e0, int t0, int L,
                                            uint32_t end, const float (&v)[kT]) {
  constexpr int kVec = Vec<Elem>::kN;
  if constexpr (kVecRows) {
#pragma unroll
    for (int q = 0; q < kT / kVec; ++q) {
      const uint32_t e = (t0 + q * kVec < L) ? e0 + q * kVec : end;
      if constexpr (sizeof(Elem) == 4) {
        b.store16_nt(make_uint4(__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                                __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])),
                     4 * e);
      } else {
        b.store16_nt(make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])),
                     2 * e);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kT; ++j) {
      const uint32_t e = (t0 + j < L) ? e0 + j : end;
      if constexpr (sizeof(Elem) == 4)
        b.store4(__float_as_uint(v[j]), 4 * e);
      else
        b.store2(uint16_t(pack_bf16x2(v[j], 0.0f)), 2 * e);
    }
  }
}

// W: waves per workgroup (2 W channels). M: states between workgroup barriers; the LDS
// rows of dB and dC have 2 M slots, so that one group of M states is written while the
// previous one is added up. kMask: read a padding mask (its own instantiation: the unmasked
// kernel's register count decides how many waves fit on a SIMD). kSeg: a segmented backward
// (the workgroup takes one segment of its channels' sequences, starting from the adjoint
// carried into it; its own instantiation, so that the whole-sequence kernel's code is not
// touched).
template <typename Elem, int W, int M, bool kVecRows, bool kMask, bool kSeg = false>
__global__ __launch_bounds__(64 * W, 4) void scan_bwd_kernel(BParams p) {
  constexpr int kVec = Vec<Elem>::kN;
  constexpr int kSteps = kCkptInterval;  // steps per interval
  constexpr int kSlots = 2 * M;
  static_assert(kT % kVec == 0, "whole 16-byte words per lane");

  // [slot][dB / dC][wave][four steps]: each wave writes its own row (the sums of its two
  // channels); the flush adds the W rows of a step in wave order.
  __shared__ float4 acc[kSlots][2][W][kSteps / 4];
  // Per (wave, half, state): the state adjoint carried from the interval to the right, and
  // the running dA sum over the intervals.
  __shared__ float s_adj[W][2][kMaxStates];
  __shared__ float s_dA[W][2][kMaxStates];
  __shared__ float s_dDb[W][2][2];  // running dD and dbias sums of each channel
  // B and C of a group's M states over the interval, widened to fp32 once per workgroup
  // rather than by every wave: [buffer][state in group][B / C][four steps]. Group k reads
  // buffer k & 1; the rows of group k + 1 go into the other one during group k.
  __shared__ float4 s_bc[2][M][2][kSteps / 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;         // which of the wave's two channels
  const int li = lane & 31;         // lane inside the channel
  const bool half_start = li == 0, half_end = li == kHalfLanes - 1;
  const int seg = kSeg ? int(blockIdx.x) / p.wgs : 0;
  const int wg = kSeg ? int(blockIdx.x) - seg * p.wgs : int(blockIdx.x);  // the channel group
  const int b = wg / p.dblocks;
  const int d0 = (wg - b * p.dblocks) * (2 * W) + 2 * wave;  // the wave's first channel
  // Uniform, but the compiler computes the clamp with a vector min/max (v_med3): taken back
  // to a scalar register here, or every buffer descriptor built from it would be treated as
  // divergent (a waterfall loop around each access).
  const int rows_here = __builtin_amdgcn_readfirstlane(
      p.dim - d0 >= 2 ? 2 : (p.dim - d0 > 0 ? p.dim - d0 : 0));
  const int d = d0 + hf;
  const bool active = hf < rows_here;
  const int N = p.dstate, L = p.seqlen;
  const int n_chunks = (L + kSteps - 1) / kSteps;
  // this segment's intervals, c_lo .. c_hi, processed last to first
  const int c_lo = kSeg ? seg * p.seg_chunks : 0;
  const int c_hi =
      kSeg ? (c_lo + p.seg_chunks < n_chunks ? c_lo + p.seg_chunks : n_chunks) - 1 : n_chunks - 1;
  const int64_t row0 = int64_t(b) * p.dim + (rows_here > 0 ? d0 : 0);
  const int64_t row = row0 + hf;  // this half's channel (meaningful when active)

  // The wave's channel rows, back to back: lane (hf, li) reads element hf * L + t.
  const uint32_t end = uint32_t(rows_here) * uint32_t(L);  // elements
  const uint32_t bytes = end * uint32_t(sizeof(Elem));
  const Buf u_buf(static_cast<const Elem*>(p.u) + row0 * L, bytes);
  const Buf dl_buf(static_cast<const Elem*>(p.delta) + row0 * L, bytes);
  const Buf do_buf(static_cast<const Elem*>(p.dout) + row0 * L, bytes);
  const Buf z_buf(static_cast<const Elem*>(p.z ? p.z : p.u) + row0 * L, p.z ? bytes : 0u);
  const Buf du_buf(static_cast<Elem*>(p.du) + row0 * L, bytes);
  const Buf dd_buf(static_cast<Elem*>(p.ddelta) + row0 * L, bytes);
  const Buf dz_buf(static_cast<Elem*>(p.z ? p.dz : p.du) + row0 * L, p.z ? bytes : 0u);
  const uint32_t bc_elems = uint32_t(N) * uint32_t(L);
  const Buf B_buf(static_cast<const Elem*>(p.B) + int64_t(b) * N * L, bc_elems * sizeof(Elem));
  const Buf C_buf(static_cast<const Elem*>(p.C) + int64_t(b) * N * L, bc_elems * sizeof(Elem));
  const uint32_t row_e = uint32_t(hf) * uint32_t(L);  // this half's row inside the buffers
  const Buf mask_buf(kMask ? p.mask + int64_t(b) * L : nullptr, kMask ? uint32_t(L) : 0u);

  const float Dd = (active && p.D) ? p.D[d] : 0.0f;
  const float bias_d = (active && p.bias) ? p.bias[d] : 0.0f;
  for (int n = li; n < N; n += kHalfLanes) {
    // e entering from the right: dfinal at the sequence's end (e_L); with segments, what
    // bwd_carry_kernel combined for this segment.
    float e = 0.0f;
    if (active) {
      if (kSeg)
        e = p.cq[(int64_t(seg) * p.rows + row) * N + n];
      else
        e = p.dfinal ? p.dfinal[row * N + n] : 0.0f;
    }
    s_adj[wave][hf][n] = e;
    s_dA[wave][hf][n] = 0.0f;
  }
  if (li < 2) s_dDb[wave][hf][li] = 0.0f;
  {
    // slots of inactive waves are read by the flush: they stay zero
    float4* flat = &acc[0][0][0][0];
    for (int i = tid; i < kSlots * 2 * W * (kSteps / 4); i += 64 * W)
      flat[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  __syncthreads();

  // Where the flush adds this workgroup's dB and dC rows: this batch row of the outputs, or
  // this workgroup's slot of partial sums. Both take the same offset (state, step) after it.
  const int64_t nl = int64_t(N) * L;
  float* const flush0 = p.partials ? p.dB + int64_t(wg) * 2 * nl : p.dB + b * nl;
  float* const flush1 = p.partials ? flush0 + nl : p.dC + b * nl;
  const int total = (c_hi - c_lo + 1) * N;  // (interval, state) pairs, in processing order

  // The staging words: one 16-byte source word per thread of the first kStageWords. The
  // first M kRowWords threads take B, the next C (a whole number of waves each, so the
  // array, and with it the buffer descriptor, is uniform in a wave); thread `tid` holds
  // state-in-group st_ms, steps [st_ws, st_ws + kVec) of the interval. A word at or past
  // the sequence's end reads zeros (put past the array).
  constexpr int kRowWords = kSteps / kVec;
  constexpr int kStageWords = M * 2 * kRowWords;
  static_assert(kStageWords <= 64 * W, "one staging word per thread");
  static_assert((M * kRowWords) % 64 == 0, "each array takes whole waves");
  const bool st_on = wave < kStageWords / 64;
  const int st_ab = __builtin_amdgcn_readfirstlane(tid / (M * kRowWords));  // 0: B, 1: C
  const int st_ms = (tid / kRowWords) % M;
  const int st_ws = (tid % kRowWords) * kVec;
  auto stage_load = [&](int grp, uint4& st_raw) {  // this thread's word of group grp
    if (st_on) {
      const int i0 = grp * M;  // uniform: the group's first (interval, state) pair
      int c = c_hi - i0 / N, n = i0 - (i0 / N) * N + st_ms;
      while (n >= N) {  // the pairs after it take the next states, then the interval before
        n -= N;
        --c;
      }
      const int t = c * kSteps + st_ws;
      const uint32_t e =
          (c >= c_lo && t < L) ? uint32_t(n) * uint32_t(L) + uint32_t(t) : bc_elems;
      st_raw = load_word<Elem, kVecRows>(st_ab == 0 ? B_buf : C_buf, e);
    }
  };
  auto stage_commit = [&](int grp, const uint4& st_raw) {
    if (st_on) {
      float v[kVec];
      widen_raw16<Elem>(st_raw, v);
      float4* dst = &s_bc[grp & 1][st_ms][st_ab][st_ws / 4];
#pragma unroll
      for (int q = 0; q < kVec / 4; ++q)
        dst[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
  };
  {
    uint4 w0;
    stage_load(0, w0);
    stage_commit(0, w0);
    __syncthreads();
  }
  // Adds the workgroup's rows of the pairs first .. first + count - 1 into dB and dC: one
  // (pair, gradient, step) item per thread and pass. (c0, n0): the interval and state of
  // pair `first`; the pairs after it take the next states, then the interval to the left.
  // A wave's 64 items share their pair and gradient (64 divides kSteps), so everything but
  // the step is uniform.
  static_assert(kSteps % 64 == 0, "a wave's flush items share a pair and a gradient");
  auto flush = [&](int first, int count, int c0, int n0) {
    for (int i0 = 64 * wave; i0 < count * 2 * kSteps; i0 += 64 * W) {
      const int k = i0 / (2 * kSteps);
      const int wc = (i0 / kSteps) & 1;  // 0: dB, 1: dC
      const int st = i0 % kSteps + lane;
      const int pair = first + k;
      int c = c0, n = n0 + k;
      while (n >= N) {
        n -= N;
        --c;
      }
      const int t = c * kSteps + st;
      const float* src = reinterpret_cast<const float*>(&acc[pair % kSlots][wc][0][0]) + st;
      float v = 0.0f;
#pragma unroll 4
      for (int w = 0; w < W; ++w) v += src[w * kSteps];
      if (t < L) {
        float* dst = (wc ? flush1 : flush0) + (int64_t(n) * L + t);
        if (p.partials)  // read once, by the reduction launch: kept out of L2's way
          __builtin_nontemporal_store(v, dst);
        else
          unsafeAtomicAdd(dst, v);
      }
    }
  };

  // A and the saved state of an (interval, state) pair, fetched one pair ahead of their use
  // (past the last pair: the first pair again, never used). Both through the wave's rows as
  // one buffer: the half's offset in a register (an inactive half's lies past the buffer and
  // reads zero), the pair's part uniform (a per-lane 64-bit address would hold two
  // registers each across the state loop).
  const Buf A_buf(p.A + int64_t(rows_here > 0 ? d0 : 0) * N, uint32_t(rows_here * N) * 4u);
  const Buf ck_buf(p.ckpt + row0 * p.n_ckpt * N, uint32_t(rows_here * p.n_ckpt * N) * 4u);
  const uint32_t a_off = uint32_t(hf * N) * 4u, ck_off = uint32_t(hf * p.n_ckpt * N) * 4u;
  auto fetch_pair = [&](int c, int n, float& A_out, float& h_out) {
    if (c < c_lo) c = c_lo, n = 0;
    A_out = __uint_as_float(A_buf.load4(a_off, uint32_t(n) * 4u));
    h_out = __uint_as_float(ck_buf.load4(ck_off, uint32_t(c * N + n) * 4u));
  };
  float A_nx, hc_nx;
  fetch_pair(c_hi, 0, A_nx, hc_nx);

  int pair = 0;
  int grp_c = c_hi, grp_n = 0;  // the current group's first pair
  for (int c = c_hi; c >= c_lo; --c) {
    const int t0 = c * kSteps + li * kT;
    const uint32_t e0 = row_e + uint32_t(t0);
    // Live across the state loop: s, s u, dL/dy, y and the two sums over the states (u
    // itself is read again after the loop).
    float su[kT], sv[kT], dyv[kT], y[kT], gdu[kT], gds[kT];
    float sdt = 0.0f;
    uint32_t pad_bits = 0;  // bit j: step t0 + j is padding (masked kernels only)
    // The padding mask of this lane's steps, read branch-free through the batch row's mask
    // (bytes past the sequence read 1: those steps are identity steps anyway).
    uint32_t mask_bytes[kT];
    if constexpr (kMask) {
#pragma unroll
      for (int j = 0; j < kT; ++j)
        mask_bytes[j] = t0 + j < L ? mask_buf.load1(uint32_t(t0 + j)) : 1u;
    }
    float dD_acc = 0.0f;
    {
      float uv[kT], xv[kT], dov[kT], zv[kT];
      load_steps<Elem, kVecRows>(u_buf, e0, t0, L, end, uv);
      load_steps<Elem, kVecRows>(dl_buf, e0, t0, L, end, xv);
      load_steps<Elem, kVecRows>(do_buf, e0, t0, L, end, dov);
      load_steps<Elem, kVecRows>(z_buf, e0, t0, L, end, zv);
      // the step size: the softplus flag tested once, around the whole loop
      if (p.softplus) {
#pragma unroll
        for (int j = 0; j < kT; ++j) sv[j] = softplus_f(xv[j] + bias_d);
      } else {
#pragma unroll
        for (int j = 0; j < kT; ++j) sv[j] = xv[j] + bias_d;
      }
#pragma unroll
      for (int j = 0; j < kT; ++j) {
        float s = sv[j];
        if (t0 + j >= L || !active) s = uv[j] = dov[j] = zv[j] = 0.0f;  // identity steps
        if constexpr (kMask) {
          if (mask_bytes[j] == 0) {  // padding: the state is kept (the step is the identity)
            s = 0.0f;
            pad_bits |= 1u << j;
          }
        }
        sv[j] = s;
        su[j] = s * uv[j];
        sdt += s;
        dyv[j] = dov[j];
      }
      // With the gate, dL/dy = dout z sigmoid(z) does not need y; only dL/dz does, and y
      // (before the gate) is summed over the states in the loop below, which recomputes
      // every h_t anyway. dout, z and the raw step size are read again after the loop
      // rather than kept live across it.
#pragma unroll
      for (int j = 0; j < kT; ++j) y[j] = Dd * uv[j];
      if (p.z) {
#pragma unroll
        for (int j = 0; j < kT; ++j) dyv[j] = dov[j] * zv[j] * sigmoid_f(zv[j]);
      }
#pragma unroll
      for (int j = 0; j < kT; ++j) {
        dD_acc = __builtin_fmaf(dyv[j], uv[j], dD_acc);
        gdu[j] = 0.0f;  // sum over states of g B (du and the step size share it)
        gds[j] = 0.0f;  // sum over states of g A a h_{t-1}
      }
      // Formed here: left to the compiler, the sum sinks to its use after the state loop
      // and keeps u live (and spilled) across it.
      asm volatile("" : "+v"(dD_acc));
    }

    for (int n = 0; n < N; ++n, ++pair) {
      const float An = A_nx, hc = hc_nx;
      const int c_nx = n + 1 < N ? c : c - 1, n_nx = n + 1 < N ? n + 1 : 0;
      fetch_pair(c_nx, n_nx, A_nx, hc_nx);
      const float a2 = An * kLog2e;
      const float G = s_adj[wave][hf][n];  // e entering the interval from the right
      float Bv[kT], Cv[kT], dA[kT], h[kT];
      // The next group's rows, fetched at the start of the group's first state and written
      // into the other buffer before its adjoint part (read only after the group's barrier).
      // Local to the state, so nothing keeps the word live across the loop.
      uint4 st_word;
      {
        const int grp = pair / M;
        if (pair % M == 0) stage_load(grp + 1, st_word);
        const float4* sB = &s_bc[grp & 1][pair % M][0][kT / 4 * li];
#pragma unroll
        for (int q = 0; q < kT / 4; ++q) {
          const float4 bq = sB[q];
          Bv[4 * q] = bq.x;
          Bv[4 * q + 1] = bq.y;
          Bv[4 * q + 2] = bq.z;
          Bv[4 * q + 3] = bq.w;
        }
      }
      // forward again from the saved state: h_t for this lane's steps
      float bseg = half_start ? hc : 0.0f;
#pragma unroll
      for (int j = 0; j < kT; ++j) {
        dA[j] = exp2_hw(sv[j] * a2);
        bseg = __builtin_fmaf(dA[j], bseg, su[j] * Bv[j]);
      }
      const float alpha = exp2_hw(sdt * a2);  // product of the lane's a_t
      {
        // C only from here on: read after the recomputation, so its registers are free
        // during it
        asm volatile("" ::: "memory");
        const float4* sC = &s_bc[(pair / M) & 1][pair % M][1][kT / 4 * li];
#pragma unroll
        for (int q = 0; q < kT / 4; ++q) {
          const float4 cq = sC[q];
          Cv[4 * q] = cq.x;
          Cv[4 * q + 1] = cq.y;
          Cv[4 * q + 2] = cq.z;
          Cv[4 * q + 3] = cq.w;
        }
      }
      {
        float aseg = alpha;
        half_scan_inclusive(aseg, bseg);  // bseg: the state after the lane's last step
      }
      const float up = shift_up_any(bseg);
      const float hin = half_start ? hc : up;  // the state entering the lane's steps
      {
        float hh = hin;
#pragma unroll
        for (int j = 0; j < kT; ++j) {
          hh = (j == kT - 1) ? bseg : __builtin_fmaf(dA[j], hh, su[j] * Bv[j]);
          h[j] = hh;
          y[j] = __builtin_fmaf(Cv[j], hh, y[j]);  // read only with a gate; a select per
                                                   // step would cost more
        }
      }
      if (pair % M == 0) stage_commit(pair / M + 1, st_word);  // before the adjoint's peak
      // adjoint: fold the lane's steps from the right, scan from the half's last lane down
      float beta = 0.0f;
#pragma unroll
      for (int j = kT - 1; j >= 0; --j) beta = dA[j] * __builtin_fmaf(Cv[j], dyv[j], beta);
      float ra = alpha, rb = beta;
      half_scan_from_right(ra, rb);
      // e entering this lane's steps from the right; the last lane's right neighbour is the
      // next interval, whose adjoint G enters unchanged
      const float an = shift_down_any(ra), bn = shift_down_any(rb);
      float v = half_end ? G : __builtin_fmaf(an, G, bn);
      if (half_start) s_adj[wave][hf][n] = __builtin_fmaf(ra, G, rb);  // into the interval
                                                                       // to the left
      // dB and dC rows of the step pairs (j, j + 4) are added across the two halves as
      // soon as both exist and go to LDS at once: four steps per lane, 8 li + 4 hf on.
      float dBr[kT / 2], dCr[kT / 2];
      const int slot = pair % kSlots;
      float* const rowB = reinterpret_cast<float*>(&acc[slot][0][wave][2 * li + hf]);
      float* const rowC = reinterpret_cast<float*>(&acc[slot][1][wave][2 * li + hf]);
      float dAn = 0.0f;
#pragma unroll
      for (int j = kT - 1; j >= 0; --j) {
        const float g = __builtin_fmaf(Cv[j], dyv[j], v);  // g_t = C_t dy_t + e_{t+1}
        const float hp = (j > 0) ? h[j - 1] : hin;
        const float ag = dA[j] * g;  // e_t = a_t g_t, the adjoint entering the step before
        const float q = ag * hp;     // g_t a_t h_{t-1}
        const float gB = g * su[j], gC = dyv[j] * h[j];
        if (j >= kT / 2) {
          dBr[j - kT / 2] = gB;
          dCr[j - kT / 2] = gC;
        } else {
          rowB[j] = sum_halves(gB, dBr[j]);
          rowC[j] = sum_halves(gC, dCr[j]);
        }
        gdu[j] = __builtin_fmaf(g, Bv[j], gdu[j]);
        gds[j] = __builtin_fmaf(q, An, gds[j]);
        dAn = __builtin_fmaf(q, sv[j], dAn);
        v = ag;
      }
      dAn = half_sum_to_last(dAn);
      if (half_end) atomicAdd(&s_dA[wave][hf][n], dAn);  // one lane per address: in order
      if ((pair + 1) % M == 0) {
        __syncthreads();  // every wave's rows of the group are in acc
        // The group's slots are written again one group later, after the next barrier,
        // which no thread passes before finishing this flush.
        flush(pair + 1 - M, M, grp_c, grp_n);
        grp_c = c_nx;
        grp_n = n_nx;
      }
    }
    // du_t = s_t sum_n g B + D dy_t and ds_t = sum_n g (A a h_{t-1} + B u_t), from the two
    // sums over the states.
    // Three phases, each storing its output before the next one's loads are issued (a
    // memory clobber between them keeps the compiler from hoisting every reload to the top,
    // which would hold them all live at once).
    {
      float uv[kT];
      load_steps<Elem, kVecRows, true>(u_buf, e0, t0, L, end, uv);
#pragma unroll
      for (int j = 0; j < kT; ++j) {
        gds[j] = __builtin_fmaf(uv[j], gdu[j], gds[j]);
        gdu[j] = __builtin_fmaf(sv[j], gdu[j], Dd * dyv[j]);
      }
      store_steps<Elem, kVecRows>(du_buf, e0, t0, L, end, gdu);
    }
    asm volatile("" ::: "memory");
    if (p.z) {
      float dz2[kT], zz[kT];
      load_steps<Elem, kVecRows, true>(do_buf, e0, t0, L, end, dz2);
      load_steps<Elem, kVecRows, true>(z_buf, e0, t0, L, end, zz);
#pragma unroll
      for (int j = 0; j < kT; ++j) {
        const float sg = sigmoid_f(zz[j]);
        dz2[j] = dz2[j] * y[j] * sg * __builtin_fmaf(zz[j], 1.0f - sg, 1.0f);
      }
      store_steps<Elem, kVecRows>(dz_buf, e0, t0, L, end, dz2);
    }
    asm volatile("" ::: "memory");
    float dd[kT], db_acc = 0.0f;
    if (p.softplus) {  // the flag tested once, around the whole loop
      float xv[kT];    // the raw step size again, for softplus' derivative
      load_steps<Elem, kVecRows, true>(dl_buf, e0, t0, L, end, xv);
#pragma unroll
      for (int j = 0; j < kT; ++j) dd[j] = gds[j] * sigmoid_f(xv[j] + bias_d);
    } else {
#pragma unroll
      for (int j = 0; j < kT; ++j) dd[j] = gds[j];
    }
#pragma unroll
    for (int j = 0; j < kT; ++j) {
      if constexpr (kMask) {
        if (pad_bits & (1u << j)) dd[j] = 0.0f;  // a padding step's step size is not used
      }
      if (t0 + j < L) db_acc += dd[j];
    }
    store_steps<Elem, kVecRows>(dd_buf, e0, t0, L, end, dd);
    {
      // this interval's dD and dbias shares, summed over the half into its last lane
      const float sD = half_sum_to_last(dD_acc), sb = half_sum_to_last(db_acc);
      if (half_end) {
        s_dDb[wave][hf][0] += sD;
        s_dDb[wave][hf][1] += sb;
      }
    }
  }
  if (total % M != 0) {  // the last, partly filled group
    __syncthreads();
    flush(total - total % M, total % M, grp_c, grp_n);
  }

  const float sD = s_dDb[wave][hf][0], sb = s_dDb[wave][hf][1];
  if (active) {
    // s_adj and s_dA were last written by lanes of this wave; LDS keeps a wave's order. With
    // segments, dh0 comes from the first one, and dA, dD and dbias go into this segment's
    // slots (the reduction adds the segments too).
    const int64_t srow = kSeg ? int64_t(seg) * p.rows + row : row;
    for (int n = li; n < N; n += kHalfLanes) {
      const float dAv = s_dA[wave][hf][n];
      if (p.dh0 && (!kSeg || seg == 0))
        p.dh0[row * N + n] = s_adj[wave][hf][n];  // e_{-1} = a_0 g_0
      if (p.partials)
        p.dA[srow * N + n] = dAv;
      else
        unsafeAtomicAdd(&p.dA[int64_t(d) * N + n], dAv);
    }
    if (half_end) {
      if (p.partials) {
        if (p.dD) p.dD[srow] = sD;
        if (p.dbias) p.dbias[srow] = sb;
      } else {
        if (p.dD) unsafeAtomicAdd(&p.dD[d], sD);
        if (p.dbias) unsafeAtomicAdd(&p.dbias[d], sb);
      }
    }
  }
}

// The carry launch of a segmented backward, for segments 1 .. nseg - 1: per (row, state), the
// state adjoint leaving the segment's first step when zero enters it from the right, and per
// row the segment's sum of step sizes. Only the adjoint's part of the backward: per interval
// (last to first) the step sizes and dL/dy of the lane's 8 steps, then per state a_t, the
// lane's fold from the right, the half's scan from the right and the carry across
// intervals. The lanes are mapped as in scan_bwd_kernel (a wave owns two channels, lane i of
// a half 8 consecutive steps of an interval); each wave is independent of the others: C is
// read straight from memory (a half's 32 lanes read 256 consecutive steps of a row), and
// nothing is staged or waited for across waves.
constexpr int kCarryWaves = 4;

template <typename Elem, bool kVecRows, bool kMask>
__global__ __launch_bounds__(64 * kCarryWaves) void bwd_carry_scan_kernel(BParams p) {
  __shared__ float s_e[kCarryWaves][2][kMaxStates];   // the adjoint carried across intervals
  __shared__ float s_a2[kCarryWaves][2][kMaxStates];  // A log2(e) of the half's channel
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, li = lane & 31;
  const bool half_start = li == 0, half_end = li == kHalfLanes - 1;
  const int dblocks = (p.dim + 2 * kCarryWaves - 1) / (2 * kCarryWaves);
  const int wgs = int(p.rows / p.dim) * dblocks;  // workgroups per segment
  const int seg = 1 + int(blockIdx.x) / wgs;
  const int wg = int(blockIdx.x) - (seg - 1) * wgs;
  const int b = wg / dblocks;
  const int d0 = (wg - b * dblocks) * (2 * kCarryWaves) + 2 * wave;
  const int rows_here = __builtin_amdgcn_readfirstlane(
      p.dim - d0 >= 2 ? 2 : (p.dim - d0 > 0 ? p.dim - d0 : 0));
  const int d = d0 + hf;
  const bool active = hf < rows_here;
  const int N = p.dstate, L = p.seqlen;
  constexpr int kSteps = kCkptInterval;
  const int n_chunks = (L + kSteps - 1) / kSteps;
  const int c_lo = seg * p.seg_chunks;
  const int c_hi = (c_lo + p.seg_chunks < n_chunks ? c_lo + p.seg_chunks : n_chunks) - 1;
  const int64_t row0 = int64_t(b) * p.dim + (rows_here > 0 ? d0 : 0);
  const int64_t row = row0 + hf;
  const uint32_t end = uint32_t(rows_here) * uint32_t(L);  // elements of the wave's rows
  const uint32_t bytes = end * uint32_t(sizeof(Elem));
  const Buf dl_buf(static_cast<const Elem*>(p.delta) + row0 * L, bytes);
  const Buf do_buf(static_cast<const Elem*>(p.dout) + row0 * L, bytes);
  const Buf z_buf(static_cast<const Elem*>(p.z ? p.z : p.delta) + row0 * L, p.z ? bytes : 0u);
  const uint32_t bc_elems = uint32_t(N) * uint32_t(L);
  const Buf C_buf(static_cast<const Elem*>(p.C) + int64_t(b) * N * L, bc_elems * sizeof(Elem));
  const uint32_t row_e = uint32_t(hf) * uint32_t(L);
  const Buf mask_buf(kMask ? p.mask + int64_t(b) * L : nullptr, kMask ? uint32_t(L) : 0u);
  const float bias_d = (active && p.bias) ? p.bias[d] : 0.0f;
  for (int n = li; n < N; n += kHalfLanes) {
    s_e[wave][hf][n] = 0.0f;
    s_a2[wave][hf][n] = active ? p.A[int64_t(d) * N + n] * kLog2e : 0.0f;
  }
  float seg_sdt = 0.0f;
  for (int c = c_hi; c >= c_lo; --c) {
    const int t0 = c * kSteps + li * kT;
    const uint32_t e0 = row_e + uint32_t(t0);
    float sv[kT], dyv[kT], sdt = 0.0f;
    {
      float xv[kT], dov[kT], zv[kT];
      load_steps<Elem, kVecRows>(dl_buf, e0, t0, L, end, xv);
      load_steps<Elem, kVecRows>(do_buf, e0, t0, L, end, dov);
      load_steps<Elem, kVecRows>(z_buf, e0, t0, L, end, zv);
      if (p.softplus) {
#pragma unroll
        for (int j = 0; j < kT; ++j) sv[j] = softplus_f(xv[j] + bias_d);
      } else {
#pragma unroll
        for (int j = 0; j < kT; ++j) sv[j] = xv[j] + bias_d;
      }
#pragma unroll
      for (int j = 0; j < kT; ++j) {
        float sj = sv[j];
        if (t0 + j >= L || !active) sj = dov[j] = zv[j] = 0.0f;  // identity steps
        if constexpr (kMask) {
          const uint32_t m = t0 + j < L ? mask_buf.load1(uint32_t(t0 + j)) : 1u;
          if (m == 0) sj = 0.0f;  // padding: the state is kept, the output still emitted
        }
        sv[j] = sj;
        sdt += sj;
        dyv[j] = p.z ? dov[j] * zv[j] * sigmoid_f(zv[j]) : dov[j];
      }
    }
    seg_sdt += sdt;
    for (int n = 0; n < N; ++n) {
      float Cv[kT];
      load_steps<Elem, kVecRows>(C_buf, uint32_t(n) * uint32_t(L) + uint32_t(t0), t0, L,
                                 bc_elems, Cv);
      const float a2 = s_a2[wave][hf][n];
      float beta = 0.0f;
#pragma unroll
      for (int j = kT - 1; j >= 0; --j)
        beta = exp2_hw(sv[j] * a2) * __builtin_fmaf(Cv[j], dyv[j], beta);
      float ra = exp2_hw(sdt * a2), rb = beta;
      half_scan_from_right(ra, rb);
      const float G = s_e[wave][hf][n];
      if (half_start) s_e[wave][hf][n] = __builtin_fmaf(ra, G, rb);
    }
  }
  const float sp = half_sum_to_last(seg_sdt);
  if (active) {
    const int64_t r = int64_t(seg) * p.rows + row;
    for (int n = li; n < N; n += kHalfLanes) p.cq[r * N + n] = s_e[wave][hf][n];
    if (half_end) p.cp[r] = sp;
  }
}

// Between the carry launch and the main one of a segmented backward: per (row, state), the
// adjoint entering each segment from the right, from the last segment down. Segment s maps
// the e entering it to the e leaving its first step, e -> exp(A sum s) e + q_s (q_s its
// adjoint from a zero start, written by the carry launch); the last segment starts from
// dfinal. Each q_s is read before its slot receives the e entering segment s, which is what
// the main launch reads (slot 0, which no carry fills, receives segment 0's).
__global__ __launch_bounds__(256) void bwd_carry_kernel(const float* A, const float* dfinal,
                                                        float* cq, const float* cp, int64_t rows,
                                                        int64_t dim, int dstate, int nseg) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * dstate) return;
  const int64_t row = i / dstate;
  const int n = int(i - row * dstate);
  const float a2 = A[(row % dim) * dstate + n] * kLog2e;
  float e = dfinal ? dfinal[i] : 0.0f;
  for (int s = nseg - 1; s >= 1; --s) {
    const int64_t r = int64_t(s) * rows + row;
    const float q = cq[r * dstate + n];
    cq[r * dstate + n] = e;
    e = __builtin_fmaf(exp2_hw(cp[r] * a2), e, q);
  }
  cq[row * dstate + n] = e;
}

// The second launch of a backward with a workspace: every summed gradient is the sum of its
// partials in a fixed order (no atomics). grid.y = 0: dB and dC, element (b, n, t) summed
// over the batch row's workgroups; grid.y = 1: dA, dD and dbias summed over the segments'
// batch rows.
struct RParams {
  const float* part;
  const float* part_dA;
  const float* part_dD;
  const float* part_dbias;
  float* dB;
  float* dC;
  float* dA;
  float* dD;      // nullable
  float* dbias;   // nullable
  int64_t batch, dim, dstate, seqlen, groups;
  int64_t seg_rows;  // rows of dA, dD and dbias partials: segments x batch rows
};

// The workgroups g of a batch row are split into kSlices runs of consecutive g; eight
// threads take one (float, or four neighbouring floats with V = 4) column, one run each, and
// the runs' sums are added through LDS in run order. Within a run, s_k adds the partials of
// g = k (mod 4) in increasing g, the tail joins s_0, and the run sum is (s_0 + s_1) +
// (s_2 + s_3): a fixed order for every element, whatever V is, with 16 loads per thread.
constexpr int kSlices = 8;
constexpr int kColumns = 256 / kSlices;

// V = 4 needs dstate * seqlen % 4 == 0 and 16-byte aligned dB and dC.
template <int V>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(RParams r) {
  typedef float vec_t __attribute__((ext_vector_type(V)));
  if (blockIdx.y == 0) {
    __shared__ vec_t runs[kSlices][kColumns];
    const int col = threadIdx.x % kColumns, slice = threadIdx.x / kColumns;
    const int64_t nl = r.dstate * r.seqlen;
    const int64_t cols = r.batch * 2 * nl / V;
    const int64_t gs = 2 * nl / V;  // vectors from one workgroup's partials to the next
    const int64_t per = (r.groups + kSlices - 1) / kSlices;
    const int64_t g0 = slice * per, g1 = g0 + per < r.groups ? g0 + per : r.groups;
    for (int64_t base = int64_t(blockIdx.x) * kColumns; base < cols;
         base += int64_t(gridDim.x) * kColumns) {  // the same trip count for the whole block
      const int64_t i = base + col;
      const int64_t bw = (i * V) / nl, e = i * V - bw * nl;  // bw = 2 b + (0: dB, 1: dC)
      const int64_t b = bw >> 1;
      vec_t run = 0.0f;
      if (i < cols) {
        const vec_t* src =
            reinterpret_cast<const vec_t*>(r.part + (b * r.groups * 2 + (bw & 1)) * nl + e);
        vec_t s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
        int64_t g = g0;
#pragma unroll 4
        for (; g + 4 <= g1; g += 4) {
          s0 += src[g * gs];
          s1 += src[(g + 1) * gs];
          s2 += src[(g + 2) * gs];
          s3 += src[(g + 3) * gs];
        }
        for (; g < g1; ++g) s0 += src[g * gs];
        run = (s0 + s1) + (s2 + s3);
      }
      runs[slice][col] = run;
      __syncthreads();
      if (slice == 0 && i < cols) {
        vec_t sum = runs[0][col];
#pragma unroll
        for (int k = 1; k < kSlices; ++k) sum += runs[k][col];
        *reinterpret_cast<vec_t*>(((bw & 1) ? r.dC : r.dB) + b * nl + e) = sum;
      }
      __syncthreads();
    }
  } else {
    const int64_t stride = int64_t(gridDim.x) * 256;
    const int64_t first = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t na = r.dim * r.dstate;
    const int64_t items = na + 2 * r.dim;
    for (int64_t i = first; i < items; i += stride) {
      const float* src;
      float* dst;
      int64_t e, gs;
      if (i < na) {
        src = r.part_dA; dst = r.dA; e = i; gs = na;
      } else if (i < na + r.dim) {
        src = r.part_dD; dst = r.dD; e = i - na; gs = r.dim;
      } else {
        src = r.part_dbias; dst = r.dbias; e = i - na - r.dim; gs = r.dim;
      }
      if (!dst) continue;
      float s = 0.0f;
      for (int64_t b = 0; b < r.seg_rows; ++b) s += src[b * gs + e];
      dst[e] = s;
    }
  }
}

// Up to five float arrays to zero (count 0: skipped); grid.y picks the array.
struct ZeroList {
  float* p[5];
  int64_t n[5];
};

__global__ __launch_bounds__(256) void fill_zero_many_kernel(ZeroList z) {
  float* p = z.p[blockIdx.y];
  const int64_t n = z.n[blockIdx.y];
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

template <typename Elem, int W, int M>
int launch_bwd_typed(const BwdArgs& a, hipStream_t s) {
  BParams p;
  p.u = a.u;
  p.delta = a.delta;
  p.A = a.A;
  p.B = a.B;
  p.C = a.C;
  p.D = a.D;
  p.z = a.z;
  p.bias = a.bias;
  p.ckpt = a.ckpt;
  p.dout = a.dout;
  p.dfinal = a.dfinal;
  p.du = a.du;
  p.ddelta = a.ddelta;
  p.dA = a.dA;
  p.dB = a.dB;
  p.dC = a.dC;
  p.dD = a.dD;
  p.dz = a.dz;
  p.dbias = a.dbias;
  p.dh0 = a.dh0;
  p.mask = a.mask;
  p.dim = int(a.dim);
  p.dstate = int(a.dstate);
  p.seqlen = int(a.seqlen);
  p.dblocks = int((a.dim + 2 * W - 1) / (2 * W));
  p.softplus = a.softplus ? 1 : 0;
  p.n_ckpt = int((a.seqlen + kCkptInterval - 1) / kCkptInterval);
  BwdWorkspace ws{};
  p.partials = a.workspace ? 1 : 0;
  const int64_t nseg = a.workspace ? a.segments : 1;
  const int64_t n_chunks = bwd_intervals(a.seqlen);
  p.nseg = int(nseg);
  p.seg_chunks = int((n_chunks + nseg - 1) / nseg);
  p.wgs = int(a.batch * p.dblocks);
  p.rows = a.batch * a.dim;
  p.cq = nullptr;
  p.cp = nullptr;
  if (nseg < 1 || (nseg > 1 && (nseg - 1) * p.seg_chunks >= n_chunks))
    return int(hipErrorInvalidValue);  // every segment holds at least one interval
  if (a.workspace) {
    if (!bwd_workspace(a.batch, a.dim, a.dstate, a.seqlen, a.io, nseg, &ws) ||
        ws.groups != p.dblocks)
      return int(hipErrorInvalidValue);
    p.dB = a.workspace + ws.part;
    p.dC = nullptr;
    p.dA = a.workspace + ws.dA;
    p.dD = a.dD ? a.workspace + ws.dD : nullptr;
    p.dbias = a.dbias ? a.workspace + ws.dbias : nullptr;
    if (nseg > 1) {
      p.cq = a.workspace + ws.cq;
      p.cp = a.workspace + ws.cp;
    }
  }
  const int64_t blocks = nseg * p.wgs;
  const dim3 grid = dim3(unsigned(blocks)), block = dim3(64 * W);
  if (nseg > 1) {
    // The carry launch: segments 1 .. nseg - 1 (segment 0's carry is never needed), one
    // workgroup per batch row, segment and 2 kCarryWaves channels.
    const int64_t cwgs = a.batch * ((a.dim + 2 * kCarryWaves - 1) / (2 * kCarryWaves));
    const dim3 cgrid = dim3(unsigned((nseg - 1) * cwgs)), cblock = dim3(64 * kCarryWaves);
    if (a.vec_ok) {
      if (a.mask)
        hipLaunchKernelGGL((bwd_carry_scan_kernel<Elem, true, true>), cgrid, cblock, 0, s, p);
      else
        hipLaunchKernelGGL((bwd_carry_scan_kernel<Elem, true, false>), cgrid, cblock, 0, s, p);
    } else {
      if (a.mask)
        hipLaunchKernelGGL((bwd_carry_scan_kernel<Elem, false, true>), cgrid, cblock, 0, s, p);
      else
        hipLaunchKernelGGL((bwd_carry_scan_kernel<Elem, false, false>), cgrid, cblock, 0, s, p);
    }
    int st = int(hipGetLastError());
    if (st != 0) return st;
    const int64_t items = p.rows * a.dstate;
    hipLaunchKernelGGL(bwd_carry_kernel, dim3(unsigned((items + 255) / 256)), dim3(256), 0, s,
                       a.A, a.dfinal, p.cq, p.cp, p.rows, a.dim, int(a.dstate), int(nseg));
    st = int(hipGetLastError());
    if (st != 0) return st;
  }
  if (nseg > 1) {
    if (a.vec_ok) {
      if (a.mask)
        hipLaunchKernelGGL((scan_bwd_kernel<Elem, W, M, true, true, true>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((scan_bwd_kernel<Elem, W, M, true, false, true>), grid, block, 0, s, p);
    } else {
      if (a.mask)
        hipLaunchKernelGGL((scan_bwd_kernel<Elem, W, M, false, true, true>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((scan_bwd_kernel<Elem, W, M, false, false, true>), grid, block, 0, s, p);
    }
  } else if (a.vec_ok) {
    if (a.mask)
      hipLaunchKernelGGL((scan_bwd_kernel<Elem, W, M, true, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((scan_bwd_kernel<Elem, W, M, true, false>), grid, block, 0, s, p);
  } else {
    if (a.mask)
      hipLaunchKernelGGL((scan_bwd_kernel<Elem, W, M, false, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((scan_bwd_kernel<Elem, W, M, false, false>), grid, block, 0, s, p);
  }
  int st = int(hipGetLastError());
  if (st != 0 || !a.workspace) return st;
  RParams r;
  r.part = a.workspace + ws.part;
  r.part_dA = a.workspace + ws.dA;
  r.part_dD = a.workspace + ws.dD;
  r.part_dbias = a.workspace + ws.dbias;
  r.dB = a.dB;
  r.dC = a.dC;
  r.dA = a.dA;
  r.dD = a.dD;        // the C-ABI layer has already cleared it when D is absent
  r.dbias = a.dbias;  // likewise for delta_bias
  r.batch = a.batch;
  r.dim = a.dim;
  r.dstate = a.dstate;
  r.seqlen = a.seqlen;
  r.groups = ws.groups;
  r.seg_rows = nseg * a.batch;
  const bool v4 = (a.dstate * a.seqlen) % 4 == 0 && reinterpret_cast<uintptr_t>(a.dB) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(a.dC) % 16 == 0;
  const int64_t cols = a.batch * 2 * a.dstate * a.seqlen / (v4 ? 4 : 1);
  int64_t gx = (cols + kColumns - 1) / kColumns;
  gx = gx < 1 ? 1 : (gx > 16384 ? 16384 : gx);
  if (v4)
    hipLaunchKernelGGL(bwd_reduce_kernel<4>, dim3(unsigned(gx), 2), dim3(256), 0, s, r);
  else
    hipLaunchKernelGGL(bwd_reduce_kernel<1>, dim3(unsigned(gx), 2), dim3(256), 0, s, r);
  return int(hipGetLastError());
}

}  // namespace

int launch_scan_bwd(const BwdArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.workspace) {  // partial sums, then the reduction launch overwrites every output
    if (a.io == Io::BF16) return launch_bwd_typed<uint16_t, kBwdWavesBf16, kBwdGroup>(a, s);
    return launch_bwd_typed<float, kBwdWavesF32, kBwdGroup>(a, s);
  }
  // Without a workspace the channel- and batch-summed gradients are accumulated with
  // atomics: zero all five in one launch (five small launches cost more than their bytes).
  ZeroList z;
  z.p[0] = a.dA;
  z.n[0] = a.dim * a.dstate;
  z.p[1] = a.dB;
  z.n[1] = a.batch * a.dstate * a.seqlen;
  z.p[2] = a.dC;
  z.n[2] = z.n[1];
  z.p[3] = a.dD;
  z.n[3] = a.dD ? a.dim : 0;
  z.p[4] = a.dbias;
  z.n[4] = a.dbias ? a.dim : 0;
  int64_t most = 0;
  for (int k = 0; k < 5; ++k) most = z.n[k] > most ? z.n[k] : most;
  if (most > 0) {
    int64_t gx = (most + 1023) / 1024;  // about four stores per thread
    gx = gx < 1 ? 1 : (gx > 4096 ? 4096 : gx);
    hipLaunchKernelGGL(fill_zero_many_kernel, dim3(unsigned(gx), 5), dim3(256), 0, s, z);
    const int st = int(hipGetLastError());
    if (st != 0) return st;
  }
  if (a.io == Io::BF16) return launch_bwd_typed<uint16_t, kBwdWavesBf16, kBwdGroup>(a, s);
  return launch_bwd_typed<float, kBwdWavesF32, kBwdGroup>(a, s);
}

}  // namespace ssm
