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
// the later step first. A lane folds its steps from the right into one operator, the wave
// scans those operators from lane 63 down to lane 0, and each lane replays its steps with
// the adjoint entering from its right, forming per step:
//   dC_t += dy_t h_t,  dB_t += g_t s_t u_t  (summed over the workgroup's channels in LDS,
//   then over workgroups: partial sums in a workspace added up in a fixed order by a second
//   launch, or float atomics when there is no workspace), du_t += g_t s_t B_t,
//   ds_t += g_t (A a_t h_{t-1} + B_t u_t), dA += g_t a_t s_t h_{t-1}.
// The mapping is the forward's: a workgroup owns K channels of one batch row, one
// wavefront per channel, and lane i owns T consecutive steps of a 64*T-step interval; the
// intervals are processed last to first, carrying the state adjoint between them.
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
};

// Inclusive scan from the right: lane i ends with the composition of the operators of
// lanes i..63, lane 63 applied first: (a, b) <- (a_i a_j, a_i b_j + b_i) for the lanes j
// to its right.
//   1. Inside each 16-lane row, four Hillis-Steele steps read the lane k to the right with
//      DPP row_shl:k (k = 1, 2, 4, 8); a lane whose source is past the row's end is not
//      written (no bound_ctrl), which is combining with the identity (1, 0).
//   2. Lane 16 r now holds row r's whole operator. The operators of the rows to the right
//      of each row are composed from lanes 16, 32 and 48 (read into scalars) and applied
//      to every lane of the row.
// gfx950 needs two wait states between a VALU write and a DPP read of the same VGPR.
__device__ __forceinline__ void wave_scan_from_right(float& a, float& b, int lane) {
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
      "s_nop 1"
      : "+v"(a), "+v"(b));
  // row operators (rows 1..3), composed from the right
  const float a3 = readlane(a, 48), b3 = readlane(b, 48);
  const float a2 = readlane(a, 32), b2 = readlane(b, 32);
  const float a1 = readlane(a, 16), b1 = readlane(b, 16);
  const float s2a = a3, s2b = b3;                                        // rows 3
  const float s1a = a2 * a3, s1b = __builtin_fmaf(a2, b3, b2);           // rows 2..3
  const float s0a = a1 * s1a, s0b = __builtin_fmaf(a1, s1b, b1);         // rows 1..3
  const int row = lane >> 4;
  float sa = 1.0f, sb = 0.0f;
  sa = (row == 0) ? s0a : sa;
  sb = (row == 0) ? s0b : sb;
  sa = (row == 1) ? s1a : sa;
  sb = (row == 1) ? s1b : sb;
  sa = (row == 2) ? s2a : sa;
  sb = (row == 2) ? s2b : sb;
  b = __builtin_fmaf(a, sb, b);
  a = a * sa;
}

// Lane i receives lane i+1's value; lane 63 receives `last` (DPP wave_shl:1).
__device__ __forceinline__ float shift_down_one(float v, float last) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(last), __float_as_int(v),
                                                    0x130, 0xf, 0xf, false));
}

// Sum over the 64 lanes, in every lane: DPP row_shr partial sums inside each row (lane 15
// of a row ends with the row's sum), then the four row sums.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
  return (readlane(v, 15) + readlane(v, 31)) + (readlane(v, 47) + readlane(v, 63));
}

// Sum over the 64 lanes, complete in lane 63: DPP row_shr partial sums inside each row, then
// row_bcast:15 and row_bcast:31 carry the row totals up (no readlanes).
__device__ __forceinline__ float wave_sum_to_last(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
  return v;
}

__device__ __forceinline__ float sigmoid_f(float x) { return rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

// kMask: read a padding mask (its own instantiation: the unmasked kernel's register count
// decides how many waves fit on a SIMD).
template <typename Elem, int T, int K, bool kVecRows, bool kMask>
__global__ __launch_bounds__(64 * K, 4) void scan_bwd_kernel(BParams p) {
  constexpr int kVec = Vec<Elem>::kN;
  constexpr int kChunk = 64 * T;
  constexpr int kBlocks = T / kVec;
  constexpr uint32_t kEsz = sizeof(Elem);
  // LDS pitch of the per-wave dB/dC rows, [wave][step j][lane]: 72 = 8 (mod 64) words, so
  // the 64 lanes of a flush read (8 steps x 8 lanes) fall on 64 different banks.
  constexpr int kPitch = 72;
  static_assert(kChunk == kCkptInterval, "one interval per saved state");
  static_assert(T % kVec == 0, "whole 16-byte words per lane");

  // [state parity][dB / dC][wave][j * kPitch + lane]: each wave writes its own rows (no
  // atomics); the flush adds the K rows of a step.
  __shared__ float acc[2][2][K][T * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / p.dblocks;
  const int d = (blockIdx.x - b * p.dblocks) * K + wave;
  const bool active = d < p.dim;
  const int N = p.dstate, L = p.seqlen;
  const int n_chunks = (L + kChunk - 1) / kChunk;
  const int64_t row = int64_t(b) * p.dim + (active ? d : 0);

  const uint32_t row_bytes = active ? uint32_t(L) * kEsz : 0u;
  const Buf u_buf(static_cast<const Elem*>(p.u) + row * L, row_bytes);
  const Buf dl_buf(static_cast<const Elem*>(p.delta) + row * L, row_bytes);
  const Buf do_buf(static_cast<const Elem*>(p.dout) + row * L, row_bytes);
  const Buf z_buf(static_cast<const Elem*>(p.z ? p.z : p.u) + row * L, p.z ? row_bytes : 0u);
  const Buf du_buf(static_cast<Elem*>(p.du) + row * L, row_bytes);
  const Buf dd_buf(static_cast<Elem*>(p.ddelta) + row * L, row_bytes);
  const Buf dz_buf(static_cast<Elem*>(p.z ? p.dz : p.du) + row * L, p.z ? row_bytes : 0u);
  const uint32_t bc_elems = uint32_t(N) * uint32_t(L);
  const Buf B_buf(static_cast<const Elem*>(p.B) + int64_t(b) * N * L, bc_elems * kEsz);
  const Buf C_buf(static_cast<const Elem*>(p.C) + int64_t(b) * N * L, bc_elems * kEsz);

  // Per-state values live in lane n of these registers.
  float A_l = 0.0f, gc_l = 0.0f, dA_l = 0.0f, Dd = 0.0f, bias_d = 0.0f;
  if (active) {
    Dd = p.D ? p.D[d] : 0.0f;
    bias_d = p.bias ? p.bias[d] : 0.0f;
    if (lane < N) {
      A_l = p.A[int64_t(d) * N + lane];
      if (p.dfinal) gc_l = p.dfinal[row * N + lane];  // e_{L-1} = dfinal
    }
  }
  const float a2_l = A_l * kLog2e;
  float dD_acc = 0.0f, db_acc = 0.0f;
  // Where the flush adds this workgroup's dB and dC rows: this batch row of the outputs, or
  // this workgroup's slot of partial sums. Both take the same offset (state, step) after it.
  const int64_t nl = int64_t(N) * L;
  float* const flush0 = p.partials ? p.dB + int64_t(blockIdx.x) * 2 * nl : p.dB + b * nl;
  float* const flush1 = p.partials ? flush0 + nl : p.dC + b * nl;

  {
    // rows of inactive waves are read by the flush: they stay zero
    float* flat = &acc[0][0][0][0];
    for (int i = tid; i < 2 * 2 * K * T * kPitch; i += 64 * K) flat[i] = 0.0f;
  }
  __syncthreads();

  // B or C words of state n for this lane's steps (zeros past the end of the sequence).
  auto load_bc = [&](const Buf& buf, int n, int tb, float (&v)[T]) {
#pragma unroll
    for (int q = 0; q < kBlocks; ++q) {
      const int t0 = tb + q * kVec;
      const uint32_t e = (t0 < L) ? uint32_t(n) * uint32_t(L) + uint32_t(t0) : bc_elems;
      widen_raw16<Elem>(load_word<Elem, kVecRows>(buf, e), &v[q * kVec]);
    }
  };

  int it = 0;  // states processed so far: selects the LDS buffer
  for (int c = n_chunks - 1; c >= 0; --c) {
    const int tb = c * kChunk + lane * T;
    float uv[T], sv[T], xv[T], dyv[T], gdu[T], gds[T];
    float sdt = 0.0f;
    uint32_t pad_bits = 0;  // bit j: step tb + j is padding (masked kernels only)
    {
      float dov[T], zv[T];
#pragma unroll
      for (int q = 0; q < kBlocks; ++q) {
        const uint32_t e = uint32_t(tb + q * kVec);
        widen_raw16<Elem>(load_word<Elem, kVecRows>(u_buf, e), &uv[q * kVec]);
        widen_raw16<Elem>(load_word<Elem, kVecRows>(dl_buf, e), &xv[q * kVec]);
        widen_raw16<Elem>(load_word<Elem, kVecRows>(do_buf, e), &dov[q * kVec]);
        widen_raw16<Elem>(load_word<Elem, kVecRows>(z_buf, e), &zv[q * kVec]);
      }
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const float x = xv[j] + bias_d;
        float s = p.softplus ? softplus_f(x) : x;
        if (tb + j >= L) s = uv[j] = dov[j] = 0.0f;  // past the end: identity steps
        if constexpr (kMask) {
          if (tb + j < L && p.mask[int64_t(b) * L + tb + j] == 0) {
            s = 0.0f;  // padding: the state is kept (the step is the identity)
            pad_bits |= 1u << j;
          }
        }
        sv[j] = s;
        sdt += s;
        dyv[j] = dov[j];
      }
      const float hc_l = (active && lane < N) ? p.ckpt[(row * p.n_ckpt + c) * N + lane] : 0.0f;

      // With the gate, dL/dy = dout z sigmoid(z) does not need y; only dL/dz does, and y
      // (before the gate) is summed over the states in the loop below, which recomputes
      // every h_t anyway. dout, z and the biased step size are read again after the loop
      // (from L2) rather than kept live across it.
      float y[T];
#pragma unroll
      for (int j = 0; j < T; ++j) y[j] = Dd * uv[j];
      if (p.z) {
#pragma unroll
        for (int j = 0; j < T; ++j) dyv[j] = dov[j] * zv[j] * sigmoid_f(zv[j]);
      }
#pragma unroll
      for (int j = 0; j < T; ++j) {
        dD_acc = __builtin_fmaf(dyv[j], uv[j], dD_acc);
        gdu[j] = 0.0f;  // sum over states of g B (du and the step size share it)
        gds[j] = 0.0f;  // sum over states of g A a h_{t-1}
      }

      for (int n = 0; n < N; ++n) {
        const int par = it & 1;
        if (active) {
          const float a2 = readlane(a2_l, n), An = readlane(A_l, n);
          const float hc = readlane(hc_l, n), G = readlane(gc_l, n);
          float Bv[T], Cv[T], dA[T], h[T];
          load_bc(B_buf, n, tb, Bv);
          load_bc(C_buf, n, tb, Cv);
          // forward again from the saved state: h_t for this lane's steps
          float bseg = (lane == 0) ? hc : 0.0f;
#pragma unroll
          for (int j = 0; j < T; ++j) {
            dA[j] = exp2_hw(sv[j] * a2);
            bseg = __builtin_fmaf(dA[j], bseg, (sv[j] * uv[j]) * Bv[j]);
          }
          const float alpha = exp2_hw(sdt * a2);  // product of the lane's a_t
          float aseg = alpha;
          wave_scan_inclusive(aseg, bseg);
          const float hin = shift_up_one(bseg, hc);  // state entering the lane's steps
          {
            float hh = hin;
#pragma unroll
            for (int j = 0; j < T; ++j) {
              hh = __builtin_fmaf(dA[j], hh, (sv[j] * uv[j]) * Bv[j]);
              h[j] = hh;
              y[j] = __builtin_fmaf(Cv[j], hh, y[j]);  // read only with a gate; a select
                                                       // per step would cost more
            }
          }
          // adjoint: fold the lane's steps from the right, scan from lane 63 down
          float beta = 0.0f;
#pragma unroll
          for (int j = T - 1; j >= 0; --j) beta = dA[j] * __builtin_fmaf(Cv[j], dyv[j], beta);
          float ra = alpha, rb = beta;
          wave_scan_from_right(ra, rb, lane);
          // lane 63's right neighbour is the next interval: the identity applied to G
          const float an = shift_down_one(ra, 1.0f), bn = shift_down_one(rb, 0.0f);
          float v = __builtin_fmaf(an, G, bn);  // e entering from the right
          const float G_next = __builtin_fmaf(readlane(ra, 0), G, readlane(rb, 0));
          gc_l = (lane == n) ? G_next : gc_l;
          float dAn = 0.0f;
#pragma unroll
          for (int j = T - 1; j >= 0; --j) {
            const float g = __builtin_fmaf(Cv[j], dyv[j], v);  // g_t = C_t dy_t + e_{t+1}
            const float hp = (j > 0) ? h[j - 1] : hin;
            const float t1 = dA[j] * hp;
            acc[par][0][wave][j * kPitch + lane] = g * (sv[j] * uv[j]);  // dB
            acc[par][1][wave][j * kPitch + lane] = dyv[j] * h[j];        // dC
            const float q = g * t1;
            gdu[j] = __builtin_fmaf(g, Bv[j], gdu[j]);
            gds[j] = __builtin_fmaf(q, An, gds[j]);
            dAn = __builtin_fmaf(q, sv[j], dAn);
            v = dA[j] * g;  // e_t = a_t g_t
          }
          dAn = readlane(wave_sum_to_last(dAn), 63);
          dA_l = (lane == n) ? dA_l + dAn : dA_l;
        }
        __syncthreads();  // every channel's share of state n is in acc[par]
        // Add the workgroup's sums for state n into dB and dC: one (gradient, step) item per
        // thread and pass, dB items first (whole waves take the same gradient). The buffer is
        // written again two states later, after the next barrier, which no thread passes
        // before finishing this loop. Every active wave overwrites its rows for every state;
        // inactive waves' rows stay zero.
        for (int i = tid; i < 2 * kChunk; i += 64 * K) {
          const int wc = i >= kChunk ? 1 : 0;  // 0: dB, 1: dC
          const int st = i - wc * kChunk;
          const int ln = st / T, j = st - ln * T;
          const int t = c * kChunk + st;
          float v = 0.0f;
#pragma unroll 4  // fully unrolled, the K loads in flight would push past 128 registers
          for (int k = 0; k < K; ++k) v += acc[par][wc][k][j * kPitch + ln];
          if (t < L) {
            float* dst = (wc ? flush1 : flush0) + (int64_t(n) * L + t);
            if (p.partials)
              *dst = v;
            else
              unsafeAtomicAdd(dst, v);
          }
        }
        ++it;
      }
      // du_t = s_t sum_n g B + D dy_t and ds_t = sum_n g (A a h_{t-1} + B u_t), from the two
      // sums over the states.
#pragma unroll
      for (int j = 0; j < T; ++j) {
        gds[j] = __builtin_fmaf(uv[j], gdu[j], gds[j]);
        gdu[j] = __builtin_fmaf(sv[j], gdu[j], Dd * dyv[j]);
      }
      if (p.z) {
        float dz2[T], zz[T];
#pragma unroll
        for (int q = 0; q < kBlocks; ++q) {
          const uint32_t e = uint32_t(tb + q * kVec);
          widen_raw16<Elem>(load_word<Elem, kVecRows>(do_buf, e), &dz2[q * kVec]);
          widen_raw16<Elem>(load_word<Elem, kVecRows>(z_buf, e), &zz[q * kVec]);
        }
#pragma unroll
        for (int j = 0; j < T; ++j) {
          const float sg = sigmoid_f(zz[j]);
          dz2[j] = dz2[j] * y[j] * sg * __builtin_fmaf(zz[j], 1.0f - sg, 1.0f);
        }
        store_lane_block<Elem, kVecRows, T>(dz_buf, uint32_t(tb), dz2);
      }
    }
    float dd[T];
    if (p.softplus) {  // the raw step size again (from L2), for softplus' derivative
#pragma unroll
      for (int q = 0; q < kBlocks; ++q)
        widen_raw16<Elem>(load_word<Elem, kVecRows>(dl_buf, uint32_t(tb + q * kVec)),
                          &xv[q * kVec]);
    }
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const float x = xv[j] + bias_d;
      dd[j] = p.softplus ? gds[j] * sigmoid_f(x) : gds[j];
      if constexpr (kMask) {
        if (pad_bits & (1u << j)) dd[j] = 0.0f;  // a padding step's step size is not used
      }
      if (tb + j < L) db_acc += dd[j];
    }
    store_lane_block<Elem, kVecRows, T>(du_buf, uint32_t(tb), gdu);
    store_lane_block<Elem, kVecRows, T>(dd_buf, uint32_t(tb), dd);
  }

  if (active) {
    if (lane < N) {
      if (p.dh0) p.dh0[row * N + lane] = gc_l;  // e_{-1} = a_0 g_0
      if (p.partials)
        p.dA[row * N + lane] = dA_l;
      else
        unsafeAtomicAdd(&p.dA[int64_t(d) * N + lane], dA_l);
    }
    const float sD = wave_sum(dD_acc), sb = wave_sum(db_acc);
    if (lane == 0) {
      if (p.partials) {
        if (p.dD) p.dD[row] = sD;
        if (p.dbias) p.dbias[row] = sb;
      } else {
        if (p.dD) unsafeAtomicAdd(&p.dD[d], sD);
        if (p.dbias) unsafeAtomicAdd(&p.dbias[d], sb);
      }
    }
  }
}

// The second launch of a backward with a workspace: every summed gradient is the sum of its
// partials in a fixed order (no atomics). grid.y = 0: dB and dC, element (b, n, t) summed
// over the batch row's workgroups; grid.y = 1: dA, dD and dbias summed over batch rows.
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
      for (int64_t b = 0; b < r.batch; ++b) s += src[b * gs + e];
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

template <typename Elem, int T, int K>
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
  p.dblocks = int((a.dim + K - 1) / K);
  p.softplus = a.softplus ? 1 : 0;
  p.n_ckpt = int((a.seqlen + kCkptInterval - 1) / kCkptInterval);
  BwdWorkspace ws{};
  p.partials = a.workspace ? 1 : 0;
  if (a.workspace) {
    if (!bwd_workspace(a.batch, a.dim, a.dstate, a.seqlen, a.io, &ws) || ws.groups != p.dblocks)
      return int(hipErrorInvalidValue);
    p.dB = a.workspace + ws.part;
    p.dC = nullptr;
    p.dA = a.workspace + ws.dA;
    p.dD = a.dD ? a.workspace + ws.dD : nullptr;
    p.dbias = a.dbias ? a.workspace + ws.dbias : nullptr;
  }
  const int64_t blocks = a.batch * p.dblocks;
  const dim3 grid = dim3(unsigned(blocks)), block = dim3(64 * K);
  if (a.vec_ok) {
    if (a.mask)
      hipLaunchKernelGGL((scan_bwd_kernel<Elem, T, K, true, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((scan_bwd_kernel<Elem, T, K, true, false>), grid, block, 0, s, p);
  } else {
    if (a.mask)
      hipLaunchKernelGGL((scan_bwd_kernel<Elem, T, K, false, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((scan_bwd_kernel<Elem, T, K, false, false>), grid, block, 0, s, p);
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
    if (a.io == Io::BF16) return launch_bwd_typed<uint16_t, 8, kBwdChannelsBf16>(a, s);
    return launch_bwd_typed<float, 8, kBwdChannelsF32>(a, s);
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
  // bf16: 16 channels per workgroup, half the dB/dC atomics of 8 at the same 4 waves per SIMD
  // (one 16-wave workgroup per CU; its per-wave rows take 144 KB of LDS). fp32 keeps 8: at
  // 16 its masked kernel spills past 128 registers.
  if (a.io == Io::BF16) return launch_bwd_typed<uint16_t, 8, kBwdChannelsBf16>(a, s);
  return launch_bwd_typed<float, 8, kBwdChannelsF32>(a, s);
}

}  // namespace ssm
