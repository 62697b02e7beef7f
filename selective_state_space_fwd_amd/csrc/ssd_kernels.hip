// Mamba-2 (SSD) forward on the gfx950 matrix cores.
//
// Mamba-2 keeps the selective recurrence but makes A one scalar per head
// (ybb.press/ai-applications/14118.html, section 2.2). Unrolled, the recurrence of one head
// is one lower-triangular (semiseparable) matrix applied to the head's channels
// (mhpq.cn/news/1077344, section 5.1); cut into blocks, the part inside a block is a
// matrix product and the blocks are joined by a scan of block-end states (same page,
// section 5.2). With cs_t the running sum of a_r = dt_r A over the block (r <= t):
//
//   y_t   = sum_{s<=t} (C_t . B_s) exp(cs_t - cs_s) dt_s x_s      (inside the block)
//         + exp(cs_t) C_t . H_in                                  (the carried state)
//   H_out = exp(cs_end) H_in + sum_s exp(cs_end - cs_s) dt_s B_s x_s^T
//
// Where a block's decay span -cs_end is moderate, exp(cs_t - cs_s) factors as
// exp(cs_t - ref) exp(ref - cs_s) (ref = cs_end / 2), and the block-diagonal part becomes
// exp(cs_t - ref) ((G o L) xs) with xs_s = exp(ref - cs_s) dt_s x_s and L the causal mask:
// no per-head block matrix is formed, and xs is the operand the state update needs too.
// Blocks of larger span use M = G o exp(cs_t - cs_s) o dt_s directly.
//
// Two launches:
//   ssd_prep_kernel: per (batch row, 64-step block), G o L with G = C^T B (MFMA over the
//     states, stored bf16) and C^T in the lane order and swizzle the block kernels' operands
//     use, shared by every head; and per (batch row, head, block), a record of the step
//     sizes, their running sums and the per-step factors (ssd_step_record).
//   ssd_chunk_kernel (up to 128 states) or ssd_fwd_kernel (256 states), one workgroup per
//     (batch row, head, 32 channels), blocks in order: per wave y = the carried state read
//     through C plus the block-diagonal product (MFMA), the D skip and gate, and the state
//     update H_out = exp(cs_end) H_in + B (w o x) (MFMA). Wherever the fp32 state or a value
//     that feeds it is an MFMA operand (H_in in the carried-state product, w o x in the
//     update), it enters as two bf16 halves, hi + lo, which keeps fp32-level accuracy.
//
// Wave layout: 2 channel blocks of 16 x kNS splits of the states (kNS = 4 for 128 states:
// 8 waves, two per SIMD; 2 otherwise). A wave holds its slice of H as MFMA accumulators.
// ssd_chunk_kernel hands the slices to every wave through LDS once per block, so each wave
// forms whole output tiles and a block needs one barrier; ssd_fwd_kernel (whose two B and
// C^T stages alone fill 128 KB of LDS at 256 states) splits the carried-state product over
// the states and sums partial outputs through LDS instead.
//
// Data movement: the next block's B and C^T (and, up to 128 states, G, x and z) travel by
// buffer-to-LDS DMA into a second stage while the current block computes, so that the
// CU's vector memory path works in the background instead of stalling every wave at one
// point.
//
// MFMA v_mfma_f32_16x16x32_bf16 lane layout (checked on the device): lane l, r = l % 16,
// g = l / 16: A operand row r, k = 8g..8g+7; B operand column r, the same k; result rows
// 4g..4g+3 of column r. The k order inside a 32-wide block is free as long as both operands
// agree, which lets H (in result layout) feed the carried-state product directly: its
// lanes hold states {4g..4g+3, 16+4g..16+4g+3} of each 32-state block, and the prep kernel
// writes C^T in that same order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_math.h"
#include "device_scan.h"
#include "scan_launch.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kQ = kSsdBlock;          // steps per block
constexpr int kMPitch = kQ + 8;        // bf16 per row of the block matrix in LDS
constexpr uint32_t kOob = 0x80000000u;  // a byte offset past every buffer: loads read 0
// Largest decay span -cs_end of a block (natural log units) that takes the separable form:
// its two factors then stay within exp(+-60).
constexpr float kSepSpan = 120.0f;

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 loads through a buffer resource (byte offsets; past the end they read 0).
__device__ __forceinline__ float4 ld_f4(const Buf& b, uint32_t off) {
  return __builtin_bit_cast(float4, b.load16(off));
}
__device__ __forceinline__ float ld_f1(const Buf& b, uint32_t off) {
  return __uint_as_float(b.load4(off));
}

// 8 consecutive bf16 of a row (elements [row + t, row + t + 8)); elements at or past len
// read 0. With kVec rows hold whole 16-byte words, so a word is wholly in or past the row.
template <bool kVec>
__device__ __forceinline__ uint4 load8(const Buf& buf, uint32_t row, int t, int len) {
  if constexpr (kVec) {
    return buf.load16(t < len ? 2u * (row + uint32_t(t)) : kOob);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = t + 2 * k;
      const uint32_t lo = buf.load2(e < len ? 2u * (row + uint32_t(e)) : kOob);
      const uint32_t hi = buf.load2(e + 1 < len ? 2u * (row + uint32_t(e) + 1) : kOob);
      w[k] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// 4 consecutive bf16 (t a multiple of 4).
template <bool kVec>
__device__ __forceinline__ uint2 load4(const Buf& buf, uint32_t row, int t, int len) {
  if constexpr (kVec) {
    return buf.load8(t < len ? 2u * (row + uint32_t(t)) : kOob);
  } else {
    uint32_t w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = t + 2 * k;
      const uint32_t lo = buf.load2(e < len ? 2u * (row + uint32_t(e)) : kOob);
      const uint32_t hi = buf.load2(e + 1 < len ? 2u * (row + uint32_t(e) + 1) : kOob);
      w[k] = lo | (hi << 16);
    }
    return make_uint2(w[0], w[1]);
  }
}

// Stores of 4 consecutive bf16; elements at or past len (or all, when !on) go to an offset
// past the buffer, where the hardware drops them. Branch-free, so the compiler's count of
// outstanding memory operations stays exact.
template <bool kVec>
__device__ __forceinline__ void store4(const Buf& buf, uint32_t row, int t, int len, bool on,
                                       const float (&v)[4]) {
  const uint2 w = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  if constexpr (kVec) {
    buf.store8(w, (on && t < len) ? 2u * (row + uint32_t(t)) : kOob);
  } else {
    const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint16_t h = uint16_t(ws[k >> 1] >> (16 * (k & 1)));
      buf.store2(h, (on && t + k < len) ? 2u * (row + uint32_t(t + k)) : kOob);
    }
  }
}

// Inclusive sum across the 64 lanes (lane 0 first): DPP row_shr inside 16-lane rows, then
// the row totals through readlanes.
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
  const float r0 = readlane(v, 15), r1 = readlane(v, 31), r2 = readlane(v, 47);
  const int row = int(threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0.0f) + (row >= 2 ? r1 : 0.0f) + (row >= 3 ? r2 : 0.0f);
}

// XOR swizzle of the 16-byte words of a C^T row in the LDS stage, so that the 16 rows an
// MFMA operand read touches fall in distinct bank groups (rows of 256 B or more: 16
// distinct words; rows of 128 B: pairs of rows share a word but not a half).
template <int N>
__device__ __forceinline__ int ct_swizzle(int t) {
  return N >= 128 ? (t & 15) : ((t >> 1) & 7);
}

// The same for 128-byte rows of 64 steps (B, x and z in their LDS stages): word w of row n
// sits in slot w ^ row_swizzle(n).
__device__ __forceinline__ int row_swizzle(int n) { return (n >> 1) & 7; }

// The hardware deals workgroups out to the eight XCDs round-robin (workgroup i to XCD
// i % 8). Renumbering them so that each XCD holds a contiguous range of logical indices
// puts the workgroups of one batch row, which share G, C^T and B, on as few XCDs (and L2s)
// as possible.
__device__ __forceinline__ int xcd_order(int lin, int n) {
  const int per = n / 8;
  return lin < 8 * per ? (lin % 8) * per + lin / 8 : lin;
}

struct SsdParams {
  const uint16_t* x;
  const uint16_t* dt;
  const float* A;
  const uint16_t* B;
  const uint16_t* C;
  const float* D;
  const uint16_t* z;
  const float* dt_bias;
  const uint8_t* mask;
  uint16_t* out;
  float* final_state;
  uint16_t* G;       // [batch, nblocks, 64, 64] bf16, G o L, rows swizzled
  uint16_t* CTp;     // [batch, nblocks, 64, dstate], states in operand order, swizzled
  float* steps;      // [batch, nheads, nblocks, 4, 64]: w, e, cs, dt of every step
  int nheads, headdim, seqlen, nblocks;
  int softplus, initial_state;
};

// ---------------------------------------------------------------- step sizes of every head

// One wave per record (batch row, head, block), lane = step: the step size dt_t (bias, softplus,
// zero at padding and past the end), its running sum cs_t over the block (a_r = dt_r A),
// and the per-step factors the block kernel applies, written as one 1 KB record
// [w | e | cs | dt] of 64 fp32 each. With ref = cs_end / 2 when the block's decay span
// -cs_end is at most kSepSpan (the separable form) and ref = cs_end otherwise:
//   w_s = exp(ref - cs_s) dt_s        (scales x_s for the state update and the block product)
//   e_t = exp(cs_t - ref) (separable) or exp(cs_t)      (the output factor)
__device__ __forceinline__ void ssd_step_record(const SsdParams& p, int64_t rec) {
  const int l = threadIdx.x & 63, L = p.seqlen;
  const int c = int(rec % p.nblocks);
  const int h = int((rec / p.nblocks) % p.nheads);
  const int64_t b = rec / (int64_t(p.nblocks) * p.nheads);
  const int t = c * kQ + l;
  const bool in = t < L;
  const uint16_t* dtrow = p.dt + (b * p.nheads + h) * L;
  float s = in ? bf16_lo(dtrow[t]) : 0.0f;
  s += p.dt_bias ? p.dt_bias[h] : 0.0f;
  s = p.softplus ? softplus_f(s) : s;
  const bool live = in && (p.mask == nullptr || p.mask[b * L + t] != 0);
  s = live ? s : 0.0f;
  const float cs = wave_prefix_sum(s * p.A[h]);
  const float cs_end = readlane(cs, 63);
  const bool sep = cs_end >= -kSepSpan;
  const float ref = sep ? 0.5f * cs_end : cs_end;
  float* out = p.steps + rec * (4 * kQ);
  out[l] = exp2_hw((ref - cs) * kLog2e) * s;
  out[kQ + l] = exp2_hw((cs - (sep ? ref : 0.0f)) * kLog2e);
  out[2 * kQ + l] = cs;
  out[3 * kQ + l] = s;
}

// ---------------------------------------------------------------- prep: G and C^T

// Workgroups [0, n_prep) take one (batch row, block) each; the ones after them take four
// step records each (one per wave), so the two kinds of work share one launch.
template <int N, bool kVec>
__global__ __launch_bounds__(256) void ssd_prep_kernel(SsdParams p, int n_prep, int64_t records) {
  constexpr int kPitch = N + 8;  // bf16 per LDS row
  __shared__ __attribute__((aligned(16))) uint16_t ct[kQ][kPitch];  // C^T of the block
  __shared__ __attribute__((aligned(16))) uint16_t bt[kQ][kPitch];  // B^T of the block
  if (int(blockIdx.x) >= n_prep) {
    const int64_t rec = int64_t(int(blockIdx.x) - n_prep) * 4 + (threadIdx.x >> 6);
    if (rec < records) ssd_step_record(p, rec);
    return;
  }
  const int logical = xcd_order(blockIdx.x, n_prep);  // one batch row's blocks together
  const int c = logical % p.nblocks, b = logical / p.nblocks, L = p.seqlen, t0 = c * kQ;
  const uint32_t bc_bytes = uint32_t(N) * uint32_t(L) * 2u;
  const Buf cbuf(p.C + size_t(b) * N * L, bc_bytes), bbuf(p.B + size_t(b) * N * L, bc_bytes);

  // Transpose the block's B and C into LDS: thread -> (states n, n + 1; steps 8 q .. + 7).
  // Each step's two states go in as one 32-bit write, and consecutive lanes take
  // consecutive state pairs, so one write instruction covers consecutive words of one row:
  // no bank conflicts. (Lanes on the same state pair would write rows 8 apart, 2 176 bytes,
  // all on one bank.) The 16-byte loads then come from different rows; the other step
  // groups of each 128-byte row are read by the neighbouring waves, from L2.
  for (int idx = threadIdx.x; idx < N * 4; idx += 256) {
    const int n = 2 * (idx % (N / 2)), q = idx / (N / 2);
    const uint4 c0 = load8<kVec>(cbuf, uint32_t(n) * L, t0 + 8 * q, L);
    const uint4 c1 = load8<kVec>(cbuf, uint32_t(n + 1) * L, t0 + 8 * q, L);
    const uint4 b0 = load8<kVec>(bbuf, uint32_t(n) * L, t0 + 8 * q, L);
    const uint4 b1 = load8<kVec>(bbuf, uint32_t(n + 1) * L, t0 + 8 * q, L);
    const uint32_t vc0[4] = {c0.x, c0.y, c0.z, c0.w}, vc1[4] = {c1.x, c1.y, c1.z, c1.w};
    const uint32_t vb0[4] = {b0.x, b0.y, b0.z, b0.w}, vb1[4] = {b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // step 8 q + 2 k: the low halves of state n's and state n + 1's words; step + 1: the
      // high halves (v_perm_b32 selector bytes: result = {hi-or-lo of src1, of src0})
      *reinterpret_cast<uint32_t*>(&ct[8 * q + 2 * k][n]) =
          __builtin_amdgcn_perm(vc1[k], vc0[k], 0x05040100u);
      *reinterpret_cast<uint32_t*>(&ct[8 * q + 2 * k + 1][n]) =
          __builtin_amdgcn_perm(vc1[k], vc0[k], 0x07060302u);
      *reinterpret_cast<uint32_t*>(&bt[8 * q + 2 * k][n]) =
          __builtin_amdgcn_perm(vb1[k], vb0[k], 0x05040100u);
      *reinterpret_cast<uint32_t*>(&bt[8 * q + 2 * k + 1][n]) =
          __builtin_amdgcn_perm(vb1[k], vb0[k], 0x07060302u);
    }
  }
  __syncthreads();

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 15, g = l >> 4;
  // G[t][s] = sum_n C[n][t] B[n][s] for s <= t, 0 above the diagonal: wave w takes rows
  // 16w..16w+15 (bf16, rows of 8 words, word q of row t in slot q ^ row_swizzle(t)).
  uint16_t* G = p.G + (size_t(b) * p.nblocks + c) * (kQ * kQ);
#pragma unroll
  for (int sj = 0; sj < kQ / 16; ++sj) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < N / 32; ++kb) {
      const uint4 a = *reinterpret_cast<const uint4*>(&ct[16 * w + r][32 * kb + 8 * g]);
      const uint4 bv = *reinterpret_cast<const uint4*>(&bt[16 * sj + r][32 * kb + 8 * g]);
      acc = mfma16(a, bv, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * w + 4 * g + i, sc = 16 * sj + r;
      const float v = sc <= t ? acc[i] : 0.0f;  // causal: zero above the diagonal
      G[t * kQ + 8 * ((sc >> 3) ^ row_swizzle(t)) + (sc & 7)] = uint16_t(pack_bf16x2(v, 0.0f));
    }
  }

  // C^T with the states of each 32-block in operand order (position 8g' + j holds state
  // 4g' + j for j < 4, 16 + 4g' + j - 4 for j >= 4), its 16-byte words XOR-swizzled per
  // row as the main kernel's LDS stage expects, so the stage is a linear copy.
  uint16_t* CT = p.CTp + (size_t(b) * p.nblocks + c) * (kQ * N);
  for (int idx = threadIdx.x; idx < kQ * N / 8; idx += 256) {
    const int t = idx / (N / 8), slot = idx % (N / 8);
    const int q = slot ^ ct_swizzle<N>(t), kb = q >> 2, gg = q & 3;
    const uint2 lo = *reinterpret_cast<const uint2*>(&ct[t][32 * kb + 4 * gg]);
    const uint2 hi = *reinterpret_cast<const uint2*>(&ct[t][32 * kb + 16 + 4 * gg]);
    *reinterpret_cast<uint4*>(&CT[t * N + 8 * slot]) = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// ---------------------------------------------------------------- the block scan, 256 states

// The launcher runs ssd_fwd_kernel for 256 states only (ssd_chunk_kernel below takes 64 and
// 128); its layout still covers every size. States split across waves: 128 states in
// quarters (8 waves, two per SIMD); 64 states in halves (a quarter would be 16, below the
// 32-deep MFMA); 256 states in halves (its two B and C^T stages alone fill 128 KB of LDS).
// It computes its step sizes itself rather than reading the step records.
template <int N>
struct StateSplit {
  static constexpr int kNS = N == 128 ? 4 : 2;
  // G, x and z staged in LDS as well (up to 128 states); at 256 they are register loads.
  static constexpr bool kStageAll = N <= 128;
};

// Per-lane loads of one block, issued a block ahead of their use into one of two register
// sets (the block loop is unrolled by two, so the sets alternate without copies).
template <int N, bool kVec, int kNS, bool kStageAll>
struct LaneLoads {
  static constexpr int kWaves = 2 * kNS;                  // 2 channel blocks x kNS state splits
  static constexpr int kEPT = kQ * kQ / (64 * kWaves);    // block-matrix entries per thread
  static constexpr int kOwn = 4 / kNS;                    // 16-step output tiles per wave
  static constexpr int kBInstr = N / 8 / kWaves;          // 1 KB copies of B (and of C^T)
  // dt and the mask byte stay narrow until use: widening them where they are loaded
  // would make the loop carry wait for them (and every memory operation before them).
  uint16_t dt;
  uint8_t live;
  // register path (kStageAll false)
  uint4 g[kStageAll ? 1 : kEPT / 8];       // bf16 G[t][s0 .. s0+kEPT)
  uint4 xo[kStageAll ? 1 : 2];             // x operands: channel r, steps 32kb + 8g .. +7
  uint2 xe[kStageAll ? 1 : kOwn], ze[kStageAll ? 1 : kOwn];  // x, z at the output positions
  // element-wise path (kVec false): words gathered through registers for the LDS stages
  uint4 bst[kVec ? 1 : kBInstr];
  uint4 xst[kWaves == 8 ? 1 : 2];
};

template <int N, bool kVec, int kNS>
__global__ __launch_bounds__(128 * kNS) void ssd_fwd_kernel(SsdParams p) {
  constexpr bool kStageAll = StateSplit<N>::kStageAll;
  using LL = LaneLoads<N, kVec, kNS, kStageAll>;
  constexpr int kWaves = LL::kWaves;
  constexpr int kNW = N / kNS;                     // states per wave
  constexpr int kNT = kNW / 16, kKB = kNW / 32;    // its 16-state tiles and 32-state k-blocks
  constexpr int kOwn = LL::kOwn, kEPT = LL::kEPT, kBInstr = LL::kBInstr;
  constexpr int kGInstr = 8 / kWaves;              // 1 KB copies of G per wave (kStageAll)
  constexpr int kRowWords = N / 8;                 // 16-byte words per C^T row
  static_assert(kKB >= 1 && kBInstr >= 1 && kEPT % 8 == 0, "unsupported split");
  static_assert(kWaves == 4 || kWaves == 8, "x and z copies assume 4 or 8 waves");
  // LDS: two stages, each array of each stage its own variable and every access to it
  // static: the compiler then knows that reading one stage does not wait for the DMA
  // filling the other. B: N x 64 bf16 (row = 8 words); C^T: 64 x N; G: 64 x 64 bf16;
  // x, z: 32 channels x 64 steps.
  constexpr int kXW = kStageAll ? 32 * 8 : 1, kGW = kStageAll ? kQ * 8 : 1;
  __shared__ __attribute__((aligned(16))) uint4 sB0[N * 8], sB1[N * 8];
  __shared__ __attribute__((aligned(16))) uint4 sCT0[kQ * kRowWords], sCT1[kQ * kRowWords];
  __shared__ __attribute__((aligned(16))) uint4 sG0[kGW], sG1[kGW];
  __shared__ __attribute__((aligned(16))) uint4 sXZ0[2 * kXW], sXZ1[2 * kXW];  // x rows, z rows
  __shared__ __attribute__((aligned(16))) float s_dt[2][kQ], s_cs[2][kQ], s_wdt[2][kQ];
  __shared__ __attribute__((aligned(16))) uint16_t sM[kQ][kMPitch];
  __shared__ f32x4 sY[kWaves][4][64];  // partial carried-state products, every step tile

  // The wave index as a scalar: branches and offsets on it stay wave-uniform.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
  const int pb = w & 1, nq = w >> 1;       // channel block, state split
  const int pgroups = (p.headdim + 31) / 32;
  const int logical = xcd_order(blockIdx.x, gridDim.x);
  const int pg = logical % pgroups, h = (logical / pgroups) % p.nheads;
  const int b = logical / (pgroups * p.nheads);
  const int P = p.headdim, L = p.seqlen, dim = p.nheads * P;
  const int p0 = pg * 32 + pb * 16;        // first channel (within the head) of this wave
  const bool wave_on = p0 < P;             // headdim % 32 == 16 leaves one block idle
  const int d = h * P + p0 + r;            // this lane's channel (operand column)
  const int xr = pb * 16 + r;              // its row in the x and z stages
  // This wave finishes step tiles nq, nq + kNS, ...: with 4 splits one each, with 2 splits
  // tiles {nq, nq + 2}, 3 of the 6 causal block products either way.

  const uint32_t row_bytes = uint32_t(dim) * uint32_t(L) * 2u;
  const Buf xbuf(p.x + size_t(b) * dim * L, row_bytes);
  const Buf zbuf(p.z ? p.z + size_t(b) * dim * L : p.x, p.z ? row_bytes : 0u);
  const Buf obuf(p.out + size_t(b) * dim * L, row_bytes);
  const Buf bbuf(p.B + size_t(b) * N * L, uint32_t(N) * uint32_t(L) * 2u);
  const Buf dtbuf(p.dt + (size_t(b) * p.nheads + h) * L, uint32_t(L) * 2u);
  const Buf mbuf(p.mask ? p.mask + size_t(b) * L : nullptr, p.mask ? uint32_t(L) : 0u);
  const Buf ctbuf(p.CTp + size_t(b) * p.nblocks * (kQ * N), uint32_t(p.nblocks) * (kQ * N * 2));
  const Buf gbuf(p.G + size_t(b) * p.nblocks * (kQ * kQ), uint32_t(p.nblocks) * (kQ * kQ * 2));
  const uint32_t xrow = uint32_t(d) * uint32_t(L);
  const uint32_t xrow0 = uint32_t(h * P + pg * 32) * uint32_t(L);  // first row of the group
  const int xvalid = P - pg * 32;          // rows of this group inside the head (16 or more)

  const float A_h = p.A[h];
  const float bias_h = p.dt_bias ? p.dt_bias[h] : 0.0f;
  const float D_d = (p.D && wave_on) ? p.D[d] : 0.0f;

  // The state slice of this wave: tile j holds states nq*kNW + 16j + 4g + i, channel r.
  f32x4 H[kNT];
  float* fs = p.final_state ? p.final_state + (size_t(b) * dim + d) * N : nullptr;
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    H[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (p.initial_state && wave_on)
      H[j] = *reinterpret_cast<const f32x4*>(fs + nq * kNW + 16 * j + 4 * g);
  }

  // Block-matrix share: row mt, columns ms0 .. ms0 + kEPT.
  const int mt = threadIdx.x / (kQ / kEPT), ms0 = (threadIdx.x % (kQ / kEPT)) * kEPT;

  // One 1 KB copy of 8 rows of 64 steps (B, x or z) into a swizzled stage: lane l fills
  // row 8 k + l / 8, slot l % 8, with step word (l % 8) ^ row_swizzle(row) of block c.
  // Rows at or past valid_rows and steps past the end read zeros.
  auto row_copy = [&](const Buf& src, uint32_t row0, int k, int c, uint4* dst, uint4& reg,
                      int valid_rows) {
    const int n = 8 * k + (l >> 3);
    const int t = c * kQ + 8 * ((l & 7) ^ row_swizzle(n));
    if constexpr (kVec) {
      const uint32_t off =
          (t < L && n < valid_rows) ? 2u * (row0 + uint32_t(n) * uint32_t(L) + uint32_t(t)) : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src.r, (lds_void_t*)&dst[k * 64], 16, off, 0, 0, 0);
    } else {
      reg = load8<false>(src, row0 + uint32_t(n) * uint32_t(L), t, n < valid_rows ? L : 0);
    }
  };
  // A 1 KB linear copy from the workspace (C^T or G of block c).
  auto lin_copy = [&](const Buf& src, uint32_t block_bytes, int k, int c, uint4* dst) {
    const uint32_t off = c < p.nblocks
                             ? uint32_t(c) * block_bytes + uint32_t(k) * 1024u + uint32_t(l) * 16u
                             : kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.r, (lds_void_t*)&dst[k * 64], 16, off, 0, 0, 0);
  };
  // The next block's copies, in three groups spread over the block.
  auto issue_b = [&](auto tag, int c, LL& ld) {
    uint4* sBs = decltype(tag)::value == 0 ? sB0 : sB1;
#pragma unroll
    for (int k = 0; k < kBInstr; ++k) row_copy(bbuf, 0u, w * kBInstr + k, c, sBs, ld.bst[k], N);
  };
  auto issue_ct_g = [&](auto tag, int c) {
    uint4* sCTs = decltype(tag)::value == 0 ? sCT0 : sCT1;
#pragma unroll
    for (int k = 0; k < kBInstr; ++k) lin_copy(ctbuf, kQ * N * 2, w * kBInstr + k, c, sCTs);
    if constexpr (kStageAll) {
      uint4* sGs = decltype(tag)::value == 0 ? sG0 : sG1;
#pragma unroll
      for (int k = 0; k < kGInstr; ++k) lin_copy(gbuf, kQ * kQ * 2, w * kGInstr + k, c, sGs);
    }
  };
  auto issue_xz = [&](auto tag, int c, LL& ld) {
    if constexpr (kStageAll) {
      uint4* sXZs = decltype(tag)::value == 0 ? sXZ0 : sXZ1;
      const int zvalid = p.z ? xvalid : 0;
      if constexpr (kWaves == 8) {  // waves 0..3 copy x, waves 4..7 copy z (no branch)
        const bool is_z = w >= 4;
        row_copy(is_z ? zbuf : xbuf, xrow0, w & 3, c, sXZs + (is_z ? kXW : 0), ld.xst[0],
                 is_z ? zvalid : xvalid);
      } else {  // every wave copies a quarter of both
        row_copy(xbuf, xrow0, w, c, sXZs, ld.xst[0], xvalid);
        row_copy(zbuf, xrow0, w, c, sXZs + kXW, ld.xst[1], zvalid);
      }
    }
  };
  auto lane_issue = [&](int c, LL& ld) {
    const int t0 = c * kQ;
    ld.dt = __builtin_amdgcn_raw_buffer_load_b16(dtbuf.r, t0 + l < L ? 2u * uint32_t(t0 + l) : kOob,
                                                 0, 0);
    ld.live = __builtin_amdgcn_raw_buffer_load_b8(mbuf.r, t0 + l < L ? uint32_t(t0 + l) : kOob, 0,
                                                  0);  // reads 0 without a mask
    if constexpr (!kStageAll) {
      const uint32_t grow = 2u * (uint32_t(c) * (kQ * kQ) + uint32_t(mt) * kQ);
#pragma unroll
      for (int q = 0; q < kEPT / 8; ++q)
        ld.g[q] = gbuf.load16(c < p.nblocks
                                  ? grow + 16u * uint32_t((ms0 / 8 + q) ^ row_swizzle(mt))
                                  : kOob);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) ld.xo[kb] = load8<kVec>(xbuf, xrow, t0 + 32 * kb + 8 * g, L);
      const int tz = p.z ? L : 0;
#pragma unroll
      for (int k = 0; k < kOwn; ++k) {
        const int te = t0 + 16 * (nq + kNS * k) + 4 * g;
        ld.xe[k] = load4<kVec>(xbuf, xrow, te, L);
        ld.ze[k] = load4<kVec>(zbuf, xrow, te, tz);
      }
    }
  };

  auto block = [&](auto tag, int c, LL& cur, LL& nxt) {
    constexpr int buf = decltype(tag)::value;  // == c & 1
    using Next = std::integral_constant<int, buf ^ 1>;
    const uint4* sBb = buf == 0 ? sB0 : sB1;
    const uint4* sCTb = buf == 0 ? sCT0 : sCT1;
    const uint4* sGb = buf == 0 ? sG0 : sG1;
    const uint4* sXb = buf == 0 ? sXZ0 : sXZ1;
    const uint4* sZb = sXb + kXW;
    const int t0 = c * kQ;
    // This block's copies (issued during the previous block, before that block's output
    // stores) have landed; the barrier below publishes the stages to all waves. Vector
    // memory operations complete in issue order, so it suffices to leave the previous
    // block's output stores outstanding: waiting for them would expose their write
    // latency once per block.
    constexpr int kStores = kOwn * (kVec ? 1 : 4);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kStores) : "memory");
    if constexpr (!kVec) {
      uint4* sBw = buf == 0 ? sB0 : sB1;
#pragma unroll
      for (int k = 0; k < kBInstr; ++k) sBw[(w * kBInstr + k) * 64 + l] = cur.bst[k];
      if constexpr (kStageAll) {
        uint4* sXZw = buf == 0 ? sXZ0 : sXZ1;
        if constexpr (kWaves == 8) {
          sXZw[(w >= 4 ? kXW : 0) + (w & 3) * 64 + l] = cur.xst[0];
        } else {
          sXZw[w * 64 + l] = cur.xst[0];
          sXZw[kXW + w * 64 + l] = cur.xst[1];
        }
      }
    }

    // Step sizes of the block, one per lane; every wave computes them, wave 0 publishes.
    float s = __uint_as_float(uint32_t(cur.dt) << 16) + bias_h;
    s = p.softplus ? softplus_f(s) : s;
    const bool live = p.mask == nullptr || cur.live != 0;
    s = (t0 + l < L && live) ? s : 0.0f;  // past the end and padding: identity
    const float cs = wave_prefix_sum(s * A_h);
    const float cs_end = readlane(cs, 63);
    if (w == 0) {
      s_dt[buf][l] = s;
      s_cs[buf][l] = cs;
      s_wdt[buf][l] = exp2_hw((cs_end - cs) * kLog2e) * s;
    }
    __syncthreads();

    // Prefetch, first group. Unconditional (past the last block the offsets read zeros),
    // so the compiler can count outstanding loads exactly and never waits for it here.
    issue_b(Next(), c + 1, nxt);
    lane_issue(c + 1, nxt);

    // Carried state: C^T H_in over this wave's states, for all 4 step tiles. H enters as
    // two bf16 halves (hi + lo): a single bf16 rounding of the state costs up to 2% of the
    // output where the state dominates it.
    uint4 hb[kKB], hl[kKB];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      uint32_t whi[4], wlo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4& a = H[2 * kb + (q >> 1)];
        const float v0 = a[2 * (q & 1)], v1 = a[2 * (q & 1) + 1];
        whi[q] = pack_bf16x2(v0, v1);
        wlo[q] = pack_bf16x2(v0 - bf16_lo(whi[q]), v1 - bf16_hi(whi[q]));
      }
      hb[kb] = make_uint4(whi[0], whi[1], whi[2], whi[3]);
      hl[kb] = make_uint4(wlo[0], wlo[1], wlo[2], wlo[3]);
    }
    f32x4 Y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Y[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const int t = 16 * i + r;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        const int slot = (nq * kNW / 8 + 4 * kb + g) ^ ct_swizzle<N>(t);
        const uint4 a = sCTb[t * kRowWords + slot];
        Y[i] = mfma16(a, hb[kb], Y[i]);
        Y[i] = mfma16(a, hl[kb], Y[i]);
      }
    }

    // Prefetch, second group.
    issue_ct_g(Next(), c + 1);

    // Block matrix M[t][s] = G[t][s] exp(cs_t - cs_s) dt_s for s <= t (bf16, LDS).
    {
      const float cst = s_cs[buf][mt];
      uint4 gw[kEPT / 8];
#pragma unroll
      for (int q = 0; q < kEPT / 8; ++q) {
        if constexpr (kStageAll)
          gw[q] = sGb[mt * 8 + ((ms0 / 8 + q) ^ row_swizzle(mt))];
        else
          gw[q] = cur.g[q];
      }
      float m[kEPT];
#pragma unroll
      for (int q = 0; q < kEPT / 4; ++q) {
        const f32x4 csq = *reinterpret_cast<const f32x4*>(&s_cs[buf][ms0 + 4 * q]);
        const f32x4 dtq = *reinterpret_cast<const f32x4*>(&s_dt[buf][ms0 + 4 * q]);
        const uint4 gg = gw[q >> 1];
        const uint32_t g01 = (q & 1) ? gg.z : gg.x, g23 = (q & 1) ? gg.w : gg.y;
        const float gq[4] = {bf16_lo(g01), bf16_hi(g01), bf16_lo(g23), bf16_hi(g23)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = gq[e] * exp2_hw((cst - csq[e]) * kLog2e) * dtq[e];
          m[4 * q + e] = ms0 + 4 * q + e <= mt ? v : 0.0f;
        }
      }
#pragma unroll
      for (int q = 0; q < kEPT / 8; ++q)
        *reinterpret_cast<uint4*>(&sM[mt][ms0 + 8 * q]) =
            make_uint4(pack_bf16x2(m[8 * q], m[8 * q + 1]), pack_bf16x2(m[8 * q + 2], m[8 * q + 3]),
                       pack_bf16x2(m[8 * q + 4], m[8 * q + 5]),
                       pack_bf16x2(m[8 * q + 6], m[8 * q + 7]));
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) sY[w][i][l] = Y[i];
    // A bare barrier: the block matrix and the partial products are LDS writes; a fence
    // here would also wait for the next block's copies just issued.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // Prefetch, third group: ahead of this block's output stores, so that the wait at the
    // next block's start can leave exactly those stores outstanding.
    issue_xz(Next(), c + 1, nxt);

    // x operands of this wave's channels (steps 32kb + 8g .. +7), and x scaled per step by
    // w_s = exp(cs_end - cs_s) dt_s, split hi + lo.
    uint4 xo[2], xh[2], xl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (kStageAll)
        xo[kb] = sXb[xr * 8 + ((4 * kb + g) ^ row_swizzle(xr))];
      else
        xo[kb] = cur.xo[kb];
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&s_wdt[buf][32 * kb + 8 * g]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&s_wdt[buf][32 * kb + 8 * g + 4]);
      const uint4 xw = xo[kb];
      const float xv[8] = {bf16_lo(xw.x) * w0[0], bf16_hi(xw.x) * w0[1],
                           bf16_lo(xw.y) * w0[2], bf16_hi(xw.y) * w0[3],
                           bf16_lo(xw.z) * w1[0], bf16_hi(xw.z) * w1[1],
                           bf16_lo(xw.w) * w1[2], bf16_hi(xw.w) * w1[3]};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hi[q] = pack_bf16x2(xv[2 * q], xv[2 * q + 1]);
        lo[q] = pack_bf16x2(xv[2 * q] - bf16_lo(hi[q]), xv[2 * q + 1] - bf16_hi(hi[q]));
      }
      xh[kb] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      xl[kb] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }

#pragma unroll
    for (int k = 0; k < kOwn; ++k) {
      const int i = nq + kNS * k;  // this wave's output tile
      f32x4 Yo = sY[pb][i][l];
#pragma unroll
      for (int q = 1; q < kNS; ++q) Yo += sY[pb + 2 * q][i][l];
      // exp(cs_t) on the carried part, then the block-diagonal product on top. Both 32-step
      // halves, also for tiles 0 and 1 whose second half of M is zero: a branch here would
      // cost more than the product (the compiler then also waits for the DMA in flight
      // before the LDS read inside it).
      const f32x4 csr = *reinterpret_cast<const f32x4*>(&s_cs[buf][16 * i + 4 * g]);
#pragma unroll
      for (int q = 0; q < 4; ++q) Yo[q] *= exp2_hw(csr[q] * kLog2e);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint4 a = *reinterpret_cast<const uint4*>(&sM[16 * i + r][32 * kb + 8 * g]);
        Yo = mfma16(a, xo[kb], Yo);
      }
      // D skip, gate, store: rows t0 + 16 i + 4 g .. +3 of channel d.
      uint2 xe, ze;
      if constexpr (kStageAll) {
        const int slot = (2 * i + (g >> 1)) ^ row_swizzle(xr);
        xe = reinterpret_cast<const uint2*>(&sXb[xr * 8 + slot])[g & 1];
        ze = reinterpret_cast<const uint2*>(&sZb[xr * 8 + slot])[g & 1];
      } else {
        xe = cur.xe[k];
        ze = cur.ze[k];
      }
      const float xv[4] = {bf16_lo(xe.x), bf16_hi(xe.x), bf16_lo(xe.y), bf16_hi(xe.y)};
      const float zv[4] = {bf16_lo(ze.x), bf16_hi(ze.x), bf16_lo(ze.y), bf16_hi(ze.y)};
      float y[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        y[q] = Yo[q] + D_d * xv[q];
        if (p.z) y[q] = gate_f(y[q], zv[q]);
      }
      store4<kVec>(obuf, xrow, t0 + 16 * i + 4 * g, L, wave_on, y);
    }

    // State: H <- exp(cs_end) H + B (w o x).
    {
      const float dec = exp2_hw(cs_end * kLog2e);
#pragma unroll
      for (int j = 0; j < kNT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) H[j][q] *= dec;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int n = nq * kNW + 16 * j + r;
        const uint4 a = sBb[n * 8 + ((4 * kb + g) ^ row_swizzle(n))];
        H[j] = mfma16(a, xh[kb], H[j]);
        H[j] = mfma16(a, xl[kb], H[j]);
      }
    }
  };

  LL la, lb;
  issue_b(std::integral_constant<int, 0>(), 0, la);
  lane_issue(0, la);
  issue_ct_g(std::integral_constant<int, 0>(), 0);
  issue_xz(std::integral_constant<int, 0>(), 0, la);
  for (int c = 0; c < p.nblocks; c += 2) {
    block(std::integral_constant<int, 0>(), c, la, lb);
    if (c + 1 < p.nblocks) block(std::integral_constant<int, 1>(), c + 1, lb, la);
  }

  if (fs && wave_on) {
#pragma unroll
    for (int j = 0; j < kNT; ++j)
      *reinterpret_cast<f32x4*>(fs + nq * kNW + 16 * j + 4 * g) = H[j];
  }
}

// ---------------------------------------------------------------- the block scan, one barrier

// Up to 128 states. Wave layout as above: 2 channel blocks of 16 x kNS state splits of 32
// states; a wave keeps its 32 x 16 slice of H as MFMA accumulators. At the end of every
// block each wave writes its slice, split hi + lo in the operand order of the carried-state
// product, to LDS; the barrier at the next block's start publishes it with the staged B,
// C^T, G, x and z of that block, and every wave then forms its own output tiles over all
// the states. One barrier per block, and no reduction of partial outputs between waves.
template <int N>
struct ChunkLayout {
  static constexpr int kNS = N == 128 ? 4 : 2;   // state splits of 32
  static constexpr int kWaves = 2 * kNS;
  static constexpr int kKB = N / 32;              // 32-state k-blocks of the whole state
  static constexpr int kOwn = 4 / kNS;            // 16-step output tiles per wave
  static constexpr int kBInstr = N / 8 / kWaves;  // 1 KB copies of B (and of C^T) per wave
  static constexpr int kGInstr = 8 / kWaves;      // of G
  static constexpr int kXZInstr = 8 / kWaves;     // of x and z (4 copies each)
};

template <int N, bool kVec>
struct ChunkLoads {
  using CL = ChunkLayout<N>;
  float4 w[4];            // w_s, s = 32 kb + 8 g + 4 k .. + 3  (index 2 kb + k)
  float4 e[CL::kOwn];     // e_t at this lane's output rows
  float cse;              // cs_end of the block
  // Element-wise path: B and x/z words for the stages. The vector path copies straight to
  // LDS and never touches these (the compiler drops them), but the copy routine still takes
  // a reference to the slot, so they are sized for its largest index on both paths.
  uint4 bst[CL::kBInstr];
  uint4 xst[CL::kXZInstr];
};

template <int N, bool kVec>
__global__ __launch_bounds__(128 * ChunkLayout<N>::kNS) void ssd_chunk_kernel(SsdParams p) {
  using CL = ChunkLayout<N>;
  using LL = ChunkLoads<N, kVec>;
  constexpr int kNS = CL::kNS, kWaves = CL::kWaves, kKB = CL::kKB, kOwn = CL::kOwn;
  constexpr int kBInstr = CL::kBInstr, kGInstr = CL::kGInstr, kXZInstr = CL::kXZInstr;
  constexpr int kRowWords = N / 8;                 // 16-byte words per C^T row
  constexpr int kXW = 32 * 8;                      // words of the x (or z) stage
  constexpr int kStores = kOwn * (kVec ? 1 : 4);
  static_assert(kBInstr >= 1 && kGInstr >= 1 && kXZInstr >= 1, "unsupported split");
  // LDS: two stages, each array of each stage its own variable (see ssd_fwd_kernel).
  __shared__ __attribute__((aligned(16))) uint4 sB0[N * 8], sB1[N * 8];
  __shared__ __attribute__((aligned(16))) uint4 sCT0[kQ * kRowWords], sCT1[kQ * kRowWords];
  __shared__ __attribute__((aligned(16))) uint4 sG0[kQ * 8], sG1[kQ * 8];
  __shared__ __attribute__((aligned(16))) uint4 sXZ0[2 * kXW], sXZ1[2 * kXW];
  __shared__ __attribute__((aligned(16))) uint4 sH0[2][kNS][2][64], sH1[2][kNS][2][64];
  // At 128 states each wave copies its block's 1 KB step record by DMA into a slot of its own
  // (dynamic LDS, kWaves KB) instead of six per-lane loads: the per-lane loads repeat each
  // address across lanes and crowd the vector memory path right after the barrier. At 64
  // states the stages alone are 80 KB, the most that lets two workgroups share a CU.
  constexpr bool kStepDma = N == 128;
  extern __shared__ __attribute__((aligned(16))) uint4 sStepDyn[];  // [kWaves][64]

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
  const int pb = w & 1, nq = w >> 1;       // channel block, state split
  const int pgroups = (p.headdim + 31) / 32;
  const int logical = xcd_order(blockIdx.x, gridDim.x);
  const int pg = logical % pgroups, h = (logical / pgroups) % p.nheads;
  const int b = logical / (pgroups * p.nheads);
  const int P = p.headdim, L = p.seqlen, dim = p.nheads * P;
  const int p0 = pg * 32 + pb * 16;
  const bool wave_on = p0 < P;
  const int d = h * P + p0 + r;
  const int xr = pb * 16 + r;

  const uint32_t row_bytes = uint32_t(dim) * uint32_t(L) * 2u;
  const Buf xbuf(p.x + size_t(b) * dim * L, row_bytes);
  const Buf zbuf(p.z ? p.z + size_t(b) * dim * L : p.x, p.z ? row_bytes : 0u);
  const Buf obuf(p.out + size_t(b) * dim * L, row_bytes);
  const Buf bbuf(p.B + size_t(b) * N * L, uint32_t(N) * uint32_t(L) * 2u);
  const Buf ctbuf(p.CTp + size_t(b) * p.nblocks * (kQ * N), uint32_t(p.nblocks) * (kQ * N * 2));
  const Buf gbuf(p.G + size_t(b) * p.nblocks * (kQ * kQ), uint32_t(p.nblocks) * (kQ * kQ * 2));
  const Buf sbuf(p.steps + (size_t(b) * p.nheads + h) * p.nblocks * (4 * kQ),
                 uint32_t(p.nblocks) * (4 * kQ * 4));
  const uint32_t xrow = uint32_t(d) * uint32_t(L);
  const uint32_t xrow0 = uint32_t(h * P + pg * 32) * uint32_t(L);
  const int xvalid = P - pg * 32;
  const float D_d = (p.D && wave_on) ? p.D[d] : 0.0f;

  // This wave's slice of H: tile j holds states 32 nq + 16 j + 4 g + i of channel r.
  f32x4 H[2];
  float* fs = p.final_state ? p.final_state + (size_t(b) * dim + d) * N : nullptr;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    H[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (p.initial_state && wave_on)
      H[j] = *reinterpret_cast<const f32x4*>(fs + 32 * nq + 16 * j + 4 * g);
  }
  // H as the B operand of the carried-state product, in two bf16 halves: lane (r, g) holds
  // k = 8 g .. 8 g + 7 of this wave's 32-state block = states {4g..4g+3, 16+4g..16+4g+3}.
  auto write_slice = [&](auto tag) {
    auto& sH = decltype(tag)::value == 0 ? sH0 : sH1;
    uint32_t whi[4], wlo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4& a = H[q >> 1];
      const float v0 = a[2 * (q & 1)], v1 = a[2 * (q & 1) + 1];
      whi[q] = pack_bf16x2(v0, v1);
      wlo[q] = pack_bf16x2(v0 - bf16_lo(whi[q]), v1 - bf16_hi(whi[q]));
    }
    sH[pb][nq][0][l] = make_uint4(whi[0], whi[1], whi[2], whi[3]);
    sH[pb][nq][1][l] = make_uint4(wlo[0], wlo[1], wlo[2], wlo[3]);
  };

  auto row_copy = [&](const Buf& src, uint32_t row0, int k, int c, uint4* dst, uint4& reg,
                      int valid_rows) {
    const int n = 8 * k + (l >> 3);
    const int t = c * kQ + 8 * ((l & 7) ^ row_swizzle(n));
    if constexpr (kVec) {
      const uint32_t off =
          (t < L && n < valid_rows) ? 2u * (row0 + uint32_t(n) * uint32_t(L) + uint32_t(t)) : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src.r, (lds_void_t*)&dst[k * 64], 16, off, 0, 0, 0);
    } else {
      reg = load8<false>(src, row0 + uint32_t(n) * uint32_t(L), t, n < valid_rows ? L : 0);
    }
  };
  auto lin_copy = [&](const Buf& src, uint32_t block_bytes, int k, int c, uint4* dst) {
    const uint32_t off = c < p.nblocks
                             ? uint32_t(c) * block_bytes + uint32_t(k) * 1024u + uint32_t(l) * 16u
                             : kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.r, (lds_void_t*)&dst[k * 64], 16, off, 0, 0, 0);
  };
  // Every copy of block c into stage `tag`, and this lane's step factors of block c.
  auto issue = [&](auto tag, int c, LL& ld) {
    constexpr int st = decltype(tag)::value;
    uint4* sBs = st == 0 ? sB0 : sB1;
    uint4* sCTs = st == 0 ? sCT0 : sCT1;
    uint4* sGs = st == 0 ? sG0 : sG1;
    uint4* sXZs = st == 0 ? sXZ0 : sXZ1;
#pragma unroll
    for (int k = 0; k < kBInstr; ++k) row_copy(bbuf, 0u, w * kBInstr + k, c, sBs, ld.bst[k], N);
#pragma unroll
    for (int k = 0; k < kBInstr; ++k) lin_copy(ctbuf, kQ * N * 2, w * kBInstr + k, c, sCTs);
#pragma unroll
    for (int k = 0; k < kGInstr; ++k) lin_copy(gbuf, kQ * kQ * 2, w * kGInstr + k, c, sGs);
    const int zvalid = p.z ? xvalid : 0;
    if constexpr (kWaves == 8) {  // waves 0..3 copy x, waves 4..7 copy z (no branch)
      const bool is_z = w >= 4;
      row_copy(is_z ? zbuf : xbuf, xrow0, w & 3, c, sXZs + (is_z ? kXW : 0), ld.xst[0],
               is_z ? zvalid : xvalid);
    } else {                      // every wave copies a quarter of both
      row_copy(xbuf, xrow0, w, c, sXZs, ld.xst[0], xvalid);
      row_copy(zbuf, xrow0, w, c, sXZs + kXW, ld.xst[kXZInstr - 1], zvalid);
    }
    if constexpr (kStepDma) {
      const uint32_t off = c < p.nblocks ? uint32_t(c) * (4 * kQ * 4) + uint32_t(l) * 16u : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sbuf.r, (lds_void_t*)&sStepDyn[w * 64], 16, off, 0,
                                               0, 0);
    } else {
      const uint32_t rb = c < p.nblocks ? uint32_t(c) * (4 * kQ * 4) : kOob;
      const bool ok = c < p.nblocks;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        ld.w[q] = ld_f4(sbuf, ok ? rb + 4u * uint32_t(32 * (q >> 1) + 8 * g + 4 * (q & 1)) : kOob);
#pragma unroll
      for (int k = 0; k < kOwn; ++k)
        ld.e[k] = ld_f4(sbuf, ok ? rb + 4u * uint32_t(kQ + 16 * (nq + kNS * k) + 4 * g) : kOob);
      ld.cse = ld_f1(sbuf, ok ? rb + 4u * uint32_t(2 * kQ + kQ - 1) : kOob);
    }
  };

  auto block = [&](auto tag, int c, LL& cur, LL& nxt) {
    constexpr int bb = decltype(tag)::value;  // == c & 1
    using Next = std::integral_constant<int, bb ^ 1>;
    const uint4* sBb = bb == 0 ? sB0 : sB1;
    const uint4* sCTb = bb == 0 ? sCT0 : sCT1;
    const uint4* sGb = bb == 0 ? sG0 : sG1;
    const uint4* sXb = bb == 0 ? sXZ0 : sXZ1;
    const uint4* sZb = sXb + kXW;
    const auto& sHb = bb == 0 ? sH0 : sH1;
    const int t0 = c * kQ;
    // This block's copies have landed (the previous block's output stores may still be in
    // flight: vector memory operations complete in issue order), then one barrier
    // publishes them and the H slices written at the previous block's end.
    // The builtin, unlike an asm wait, is seen by the compiler's own wait insertion, which
    // then knows these copies have landed. Operand: vmcnt = kStores in bits 3:0 (its high
    // bits 15:14 zero); expcnt (6:4) and lgkmcnt (11:8) at their maxima, i.e. not waited on.
    static_assert(kStores < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0xF70 | kStores);
    asm volatile("" ::: "memory");
    if constexpr (kStepDma) {
      // This wave's step record, landed with the copies above.
      static_assert(kOwn == 1, "one output tile per wave at 128 states");
      const float4* rec = reinterpret_cast<const float4*>(&sStepDyn[w * 64]);
#pragma unroll
      for (int q = 0; q < 4; ++q) cur.w[q] = rec[8 * (q >> 1) + 2 * g + (q & 1)];
      cur.e[0] = rec[(kQ + 16 * nq + 4 * g) / 4];
      cur.cse = reinterpret_cast<const float*>(rec)[2 * kQ + kQ - 1];
    }
    if constexpr (!kVec) {
      uint4* sBw = bb == 0 ? sB0 : sB1;
      uint4* sXZw = bb == 0 ? sXZ0 : sXZ1;
#pragma unroll
      for (int k = 0; k < kBInstr; ++k) sBw[(w * kBInstr + k) * 64 + l] = cur.bst[k];
      if constexpr (kWaves == 8) {
        sXZw[(w >= 4 ? kXW : 0) + (w & 3) * 64 + l] = cur.xst[0];
      } else {
        sXZw[w * 64 + l] = cur.xst[0];
        sXZw[kXW + w * 64 + l] = cur.xst[kXZInstr - 1];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // The carried-state product and the B rows of this wave's states (for the state update)
    // read this stage before the next block's copies are issued: the compiler cannot always
    // tell such a read from the LDS the copies write, and would otherwise wait for them.
    // Carried state over all N states: C^T H for this wave's output tiles.
    f32x4 Yc[kOwn];
#pragma unroll
    for (int k = 0; k < kOwn; ++k) {
      const int t = 16 * (nq + kNS * k) + r;
      Yc[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        const uint4 a = sCTb[t * kRowWords + ((4 * kb + g) ^ ct_swizzle<N>(t))];
        Yc[k] = mfma16(a, sHb[pb][kb][0][l], Yc[k]);
        Yc[k] = mfma16(a, sHb[pb][kb][1][l], Yc[k]);
      }
    }
    uint4 bop[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = 32 * nq + 16 * j + r;
        bop[kb][j] = sBb[n * 8 + ((4 * kb + g) ^ row_swizzle(n))];
      }
    asm volatile("" ::: "memory");
    issue(Next(), c + 1, nxt);

    const float cs_end = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cur.cse)));
    const bool sep = cs_end >= -kSepSpan;     // the same test as the step kernel's
    const float ref = sep ? 0.5f * cs_end : cs_end;

    // x operands of this wave's channels (steps 32 kb + 8 g .. + 7) and x scaled by w_s,
    // split hi + lo.
    uint4 xo[2], xh[2], xl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      xo[kb] = sXb[xr * 8 + ((4 * kb + g) ^ row_swizzle(xr))];
      const float4 w0 = cur.w[2 * kb], w1 = cur.w[2 * kb + 1];
      const uint4 xw = xo[kb];
      const float xv[8] = {bf16_lo(xw.x) * w0.x, bf16_hi(xw.x) * w0.y,
                           bf16_lo(xw.y) * w0.z, bf16_hi(xw.y) * w0.w,
                           bf16_lo(xw.z) * w1.x, bf16_hi(xw.z) * w1.y,
                           bf16_lo(xw.w) * w1.z, bf16_hi(xw.w) * w1.w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hi[q] = pack_bf16x2(xv[2 * q], xv[2 * q + 1]);
        lo[q] = pack_bf16x2(xv[2 * q] - bf16_lo(hi[q]), xv[2 * q + 1] - bf16_hi(hi[q]));
      }
      xh[kb] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      xl[kb] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }

    // B (w o x) for the state update. It needs only this block's operands, so it is issued
    // here, ahead of the output arithmetic, which the matrix cores then overlap.
    f32x4 T[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        T[jt] = mfma16(bop[kb][jt], xh[kb], T[jt]);
        T[jt] = mfma16(bop[kb][jt], xl[kb], T[jt]);
      }
    }

    // Outputs: separable, y = e_t (exp(ref) C^T H + (G o L) (w o x)); otherwise
    // y = e_t C^T H + M x with M[t][s] = G[t][s] exp(cs_t - cs_s) dt_s formed in registers,
    // in the operand layout (lane (r, g): row t, s = 32 kb + 8 g .. + 7).
    const float er = sep ? exp2_hw(ref * kLog2e) : 1.0f;
#pragma unroll
    for (int k = 0; k < kOwn; ++k) {
      const int i = nq + kNS * k;
      const int t = 16 * i + r;
      f32x4 Yd = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (sep) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint4 a = sGb[t * 8 + ((4 * kb + g) ^ row_swizzle(t))];
          Yd = mfma16(a, xh[kb], Yd);
          Yd = mfma16(a, xl[kb], Yd);
        }
      } else {
        const uint32_t rb = uint32_t(c) * (4 * kQ * 4);
        const float cst = ld_f1(sbuf, rb + 4u * uint32_t(2 * kQ + t));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int s0 = 32 * kb + 8 * g;
          const uint4 gw = sGb[t * 8 + ((4 * kb + g) ^ row_swizzle(t))];
          const float4 c0 = ld_f4(sbuf, rb + 4u * uint32_t(2 * kQ + s0));
          const float4 c1 = ld_f4(sbuf, rb + 4u * uint32_t(2 * kQ + s0 + 4));
          const float4 d0 = ld_f4(sbuf, rb + 4u * uint32_t(3 * kQ + s0));
          const float4 d1 = ld_f4(sbuf, rb + 4u * uint32_t(3 * kQ + s0 + 4));
          const float cs8[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
          const float dt8[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
          const uint32_t gq[4] = {gw.x, gw.y, gw.z, gw.w};
          uint32_t m[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[2];
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
              const int j = 2 * q + e2;
              const float gv = e2 ? bf16_hi(gq[q]) : bf16_lo(gq[q]);
              const float mv = gv * exp2_hw((cst - cs8[j]) * kLog2e) * dt8[j];
              v[e2] = s0 + j <= t ? mv : 0.0f;
            }
            m[q] = pack_bf16x2(v[0], v[1]);
          }
          Yd = mfma16(make_uint4(m[0], m[1], m[2], m[3]), xo[kb], Yd);
        }
      }
      // D skip, gate, store: rows t0 + 16 i + 4 g .. + 3 of channel d.
      const int slot = (2 * i + (g >> 1)) ^ row_swizzle(xr);
      const uint2 xe = reinterpret_cast<const uint2*>(&sXb[xr * 8 + slot])[g & 1];
      const uint2 ze = reinterpret_cast<const uint2*>(&sZb[xr * 8 + slot])[g & 1];
      const float xv[4] = {bf16_lo(xe.x), bf16_hi(xe.x), bf16_lo(xe.y), bf16_hi(xe.y)};
      const float zv[4] = {bf16_lo(ze.x), bf16_hi(ze.x), bf16_lo(ze.y), bf16_hi(ze.y)};
      const float ev[4] = {cur.e[k].x, cur.e[k].y, cur.e[k].z, cur.e[k].w};
      float y[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float yb = sep ? ev[q] * __builtin_fmaf(er, Yc[k][q], Yd[q])
                             : __builtin_fmaf(ev[q], Yc[k][q], Yd[q]);
        y[q] = __builtin_fmaf(D_d, xv[q], yb);
        if (p.z) y[q] = gate_f(y[q], zv[q]);
      }
      store4<kVec>(obuf, xrow, t0 + 16 * i + 4 * g, L, wave_on, y);
    }

    // State: H <- exp(cs_end) H + exp(cs_end - ref) B (w o x), with T = B (w o x) formed above.
    const float alpha = exp2_hw(cs_end * kLog2e);
    const float beta = sep ? exp2_hw((cs_end - ref) * kLog2e) : 1.0f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) H[j][q] = __builtin_fmaf(H[j][q], alpha, T[j][q] * beta);
    write_slice(Next());
  };

  LL la, lb;
  write_slice(std::integral_constant<int, 0>());
  issue(std::integral_constant<int, 0>(), 0, la);
  // The block-top wait leaves the last kStores operations in flight, which from the second
  // block on are the previous block's output stores. The first block has none behind its
  // copies: waiting for them in full here lets the compiler see, on entry to the loop, that
  // nothing but stores can be pending, so it adds no full wait of its own inside the loop.
  if constexpr (kStepDma) __builtin_amdgcn_s_waitcnt(0xF70);
  for (int c = 0; c < p.nblocks; c += 2) {
    block(std::integral_constant<int, 0>(), c, la, lb);
    if (c + 1 < p.nblocks) block(std::integral_constant<int, 1>(), c + 1, lb, la);
  }

  if (fs && wave_on) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      *reinterpret_cast<f32x4*>(fs + 32 * nq + 16 * j + 4 * g) = H[j];
  }
}

template <int N, bool kVec>
int launch_n(const SsdArgs& a, const SsdParams& p, hipStream_t s) {
  const int64_t records = a.batch * a.nheads * p.nblocks;
  const int n_prep = int(p.nblocks * a.batch);
  const dim3 pgrid = dim3(unsigned(n_prep + (records + 3) / 4));
  hipLaunchKernelGGL((ssd_prep_kernel<N, kVec>), pgrid, dim3(256), 0, s, p, n_prep, records);
  const dim3 grid = dim3(unsigned((a.headdim + 31) / 32 * a.nheads * a.batch));
  if constexpr (N <= 128) {
    constexpr int kNS = ChunkLayout<N>::kNS;
    const size_t step_lds = N == 128 ? size_t(2 * kNS) * 1024 : 0;  // one 1 KB slot per wave
    hipLaunchKernelGGL((ssd_chunk_kernel<N, kVec>), grid, dim3(128 * kNS), step_lds, s, p);
  } else {
    constexpr int kNS = StateSplit<N>::kNS;
    hipLaunchKernelGGL((ssd_fwd_kernel<N, kVec, kNS>), grid, dim3(128 * kNS), 0, s, p);
  }
  return int(hipGetLastError());
}

template <int N>
int launch_vec(const SsdArgs& a, const SsdParams& p, hipStream_t s) {
  return a.vec_ok ? launch_n<N, true>(a, p, s) : launch_n<N, false>(a, p, s);
}

}  // namespace

int launch_ssd_fwd(const SsdArgs& a, void* stream) {
  SsdParams p;
  p.x = static_cast<const uint16_t*>(a.x);
  p.dt = static_cast<const uint16_t*>(a.dt);
  p.A = a.A;
  p.B = static_cast<const uint16_t*>(a.B);
  p.C = static_cast<const uint16_t*>(a.C);
  p.D = a.D;
  p.z = static_cast<const uint16_t*>(a.z);
  p.dt_bias = a.dt_bias;
  p.mask = a.mask;
  p.out = static_cast<uint16_t*>(a.out);
  p.final_state = a.final_state;
  p.nheads = int(a.nheads);
  p.headdim = int(a.headdim);
  p.seqlen = int(a.seqlen);
  p.nblocks = int((a.seqlen + kQ - 1) / kQ);
  p.softplus = a.softplus ? 1 : 0;
  p.initial_state = a.initial_state ? 1 : 0;
  p.G = static_cast<uint16_t*>(a.workspace);
  p.CTp = p.G + size_t(a.batch) * p.nblocks * kQ * kQ;
  p.steps = reinterpret_cast<float*>(p.CTp + size_t(a.batch) * p.nblocks * kQ * a.dstate);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.dstate) {
    case 64:
      return launch_vec<64>(a, p, s);
    case 128:
      return launch_vec<128>(a, p, s);
    case 256:
      return launch_vec<256>(a, p, s);
    default:
      return int(hipErrorInvalidValue);
  }
}

}  // namespace ssm
