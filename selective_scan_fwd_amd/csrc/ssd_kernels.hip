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
// Two kernels:
//   ssd_prep_kernel, one workgroup per (batch row, 64-step block): G = C^T B of the block
//     (MFMA over the states) and C^T in the lane order the main kernel's operands use.
//     Both depend only on the batch row, so every head reuses them (from L2).
//   ssd_fwd_kernel, one workgroup per (batch row, head, 32 channels), blocks in order:
//     the decayed block matrix M = G o exp(cs_t - cs_s) o dt_s (bf16, LDS), then per wave
//     Y = exp(cs_t) C^T H_in + M x (MFMA), the D skip and gate, and
//     H_out = exp(cs_end) H_in + B (w o x) (MFMA). Wherever the fp32 state or a value
//     that feeds it is an MFMA operand (H_in in the carried-state product, w o x in the
//     update), it enters as two bf16 halves, hi + lo, which keeps fp32-level accuracy.
//
// Wave layout of ssd_fwd_kernel: 4 waves = 2 channel blocks of 16 x 2 halves of the
// states. A wave holds its (states/2 x 16) slice of H as MFMA accumulators; the two waves
// of a channel block split the carried-state product over the states and exchange partial
// outputs through LDS.
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

constexpr int kQ = kSsdBlock;          // steps per block
constexpr int kMPitch = kQ + 8;        // bf16 per row of the block matrix in LDS
constexpr uint32_t kOob = 0x80000000u;  // a byte offset past every buffer: loads read 0

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
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

typedef __attribute__((address_space(3))) void lds_void_t;

// XOR swizzle of the 16-byte words of a C^T row in the LDS stage, so that the 16 rows an
// MFMA operand read touches fall in distinct bank groups (rows of 256 B or more: 16
// distinct words; rows of 128 B: pairs of rows share a word but not a half).
template <int N>
__device__ __forceinline__ int ct_swizzle(int t) {
  return N >= 128 ? (t & 15) : ((t >> 1) & 7);
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
  float* G;          // [batch, nblocks, 64, 64]
  uint16_t* CTp;     // [batch, nblocks, 64, dstate], states in operand order
  int nheads, headdim, seqlen, nblocks;
  int softplus, initial_state;
};

// ---------------------------------------------------------------- prep: G and C^T

template <int N, bool kVec>
__global__ __launch_bounds__(256) void ssd_prep_kernel(SsdParams p) {
  constexpr int kPitch = N + 8;  // bf16 per LDS row
  __shared__ __attribute__((aligned(16))) uint16_t ct[kQ][kPitch];  // C^T of the block
  __shared__ __attribute__((aligned(16))) uint16_t bt[kQ][kPitch];  // B^T of the block
  const int c = blockIdx.x, b = blockIdx.y, L = p.seqlen, t0 = c * kQ;
  const uint32_t bc_bytes = uint32_t(N) * uint32_t(L) * 2u;
  const Buf cbuf(p.C + size_t(b) * N * L, bc_bytes), bbuf(p.B + size_t(b) * N * L, bc_bytes);

  // Transpose the block's B and C into LDS: thread -> (state n, 8 steps).
  for (int idx = threadIdx.x; idx < N * 8; idx += 256) {
    const int n = idx >> 3, q = idx & 7;
    const uint4 wc = load8<kVec>(cbuf, uint32_t(n) * L, t0 + 8 * q, L);
    const uint4 wb = load8<kVec>(bbuf, uint32_t(n) * L, t0 + 8 * q, L);
    const uint32_t vc[4] = {wc.x, wc.y, wc.z, wc.w}, vb[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ct[8 * q + 2 * k][n] = uint16_t(vc[k]);
      ct[8 * q + 2 * k + 1][n] = uint16_t(vc[k] >> 16);
      bt[8 * q + 2 * k][n] = uint16_t(vb[k]);
      bt[8 * q + 2 * k + 1][n] = uint16_t(vb[k] >> 16);
    }
  }
  __syncthreads();

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 15, g = l >> 4;
  // G[t][s] = sum_n C[n][t] B[n][s]: wave w takes rows 16w..16w+15.
  float* G = p.G + (size_t(b) * p.nblocks + c) * (kQ * kQ);
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
    for (int i = 0; i < 4; ++i) G[(16 * w + 4 * g + i) * kQ + 16 * sj + r] = acc[i];
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

// ---------------------------------------------------------------- the block scan

// Per-lane loads of one block, issued a block ahead of their use into one of two register
// sets (the block loop is unrolled by two, so the sets alternate without copies).
template <int N, bool kVec>
struct LaneLoads {
  static constexpr int kStageWords = kVec ? 1 : N / 32;  // B words staged through registers
  // dt and the mask byte stay narrow until use: widening them where they are loaded
  // would make the loop carry wait for them (and every memory operation before them).
  uint16_t dt;
  uint8_t live;
  uint4 g[4];          // G[t][s0 .. s0+15]: this thread's share of the block matrix
  uint4 xo[2];         // x operands: channel r, steps 32kb + 8g .. +7
  uint2 xe[2], ze[2];  // x and z at this lane's output positions (its two step tiles)
  uint4 bst[kStageWords];  // element-wise path: B words bound for the LDS stage
};

template <int N, bool kVec>
__global__ __launch_bounds__(256) void ssd_fwd_kernel(SsdParams p) {
  constexpr int kNH = N / 2, kNT = N / 32, kKB = N / 64;
  constexpr int kRowWords = N / 8;                 // 16-byte words per C^T row
  constexpr int kStageInstr = N / 32;              // 1 KB DMA copies per wave per array
  // LDS: two stages of B (N x 64 bf16, row = 8 words) and C^T (64 x N bf16), each stage
  // its own variable and every access to it static: the compiler then knows that reading
  // one stage does not wait for the DMA filling the other.
  __shared__ __attribute__((aligned(16))) uint4 sB0[N * 8], sB1[N * 8];
  __shared__ __attribute__((aligned(16))) uint4 sCT0[kQ * kRowWords], sCT1[kQ * kRowWords];
  __shared__ __attribute__((aligned(16))) float s_dt[2][kQ], s_cs[2][kQ], s_wdt[2][kQ];
  __shared__ __attribute__((aligned(16))) uint16_t sM[kQ][kMPitch];
  __shared__ f32x4 sY[4][2][64];

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 15, g = l >> 4;
  const int pb = w & 1, nh = w >> 1;
  const int pg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int P = p.headdim, L = p.seqlen, dim = p.nheads * P;
  const int p0 = pg * 32 + pb * 16;        // first channel (within the head) of this wave
  const bool wave_on = p0 < P;             // headdim % 32 == 16 leaves one block idle
  const int d = h * P + p0 + r;            // this lane's channel (operand column)
  // Step tiles: this wave finishes tiles nh and nh + 2 (3 causal block products each
  // way) and hands the partial carried-state product of the other two to its partner.
  const int own0 = nh, own1 = nh + 2, oth0 = 1 - nh, oth1 = 3 - nh;

  const uint32_t row_bytes = uint32_t(dim) * uint32_t(L) * 2u;
  const Buf xbuf(p.x + size_t(b) * dim * L, row_bytes);
  const Buf zbuf(p.z ? p.z + size_t(b) * dim * L : p.x, p.z ? row_bytes : 0u);
  const Buf obuf(p.out + size_t(b) * dim * L, row_bytes);
  const Buf bbuf(p.B + size_t(b) * N * L, uint32_t(N) * uint32_t(L) * 2u);
  const Buf dtbuf(p.dt + (size_t(b) * p.nheads + h) * L, uint32_t(L) * 2u);
  const Buf mbuf(p.mask ? p.mask + size_t(b) * L : nullptr, p.mask ? uint32_t(L) : 0u);
  const uint16_t* CTb = p.CTp + size_t(b) * p.nblocks * (kQ * N);
  const Buf ctbuf(CTb, uint32_t(p.nblocks) * uint32_t(kQ * N * 2));
  const uint32_t xrow = uint32_t(d) * uint32_t(L);

  const float A_h = p.A[h];
  const float bias_h = p.dt_bias ? p.dt_bias[h] : 0.0f;
  const float D_d = (p.D && wave_on) ? p.D[d] : 0.0f;

  // The state slice of this wave: tile j holds states nh*N/2 + 16j + 4g + i, channel r.
  f32x4 H[kNT];
  float* fs = p.final_state ? p.final_state + (size_t(b) * dim + d) * N : nullptr;
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    H[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (p.initial_state && wave_on)
      H[j] = *reinterpret_cast<const f32x4*>(fs + nh * kNH + 16 * j + 4 * g);
  }

  const float* Gb = p.G + size_t(b) * p.nblocks * (kQ * kQ);
  const int mt = threadIdx.x >> 2, ms0 = (threadIdx.x & 3) * 16;  // block-matrix share

  // B stage word for DMA copy k of this wave: row n = 8 (w kStageInstr + k) + l / 8, slot
  // l % 8 holding step word (l % 8) ^ ((n >> 1) & 7) of the block (zeros past the end).
  auto b_stage_offset = [&](int c, int k) -> uint32_t {
    const int n = 8 * (w * kStageInstr + k) + (l >> 3);
    const int t = c * kQ + 8 * ((l & 7) ^ ((n >> 1) & 7));
    return t < L ? 2u * (uint32_t(n) * uint32_t(L) + uint32_t(t)) : kOob;
  };
  // Copy block c's B and C^T into LDS stage c & 1 (DMA; the element-wise path gathers B
  // through registers and writes it at the start of block c).
  auto stage_issue = [&](auto tag, int c, LaneLoads<N, kVec>& ld) {
    uint4* sBs = decltype(tag)::value == 0 ? sB0 : sB1;
    uint4* sCTs = decltype(tag)::value == 0 ? sCT0 : sCT1;
    const bool in = c < p.nblocks;
#pragma unroll
    for (int k = 0; k < kStageInstr; ++k) {
      const int idx = w * kStageInstr + k;
      const uint32_t ct_off =
          in ? uint32_t(c) * uint32_t(kQ * N * 2) + uint32_t(idx) * 1024u + uint32_t(l) * 16u
             : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ctbuf.r, (lds_void_t*)&sCTs[idx * 64], 16,
                                               ct_off, 0, 0, 0);
      if constexpr (kVec) {
        const uint32_t off = b_stage_offset(c, k);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(bbuf.r, (lds_void_t*)&sBs[idx * 64], 16, off,
                                                 0, 0, 0);
      } else {
        const int n = 8 * idx + (l >> 3);
        ld.bst[k] = load8<false>(bbuf, uint32_t(n) * uint32_t(L),
                                 c * kQ + 8 * ((l & 7) ^ ((n >> 1) & 7)), L);
      }
    }
  };
  auto lane_issue = [&](int c, LaneLoads<N, kVec>& ld) {
    const int t0 = c * kQ;
    ld.dt = __builtin_amdgcn_raw_buffer_load_b16(dtbuf.r, t0 + l < L ? 2u * uint32_t(t0 + l) : kOob,
                                                 0, 0);
    ld.live = __builtin_amdgcn_raw_buffer_load_b8(mbuf.r, t0 + l < L ? uint32_t(t0 + l) : kOob, 0,
                                                  0);  // reads 0 without a mask
    const int cg = c < p.nblocks ? c : c - 1;  // past the last block: a harmless reload
    const uint4* gp = reinterpret_cast<const uint4*>(Gb + (size_t(cg) * kQ + mt) * kQ + ms0);
#pragma unroll
    for (int q = 0; q < 4; ++q) ld.g[q] = gp[q];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) ld.xo[kb] = load8<kVec>(xbuf, xrow, t0 + 32 * kb + 8 * g, L);
    ld.xe[0] = load4<kVec>(xbuf, xrow, t0 + 16 * own0 + 4 * g, L);
    ld.xe[1] = load4<kVec>(xbuf, xrow, t0 + 16 * own1 + 4 * g, L);
    const int tz = p.z ? L : 0;
    ld.ze[0] = load4<kVec>(zbuf, xrow, t0 + 16 * own0 + 4 * g, tz);
    ld.ze[1] = load4<kVec>(zbuf, xrow, t0 + 16 * own1 + 4 * g, tz);
  };

  auto block = [&](auto tag, int c, LaneLoads<N, kVec>& cur, LaneLoads<N, kVec>& nxt) {
    constexpr int buf = decltype(tag)::value;  // == c & 1
    const uint4* sBb = buf == 0 ? sB0 : sB1;
    const uint4* sCTb = buf == 0 ? sCT0 : sCT1;
    const int t0 = c * kQ;
    // This block's DMA (issued during the previous block, before that block's lane loads
    // and output stores) has landed; the barrier below publishes the stage to all waves.
    // Vector memory operations complete in issue order, so it suffices to leave the
    // previous block's output stores outstanding: waiting for them (vmcnt(0)) would expose
    // their write latency once per block.
    if constexpr (kVec)
      asm volatile("s_waitcnt vmcnt(2)" ::: "memory");  // two 8-byte stores per block
    else
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // eight 2-byte stores per block
    if constexpr (!kVec) {
#pragma unroll
      for (int k = 0; k < kStageInstr; ++k)
        (buf == 0 ? sB0 : sB1)[(w * kStageInstr + k) * 64 + l] = cur.bst[k];
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

    // Unconditional (past the last block the offsets read zeros), so the compiler can
    // count outstanding loads exactly and never waits for this prefetch inside the block.
    stage_issue(std::integral_constant<int, buf ^ 1>(), c + 1, nxt);
    lane_issue(c + 1, nxt);

    // Block matrix M[t][s] = G[t][s] exp(cs_t - cs_s) dt_s for s <= t (bf16, LDS).
    {
      const float cst = s_cs[buf][mt];
      float m[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 csq = *reinterpret_cast<const f32x4*>(&s_cs[buf][ms0 + 4 * q]);
        const f32x4 dtq = *reinterpret_cast<const f32x4*>(&s_dt[buf][ms0 + 4 * q]);
        const float gq[4] = {__uint_as_float(cur.g[q].x), __uint_as_float(cur.g[q].y),
                             __uint_as_float(cur.g[q].z), __uint_as_float(cur.g[q].w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = gq[e] * exp2_hw((cst - csq[e]) * kLog2e) * dtq[e];
          m[4 * q + e] = ms0 + 4 * q + e <= mt ? v : 0.0f;
        }
      }
      uint32_t mw[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) mw[q] = pack_bf16x2(m[2 * q], m[2 * q + 1]);
      *reinterpret_cast<uint4*>(&sM[mt][ms0]) = make_uint4(mw[0], mw[1], mw[2], mw[3]);
      *reinterpret_cast<uint4*>(&sM[mt][ms0 + 8]) = make_uint4(mw[4], mw[5], mw[6], mw[7]);
    }

    // Carried state: C^T H_in over this wave's half of the states, for all 4 step tiles
    // (own tiles first). H enters as two bf16 halves (hi + lo): a single bf16 rounding of
    // the state costs up to 2% of the output where the state dominates it.
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
    const int tiles[4] = {own0, own1, oth0, oth1};
    f32x4 Y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Y[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const int t = 16 * tiles[i] + r;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        const int slot = (nh * kNH / 8 + 4 * kb + g) ^ ct_swizzle<N>(t);
        const uint4 a = sCTb[t * kRowWords + slot];
        Y[i] = mfma16(a, hb[kb], Y[i]);
        Y[i] = mfma16(a, hl[kb], Y[i]);
      }
    }
    sY[w][0][l] = Y[2];
    sY[w][1][l] = Y[3];
    // A bare barrier: the block matrix and the partial products are LDS writes; a fence
    // here would also wait for the next block's DMA and lane loads just issued.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    f32x4 Yo[2] = {Y[0] + sY[w ^ 2][0][l], Y[1] + sY[w ^ 2][1][l]};
    // exp(cs_t) on the carried part, then the block-diagonal product on top.
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = k == 0 ? own0 : own1;
      const f32x4 csr = *reinterpret_cast<const f32x4*>(&s_cs[buf][16 * i + 4 * g]);
#pragma unroll
      for (int q = 0; q < 4; ++q) Yo[k][q] *= exp2_hw(csr[q] * kLog2e);
#pragma unroll
      for (int kb = 0; kb <= k; ++kb) {  // tile nh needs steps 0..31, tile nh + 2 all 64
        const uint4 a = *reinterpret_cast<const uint4*>(&sM[16 * i + r][32 * kb + 8 * g]);
        Yo[k] = mfma16(a, cur.xo[kb], Yo[k]);
      }
    }
    // D skip, gate, store: rows t0 + 16 i + 4 g .. +3 of channel d.
    {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int i = k == 0 ? own0 : own1;
        const float xv[4] = {bf16_lo(cur.xe[k].x), bf16_hi(cur.xe[k].x), bf16_lo(cur.xe[k].y),
                             bf16_hi(cur.xe[k].y)};
        const float zv[4] = {bf16_lo(cur.ze[k].x), bf16_hi(cur.ze[k].x), bf16_lo(cur.ze[k].y),
                             bf16_hi(cur.ze[k].y)};
        float y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          y[q] = Yo[k][q] + D_d * xv[q];
          if (p.z) y[q] = gate_f(y[q], zv[q]);
        }
        store4<kVec>(obuf, xrow, t0 + 16 * i + 4 * g, L, wave_on, y);
      }
    }

    // State: H <- exp(cs_end) H + B (wdt o x), x scaled per step and split hi + lo.
    const float dec = exp2_hw(cs_end * kLog2e);
#pragma unroll
    for (int j = 0; j < kNT; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) H[j][q] *= dec;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&s_wdt[buf][32 * kb + 8 * g]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&s_wdt[buf][32 * kb + 8 * g + 4]);
      const uint4 xw = cur.xo[kb];
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
      const uint4 xh = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      const uint4 xl = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int n = nh * kNH + 16 * j + r;
        const uint4 a = sBb[n * 8 + ((4 * kb + g) ^ ((n >> 1) & 7))];
        H[j] = mfma16(a, xh, H[j]);
        H[j] = mfma16(a, xl, H[j]);
      }
    }
  };

  LaneLoads<N, kVec> la, lb;
  stage_issue(std::integral_constant<int, 0>(), 0, la);
  lane_issue(0, la);
  for (int c = 0; c < p.nblocks; c += 2) {
    block(std::integral_constant<int, 0>(), c, la, lb);
    if (c + 1 < p.nblocks) block(std::integral_constant<int, 1>(), c + 1, lb, la);
  }

  if (fs && wave_on) {
#pragma unroll
    for (int j = 0; j < kNT; ++j)
      *reinterpret_cast<f32x4*>(fs + nh * kNH + 16 * j + 4 * g) = H[j];
  }
}

template <int N, bool kVec>
int launch_n(const SsdArgs& a, const SsdParams& p, hipStream_t s) {
  const dim3 pgrid = dim3(unsigned(p.nblocks), unsigned(a.batch));
  hipLaunchKernelGGL((ssd_prep_kernel<N, kVec>), pgrid, dim3(256), 0, s, p);
  const dim3 grid = dim3(unsigned((a.headdim + 31) / 32), unsigned(a.nheads), unsigned(a.batch));
  hipLaunchKernelGGL((ssd_fwd_kernel<N, kVec>), grid, dim3(256), 0, s, p);
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
  p.G = static_cast<float*>(a.workspace);
  p.CTp = reinterpret_cast<uint16_t*>(static_cast<char*>(a.workspace) +
                                      size_t(a.batch) * p.nblocks * kQ * kQ * sizeof(float));
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
