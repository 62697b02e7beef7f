// Selective-scan forward for gfx950 (CDNA4, wave64).
//
// What is computed (per batch row b, channel d, state n; see include/ssm_scan.h):
//   dA_t = exp(dt_t * A[d,n]), dBu_t = dt_t * B[b,n,t] * u_t, h_t = dA_t h_{t-1} + dBu_t,
//   y_t = sum_n C[b,n,t] h_t[n] + D[d] u_t, out = y_t * silu(z_t)
// (ybb.press, "Mamba state-space model: from theory to production CUDA kernel
// optimisation", sections 1.2, 2.3, 7.1; jsqmd.com, "Blelloch parallel scan as the engine
// of Mamba.py", section 3.2).
//
// How: one fused kernel. Every streamed byte is read from HBM once and written once; the
// state never leaves the chip (the fusion argument of mhpq.cn/news/1077344 section 3.2).
//
//   * A workgroup owns K channels of one batch row (one 64-lane wavefront per channel) and
//     walks the time axis in chunks of 64*T steps; lane i of a wave owns the T consecutive
//     steps [t0 + i*T, t0 + i*T + T) of its channel (the lane-holds-consecutive-steps
//     mapping of mhpq.cn/news/1057127 section 1).
//   * B and C are shared by every channel of a batch row. The workgroup stages them in LDS
//     once per chunk, already widened to fp32, a group of G states at a time, double
//     buffered: the global loads of the next group are in flight while the current group
//     is computed (the tiling / double-buffering idea of ybb.press sections 3.3 and 4.3,
//     with parameters kept on chip). The LDS layout is lane-interleaved: for a fixed state
//     and quad of steps, the 64 lanes read 64 consecutive 16-byte words (in fp32 stages
//     permuted within groups of eight, so that the stage's writes are conflict free too),
//     so each ds_read_b128 is bank-conflict free.
//   * Per state n (diagonal A: the N chains are independent, mhpq.cn/news/1057127
//     section 1):
//       1. discretise the lane's T steps: dA = exp2(dt * A*log2 e), dBu = (dt*u) * B;
//       2. fold them into the lane's segment operator (a, b): a = exp2(A*log2 e * sum dt)
//          and b = the segment's state from a zero start (lane 0 starts from the chunk's
//          carry-in instead);
//       3. inclusive wave64 Hillis-Steele scan of (a, b) under the combine
//          (a1,b1) o (a2,b2) = (a2 a1, a2 b1 + b2) (ybb.press section 3.2; mhpq.cn/news/
//          1077344 sections 2.2-2.3): six DPP steps, each one v_fmac_f32_dpp and one
//          v_mul_f32_dpp (row_shr 1, 2, 4, 8 inside 16-lane rows, then row_bcast 15 and 31);
//       4. lane i's carry-in is lane i-1's inclusive state (DPP wave_shr:1); lane 63's is
//          the carry into the next chunk (a chunked scan with a serial carry between
//          chunks, mhpq.cn/news/1077344 section 2.4; mhpq.cn/news/1057127 section 3);
//       5. replay the T steps from the carry-in, accumulating y += C h.
//   * After the last state of a chunk: D skip, silu gate, rounding to the storage type,
//     16-byte stores.
// No MFMA: nothing here is a dense contraction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "device_math.h"
#include "device_scan.h"
#include "scan_launch.h"

namespace ssm {
namespace {

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
  float* ckpt;  // nullable: states at every kCkptInterval steps, [rows, n_ckpt, dstate]
  const uint8_t* mask;  // nullable: [batch, seqlen], 0 = padding step (state kept)
  int dim, dstate, seqlen;
  int dblocks;  // ceil(dim / K)
  int softplus, initial_state;
  int n_ckpt;
};

typedef __attribute__((address_space(3))) void lds_void_t;

// Co-resident waves issue oldest first: the workgroups that share a compute unit then finish
// one after another, and the last one runs alone at low occupancy at the end of the launch.
// Giving the waves with more work left the higher priority evens out their progress instead:
// four bands by the share of the wave's state groups still to run (`left` of `total`).
__device__ __forceinline__ void set_priority_by_work_left(int left, int total) {
  const int band = (left * 4 - 1) / total;  // 3: the most left, 0: the least
  if (band >= 3) __builtin_amdgcn_s_setprio(3);
  else if (band == 2) __builtin_amdgcn_s_setprio(2);
  else if (band == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Elem: float (fp32 storage) or uint16_t (bf16 bits).
// T: steps per lane; K: channels (wavefronts) per workgroup; G: states per LDS stage.
// kVecRows: every streamed row starts 16-byte aligned and holds whole 16-byte words.
// kDmaInputs: u and delta of the next chunk travel by buffer-to-LDS DMA (no registers)
// instead of a register prefetch.
// kCkpt: also write the saved states of a training forward; kMask: read a padding mask.
// Each is a separate instantiation, so the plain forward carries neither (its register
// count decides how many waves fit on a SIMD).
// S: wavefronts per channel. With S = 2 the two waves of a channel split its states (a stage
// holds G states for each), both run the per-step work, and at the end of a chunk the second
// hands its share of y to the first through LDS; for launches with too few channels to give
// every SIMD two waves. Each wave carries, and saves, the states it scans.
template <typename Elem, int T, int K, int G, bool kVecRows, bool kDmaInputs, bool kCkpt,
          bool kMask, int S = 1, int kN = 0, bool kLate = false>
// The bf16 saved-state forms and the unrolled fixed-state form are held to four waves per
// SIMD (128 VGPRs): unbounded, the saved-state store's per-lane offset, or the unrolled
// schedule, takes them two registers past it.
__global__ __launch_bounds__(64 * K * S)
__attribute__((amdgpu_waves_per_eu(sizeof(Elem) == 2 && kVecRows && (kCkpt || kN != 0) ? 4 : 1)))
void
scan_fwd_kernel(KParams p) {
  constexpr int kVec = Vec<Elem>::kN;          // elements per 16-byte word
  constexpr int kChunk = 64 * T;               // steps per chunk
  static_assert(kChunk % kCkptInterval == 0 && kCkptInterval % T == 0,
                "saved states sit at chunk starts and at lane boundaries inside a chunk");
  constexpr int kQuads = T / 4;                // float4 LDS words per lane per state
  constexpr int kWordsPerState = kChunk / kVec;      // 16-byte words per state per chunk
  constexpr int kGS = G * S;                   // states per stage (G for each wave of a channel)
  constexpr int kArrayWords = kGS * kWordsPerState;  // words per array (B or C) per stage
  constexpr int kStageWords = 2 * kArrayWords;       // B words, then C words
  constexpr int kThreads = 64 * K * S;
  constexpr int kWordsPerLane = (kStageWords + kThreads - 1) / kThreads;
  constexpr int kBlocks = T / kVec;            // 16-byte words per lane per chunk
  constexpr uint32_t kEsz = sizeof(Elem);
  constexpr bool kBf16 = kEsz == 2;
  static_assert(T % 8 == 0, "a lane block must hold whole 16-byte bf16 words");
  static_assert(kArrayWords % 64 == 0, "each wavefront stages words of one array only");
  static_assert(!kDmaInputs || kVecRows, "input DMA moves whole aligned 16-byte words");
  static_assert(S == 1 || S == 2, "one or two waves per channel");
  static_assert(kN == 0 || (kN % (G * S) == 0 && kN <= 64), "a fixed state count: whole groups");
  // kLate: the next chunk's u and delta are loaded after the current chunk's state groups,
  // ahead of its gate and stores, rather than at its first group: the prefetch registers
  // (fp32: 32) are then live only through the chunk's tail, which leaves room for a third
  // wave per SIMD.
  static_assert(!kLate || !kDmaInputs, "late loads are register loads");

  // Staging: [buffer][B=0 / C=1][state-in-group][quad][lane] as float4 (fp32 slots).
  __shared__ float4 lds_bc[2][2][kGS * kQuads * 64];
  // Next chunk's u and delta words, per wavefront: [wave][u=0 / delta=1][word][lane].
  __shared__ uint4 lds_in[kDmaInputs ? K * S : 1][2][kBlocks][64];
  // S = 2: the second wave's share of y at the end of a chunk, [channel][quad][lane].
  __shared__ float4 lds_y[S == 2 ? K : 1][S == 2 ? kQuads : 1][64];
  // Late-load two-wave form: each wave of a channel forms the step sizes and dt u of half of
  // every lane's steps and takes the other half from its partner here:
  // [channel][dt / du][quad][lane].
  __shared__ float4 lds_steps[kLate ? K : 1][2][kLate ? kQuads : 1][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = S == 1 ? 0 : wave / K;     // which share of the states this wave scans
  const int slot = S == 1 ? wave : wave % K;  // its channel within the workgroup
  const int b = blockIdx.x / p.dblocks;
  const int d = (blockIdx.x - b * p.dblocks) * K + slot;
  const bool active = d < p.dim;  // a wave past the last channel stages, syncs, stores nothing
  const int N = kN ? kN : p.dstate, L = p.seqlen;
  const int64_t row = int64_t(b) * p.dim + (active ? d : 0);
  const uint32_t row_bytes = active ? uint32_t(L) * kEsz : 0u;

  const Buf u_buf(static_cast<const Elem*>(p.u) + row * L, row_bytes);
  const Buf dl_buf(static_cast<const Elem*>(p.delta) + row * L, row_bytes);
  const Buf z_buf(p.z ? static_cast<const Elem*>(p.z) + row * L : nullptr,
                  p.z ? row_bytes : 0u);
  const Buf out_buf(static_cast<Elem*>(p.out) + row * L, row_bytes);
  const uint32_t bc_elems = uint32_t(N) * uint32_t(L);
  const Buf B_buf(static_cast<const Elem*>(p.B) + int64_t(b) * N * L, bc_elems * kEsz);
  const Buf C_buf(static_cast<const Elem*>(p.C) + int64_t(b) * N * L, bc_elems * kEsz);

  float Dd = 0.0f, bias_d = 0.0f, a2_lane = 0.0f, hc_lane = 0.0f;
  if (active) {
    Dd = p.D ? p.D[d] : 0.0f;
    bias_d = p.bias ? p.bias[d] : 0.0f;
    // Per-state values live one per lane: lane n holds A[d,n]*log2(e) and the carry h[n].
    if (lane < N) {
      a2_lane = p.A[int64_t(d) * N + lane] * kLog2e;
      if (p.initial_state) hc_lane = p.final_state[row * N + lane];
    }
  }

  // With the state count fixed at compile time, the state loop is unrolled and each of this
  // wave's states (own state j is state own_state(j): G of every stage of kGS) keeps its
  // A log2(e) and carry in scalar registers: no readlane of either and no writelane of the
  // carry per state (the carry is read out of lane 63 straight into its register).
  constexpr int kOwnN = kN / S;
  auto own_state = [&](int j) { return (j / G) * kGS + half * G + j % G; };
  float a2_s[kN ? kOwnN : 1], hc_s[kN ? kOwnN : 1];
  if constexpr (kN != 0) {
#pragma unroll
    for (int j = 0; j < kOwnN; ++j) {
      a2_s[j] = readlane(a2_lane, own_state(j));
      hc_s[j] = readlane(hc_lane, own_state(j));
    }
  }

  const int n_groups = (N + kGS - 1) / kGS;
  const int n_chunks = (L + kChunk - 1) / kChunk;

  // fp32 stages are written one 16-byte word per thread, consecutive threads on consecutive
  // quads of one lane's steps: unswizzled, the four quads of a lane sit 1 KB apart, on the
  // same banks, and every write instruction conflicts four ways. Lane l's word of quad q goes
  // to slot l ^ 2q of the quad's row instead: a write instruction's eight lanes per LDS pass
  // then fill all 32 banks, and a read of one quad by 64 lanes stays a permutation of
  // consecutive slots within each group of eight. (bf16 stages are written as 16-bit halves
  // in another order, and keep the plain layout.)
  auto swz = [](int q, int l) { return kBf16 ? l : (l ^ (2 * q)); };

  // ---- B/C staging. Word w of a stage: array w / kArrayWords, state-in-group
  // (w % kArrayWords) / kWordsPerState, steps [s, s + kVec) with
  // s = (w % kWordsPerState) * kVec; in LDS at lane s / T, quad (s % T) / 4.
  int st_a[kWordsPerLane], st_nl[kWordsPerLane], st_s[kWordsPerLane], st_idx[kWordsPerLane];
#pragma unroll
  for (int k = 0; k < kWordsPerLane; ++k) {
    const int w = k * kThreads + tid;
    const int wa = w % kArrayWords;
    // w / kArrayWords is the same for the whole wavefront (kArrayWords % 64 == 0)
    st_a[k] = __builtin_amdgcn_readfirstlane(w / kArrayWords);
    st_nl[k] = (w < kStageWords) ? wa / kWordsPerState : kGS;  // kGS: this lane holds no word
    st_s[k] = (wa % kWordsPerState) * kVec;
    st_idx[k] = (st_nl[k] * kQuads + (st_s[k] % T) / 4) * 64 + swz((st_s[k] % T) / 4, st_s[k] / T);
  }
  uint4 raw[kWordsPerLane];
  // Stage `it` (chunk it / n_groups, group it % n_groups); past the end it reads zeros.
  auto stage_issue = [&](int it) {
    const int c = it / n_groups, g = it - c * n_groups;
#pragma unroll
    for (int k = 0; k < kWordsPerLane; ++k) {
      const int n = g * kGS + st_nl[k];
      const int t = c * kChunk + st_s[k];
      const bool ok = st_nl[k] < kGS && n < N && t < L;
      const uint32_t e = ok ? uint32_t(n) * uint32_t(L) + uint32_t(t) : bc_elems;
      raw[k] = load_word<Elem, kVecRows>(st_a[k] == 0 ? B_buf : C_buf, e);
    }
  };
  auto stage_commit = [&](int buf) {
#pragma unroll
    for (int k = 0; k < kWordsPerLane; ++k) {
      if (st_a[k] < 2 && st_nl[k] < kGS) {
        float4* base = &lds_bc[buf][0][0] + st_a[k] * (kGS * kQuads * 64) + st_idx[k];
        if constexpr (kBf16) {
          // bf16 is the top half of an fp32: store each value into the upper 16 bits of its
          // slot; the lower halves were zeroed once and are never written again.
          uint16_t* h = reinterpret_cast<uint16_t*>(base);
          const uint32_t ws[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int j0 = 2 * m, j1 = 2 * m + 1;  // steps s + j0 (low half), s + j1 (high)
            h[(j0 / 4) * 64 * 8 + (j0 % 4) * 2 + 1] = uint16_t(ws[m]);
            h[(j1 / 4) * 64 * 8 + (j1 % 4) * 2 + 1] = uint16_t(ws[m] >> 16);
          }
        } else {
          *base = __builtin_bit_cast(float4, raw[k]);
        }
      }
      // Consume the word on every path, so the load is waited for here even by lanes with
      // nothing to store, and no wait for it is left pending into the next stage.
      asm volatile("" ::"v"(raw[k].x));
    }
  };

  // ---- inputs of a chunk. With DMA, u and delta land in this wave's LDS words; z is
  // loaded into registers at the start of the chunk's last group. Past the last chunk the
  // offsets fall outside the row and read zeros.
  // In the late-load two-wave form each wave loads the u and delta of its own half of the
  // lane's steps (blocks [half kOwnBlocks, (half + 1) kOwnBlocks)); otherwise all of them.
  constexpr int kOwnBlocks = kLate ? kBlocks / 2 : kBlocks;
  static_assert(!kLate || (S == 2 && kBlocks % 2 == 0 && !kDmaInputs),
                "late loads: two waves, register loads, even halves");
  uint4 nu[kDmaInputs ? 1 : kOwnBlocks], nd[kDmaInputs ? 1 : kOwnBlocks], zraw[kBlocks];
  auto load_inputs = [&](int c) {
    const uint32_t tb = uint32_t(c) * kChunk + uint32_t(lane) * T;
    if constexpr (kDmaInputs) {
#pragma unroll
      for (int q = 0; q < kBlocks; ++q) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(u_buf.r, (lds_void_t*)&lds_in[wave][0][q][0], 16,
                                                 (tb + q * kVec) * kEsz, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(dl_buf.r, (lds_void_t*)&lds_in[wave][1][q][0], 16,
                                                 (tb + q * kVec) * kEsz, 0, 0, 0);
      }
    } else {
      const uint32_t ob = kLate ? uint32_t(half * kOwnBlocks * kVec) : 0u;  // uniform
#pragma unroll
      for (int q = 0; q < kOwnBlocks; ++q) {
        nu[q] = load_word<Elem, kVecRows>(u_buf, tb + ob + q * kVec);
        nd[q] = load_word<Elem, kVecRows>(dl_buf, tb + ob + q * kVec);
      }
    }
  };
  auto load_z = [&](int c) {
    const uint32_t tb = uint32_t(c) * kChunk + uint32_t(lane) * T;
#pragma unroll
    for (int q = 0; q < kBlocks; ++q) zraw[q] = load_word<Elem, kVecRows>(z_buf, tb + q * kVec);
  };

  float dt[T], du[T], y[T];
  float sdt = 0.0f;

  // Training forward: this row's saved states, [n_ckpt][N] fp32.
  const Buf ck_buf(kCkpt ? p.ckpt + row * int64_t(p.n_ckpt) * N : nullptr,
                   kCkpt && active ? uint32_t(p.n_ckpt) * uint32_t(N) * 4u : 0u);
  // The saved states inside a chunk are the states after steps kCkptInterval - 1,
  // 2 kCkptInterval - 1, ... of the chunk: the inclusive scan results of the lanes whose
  // segments end there (every kLanesPerCkpt-th lane, except the chunk's last, whose state
  // is the next chunk's first). Saved state k of the row sits at k * N.
  constexpr int kLanesPerCkpt = kCkptInterval / T;
  constexpr int kCkptPerChunk = kChunk / kCkptInterval;
  // Every lane stores its inclusive state at once: the lanes that hold a saved state at
  // their byte offset (set per chunk), the others far past the buffer, where the range
  // check drops the store; the state's part of the offset is uniform.
  const bool ck_lane = lane % kLanesPerCkpt == kLanesPerCkpt - 1 && lane != 63;
  uint32_t ck_lane_off = 0x80000000u;

  // One state group: the B/C words of stage `it` (chunk c) are in lds_bc[it & 1].
  auto compute_group = [&](int it, int c, int g) {
    const int buf = it & 1;
#pragma unroll
    for (int nl = 0; nl < G; ++nl) {
      const int sl = half * G + nl;  // state within the stage
      const int n = g * kGS + sl;
      if (n < N) {
        float a2, hc;
        if constexpr (kN != 0) {
          a2 = a2_s[g * G + nl];
          hc = hc_s[g * G + nl];
        } else {
          a2 = readlane(a2_lane, n);
          hc = readlane(hc_lane, n);
        }
        const float4* Bq = &lds_bc[buf][0][sl * kQuads * 64];
        const float4* Cq = &lds_bc[buf][1][sl * kQuads * 64];
        // All of this state's B words are requested at once, and its C words before the
        // wave scan, so LDS latency overlaps the exps and the scan.
        float4 bq[kQuads], cq[kQuads];
#pragma unroll
        for (int q = 0; q < kQuads; ++q) bq[q] = Bq[q * 64 + swz(q, lane)];
        float dA[T], dBu[T];
#pragma unroll
        for (int j = 0; j < T; ++j) dA[j] = exp2_hw(dt[j] * a2);
        float bseg = (lane == 0) ? hc : 0.0f;
#pragma unroll
        for (int q = 0; q < kQuads; ++q) {
          const float bb[4] = {bq[q].x, bq[q].y, bq[q].z, bq[q].w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 4 * q + r;
            dBu[j] = du[j] * bb[r];
            bseg = __builtin_fmaf(dA[j], bseg, dBu[j]);
          }
        }
#pragma unroll
        for (int q = 0; q < kQuads; ++q) cq[q] = Cq[q * 64 + swz(q, lane)];
        float aseg = exp2_hw(sdt * a2);
        wave_scan_inclusive(aseg, bseg);  // bseg: state at the end of this lane's steps
        float h = shift_up_one(bseg, hc);  // state entering this lane's steps
        if constexpr (kN != 0)  // carry into the next chunk
          hc_s[g * G + nl] = readlane(bseg, 63);
        else
          hc_lane = writelane(hc_lane, readlane(bseg, 63), n);
        if constexpr (kCkpt) {
          // (past the last saved state the offset is beyond the buffer: dropped as well)
          ck_buf.store4(__float_as_uint(bseg), ck_lane_off, uint32_t(n) * 4u);
        }
        // Replay the lane's steps from the carried-in state. The state after the last step
        // is the scan's inclusive result itself.
#pragma unroll
        for (int q = 0; q < kQuads; ++q) {
          const float cc[4] = {cq[q].x, cq[q].y, cq[q].z, cq[q].w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 4 * q + r;
            h = (j == T - 1) ? bseg : __builtin_fmaf(dA[j], h, dBu[j]);
            y[j] = __builtin_fmaf(cc[r], h, y[j]);
          }
        }
      }
    }
  };

  if constexpr (kBf16) {
    float4* flat = &lds_bc[0][0][0];
    for (int i = tid; i < 2 * 2 * kGS * kQuads * 64; i += kThreads)
      flat[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    __syncthreads();
  }
  stage_issue(0);
  load_inputs(0);
  stage_commit(0);
  __syncthreads();

  // The states whose carries (and saved states) lane `lane` of this wave holds.
  const bool own = S == 1 || (lane % kGS) / G == half;
  for (int c = 0; c < n_chunks; ++c) {
    const int tb = c * kChunk + lane * T;
    sdt = 0.0f;
    if constexpr (kCkpt && kN != 0) {  // the carries, one per lane again, for that store
#pragma unroll
      for (int j = 0; j < kOwnN; ++j) hc_lane = writelane(hc_lane, hc_s[j], own_state(j));
    }
    if (kCkpt && active && lane < N && own)  // the state entering the chunk
      ck_buf.store4(__float_as_uint(hc_lane), uint32_t(kCkptPerChunk * c * N + lane) * 4u);
    if constexpr (kCkpt)
      ck_lane_off = ck_lane ? uint32_t((kCkptPerChunk * c + lane / kLanesPerCkpt + 1) * N) * 4u
                            : 0x80000000u;
    {
      const bool tail = (c + 1) * kChunk > L;
      // Each flag is tested once per chunk, around whole loops: a test per step would be
      // turned into a select per step, paid on every chunk.
      if constexpr (!kLate) {
#pragma unroll
        for (int q = 0; q < kBlocks; ++q) {
          uint4 wu, wd;
          if constexpr (kDmaInputs) {
            wu = lds_in[wave][0][q][lane];
            wd = lds_in[wave][1][q][lane];
          } else {
            wu = nu[q];
            wd = nd[q];
          }
          float uv[kVec], dr[kVec];
          widen_raw16<Elem>(wu, uv);
          widen_raw16<Elem>(wd, dr);
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            const int j = q * kVec + e;
            dt[j] = dr[e] + bias_d;
            du[j] = uv[e];  // u for now; times the step size below
            y[j] = half == 0 ? Dd * uv[e] : 0.0f;  // the D skip once per channel
          }
        }
        if (p.softplus) {
#pragma unroll
          for (int j = 0; j < T; ++j) dt[j] = softplus_f(dt[j]);
        }
        if (tail) {  // steps past L: identity (dA = 1, dBu = 0)
#pragma unroll
          for (int j = 0; j < T; ++j) dt[j] = (tb + j < L) ? dt[j] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < T; ++j) du[j] *= dt[j];
        if constexpr (kMask) {
          // A padding step keeps the state: a zero step size makes it the identity (dA = 1,
          // dBu = 0) while y still reads the state.
          const uint8_t* m = p.mask + int64_t(b) * L;
#pragma unroll
          for (int j = 0; j < T; ++j) {
            const bool live = (tb + j < L) && m[tb + j] != 0;
            dt[j] = live ? dt[j] : 0.0f;
            du[j] = live ? du[j] : 0.0f;
          }
        }
      } else {
        // Late-load two-wave form: each wave forms the step sizes and dt u of its own half
        // of the lane's steps (lo = half T / 2 on), the same way, writes them to LDS and,
        // after a barrier, reads all T back in order. The D skip goes into the y share of
        // the wave that owns the step (the two shares are summed at the chunk's end).
        constexpr int kH = T / 2;
        const int lo = half * kH;
        const float d_first = half == 0 ? Dd : 0.0f, d_second = half == 0 ? 0.0f : Dd;
        float odt[kH], odu[kH];
#pragma unroll
        for (int q = 0; q < kOwnBlocks; ++q) {
          float uv[kVec], dr[kVec];
          widen_raw16<Elem>(nu[q], uv);
          widen_raw16<Elem>(nd[q], dr);
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            const int k = q * kVec + e;
            odt[k] = dr[e] + bias_d;
            odu[k] = uv[e];
            y[k] = d_first * uv[e];
            y[kH + k] = d_second * uv[e];
          }
        }
        if (p.softplus) {
#pragma unroll
          for (int k = 0; k < kH; ++k) odt[k] = softplus_f(odt[k]);
        }
        if (tail) {
#pragma unroll
          for (int k = 0; k < kH; ++k) odt[k] = (tb + lo + k < L) ? odt[k] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < kH; ++k) odu[k] *= odt[k];
        if constexpr (kMask) {
          const uint8_t* m = p.mask + int64_t(b) * L;
#pragma unroll
          for (int k = 0; k < kH; ++k) {
            const bool live = (tb + lo + k < L) && m[tb + lo + k] != 0;
            odt[k] = live ? odt[k] : 0.0f;
            odu[k] = live ? odu[k] : 0.0f;
          }
        }
#pragma unroll
        for (int q = 0; q < kH / 4; ++q) {
          lds_steps[slot][0][lo / 4 + q][lane] =
              make_float4(odt[4 * q], odt[4 * q + 1], odt[4 * q + 2], odt[4 * q + 3]);
          lds_steps[slot][1][lo / 4 + q][lane] =
              make_float4(odu[4 * q], odu[4 * q + 1], odu[4 * q + 2], odu[4 * q + 3]);
        }
        __syncthreads();
        const int po = kH - lo;  // the partner's first step
        float pdt[kH], pdu[kH];
#pragma unroll
        for (int q = 0; q < kH / 4; ++q) {
          const float4 a = lds_steps[slot][0][po / 4 + q][lane];
          const float4 u4 = lds_steps[slot][1][po / 4 + q][lane];
          pdt[4 * q] = a.x;
          pdt[4 * q + 1] = a.y;
          pdt[4 * q + 2] = a.z;
          pdt[4 * q + 3] = a.w;
          pdu[4 * q] = u4.x;
          pdu[4 * q + 1] = u4.y;
          pdu[4 * q + 2] = u4.z;
          pdu[4 * q + 3] = u4.w;
        }
#pragma unroll
        for (int k = 0; k < kH; ++k) {
          dt[k] = half == 0 ? odt[k] : pdt[k];
          du[k] = half == 0 ? odu[k] : pdu[k];
          dt[kH + k] = half == 0 ? pdt[k] : odt[k];
          du[kH + k] = half == 0 ? pdu[k] : odu[k];
        }
      }
#pragma unroll
      for (int j = 0; j < T; ++j) sdt += dt[j];
    }

    auto group_step = [&](int g) {
      const int it = c * n_groups + g;
      set_priority_by_work_left(n_chunks * n_groups - it, n_chunks * n_groups);
      stage_issue(it + 1);  // next stage's loads fly while this one computes
      if (g == 0) {
        // The inputs of this chunk have been read out of LDS (DMA) or consumed from
        // registers; fetch the next chunk's. Loads complete in order, so the first wait
        // that covers them is the commit of the next group.
        if constexpr (kDmaInputs) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if constexpr (!kLate) load_inputs(c + 1);
        asm volatile("" ::: "memory");  // the DMA stays ahead of the z loads below
      }
      if (g == n_groups - 1 && half == 0) load_z(c);
      if (active) compute_group(it, c, g);
      stage_commit((it + 1) & 1);
      if constexpr (kDmaInputs) {
        // A bare s_barrier: with a release fence the compiler would wait for the DMA of the
        // next chunk's u and delta at the first barrier after it is issued, exposing its
        // latency once per chunk. The DMA writes only this wave's own lds_in slot, read
        // after the chunk's last barrier, so it only has to land by then: at the last group
        // the wave waits for all its vector-memory operations (the DMA, and the z loads of
        // this group, read after the barrier anyway). Commits are LDS writes, complete
        // before every barrier.
        if (g == n_groups - 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      } else {
        __syncthreads();
      }
    };
    if constexpr (kN != 0) {
#pragma unroll
      for (int g = 0; g < (kN + kGS - 1) / kGS; ++g) group_step(g);
    } else {
      for (int g = 0; g < n_groups; ++g) group_step(g);
    }

    if constexpr (kLate) load_inputs(c + 1);
    if constexpr (S == 2) {
      // The second wave's share of y joins the first's; the first then gates and stores.
      // lds_y is written again only at the end of the next chunk, after at least one more
      // barrier, by which time the first wave has read it.
      if (half == 1) {
#pragma unroll
        for (int q = 0; q < kQuads; ++q)
          lds_y[slot][q][lane] = make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]);
      }
      __syncthreads();
      if (half == 0) {
#pragma unroll
        for (int q = 0; q < kQuads; ++q) {
          const float4 o = lds_y[slot][q][lane];
          y[4 * q] += o.x;
          y[4 * q + 1] += o.y;
          y[4 * q + 2] += o.z;
          y[4 * q + 3] += o.w;
        }
      }
    }
    if (half == 0) {  // the gate and the store: once per channel
      if (p.z) {
#pragma unroll
        for (int q = 0; q < kBlocks; ++q) {
          float zv[kVec];
          widen_raw16<Elem>(zraw[q], zv);
#pragma unroll
          for (int e = 0; e < kVec; ++e) y[q * kVec + e] = gate_f(y[q * kVec + e], zv[e]);
        }
      }
      store_lane_block<Elem, kVecRows, T>(out_buf, uint32_t(tb), y);
    }
  }

  if constexpr (kN != 0) {
#pragma unroll
    for (int j = 0; j < kOwnN; ++j) hc_lane = writelane(hc_lane, hc_s[j], own_state(j));
  }
  if (active && p.final_state && lane < N && own) p.final_state[row * N + lane] = hc_lane;
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
  // The forward kernel never uses the final a, so the routine skips the last a-update;
  // finish it here (row_bcast:31 into rows 2 and 3) so the whole a-scan is checked too.
  const float a31 = __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(1.0f), __float_as_int(av), 0x143, 0xc, 0xf, false));
  a_out[i] = av * a31;
  b_out[i] = bv;
}


// Whether an fp32 launch splits each channel's states over two waves. One wave per channel
// leaves most SIMDs with a single wave when there are few channels. A two-wave workgroup (K
// channels, 2K waves at about 192 VGPRs, two waves per SIMD) fills a compute unit, so the
// split pays only while every workgroup runs at once: past one workgroup per compute unit the
// second wave of each channel would wait for a second, partly empty round.
bool fp32_split(int64_t workgroups, int waves_per_channel) {
  if (waves_per_channel != 0) return waves_per_channel == 2;
  const int cus = device_cus();
  return cus > 0 && workgroups <= cus;
}

// fp32 channels too many for the two-wave form in four-channel workgroups to run in one round
// (more workgroups than compute units), but few enough for six-channel ones: those take the
// two-wave form with six channels per workgroup and late input loads, at most 168 VGPRs,
// i.e. one 12-wave workgroup (three waves per SIMD) per compute unit, one round. Aligned
// rows only, and not when the caller fixes the waves per channel.
bool fp32_wide_split(const FwdArgs& a) {
  if (a.waves_per_channel != 0 || !a.vec_ok) return false;
  const int cus = device_cus();
  const int64_t four = a.batch * ((a.dim + 3) / 4), six = a.batch * ((a.dim + 5) / 6);
  return cus > 0 && four > cus && six <= cus;
}

template <typename Elem, int T, int K, int G, bool kVecRows, bool kDma, bool kCkpt, bool kMask,
          int S, bool kLate>
void launch_form(dim3 grid, dim3 block, hipStream_t s, const KParams& p) {
  // 16 states on aligned rows: the form with the state count fixed (the same arithmetic, bit
  // for bit, as the general one).
  if constexpr (kVecRows) {
    if (p.dstate == 16) {
      hipLaunchKernelGGL(
          (scan_fwd_kernel<Elem, T, K, G, kVecRows, kDma, kCkpt, kMask, S, 16, kLate>), grid,
          block, 0, s, p);
      return;
    }
  }
  hipLaunchKernelGGL((scan_fwd_kernel<Elem, T, K, G, kVecRows, kDma, kCkpt, kMask, S, 0, kLate>),
                     grid, block, 0, s, p);
}

template <typename Elem, int T, int K, int G, bool kVecRows, bool kDma, bool kMask, bool kLate>
void launch_flavour(bool ckpt, bool split, dim3 grid, dim3 block, hipStream_t s,
                    const KParams& p) {
  // The training forward takes the same form as the plain one, so that both write the same
  // output bit for bit. The late-load shape exists only as the two-wave form.
  if ((sizeof(Elem) == 4 && split) || kLate) {
    if constexpr (sizeof(Elem) == 4) {
      const dim3 block2(block.x * 2);
      if (ckpt)
        launch_form<Elem, T, K, G, kVecRows, kDma, true, kMask, 2, kLate>(grid, block2, s, p);
      else
        launch_form<Elem, T, K, G, kVecRows, kDma, false, kMask, 2, kLate>(grid, block2, s, p);
    }
  } else if constexpr (!kLate) {
    if (ckpt)
      launch_form<Elem, T, K, G, kVecRows, kDma, true, kMask, 1, false>(grid, block, s, p);
    else
      launch_form<Elem, T, K, G, kVecRows, kDma, false, kMask, 1, false>(grid, block, s, p);
  }
}

template <typename Elem, int T, int K, int G, bool kDma, bool kLate = false>
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
  p.dim = int(a.dim);
  p.dstate = int(a.dstate);
  p.seqlen = int(a.seqlen);
  p.dblocks = int((a.dim + K - 1) / K);
  p.softplus = a.softplus ? 1 : 0;
  p.initial_state = a.initial_state ? 1 : 0;
  p.ckpt = a.ckpt;
  p.mask = a.mask;
  p.n_ckpt = int((a.seqlen + kCkptInterval - 1) / kCkptInterval);
  const int64_t blocks = a.batch * p.dblocks;
  const dim3 grid = dim3(unsigned(blocks)), block = dim3(64 * K);
  const bool ck = a.ckpt != nullptr;
  const bool split = sizeof(Elem) == 4 && fp32_split(blocks, a.waves_per_channel);
  if (a.vec_ok) {
    if (a.mask)
      launch_flavour<Elem, T, K, G, true, kDma, true, kLate>(ck, split, grid, block, s, p);
    else
      launch_flavour<Elem, T, K, G, true, kDma, false, kLate>(ck, split, grid, block, s, p);
  } else if constexpr (!kLate) {
    if (a.mask)
      launch_flavour<Elem, T, K, G, false, false, true, false>(ck, split, grid, block, s, p);
    else
      launch_flavour<Elem, T, K, G, false, false, false, false>(ck, split, grid, block, s, p);
  }
  return int(hipGetLastError());
}

}  // namespace

// Compute units of the current device, read once per device (declared in scan_launch.h).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Launch shapes: steps per lane, channels per workgroup, states per LDS stage.
#ifndef SSM_BF16_T
#define SSM_BF16_T 16
#endif
#ifndef SSM_BF16_K
#define SSM_BF16_K 8
#endif
#ifndef SSM_BF16_DMA
#define SSM_BF16_DMA true
#endif
#ifndef SSM_BF16_G
#define SSM_BF16_G 2
#endif
#ifndef SSM_F32_T
#define SSM_F32_T 16
#endif
#ifndef SSM_F32_K
#define SSM_F32_K 4
#endif
#ifndef SSM_F32_G
#define SSM_F32_G 2
#endif
#ifndef SSM_F32_DMA
#define SSM_F32_DMA false
#endif

int launch_scan_fwd(const FwdArgs& a, void* stream) {
  return a.seqlen <= kShortMaxSeqlen ? launch_scan_short(a, stream) : launch_scan_chunked(a, stream);
}

int launch_scan_chunked(const FwdArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.io == Io::BF16) return launch_typed<uint16_t, SSM_BF16_T, SSM_BF16_K, SSM_BF16_G, SSM_BF16_DMA>(a, s);
  if (fp32_wide_split(a)) return launch_typed<float, SSM_F32_T, 6, SSM_F32_G, false, true>(a, s);
  return launch_typed<float, SSM_F32_T, SSM_F32_K, SSM_F32_G, SSM_F32_DMA>(a, s);
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
